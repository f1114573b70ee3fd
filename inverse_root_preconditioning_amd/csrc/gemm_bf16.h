// Half-width-input batched products for gfx950 (V_MFMA_F32_32X32X16_BF16 and
// V_MFMA_F32_32X32X16_F16, fp32 accumulate) and the casts that prepare their
// operands.
//
// Every 16-bit product here is in "NT" form, C_i = A_i Bt_i^T with A and Bt
// row-major 16-bit stacks, so both operands are read along k with 16-byte
// loads.  Operands that are needed transposed are produced transposed by
// the cast kernels (or by the epilogue of the previous step).  Tiles are
// 128 x 128 per workgroup (4 waves of 64 x 64), k staged 64 at a time.
#pragma once

#include "gemm_f32.h"

namespace shp {

constexpr int kBK16 = 64;
constexpr int kLd16 = kBK16 + 8;  // LDS row stride in bf16 elements (144 bytes)

struct EpiStoreBf16 {
  static constexpr bool kSym = false;
  static constexpr bool kReduce = false;
  struct Job {
    uint16_t* out;
  };
  struct Tile {
    uint16_t* out;
    int B;
    __device__ Tile(const Job& j, int64_t item, int B_) : B(B_) { out = j.out + item * (int64_t)B_ * B_; }
    __device__ __forceinline__ float store(int row, int col, float v) {
      stg(out + (int64_t)row * B + col, f32_to_bf16_bits(v));
      return 0.f;
    }
    __device__ void partial(int, float) {}
  };
};

template <class Epi>
struct H16Launch {
  const uint16_t* a[2];
  const uint16_t* bt[2];
  typename Epi::Job e[2];
  int64_t nitems;      // items per job
  int B;
  int tiles_n;
  int tiles_per_item;
  int sym;
  uint32_t total;      // njobs * nitems * tiles_per_item
};

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

template <int FMT>
__device__ __forceinline__ floatx16 mfma_h16(const u32x4& a, const u32x4& b, const floatx16& c) {
  if constexpr (FMT == H16_F16) {
    halfx8 x, y;
    __builtin_memcpy(&x, &a, sizeof(x));
    __builtin_memcpy(&y, &b, sizeof(y));
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, c, 0, 0, 0);
  } else {
    bf16x8 x, y;
    __builtin_memcpy(&x, &a, sizeof(x));
    __builtin_memcpy(&y, &b, sizeof(y));
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
  }
}

// C_i = A_i Bt_i^T for 16-bit (bf16 or fp16) row-major stacks, fp32 accumulate.
template <class Epi, int FMT>
__global__ void __launch_bounds__(256, 2) gemm_h16_nt_kernel(const H16Launch<Epi> P) {
  constexpr int BM = 128, BN = 128, TM = 2, TN = 2;
  constexpr int kTile = BM * kLd16;  // 16-bit elements of one operand tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * kTile];

  const uint32_t lid = xcd_remap(blockIdx.x, P.total);
  const uint32_t per_job = (uint32_t)P.nitems * P.tiles_per_item;
  const int job = lid / per_job;
  const uint32_t rem = lid - job * per_job;
  const int64_t item = rem / P.tiles_per_item;
  int t = rem - (uint32_t)item * P.tiles_per_item;
  int tm, tn;
  if (!P.sym) {
    tm = t / P.tiles_n;
    tn = t - tm * P.tiles_n;
  } else {
    tm = 0;
    int rowlen = P.tiles_n;
    while (t >= rowlen) {
      t -= rowlen;
      ++tm;
      --rowlen;
    }
    tn = tm + t;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t off = item * (int64_t)P.B * P.B;
  const uint16_t* A = P.a[job] + off;
  const uint16_t* Bt = P.bt[job] + off;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int rr = lane & 31, h = lane >> 5;

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it;
      const int row = idx >> 3, ch = idx & 7;
      ra[it] = ldg(reinterpret_cast<const u32x4*>(A + (int64_t)(m0 + row) * P.B + k0 + ch * 8));
      rb[it] = ldg(reinterpret_cast<const u32x4*>(Bt + (int64_t)(n0 + row) * P.B + k0 + ch * 8));
    }
  };
  auto sstore = [&](uint16_t* buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + 256 * it;
      const int row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(buf + row * kLd16 + ch * 8) = ra[it];
      *reinterpret_cast<u32x4*>(buf + kTile + row * kLd16 + ch * 8) = rb[it];
    }
  };

  const int nstages = P.B / kBK16;
  gload(0);
  sstore(lds);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const uint16_t* cur = lds + (s & 1) * 2 * kTile;
    if (s + 1 < nstages) gload((s + 1) * kBK16);
#pragma unroll
    for (int ks = 0; ks < kBK16 / 16; ++ks) {
      u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(cur + (wm + 32 * i + rr) * kLd16 + ks * 16 + h * 8);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(cur + kTile + (wn + 32 * j + rr) * kLd16 + ks * 16 + h * 8);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_h16<FMT>(fa[i], fb[j], acc[i][j]);
    }
    if (s + 1 < nstages) sstore(lds + ((s + 1) & 1) * 2 * kTile);
    __syncthreads();
  }

  typename Epi::Tile tile(P.e[job], item, P.B);
  if constexpr (Epi::kSym) {
    static_assert(sizeof(lds) >= sizeof(float) * BM * (BN + 1), "LDS too small for the transpose");
    if (P.sym) {
      sym_epilogue<TM, TN, 1>(tile, acc, reinterpret_cast<float*>(lds), m0, n0, wm, wn, lane, tm == tn);
      return;
    }
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        const int col = n0 + wn + 32 * j + rr;
        part += tile.store(row, col, acc[i][j][e]);
      }
  if constexpr (Epi::kReduce) {
    __shared__ float red[4];
    const float tot = block_sum<256>(part, red);
    if (threadIdx.x == 0) tile.partial(tm * P.tiles_n + tn, tot);
  }
}

// ---------------------------------------------------------------------------
// fp32 -> bf16 casts over 64 x 64 tiles, optionally transposed, from a dense
// stack or through block descriptors (zero outside the block).
// ---------------------------------------------------------------------------
struct CastArgs {
  Operand src;
  uint16_t* out;    // bf16 copy (may be null)
  uint16_t* out_t;  // bf16 transposed copy (may be null)
  int B;
  int tiles;        // (B / 64)^2
};

__global__ void __launch_bounds__(256) bf16_cast_kernel(const CastArgs P) {
  __shared__ float t[64][65];
  const int64_t item = blockIdx.x / P.tiles;
  const int tt = blockIdx.x - (int)(item * P.tiles);
  const int per = P.B / 64;
  const int r0 = (tt / per) * 64, c0 = (tt % per) * 64;
  const OperandView v = operand_view(P.src, item, P.B);
  const int tid = threadIdx.x;
  const int cr = tid >> 4, cc = (tid & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + cr + 16 * i, col = c0 + cc;
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    if (row < v.rows) {
      const float* src = v.p + (int64_t)row * v.ld + col;
      if (v.vec && col + 3 < v.cols) {
        x = ldg(reinterpret_cast<const floatx4*>(src));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < v.cols) x[e] = ldg(src + e);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) t[cr + 16 * i][cc + e] = x[e];
  }
  __syncthreads();
  const int64_t base = item * (int64_t)P.B * P.B;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = cr + 16 * i;
    if (P.out) {
      u32x2 w;
      w.x = (uint32_t)f32_to_bf16_bits(t[lr][cc]) | ((uint32_t)f32_to_bf16_bits(t[lr][cc + 1]) << 16);
      w.y = (uint32_t)f32_to_bf16_bits(t[lr][cc + 2]) | ((uint32_t)f32_to_bf16_bits(t[lr][cc + 3]) << 16);
      stg(reinterpret_cast<u32x2*>(P.out + base + (int64_t)(r0 + lr) * P.B + c0 + cc), w);
    }
    if (P.out_t) {
      u32x2 w;
      w.x = (uint32_t)f32_to_bf16_bits(t[cc][lr]) | ((uint32_t)f32_to_bf16_bits(t[cc + 1][lr]) << 16);
      w.y = (uint32_t)f32_to_bf16_bits(t[cc + 2][lr]) | ((uint32_t)f32_to_bf16_bits(t[cc + 3][lr]) << 16);
      stg(reinterpret_cast<u32x2*>(P.out_t + base + (int64_t)(c0 + lr) * P.B + r0 + cc), w);
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
static inline int bf16_cast_launch(const Operand& src, uint16_t* out, uint16_t* out_t, int64_t n, int B,
                                   hipStream_t st) {
  CastArgs a;
  a.src = src;
  a.out = out;
  a.out_t = out_t;
  a.B = B;
  a.tiles = (B / 64) * (B / 64);
  const uint64_t grid = (uint64_t)n * a.tiles;
  if (grid == 0) return SHAMPOO_OK;
  if (grid > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  hipLaunchKernelGGL(bf16_cast_kernel, dim3((uint32_t)grid), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
}

// bf16 copy (transpose == false) or transposed copy of a dense fp32 stack.
static inline int bf16_cast(const float* src, uint16_t* dst, int64_t n, int B, bool transpose, hipStream_t st) {
  const Operand o{src, nullptr};
  return bf16_cast_launch(o, transpose ? nullptr : dst, transpose ? dst : nullptr, n, B, st);
}

// bf16 copies of zero-padded gradient blocks: G (g16) and/or G^T (gt16).
static inline int bf16_gather(const shampoo_block* d, int64_t n, int B, uint16_t* g16, uint16_t* gt16,
                              hipStream_t st) {
  const Operand o{nullptr, d};
  return bf16_cast_launch(o, g16, gt16, n, B, st);
}

// One launch of up to two NT products of 16-bit stacks with the same epilogue type.
template <class Epi>
static inline int h16_gemm_nt(const uint16_t* const* a, const uint16_t* const* bt, const typename Epi::Job* e,
                              int njobs, int64_t n, int B, bool sym, int fmt, hipStream_t st) {
  if (B % 128 != 0) return SHAMPOO_EUNSUPPORTED;
  H16Launch<Epi> P;
  memset(&P, 0, sizeof(P));
  for (int j = 0; j < njobs; ++j) {
    P.a[j] = a[j];
    P.bt[j] = bt[j];
    P.e[j] = e[j];
  }
  P.nitems = n;
  P.B = B;
  P.tiles_n = B / 128;
  P.tiles_per_item = sym ? P.tiles_n * (P.tiles_n + 1) / 2 : P.tiles_n * P.tiles_n;
  P.sym = sym ? 1 : 0;
  const uint64_t total = (uint64_t)njobs * n * P.tiles_per_item;
  if (total == 0) return SHAMPOO_OK;
  if (total > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  P.total = (uint32_t)total;
  if (fmt == H16_F16)
    hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_F16>), dim3(P.total), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_BF16>), dim3(P.total), dim3(256), 0, st, P);
  return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
}

template <class Epi>
static inline int bf16_gemm_nt(const uint16_t* a, const uint16_t* bt, const typename Epi::Job& e, int64_t n,
                               int B, bool sym, hipStream_t st) {
  return h16_gemm_nt<Epi>(&a, &bt, &e, 1, n, B, sym, H16_BF16, st);
}

static inline int bf16_gemm_nt_store(const uint16_t* a, const uint16_t* bt, const EpiStore::Job& e, int64_t n,
                                     int B, bool sym, hipStream_t st) {
  return bf16_gemm_nt<EpiStore>(a, bt, e, n, B, sym, st);
}

static inline int bf16_gemm_nt_clenshaw(const uint16_t* a, const uint16_t* bt, const EpiClenshaw::Job& e,
                                        int64_t n, int B, bool sym, hipStream_t st) {
  return bf16_gemm_nt<EpiClenshaw>(a, bt, e, n, B, sym, st);
}

static inline int bf16_gemm_nt_bf16out(const uint16_t* a, const uint16_t* bt, uint16_t* out, int64_t n, int B,
                                       hipStream_t st) {
  EpiStoreBf16::Job j{out};
  return bf16_gemm_nt<EpiStoreBf16>(a, bt, j, n, B, false, st);
}

static inline int bf16_gemm_nt_desc(const uint16_t* a, const uint16_t* bt, const shampoo_block* u, int64_t n,
                                    int B, hipStream_t st) {
  EpiStoreDesc::Job j{u};
  return bf16_gemm_nt<EpiStoreDesc>(a, bt, j, n, B, false, st);
}

}  // namespace shp
