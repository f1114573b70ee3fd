// Half-width-input batched products for gfx950 (V_MFMA_F32_32X32X16_BF16 and
// V_MFMA_F32_32X32X16_F16, fp32 accumulate) and the casts that prepare their
// operands.
//
// Every 16-bit product here is in "NT" form, C_i = A_i Bt_i^T with A and Bt
// row-major 16-bit stacks, so both operands are read along k with 16-byte
// loads.  Operands that are needed transposed are produced transposed by
// the cast kernels (or by the epilogue of the previous step).  Tiles are
// 256 x 256 per workgroup for full products when B % 256 == 0, else 128 x
// 128; k is staged 64 at a time.
#pragma once

#include "gemm_f32.h"

namespace shp {

constexpr int kBK16 = 64;
constexpr int kLd16 = kBK16 + 8;  // LDS row stride in bf16 elements (144 bytes)

struct EpiStoreBf16 {
  static constexpr bool kSym = false;
  static constexpr bool kReduce = false;
  static constexpr bool kBigSym = false, kBigFull = true;
  static constexpr bool kH16BigSym = false, kH16BigFull = true;
  static constexpr int kH16BigWaves = 16;
  struct Job {
    uint16_t* out;
  };
  struct Tile {
    uint16_t* out;
    int B;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : B(B_) { out = j.out + item * (int64_t)B_ * B_; }
    __device__ __forceinline__ float store(int row, int col, float v) {
      stg(out + (int64_t)row * B + col, f32_to_bf16_bits(v));
      return 0.f;
    }
    __device__ void partial(int, float) {}
  };
};

template <class Epi>
struct H16Launch {
  using EpiT = Epi;
  const uint16_t* a[2];
  const uint16_t* bt[2];
  typename Epi::Job e[2];
  int64_t nitems;      // items per job
  int B;
  int tiles_n;
  int tiles_per_item;
  uint32_t total;      // njobs * nitems * tiles_per_item
  // Operands stored only in their 256 x 256 tiles on and above the diagonal
  // (symmetric matrices; gemm_h16_big_kernel): bit 2 j (H16_UPPER_A) for A of
  // job j, bit 2 j + 1 (H16_UPPER_B) for its Bt.  Row panel I of such an
  // operand takes its k-blocks K < I from tile (K, I), transposed.
  int upper;
};

enum { H16_UPPER_A = 1, H16_UPPER_B = 2 };

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

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

// Workgroup shapes of the 16-bit product.  The LDS traffic per MFMA falls
// with the wave tile: 64 x 64 wave tiles read 1 KB of fragments per 32 x 32 x 16
// MFMA, 64 x 128 ones 0.75 KB, and the 256 x 256 workgroup tile halves the
// staging writes per MFMA as well.
//   H16_T128: 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per CU.
//   H16_T256: 256 x 256 tiles, 8 waves (4 x 2) of 64 x 128, one workgroup per
//             CU (144 KB of LDS); full products with B % 256 == 0.
enum { H16_T128 = 0, H16_T256 = 1 };

template <int CFG>
struct H16Shape {
  static constexpr int BM = CFG == H16_T256 ? 256 : 128;
  static constexpr int WR = CFG == H16_T256 ? 4 : 2;   // waves along rows
  static constexpr int WC = 2;                          // waves along columns
  static constexpr int NT = 64 * WR * WC;
  static constexpr int TM = BM / WR / 32, TN = BM / WC / 32;
  static constexpr int MINW = CFG == H16_T256 ? 1 : 2;
};

// Output tile edge of the 16-bit products: 256 x 256 tiles whenever B is a
// multiple of 256 (symmetric products too: their diagonal tiles skip the
// 32 x 32 blocks that lie below the diagonal), 128 x 128 otherwise.
__host__ __device__ constexpr int h16_tile_of(int B, bool sym) { return (B % 256 == 0) ? 256 : 128; }

// C_i = A_i Bt_i^T for 16-bit (bf16 or fp16) row-major stacks, fp32 accumulate.
// k is staged kBK16 deep through two padded LDS buffers (loads of stage s + 1
// are in registers while stage s is multiplied); the fragments of the next
// 16-deep k step are read before the MFMAs of the current one, across the
// stage boundary too.
template <class Epi, int FMT, int CFG, bool SYM>
__global__ void __launch_bounds__(H16Shape<CFG>::NT, H16Shape<CFG>::MINW)
    gemm_h16_nt_kernel(const H16Launch<Epi> P) {
  using S = H16Shape<CFG>;
  constexpr int BM = S::BM, BN = S::BM, NT = S::NT, TM = S::TM, TN = S::TN, WC = S::WC;
  constexpr int CPR = kBK16 / 8;          // 16-byte chunks per staged row
  constexpr int LA = BM * CPR / NT;       // 16-byte loads per thread per operand and stage
  constexpr int kA = BM * kLd16, kStage = 2 * kA;
  constexpr int KS = kBK16 / 16;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];

  const uint32_t lid = xcd_remap(blockIdx.x, P.total);
  const uint32_t per_job = (uint32_t)P.nitems * P.tiles_per_item;
  const int job = lid / per_job;
  const uint32_t rem = lid - job * per_job;
  const int64_t item = rem / P.tiles_per_item;
  int t = rem - (uint32_t)item * P.tiles_per_item;
  int tm, tn;
  if constexpr (!SYM) {
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
  // uniform selects, not an index into the argument arrays (which would put
  // the arguments in scratch memory)
  const uint16_t* A = (job == 0 ? P.a[0] : P.a[1]) + off;
  const uint16_t* Bt = (job == 0 ? P.bt[0] : P.bt[1]) + off;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = (wave / WC) * 32 * TM, wn = (wave % WC) * 32 * TN;
  const int rr = lane & 31, h = lane >> 5;
  // On a diagonal tile of a symmetric product a wave whose block lies wholly
  // below the diagonal holds only entries that are never written: it skips
  // its fragment reads and MFMAs but still stages operands and meets every
  // barrier.
  const bool active = !(SYM && tm == tn && wm >= wn + 32 * TN);

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 ra[LA], rb[LA];
  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int idx = tid + NT * it;
      const int row = idx / CPR, ch = idx % CPR;
      ra[it] = ldg(reinterpret_cast<const u32x4*>(A + (int64_t)(m0 + row) * P.B + k0 + ch * 8));
      rb[it] = ldg(reinterpret_cast<const u32x4*>(Bt + (int64_t)(n0 + row) * P.B + k0 + ch * 8));
    }
  };
  auto sstore = [&](uint16_t* buf) {
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int idx = tid + NT * it;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(buf + row * kLd16 + ch * 8) = ra[it];
      *reinterpret_cast<u32x4*>(buf + kA + row * kLd16 + ch * 8) = rb[it];
    }
  };
  auto frags = [&](const uint16_t* buf, int ks, u32x4(&fa)[TM], u32x4(&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = *reinterpret_cast<const u32x4*>(buf + (wm + 32 * i + rr) * kLd16 + ks * 16 + h * 8);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const u32x4*>(buf + kA + (wn + 32 * j + rr) * kLd16 + ks * 16 + h * 8);
  };

  const int nstages = P.B / kBK16;
  gload(0);
  sstore(lds);
  __syncthreads();
  u32x4 ca[TM] = {}, cb[TN] = {};
  if (active) frags(lds, 0, ca, cb);
  for (int s = 0; s < nstages; ++s) {
    const uint16_t* cur = lds + (s & 1) * kStage;
    if (s + 1 < nstages) gload((s + 1) * kBK16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 na[TM], nb[TN];  // the next k step's fragments (kept as they are when none are read)
#pragma unroll
      for (int i = 0; i < TM; ++i) na[i] = ca[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) nb[j] = cb[j];
      if (ks + 1 < KS) {
        if (active) frags(cur, ks + 1, na, nb);
      } else if (s + 1 < nstages) {
        uint16_t* nxt = lds + ((s + 1) & 1) * kStage;
        sstore(nxt);
        __syncthreads();
        if (active) frags(nxt, 0, na, nb);
      }
      if (active) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_h16<FMT>(ca[i], cb[j], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) ca[i] = na[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) cb[j] = nb[j];
    }
  }
  __syncthreads();  // the LDS is reused by the epilogue

  typename Epi::Tile tile(*(job == 0 ? &P.e[0] : &P.e[1]), item, P.B);
  float part = 0.f;
  if constexpr (CFG == H16_T256) {
    constexpr int PH = (sizeof(lds) >= sizeof(float) * BM * (BN + 1)) ? 1 : 2;
    static_assert(sizeof(lds) >= sizeof(float) * (BM / PH) * (BN + 4), "LDS too small for the staging");
    constexpr bool kDirect = [] {
      if constexpr (Epi::kSym) return Epi::kDirect && !Epi::kReduce && SYM;
      return false;
    }();
    if constexpr (kDirect)
      sym_epilogue_direct<TM, TN, 8>(tile, acc, m0, n0, wm, wn, lane, tm == tn, (1 << (TM * TN)) - 1);
    else
      part = staged_epilogue<TM, TN, BM, BN, NT, PH, Epi>(tile, acc, reinterpret_cast<float*>(lds), m0, n0, wm,
                                                          wn, lane, SYM, tm == tn);
  } else {
    if constexpr (Epi::kSym && SYM) {
      constexpr int PH = (sizeof(lds) >= sizeof(float) * BM * (BN + 1)) ? 1 : 2;
      static_assert(sizeof(lds) >= sizeof(float) * (BM / PH) * (BN + 1), "LDS too small for the transpose");
      {
        if constexpr (Epi::kDirect && !Epi::kReduce)
          sym_epilogue_direct<TM, TN, 8>(tile, acc, m0, n0, wm, wn, lane, tm == tn, (1 << (TM * TN)) - 1);
        else
          part = sym_epilogue<TM, TN, BM, BN, NT, PH, Epi::kReduce>(tile, acc, reinterpret_cast<float*>(lds), m0,
                                                                     n0, wm, wn, lane, tm == tn);
      }
    }
    if constexpr (!(Epi::kSym && SYM)) {
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
    }
  }
  if constexpr (Epi::kReduce) {
    __shared__ float red[NT / kWave];
    const float tot = block_sum<NT>(part, red);
    if (threadIdx.x == 0) {
      tile.partial(tm * P.tiles_n + tn, tot);
      if (SYM && tm != tn) tile.partial(tn * P.tiles_n + tm, tot);  // the mirrored tile
    }
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
      w.x = pack_bf16x2(t[lr][cc], t[lr][cc + 1]);
      w.y = pack_bf16x2(t[lr][cc + 2], t[lr][cc + 3]);
      stg(reinterpret_cast<u32x2*>(P.out + base + (int64_t)(r0 + lr) * P.B + c0 + cc), w);
    }
    if (P.out_t) {
      u32x2 w;
      w.x = pack_bf16x2(t[cc][lr], t[cc + 1][lr]);
      w.y = pack_bf16x2(t[cc + 2][lr], t[cc + 3][lr]);
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
// ---------------------------------------------------------------------------
// 16-bit products on 256 x 256 tiles (B a multiple of 256, epilogues that fit
// 128 VGPRs): 16 waves of 64 x 64 (2 x 2 blocks of the 32 x 32 x 16 MFMA),
// one workgroup per CU.  Each thread moves two 16-byte pieces of A and two of
// Bt per 64-deep k stage straight into LDS (global_load_lds_dwordx4) into the
// other of two stage buffers while the MFMAs run on the current one; a stage
// ends with a wait for its loads and one barrier.  Rows are stored as 8
// chunks of 16 bytes with the chunk index XOR-ed by (row ^ (row >> 3)) & 7,
// so the fragment reads of 16 consecutive rows cover all 64 banks.  Waves are
// placed, and their blocks on diagonal tiles of symmetric products assigned,
// as in gemm_f32_big_kernel.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int h16_swz(int row) { return (row ^ (row >> 3)) & 7; }

// Transposed operand stages (H16Launch::upper): 64 k-rows of 256 columns, the
// 16-byte chunk index of row kr XOR-ed with h16_tswz(kr), so that the
// column-wise fragment reads of 4 rows (ds_read_b64_tr_b16) fall on 4
// different quarters of the 64 banks.
__device__ __forceinline__ int h16_tswz(int kr) { return 4 * (kr & 3); }

// Epilogues whose large-tile kernel is built with the transposed stages, so
// that its operands may be kept on and above the diagonal only
// (H16Launch::upper).
template <class T, class = void>
struct has_upper_operands : std::false_type {};
template <class T>
struct has_upper_operands<T, std::void_t<decltype(T::kH16Upper)>> : std::integral_constant<bool, T::kH16Upper> {};

// 8 waves of 64 x 128 on a 256 x 256 tile: wave w takes block row r (64
// rows) and column half c (128 columns) from a fixed placement.  On a
// diagonal tile of a symmetric product a wave computes only its 32 x 32
// blocks (bit 4 i + j for block row i, column j) on or above the diagonal,
// and waves 4 and 5, whose placements lie wholly below it, each take one
// block from waves 2 and 3 (at their placements), so that the two waves of
// every SIMD (w and w + 4 share one) compute 9 of the tile's 36 upper blocks.
// Off-diagonal tiles: every wave computes its whole 64 x 128 block.
constexpr uint32_t kH16Place8 = 0x27645031u;  // 4 bits 2 r + c per wave, w = 0 in the low bits
constexpr int kH16Donated = 0x80;             // block (1, 3) of waves 2 and 3, computed by waves 4 and 5
__device__ __forceinline__ void h16_wave_role8(bool dtile, int wave, int& wm, int& wn, int& mask) {
  const bool helper = dtile && (wave == 4 || wave == 5);
  const int place = (int)((kH16Place8 >> (4 * (helper ? wave - 2 : wave))) & 15);
  const int r = place >> 1, c = place & 1;
  wm = 64 * r;
  wn = 128 * c;
  mask = 0xFF;
  if (dtile) {
    mask = 0;
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 4; ++j)
        if (4 * c + j >= 2 * r + i) mask |= 1 << (4 * i + j);
    if (wave == 2 || wave == 3) mask &= ~kH16Donated;
    if (helper) mask = kH16Donated;
  }
}

// WAVES = 16: 4 x 4 waves of 64 x 64 (128 VGPRs each).  WAVES = 8: 4 x 2 waves
// of 64 x 128 (256 VGPRs each), for epilogues that want registers to load
// ahead.  On a diagonal tile of a symmetric product the 8-wave layout places
// its waves by h16_wave_role8 for the register-direct symmetric epilogue;
// for the LDS-staged one (plain 4 x 2 order) the waves wholly below the
// diagonal idle and the others compute their whole block.
template <class Epi, int FMT, bool SYM, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, 1) gemm_h16_big_kernel(const H16Launch<Epi> P) {
  static_assert(WAVES == 16 || WAVES == 8, "wave layouts");
  constexpr int TM = 2, TN = WAVES == 16 ? 2 : 4, BM = kBigTile, BN = kBigTile, BKS = 64, NT = 64 * WAVES;
  constexpr int kFull = (1 << (TM * TN)) - 1;
  constexpr int CPR = BKS / 8;                           // 16-byte chunks per staged row
  constexpr int kA = BM * BKS, kStage = (BM + BN) * BKS;  // 16-bit elements
  constexpr int LA = BM * CPR / NT;                      // chunks of A (and of Bt) per thread and stage
  constexpr int KS = BKS / 16;
  // Phases of the LDS-staged epilogue (8 waves): two of 128 rows, four waves
  // staging at a time (C^p M of fp16 coupled Newton 1.70 -> 1.65 ms per launch
  // against four phases of 64 rows), which takes 130 KB of LDS beside the
  // 128 KB of stage buffers; the 16-wave register epilogues stage per wave.
  constexpr int PH = WAVES == 8 ? 2 : 4;
  constexpr int kStageFloats = 2 * kStage / 2;           // the stage buffers, counted in floats
  constexpr int kStaged = (BM / PH) * (BN + 4) + NT / kWave;  // one phase's rows and the reduction slots
  constexpr int kFloats = kStaged > kStageFloats ? kStaged : kStageFloats;
  static_assert(LA * NT == BM * CPR && BN == BM, "chunking");
  static_assert(kFloats * 4 <= 160 * 1024, "fits the LDS");
  // One LDS object only (see gemm_f32_big_kernel).
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kFloats];
  float* const red = reinterpret_cast<float*>(lds) + kFloats - NT / kWave;

  int job, tm, tn;
  int64_t item;
  decode_tile<SYM>(P, xcd_remap(blockIdx.x, P.total), job, item, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int B = P.B;
  const int64_t off = item * (int64_t)B * B;
  const uint16_t* A = (job == 0 ? P.a[0] : P.a[1]) + off;
  const uint16_t* Bt = (job == 0 ? P.bt[0] : P.bt[1]) + off;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The 8-wave layout runs epilogues other than the register-direct symmetric
  // one through LDS (staged_epilogue), so that no accumulator register is live
  // while their loads are in flight; its idle waves hold zeros, which that
  // path neither writes below the diagonal nor counts.
  constexpr bool kDirectSym = [] {
    if constexpr (Epi::kSym) return Epi::kDirect && !Epi::kReduce && SYM;
    return false;
  }();
  int wm, wn, mask;
  if constexpr (WAVES == 16) {
    big_wave_role(SYM && tm == tn, wave, wm, wn, mask);
  } else if constexpr (kDirectSym) {
    h16_wave_role8(tm == tn, wave, wm, wn, mask);
  } else {
    wm = (wave >> 1) * 64;
    wn = (wave & 1) * 128;
    mask = (SYM && tm == tn && wm >= wn + 128) ? 0 : kFull;
  }
  const int rr = lane & 31, h = lane >> 5;

  constexpr bool kUpper = has_upper_operands<Epi>::value;
  // Element offsets of this thread's 16-byte chunks from the item's base, for
  // plain stages and (kUpper) transposed ones; 32 bits hold them (B <= 16384,
  // so B * B < 2^31).  A stage picks its base as a uniform value and each
  // chunk's offset with a select, so that the load addresses carry no branch.
  uint32_t offA[LA], offB[LA], offAT[kUpper ? LA : 1], offBT[kUpper ? LA : 1];
#pragma unroll
  for (int it = 0; it < LA; ++it) {
    const int c = it * NT + tid, row = c / CPR, cs = (c % CPR) ^ h16_swz(c / CPR);
    offA[it] = (uint32_t)(m0 + row) * (uint32_t)B + 8 * cs;
    offB[it] = (uint32_t)(n0 + row) * (uint32_t)B + 8 * cs;
    if constexpr (kUpper) {
      // transposed stage: row kr of the 64 k-rows, 16-byte chunk cc of its 256 columns (h16_tswz)
      const int kr = c / (BM / 8), cc = c % (BM / 8);
      offAT[it] = (uint32_t)kr * (uint32_t)B + m0 + 8 * (cc ^ h16_tswz(kr));
      offBT[it] = (uint32_t)kr * (uint32_t)B + n0 + 8 * (cc ^ h16_tswz(kr));
    }
  }
  const int nstages = B / BKS;
  // stages whose A (Bt) panel comes transposed from the upper tiles: the
  // k-blocks left of the diagonal tile of row block tm (tn)
  const int up = kUpper ? (P.upper >> (2 * job)) & 3 : 0;
  const int ntA = (up & H16_UPPER_A) ? min(m0 / BKS, nstages) : 0;
  const int ntB = (up & H16_UPPER_B) ? min(n0 / BKS, nstages) : 0;
  auto issue = [&](uint16_t* __restrict__ buf, int s) __attribute__((always_inline)) {
    const int k0 = min(s, nstages - 1) * BKS;
    const bool tA = kUpper && s < ntA, tB = kUpper && s < ntB;
    // k-columns k0.. of the plain panel, or k-rows k0.. of the transposed one
    const uint16_t* const baseA = A + (tA ? (int64_t)k0 * B : (int64_t)k0);
    const uint16_t* const baseB = Bt + (tB ? (int64_t)k0 * B : (int64_t)k0);
    // the offsets picked by uniform masks on their values (a plain select let
    // the compiler pick between the two arrays in memory instead)
    const uint32_t mA = tA ? ~0u : 0u, mB = tB ? ~0u : 0u;
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      uint32_t oa = offA[it], ob = offB[it];
      if constexpr (kUpper) {
        oa = (offAT[it] & mA) | (oa & ~mA);
        ob = (offBT[it] & mB) | (ob & ~mB);
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(baseA + oa),
                                       (__attribute__((address_space(3))) void*)(buf + (it * NT + wave * 64) * 8),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(baseB + ob),
                                       (__attribute__((address_space(3))) void*)(buf + kA + (it * NT + wave * 64) * 8),
                                       16, 0, 0);
    }
  };
  constexpr int kWaitAll = 0 | (7 << 4);  // vmcnt(0) lgkmcnt(0)

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint16_t* const b0 = lds;
  uint16_t* const b1 = lds + kStage;
  issue(b0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();

  auto mainloop = [&](auto M) __attribute__((always_inline)) {
    constexpr int kMask = decltype(M)::value;
    // One stage: the loads for stage s + 1 into `wr` (read at stage s - 1,
    // free since that stage's barrier), then the MFMAs on `rd`.  TA (TB): A
    // (Bt) was staged transposed ([k][m], h16_tswz).
    auto step = [&](auto TAc, auto TBc, const uint16_t* __restrict__ rd, uint16_t* __restrict__ wr, int s)
        __attribute__((always_inline)) {
      constexpr bool TA = decltype(TAc)::value, TB = decltype(TBc)::value;
      issue(wr, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kMask != 0) {
        // block rows i and columns j that any computed block uses
        constexpr int kRows = [] {
          int r = 0;
          for (int i = 0; i < TM; ++i)
            if ((kMask >> (i * TN)) & ((1 << TN) - 1)) r |= 1 << i;
          return r;
        }();
        constexpr int kCols = [] {
          int c = 0;
          for (int i = 0; i < TM; ++i) c |= (kMask >> (i * TN)) & ((1 << TN) - 1);
          return c;
        }();
        auto frag = [&](const uint16_t* base, int row, int ks) __attribute__((always_inline)) {
          return *reinterpret_cast<const u32x4*>(base + (row * CPR + ((2 * ks + h) ^ h16_swz(row))) * 8);
        };
        // The fragment of rows col .. col + 31 from a transposed stage: in each
        // group of 16 lanes, lane 4 p + q addresses k-row 16 ks + 8 h + p (+ 4)
        // at column col + 16 (group & 1) + 4 q, and ds_read_b64_tr_b16 hands
        // lane t of the group column t of those at the 4 rows: 8 consecutive k
        // of one row of the operand, as the MFMA takes them (A and Bt alike).
        auto fragT = [&](const uint16_t* base, int col, int ks) __attribute__((always_inline)) {
          const int p = (lane >> 2) & 3, m = col + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          u32x4 r;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int kr = 16 * ks + 8 * h + p + 4 * half;
            const uint16_t* a = base + (kr * (BM / 8) + ((m >> 3) ^ h16_tswz(kr))) * 8 + (m & 7);
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)a);
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            r[2 * half] = w.x;
            r[2 * half + 1] = w.y;
          }
          return r;
        };
        auto fragA = [&](const uint16_t* base, int i, int ks) __attribute__((always_inline)) {
          if constexpr (TA)
            return fragT(base, wm + 32 * i, ks);
          else
            return frag(base, wm + 32 * i + rr, ks);
        };
        auto fragB = [&](const uint16_t* base, int j, int ks) __attribute__((always_inline)) {
          if constexpr (TB)
            return fragT(base, wn + 32 * j, ks);
          else
            return frag(base, wn + 32 * j + rr, ks);
        };
        u32x4 ca[2][TM], cb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if ((kRows >> i) & 1) ca[0][i] = fragA(rd, i, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if ((kCols >> j) & 1) cb[0][j] = fragB(rd + kA, j, 0);
        // LDS reads per k-step (a transposed fragment takes two) and MFMAs per k-step
        constexpr int kReads = (TA ? 2 : 1) * __builtin_popcount(kRows) + (TB ? 2 : 1) * __builtin_popcount(kCols);
        constexpr int kMfma = __builtin_popcount(kMask);
        constexpr int kPairs = kReads < kMfma ? kReads : kMfma;
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = ks & 1;
          if (ks + 1 < KS) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
              if ((kRows >> i) & 1) ca[c ^ 1][i] = fragA(rd, i, ks + 1);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              if ((kCols >> j) & 1) cb[c ^ 1][j] = fragB(rd + kA, j, ks + 1);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              if ((kMask >> (i * TN + j)) & 1) acc[i][j] = mfma_h16<FMT>(ca[c][i], cb[c][j], acc[i][j]);
          // Interleave the next k-step's fragment reads with this k-step's
          // MFMAs (one MFMA, one LDS read), so that their latency runs under
          // the matrix core instead of ahead of it; left to itself the
          // scheduler issued all reads, waited for them, then the MFMAs.
          if (ks + 1 < KS) {
#pragma unroll
            for (int q = 0; q < kPairs; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (kMfma > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPairs, 0);
            if constexpr (kReads > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kPairs, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int s = 0;
    if constexpr (kUpper) {  // the transposed stages come first; ntA and ntB are multiples of 4
      const int both = min(ntA, ntB);
      for (; s + 2 <= both; s += 2) {
        step(T_{}, T_{}, b0, b1, s);
        step(T_{}, T_{}, b1, b0, s + 1);
      }
      for (; s + 2 <= ntA; s += 2) {
        step(T_{}, F_{}, b0, b1, s);
        step(T_{}, F_{}, b1, b0, s + 1);
      }
      for (; s + 2 <= ntB; s += 2) {
        step(F_{}, T_{}, b0, b1, s);
        step(F_{}, T_{}, b1, b0, s + 1);
      }
    }
    for (; s + 2 <= nstages; s += 2) {
      step(F_{}, F_{}, b0, b1, s);
      step(F_{}, F_{}, b1, b0, s + 1);
    }
    if (s < nstages) step(F_{}, F_{}, b0, b1, s);
  };
  if constexpr (SYM && WAVES == 16) {
    switch (mask) {
      case 0xF: mainloop(std::integral_constant<int, 0xF>{}); break;
      case 0xB: mainloop(std::integral_constant<int, 0xB>{}); break;
      case 0x7: mainloop(std::integral_constant<int, 0x7>{}); break;
      case 0x8: mainloop(std::integral_constant<int, 0x8>{}); break;
      default: mainloop(std::integral_constant<int, 0>{}); break;
    }
  } else if constexpr (SYM && kDirectSym) {
    switch (mask) {  // the masks h16_wave_role8 hands out
      case 0xFF: mainloop(std::integral_constant<int, 0xFF>{}); break;
      case 0x6F: mainloop(std::integral_constant<int, 0x6F>{}); break;
      case 0x8C: mainloop(std::integral_constant<int, 0x8C>{}); break;
      default: mainloop(std::integral_constant<int, kH16Donated>{}); break;
    }
  } else if constexpr (SYM) {
    if (mask)
      mainloop(std::integral_constant<int, kFull>{});
    else
      mainloop(std::integral_constant<int, 0>{});
  } else {
    mainloop(std::integral_constant<int, kFull>{});
  }
  __syncthreads();  // every load has landed (each stage ended with vmcnt(0)); the epilogue may reuse LDS

  if constexpr (WAVES == 8 && !kDirectSym) {
    typename Epi::Tile tile(*(job == 0 ? &P.e[0] : &P.e[1]), item, P.B);
    const float part = staged_epilogue<TM, TN, BM, BN, NT, PH, Epi, !SYM>(tile, acc, reinterpret_cast<float*>(lds),
                                                                          m0, n0, wm, wn, lane, SYM, tm == tn);
    if constexpr (Epi::kReduce) {
      const float tot = block_sum<NT>(part, red);
      if (threadIdx.x == 0) {
        tile.partial(tm * P.tiles_n + tn, tot);
        if (SYM && tm != tn) tile.partial(tn * P.tiles_n + tm, tot);  // the mirrored tile
      }
    }
  } else {
    constexpr int SP = WAVES == 16 ? 1 : 2;  // mirrored half staged per block (16 waves) or block pair (8)
    static_assert(NT / kWave * 32 * (32 * SP + 4) + NT / kWave <= kFloats, "staging and reduction fit the buffers");
    gemm_epilogue<TM, TN, BM, BN, NT, PH, SYM, WAVES == 16 ? 1 : 8, SP>(P, job, item, tm, tn, acc,
                                                                     reinterpret_cast<float*>(lds), red, m0, n0, wm,
                                                                     wn, lane, mask);
  }
}

template <class Epi>
static inline int h16_gemm_nt(const uint16_t* const* a, const uint16_t* const* bt, const typename Epi::Job* e,
                              int njobs, int64_t n, int B, bool sym, int fmt, hipStream_t st, int upper = 0) {
  if (B % 128 != 0) return SHAMPOO_EUNSUPPORTED;
  if (!Epi::kSym && sym) return SHAMPOO_EINVAL;  // no symmetric epilogue
  const bool big = B % kBigTile == 0 && (sym ? Epi::kH16BigSym : Epi::kH16BigFull);
  const int T = big ? kBigTile : h16_tile_of(B, sym);
  H16Launch<Epi> P;
  memset(&P, 0, sizeof(P));
  for (int j = 0; j < njobs; ++j) {
    P.a[j] = a[j];
    P.bt[j] = bt[j];
    P.e[j] = e[j];
  }
  P.nitems = n;
  P.B = B;
  P.tiles_n = B / T;
  P.tiles_per_item = sym ? P.tiles_n * (P.tiles_n + 1) / 2 : P.tiles_n * P.tiles_n;
  // operands kept on and above the diagonal: only the large-tile kernel reads them
  if (upper != 0 && (!(big && has_upper_operands<Epi>::value) || (upper >> (2 * njobs)) != 0)) return SHAMPOO_EINVAL;
  P.upper = upper;
  const uint64_t total = (uint64_t)njobs * n * P.tiles_per_item;
  if (total == 0) return SHAMPOO_OK;
  if (total > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  P.total = (uint32_t)total;
  if (big) {
    bool launched = false;
    constexpr int W = Epi::kH16BigWaves;
    if constexpr (Epi::kSym && Epi::kH16BigSym) {
      if (sym) {
        if (fmt == H16_F16)
          hipLaunchKernelGGL((gemm_h16_big_kernel<Epi, H16_F16, true, W>), dim3(P.total), dim3(64 * W), 0, st, P);
        else
          hipLaunchKernelGGL((gemm_h16_big_kernel<Epi, H16_BF16, true, W>), dim3(P.total), dim3(64 * W), 0, st, P);
        launched = true;
      }
    }
    if constexpr (Epi::kH16BigFull) {
      if (!sym) {
        if (fmt == H16_F16)
          hipLaunchKernelGGL((gemm_h16_big_kernel<Epi, H16_F16, false, W>), dim3(P.total), dim3(64 * W), 0, st, P);
        else
          hipLaunchKernelGGL((gemm_h16_big_kernel<Epi, H16_BF16, false, W>), dim3(P.total), dim3(64 * W), 0, st, P);
        launched = true;
      }
    }
    if (!launched) return SHAMPOO_EUNSUPPORTED;  // unreachable: `big` chose this kernel
    return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
  }
  if (T == 256) {
    constexpr int NT = H16Shape<H16_T256>::NT;
    if constexpr (Epi::kSym) {
      if (sym) {
        if (fmt == H16_F16)
          hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_F16, H16_T256, true>), dim3(P.total), dim3(NT), 0, st, P);
        else
          hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_BF16, H16_T256, true>), dim3(P.total), dim3(NT), 0, st, P);
        return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
      }
    }
    if (fmt == H16_F16)
      hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_F16, H16_T256, false>), dim3(P.total), dim3(NT), 0, st, P);
    else
      hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_BF16, H16_T256, false>), dim3(P.total), dim3(NT), 0, st, P);
  } else {
    constexpr int NT = H16Shape<H16_T128>::NT;
    if constexpr (Epi::kSym) {
      if (sym) {
        if (fmt == H16_F16)
          hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_F16, H16_T128, true>), dim3(P.total), dim3(NT), 0, st, P);
        else
          hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_BF16, H16_T128, true>), dim3(P.total), dim3(NT), 0, st, P);
        return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
      }
    }
    if (fmt == H16_F16)
      hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_F16, H16_T128, false>), dim3(P.total), dim3(NT), 0, st, P);
    else
      hipLaunchKernelGGL((gemm_h16_nt_kernel<Epi, H16_BF16, H16_T128, false>), dim3(P.total), dim3(NT), 0, st, P);
  }
  return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
}

template <class Epi>
static inline int bf16_gemm_nt(const uint16_t* a, const uint16_t* bt, const typename Epi::Job& e, int64_t n,
                               int B, bool sym, hipStream_t st) {
  return h16_gemm_nt<Epi>(&a, &bt, &e, 1, n, B, sym, H16_BF16, st);
}

// The bf16 EMA Gram products (L <- beta L + alpha G G^T in place) on the
// large tiles: the 8-wave layout, whose registers let the epilogue request the
// old factor 4 groups ahead.  It reads the old factor at the entry's own
// position (4 rows of one column per group): the product is updated in place
// and the mirrored writes of a tile land on its transposed positions.
struct EpiStoreEma : EpiStore {
  static constexpr int kH16BigWaves = 8;
  struct Tile : EpiStore::Tile {
    static constexpr int kPrefetch = 4;
    struct Pre {
      floatx4 x;
    };
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : EpiStore::Tile(j, item, B_) {}
    __device__ __forceinline__ Pre prefetch4(int r, int c) const {
      Pre p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p.x[e] = ldg(cin + (int64_t)(r + e) * B + c);
      return p;
    }
    __device__ __forceinline__ floatx4 value4p(int r, int c, const floatx4& v, const Pre& p) const {
      floatx4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = mult * v[e];
        x += beta * p.x[e];
        o[e] = ident ? ((r + e == c) ? 1.f : 0.f) : x;
      }
      return o;
    }
    __device__ __forceinline__ floatx4 value4(int r, int c, const floatx4& v) const {
      return value4p(r, c, v, prefetch4(r, c));
    }
  };
};

static inline int bf16_gemm_nt_store(const uint16_t* a, const uint16_t* bt, const EpiStore::Job& e, int64_t n,
                                     int B, bool sym, hipStream_t st) {
  if (!(sym && B % kBigTile == 0 && e.cin != nullptr && e.out != nullptr && e.out16 == nullptr &&
        e.scale == nullptr && e.status == nullptr))
    return bf16_gemm_nt<EpiStore>(a, bt, e, n, B, sym, st);
  H16Launch<EpiStoreEma> P;
  memset(&P, 0, sizeof(P));
  P.a[0] = a;
  P.bt[0] = bt;
  P.e[0] = e;
  P.nitems = n;
  P.B = B;
  P.tiles_n = B / kBigTile;
  P.tiles_per_item = P.tiles_n * (P.tiles_n + 1) / 2;
  const uint64_t total = (uint64_t)n * P.tiles_per_item;
  if (total == 0) return SHAMPOO_OK;
  if (total > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  P.total = (uint32_t)total;
  constexpr int W = EpiStoreEma::kH16BigWaves;
  hipLaunchKernelGGL((gemm_h16_big_kernel<EpiStoreEma, H16_BF16, true, W>), dim3(P.total), dim3(64 * W), 0, st, P);
  return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP;
}

// a_upper: `a` (the previous Clenshaw term) holds only its tiles on and above
// the diagonal (EpiClenshaw::Job::upper16); the large-tile kernel then reads
// the rest of its row panels from those tiles, transposed.
static inline int bf16_gemm_nt_clenshaw(const uint16_t* a, const uint16_t* bt, const EpiClenshaw::Job& e,
                                        int64_t n, int B, bool sym, bool a_upper, hipStream_t st) {
  return h16_gemm_nt<EpiClenshaw>(&a, &bt, &e, 1, n, B, sym, H16_BF16, st, a_upper ? H16_UPPER_A : 0);
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
