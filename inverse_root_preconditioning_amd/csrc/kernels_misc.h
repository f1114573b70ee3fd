// Reductions, power-iteration panel steps and elementwise prologues.
#pragma once

#include "gemm_f32.h"

namespace shp {

// ---------------------------------------------------------------------------
// Trace and damping: sc[f].trace = tr(F_f), sc[f].eps = eps_rel tr / B.
// One workgroup per factor, fixed-order sum.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) trace_kernel(const float* __restrict__ F, int B, float eps_rel,
                                                    shampoo_scale* __restrict__ sc) {
  __shared__ float red[4];
  const int64_t f = blockIdx.x;
  const float* A = F + f * (int64_t)B * B;
  float s = 0.f;
  for (int i = threadIdx.x; i < B; i += 256) s += A[(int64_t)i * B + i];
  const float t = block_sum<256>(s, red);
  if (threadIdx.x == 0) {
    sc[f].trace = t;
    sc[f].eps = eps_rel * t / (float)B;
  }
}

// ---------------------------------------------------------------------------
// Range of the scale stage.  The power iteration and the Frobenius norm sum
// squares of entries of size ~ the factor's eigenvalues, which leave fp32's
// range for factors with entries beyond ~1e18 or below ~1e-19 although the
// factor itself and every later step (which work on F / c) are fine there.
// Both therefore work on F 2^-e, with 2^e the power of two just above the
// mean eigenvalue |tr F| / B, and scale the result back by 2^e.  Scaling by a
// power of two is exact, so inside the old range the results are unchanged.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int range_exp(float trace, int B) {
  const float m = fabsf(trace) / (float)B;
  if (!(m >= FLT_MIN) || !(m <= FLT_MAX)) return 0;  // zero, subnormal, NaN or infinite trace
  const int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 126;  // m in [2^(e-1), 2^e)
  return e < -125 ? -125 : (e > 125 ? 125 : e);
}

// 2^e for -126 <= e <= 127.
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// ---------------------------------------------------------------------------
// Frobenius norm: sum of squares of F 2^-e (range_exp) in `chunks` slices per
// factor, then one wave per factor finishes
// ||F + eps I||_F^2 2^-2e = sum (F 2^-e)^2 + 2 (eps 2^-e)(tr 2^-e) + B (eps 2^-e)^2.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sumsq_kernel(const float* __restrict__ F, int B, int chunks,
                                                    const shampoo_scale* __restrict__ sc,
                                                    float* __restrict__ partials) {
  __shared__ float red[4];
  const int64_t f = blockIdx.x / chunks;
  const int chunk = blockIdx.x - (int)(f * chunks);
  const int64_t per_factor = (int64_t)B * B;
  const int64_t n4 = per_factor / 4;
  const int64_t len = (n4 + chunks - 1) / chunks;
  const int64_t lo = chunk * len, hi = min(n4, lo + len);
  const floatx4* p = reinterpret_cast<const floatx4*>(F + f * per_factor);
  const float r = pow2f(-range_exp(sc[f].trace, B));
  float s = 0.f;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
    floatx4 v = p[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= r;
    s += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  const float t = block_sum<256>(s, red);
  if (threadIdx.x == 0) partials[f * chunks + chunk] = t;
}

__device__ __forceinline__ int32_t scale_status(float trace, float lam) {
  int32_t st = 0;
  if (!isfinite(trace)) {
    st |= SHAMPOO_BLK_NONFINITE;
  } else if (trace == 0.f) {
    st |= SHAMPOO_BLK_ZERO;
  }
  if (!isfinite(lam)) {
    st |= SHAMPOO_BLK_NONFINITE;
  } else if (lam <= 0.f && !(st & SHAMPOO_BLK_ZERO)) {
    st |= SHAMPOO_BLK_NONPOS_RQ;
  }
  return st;
}

// One wave per factor.
__global__ void __launch_bounds__(64) frob_finalize_kernel(const float* __restrict__ partials, int chunks,
                                                          int B, shampoo_scale* __restrict__ sc,
                                                          int32_t* __restrict__ status) {
  const int64_t f = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i < chunks; i += 64) s += partials[f * chunks + i];
  s = wave_sum(s);
  if (threadIdx.x == 0) {
    const float tr = sc[f].trace, eps = sc[f].eps;
    const int ex = range_exp(tr, B);
    const float r = pow2f(-ex), trr = tr * r, epsr = eps * r;
    const float n2 = s + 2.f * epsr * trr + (float)B * epsr * epsr;
    const float lam = sqrtf(n2) * pow2f(ex);
    sc[f].lambda = lam;
    sc[f].c = lam;
    status[f] = scale_status(tr, lam);
  }
}

// ---------------------------------------------------------------------------
// Power iteration.  Each step computes W = (F + eps I) V diag(s) for one
// PANEL-row panel of one factor on MFMA (32 x 32 blocks, K = B), where
// s_j = 1 / ||previous W column j|| (1 on the first step), and writes
// per-panel column sums of W^2 (next step's norms) and, on the last step,
// of v~_j w_j with v~ = V diag(s) (the Rayleigh quotients).  With a 128-row
// panel each of the 4 waves owns one 32-row block; with a 64-row panel two
// waves share a block and split the k-groups, summed through LDS.
// ---------------------------------------------------------------------------
constexpr int kPiCols = 32;

struct PiArgs {
  const float* F;
  const float* vin;        // [nf][B][ldv]
  int ldv;                 // r for the caller's start vectors, 32 for W buffers
  int r;                   // valid columns
  float* wout;             // [nf][B][32] (unused on the last step)
  const float* norm_in;    // [nf][npanels][32] or null on the first step
  float* norm_out;         // [nf][npanels][32]
  float* rq_out;           // [nf][npanels][32], last step only
  const shampoo_scale* sc; // eps
  int B;
  int npanels;
  int npanels_in;          // panels of norm_in (those of the previous step)
  uint32_t total;          // nf * npanels
  int last;
};

template <int PANEL>
__global__ void __launch_bounds__(256, 2) pi_step_kernel(const PiArgs P) {
  constexpr int RB = PANEL / 32;  // row blocks per panel
  constexpr int KS = 4 / RB;      // waves sharing a row block (k split)
  constexpr int BK = 32;
  using SA = Stager<PANEL, KCONTIG, false, BK>;
  using SV = Stager<kPiCols, MNCONTIG, true, BK>;
  __shared__ __attribute__((aligned(16))) float lds[2 * (SA::kFloats + SV::kFloats)];
  __shared__ float s_col[kPiCols];
  __shared__ float colsum[2][RB][kPiCols];

  const uint32_t lid = xcd_remap(blockIdx.x, P.total);
  const int64_t f = lid / P.npanels;
  const int panel = lid - (uint32_t)f * P.npanels;
  const int m0 = panel * PANEL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rb = wave % RB, ks = wave / RB;

  if (threadIdx.x < kPiCols) {
    const int j = threadIdx.x;
    float s = 0.f;
    if (j < P.r) {
      if (P.norm_in == nullptr) {
        s = 1.f;
      } else {
        float n2 = 0.f;
        for (int p = 0; p < P.npanels_in; ++p) n2 += P.norm_in[(f * P.npanels_in + p) * kPiCols + j];
        s = (n2 > 0.f) ? 1.f / sqrtf(n2) : ((n2 == 0.f) ? 0.f : n2);  // NaN propagates
      }
    }
    s_col[j] = s;
  }

  OperandView va;
  va.p = P.F + f * (int64_t)P.B * P.B;
  va.ld = P.B;
  va.rows = P.B;
  va.cols = P.B;
  va.vec = true;
  OperandView vv;
  vv.p = P.vin + f * (int64_t)P.B * P.ldv;
  vv.ld = P.ldv;
  vv.rows = P.B;
  vv.cols = P.r;
  vv.vec = (P.ldv & 3) == 0;

  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  // Two register sets keep the loads of stages s + 1 and s + 2 in flight
  // while stage s is multiplied (the kernel streams F once; the MFMA work is
  // small), two LDS buffers hold stages s and s + 1.
  SA sa[2];
  SV sv[2];
  const int stage = SA::kFloats + SV::kFloats;
  const int nstages = P.B / BK;
  sa[0].load(va, m0, 0);
  sv[0].load(vv, 0, 0);
  if (nstages > 1) {
    sa[1].load(va, m0, BK);
    sv[1].load(vv, 0, BK);
  }
  sa[0].store(lds);
  sv[0].store(lds + SA::kFloats);
  __syncthreads();
  auto step = [&](auto cur_c, int s) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    float* bufA = lds + cur * stage;
    float* bufV = bufA + SA::kFloats;
    if (s + 2 < nstages) {  // set `cur` was stored at the previous step: reuse it for stage s + 2
      sa[cur].load(va, m0, (s + 2) * BK);
      sv[cur].load(vv, 0, (s + 2) * BK);
    }
#pragma unroll
    for (int gg = 0; gg < BK / 8 / KS; ++gg) {
      const int g = gg * KS + ks;
      const floatx4 fa = SA::frag(bufA, rb * 32, g, lane);
      const floatx4 fv = SV::frag(bufV, 0, g, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q], fv[q], acc, 0, 0, 0);
    }
    if (s + 1 < nstages) {
      float* nA = lds + (cur ^ 1) * stage;
      sa[cur ^ 1].store(nA);
      sv[cur ^ 1].store(nA + SA::kFloats);
    }
    __syncthreads();
  };
  for (int s = 0; s < nstages; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nstages) step(std::integral_constant<int, 1>{}, s + 1);
  }

  if (KS > 1) {  // waves with ks > 0 hand their partial sums to ks == 0 (lds is free now)
    if (ks == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) lds[(rb * 16 + e) * 64 + lane] = acc[e];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += lds[(rb * 16 + e) * 64 + lane];
    }
  }

  const int j = lane & 31;
  if (ks == 0) {
    const float sj = s_col[j];
    const float eps = P.sc[f].eps;
    const float rinv = pow2f(-range_exp(P.sc[f].trace, P.B));
    float nsum = 0.f, rsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + rb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const float v = (j < P.r) ? ldg(vv.p + (int64_t)row * P.ldv + j) * sj : 0.f;
      const float w = (acc[e] * sj + eps * v) * rinv;
      if (!P.last) stg(P.wout + (f * P.B + row) * kPiCols + j, w);
      nsum += w * w;
      rsum += v * w;
    }
    nsum += __shfl_xor(nsum, 32, kWave);
    rsum += __shfl_xor(rsum, 32, kWave);
    if (lane < 32) {
      colsum[0][rb][j] = nsum;
      colsum[1][rb][j] = rsum;
    }
  }
  __syncthreads();
  if (threadIdx.x < kPiCols) {
    const int c = threadIdx.x;
    const int64_t o = (f * P.npanels + panel) * kPiCols + c;
    float n = 0.f, q = 0.f;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      n += colsum[0][b][c];
      q += colsum[1][b][c];
    }
    P.norm_out[o] = n;
    if (P.last) P.rq_out[o] = q;
  }
}

// The same step for 128-row panels when V has 32 columns per row (every step
// after the first): F and V go straight into LDS (global_load_lds_dwordx4)
// through a ring of three 32-deep stages, two stages ahead of the MFMAs, with
// one barrier per stage.  F is stored [row][8 quads of 4 k] with the quad index
// XOR-ed by (row ^ (row >> 3)) & 7 (conflict-free fragment reads on 64 banks),
// V as [k][32].  The arithmetic and its order are those of pi_step_kernel<128>.
__global__ void __launch_bounds__(256, 2) pi_step_dma_kernel(const PiArgs P) {
  constexpr int PANEL = 128, BK = 32;
  constexpr int kF = PANEL * BK, kV = BK * kPiCols, kStage = kF + kV;  // floats
  constexpr int NL = 5;                                                  // loads per thread and stage
  constexpr int kWaitAhead = NL | (7 << 4);                              // vmcnt(5) lgkmcnt(0)
  // One LDS object (see gemm_f32_big_kernel): the ring, then s_col and the column sums.
  __shared__ __attribute__((aligned(16))) float lds[3 * kStage + kPiCols + 2 * 4 * kPiCols];
  float* const s_col = lds + 3 * kStage;
  float* const colsum = s_col + kPiCols;  // [2][4 row blocks][32]
  const uint32_t lid = xcd_remap(blockIdx.x, P.total);
  const int64_t f = lid / P.npanels;
  const int panel = lid - (uint32_t)f * P.npanels;
  const int m0 = panel * PANEL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < kPiCols) {
    const int j = tid;
    float s = 0.f;
    if (j < P.r) {
      if (P.norm_in == nullptr) {
        s = 1.f;
      } else {
        float n2 = 0.f;
        for (int p = 0; p < P.npanels_in; ++p) n2 += P.norm_in[(f * P.npanels_in + p) * kPiCols + j];
        s = (n2 > 0.f) ? 1.f / sqrtf(n2) : ((n2 == 0.f) ? 0.f : n2);  // NaN propagates
      }
    }
    s_col[j] = s;
  }
  const int B = P.B;
  const float* Fp = P.F + f * (int64_t)B * B;
  const float* Vp = P.vin + f * (int64_t)B * kPiCols;
  auto swz = [](int row) { return (row ^ (row >> 3)) & 7; };
  // F: 4 pieces per thread and stage (wave instruction it * 4 + wave covers rows 8 (it * 4 + wave) ..);
  // V: one piece (row tid / 8, columns 4 (tid % 8) ..)
  const float* srcF[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (it * 4 + wave) * 8 + (lane >> 3);
    srcF[it] = Fp + (int64_t)(m0 + row) * B + 4 * ((lane & 7) ^ swz(row));
  }
  const float* srcV = Vp + (int64_t)(tid >> 3) * kPiCols + 4 * (tid & 7);
  const int nstages = B / BK;
  auto issue = [&](float* __restrict__ buf, int s) __attribute__((always_inline)) {
    const int k0 = min(s, nstages - 1) * BK;  // past the end: the last stage again, never read
#pragma unroll
    for (int it = 0; it < 4; ++it)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcF[it] + k0),
                                       (__attribute__((address_space(3))) void*)(buf + (it * 4 + wave) * 64 * 4),
                                       16, 0, 0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcV + (int64_t)k0 * kPiCols),
                                     (__attribute__((address_space(3))) void*)(buf + kF + wave * 64 * 4), 16, 0, 0);
  };
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  float* const b0 = lds;
  float* const b1 = lds + kStage;
  float* const b2 = lds + 2 * kStage;
  issue(b0, 0);
  issue(b1, 1);
  __builtin_amdgcn_s_waitcnt(kWaitAhead);
  __builtin_amdgcn_s_barrier();
  auto step = [&](const float* __restrict__ rd, float* __restrict__ wr, int s) __attribute__((always_inline)) {
    issue(wr, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    const int row = wave * 32 + (lane & 31);
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
      const int quad = 2 * g + (lane >> 5);
      const floatx4 fa = *reinterpret_cast<const floatx4*>(rd + row * BK + 4 * (quad ^ swz(row)));
      const float* vq = rd + kF + (8 * g + 4 * (lane >> 5)) * kPiCols + (lane & 31);
      floatx4 fv;
#pragma unroll
      for (int e = 0; e < 4; ++e) fv[e] = vq[e * kPiCols];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q], fv[q], acc, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitAhead);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int s = 0;
  for (; s + 3 <= nstages; s += 3) {
    step(b0, b2, s);
    step(b1, b0, s + 1);
    step(b2, b1, s + 2);
  }
  if (s < nstages) step(b0, b2, s);
  if (s + 1 < nstages) step(b1, b0, s + 1);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // the loads issued past the end

  const int j = lane & 31;
  const float sj = s_col[j];
  const float eps = P.sc[f].eps;
  const float rinv = pow2f(-range_exp(P.sc[f].trace, P.B));
  float nsum = 0.f, rsum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = m0 + wave * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    const float v = (j < P.r) ? ldg(Vp + (int64_t)row * kPiCols + j) * sj : 0.f;
    const float w = (acc[e] * sj + eps * v) * rinv;
    if (!P.last) stg(P.wout + (f * B + row) * kPiCols + j, w);
    nsum += w * w;
    rsum += v * w;
  }
  nsum += __shfl_xor(nsum, 32, kWave);
  rsum += __shfl_xor(rsum, 32, kWave);
  if (lane < 32) {
    colsum[wave * kPiCols + j] = nsum;
    colsum[(4 + wave) * kPiCols + j] = rsum;
  }
  __syncthreads();
  if (tid < kPiCols) {
    const int c = tid;
    const int64_t o = (f * P.npanels + panel) * kPiCols + c;
    float n = 0.f, q = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      n += colsum[b * kPiCols + c];
      q += colsum[(4 + b) * kPiCols + c];
    }
    P.norm_out[o] = n;
    if (P.last) P.rq_out[o] = q;
  }
}

// The same step for 256-column panels when V has 32 columns per row and B is
// a multiple of 256, reading F by columns: F is symmetric (the factors are
// formed as symmetric products), so W = F V = F^T V and a stage can take 16
// whole rows k of the panel's 256 columns (1 KB each), the access shape HBM
// serves fastest, instead of 128-byte pieces of many rows.  8 waves, each
// 32 columns of the panel (rows of W); k staged 16 deep through a ring of
// four stages, three ahead, one barrier per stage.  Rows 2t and 2t + 1 of F
// sit 1152 bytes apart in LDS, so that the two k rows one MFMA reads (lanes
// 0..31 and 32..63) fall on different banks; V is [k][32].
__global__ void __launch_bounds__(512, 2) pi_step_col_kernel(const PiArgs P) {
  constexpr int PANEL = 256, BK = 16, NW = 8, NB = 4;
  // F row r at r PANEL + ((r + 1) / 2) 32 floats: rows 2t and 2t + 1 are 128 bytes off modulo 256
  auto frow = [](int r) { return r * PANEL + ((r + 1) >> 1) * 32; };
  constexpr int kF = (BK - 1) * PANEL + (BK / 2) * 32 + PANEL, kV = BK * kPiCols, kStage = kF + kV;  // floats
  constexpr int NL = 3;                                // loads per thread and stage
  constexpr int kWaitAhead = (NL * (NB - 2)) | (7 << 4);
  // One LDS object (see gemm_f32_big_kernel): the ring, then s_col and the column sums.
  __shared__ __attribute__((aligned(16))) float lds[NB * kStage + kPiCols + 2 * NW * kPiCols];
  float* const s_col = lds + NB * kStage;
  float* const colsum = s_col + kPiCols;  // [2 (W², ṽ·w)][8 row blocks][32]
  const uint32_t lid = xcd_remap(blockIdx.x, P.total);
  const int64_t f = lid / P.npanels;
  const int panel = lid - (uint32_t)f * P.npanels;
  const int m0 = panel * PANEL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < kPiCols) {
    const int j = tid;
    float s = 0.f;
    if (j < P.r) {
      if (P.norm_in == nullptr) {
        s = 1.f;
      } else {
        float n2 = 0.f;
        for (int p = 0; p < P.npanels_in; ++p) n2 += P.norm_in[(f * P.npanels_in + p) * kPiCols + j];
        s = (n2 > 0.f) ? 1.f / sqrtf(n2) : ((n2 == 0.f) ? 0.f : n2);  // NaN propagates
      }
    }
    s_col[j] = s;
  }
  const int B = P.B;
  const float* Fp = P.F + f * (int64_t)B * B;
  const float* Vp = P.vin + f * (int64_t)B * kPiCols;
  // F: wave instruction it of wave w loads row k = 2 w + it of the stage, its 256 columns;
  // V: 4-byte pieces, wave w loads rows 2 w and 2 w + 1 (lanes 0..31 and 32..63)
  const float* srcF[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) srcF[it] = Fp + (int64_t)(2 * wave + it) * B + m0 + 4 * lane;
  const float* srcV = Vp + (int64_t)(2 * wave + (lane >> 5)) * kPiCols + (lane & 31);
  const int nstages = B / BK;
  auto issue = [&](float* __restrict__ buf, int s) __attribute__((always_inline)) {
    const int64_t k0 = min(s, nstages - 1) * BK;  // past the end: the last stage again, never read
#pragma unroll
    for (int it = 0; it < 2; ++it)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcF[it] + k0 * B),
                                       (__attribute__((address_space(3))) void*)(buf + frow(2 * wave + it)),
                                       16, 0, 0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcV + k0 * kPiCols),
                                     (__attribute__((address_space(3))) void*)(buf + kF + wave * 64), 4, 0, 0);
  };
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < NB - 1; ++p) issue(lds + p * kStage, p);
  __builtin_amdgcn_s_waitcnt(kWaitAhead);
  __builtin_amdgcn_s_barrier();
  const int h = lane >> 5, mcol = wave * 32 + (lane & 31);
  auto step = [&](const float* __restrict__ rd, float* __restrict__ wr, int s) __attribute__((always_inline)) {
    issue(wr, s + NB - 1);
    __builtin_amdgcn_sched_barrier(0);
    float fa[BK / 2], fv[BK / 2];
#pragma unroll
    for (int t = 0; t < BK / 2; ++t) {
      fa[t] = rd[frow(2 * t + h) + mcol];                    // F[k][m] = F[m][k]
      fv[t] = rd[kF + (2 * t + h) * kPiCols + (lane & 31)];  // V[k][j]
    }
#pragma unroll
    for (int t = 0; t < BK / 2; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[t], fv[t], acc, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitAhead);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int s = 0;
  for (; s + NB <= nstages; s += NB) {
    step(lds, lds + 3 * kStage, s);
    step(lds + kStage, lds, s + 1);
    step(lds + 2 * kStage, lds + kStage, s + 2);
    step(lds + 3 * kStage, lds + 2 * kStage, s + 3);
  }
  if (s < nstages) step(lds, lds + 3 * kStage, s);
  if (s + 1 < nstages) step(lds + kStage, lds, s + 1);
  if (s + 2 < nstages) step(lds + 2 * kStage, lds + kStage, s + 2);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // the loads issued past the end

  const int j = lane & 31;
  const float sj = s_col[j];
  const float eps = P.sc[f].eps;
  const float rinv = pow2f(-range_exp(P.sc[f].trace, P.B));
  float nsum = 0.f, rsum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = m0 + wave * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
    const float v = (j < P.r) ? ldg(Vp + (int64_t)row * kPiCols + j) * sj : 0.f;
    const float w = (acc[e] * sj + eps * v) * rinv;
    if (!P.last) stg(P.wout + (f * B + row) * kPiCols + j, w);
    nsum += w * w;
    rsum += v * w;
  }
  nsum += __shfl_xor(nsum, 32, kWave);
  rsum += __shfl_xor(rsum, 32, kWave);
  if (lane < 32) {
    colsum[wave * kPiCols + j] = nsum;
    colsum[(NW + wave) * kPiCols + j] = rsum;
  }
  __syncthreads();
  if (tid < kPiCols) {
    const int c = tid;
    const int64_t o = (f * P.npanels + panel) * kPiCols + c;
    float n = 0.f, q = 0.f;
#pragma unroll
    for (int b = 0; b < NW; ++b) {
      n += colsum[b * kPiCols + c];
      q += colsum[(NW + b) * kPiCols + c];
    }
    P.norm_out[o] = n;
    if (P.last) P.rq_out[o] = q;
  }
}

// One wave per factor: lambda = 2^e max_j q_j (the steps worked on F 2^-e, see
// range_exp), c = safety lambda, status bits.
__global__ void __launch_bounds__(64) pi_finalize_kernel(const float* __restrict__ rq, int npanels, int r, int B,
                                                        float safety, shampoo_scale* __restrict__ sc,
                                                        int32_t* __restrict__ status) {
  const int64_t f = blockIdx.x;
  const int j = threadIdx.x;
  float q = -INFINITY;
  int nan = 0;
  if (j < r) {
    q = 0.f;
    for (int p = 0; p < npanels; ++p) q += rq[(f * npanels + p) * kPiCols + j];
    nan = (q != q);
  }
  const float lam0 = wave_max(nan ? -INFINITY : q);
  const int any_nan = __any(nan);
  if (j == 0) {
    const float tr = sc[f].trace;
    const float lam = any_nan ? __int_as_float(0x7fc00000) : lam0 * pow2f(range_exp(tr, B));
    sc[f].lambda = lam;
    sc[f].c = safety * lam;
    status[f] = scale_status(tr, lam);
  }
}

// ---------------------------------------------------------------------------
// Elementwise passes over whole B x B items (float4 per thread).  Each
// workgroup covers `per_block` float4 of one item and writes one partial of
// the residual sum for it.
// ---------------------------------------------------------------------------
enum {
  EW_NDB_START = 0,   // y = a x + b I (optional store), e = (3 I - y) / 2, sum (I - y)^2
  EW_CN_START = 1,    // m = a x + b I, c = ((p+1) I - m) / p, sum (I - m)^2
  EW_CHEBY_START = 2, // as = a x + b I, bd = cd I, bd1 = cd1 I + 2 cd (2 as - I)
  EW_SCALE_COPY = 3,  // out = mult x (mult = extra c^pexp), I if degenerate
  EW_CHEBY_LINEAR = 4, // out = mult (c0 I + c1 (2 (a x + b I) - I)), I if degenerate
  EW_CN16_START = 5   // as EW_CN_START, m and c written only as 16-bit copies (h0, h1)
};

struct EwArgs {
  const float* x;              // input stack
  float* out0;                 // y | m | as | out
  float* out1;                 // e | c | bd
  float* out2;                 //     |    | bd1
  float* partials;             // [nf][chunks] or null
  const shampoo_scale* sc;     // per-factor c and eps (null: a = ua, b = ub)
  const int32_t* status;
  float ua, ub;                // uniform a, b when sc == null
  float p;                     // root order
  float c0, c1;                // Chebyshev coefficients (c_d, c_{d-1} or c_0, c_1)
  float pexp, extra;           // scale copy: mult = extra c^pexp
  uint16_t* h0;                // 16-bit outputs (EW_CN16_START)
  uint16_t* h1;
  int fmt16;
  int B;
  int chunks;                  // workgroups per item
};

template <int MODE>
__global__ void __launch_bounds__(256) ew_kernel(const EwArgs P) {
  __shared__ float red[4];
  const int64_t f = blockIdx.x / P.chunks;
  const int chunk = blockIdx.x - (int)(f * P.chunks);
  const int64_t n = (int64_t)P.B * P.B;
  const int64_t n4 = n / 4;
  const int64_t len = (n4 + P.chunks - 1) / P.chunks;
  const int64_t lo = chunk * len, hi = min(n4, lo + len);
  const int64_t off = f * n;

  float a = P.ua, b = P.ub, mult = 1.f;
  bool ident = false;
  if (P.sc != nullptr) {
    const float c = safe_c(P.sc, P.status, f);
    if (MODE == EW_SCALE_COPY || MODE == EW_CHEBY_LINEAR) {
      mult = P.extra * powf(c, P.pexp);
      if (MODE == EW_CHEBY_LINEAR) {
        a = 1.f / c;
        b = P.sc[f].eps / c;
      }
    } else {
      a = 1.f / c;
      b = P.sc[f].eps / c;
    }
    if (P.status != nullptr && degenerate(P.status[f])) {
      ident = true;
      if (MODE != EW_SCALE_COPY && MODE != EW_CHEBY_LINEAR) {
        a = 0.f;
        b = 0.f;
      }
    }
  }
  const float pinv = 1.f / P.p, p1 = P.p + 1.f;
  float part = 0.f;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
    const floatx4 xv = ldg(reinterpret_cast<const floatx4*>(P.x + off + 4 * i));
    floatx4 o0, o1, o2;
    const int row = (int)((4 * i) / P.B);
    const int col0 = (int)(4 * i - (int64_t)row * P.B);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = (row == col0 + e) ? 1.f : 0.f;
      const float y = a * xv[e] + b * d;
      if (MODE == EW_NDB_START) {
        o0[e] = y;
        o1[e] = 1.5f * d - 0.5f * y;
        part += (d - y) * (d - y);
      } else if (MODE == EW_CN_START || MODE == EW_CN16_START) {
        o0[e] = y;
        o1[e] = (p1 * d - y) * pinv;
        part += (d - y) * (d - y);
      } else if (MODE == EW_CHEBY_START) {
        o0[e] = y;
        o1[e] = P.c0 * d;
        o2[e] = P.c1 * d + 2.f * P.c0 * (2.f * y - d);
      } else if (MODE == EW_SCALE_COPY) {
        o0[e] = ident ? d : mult * xv[e];
      } else {
        o0[e] = ident ? d : mult * (P.c0 * d + P.c1 * (2.f * y - d));
      }
    }
    if (MODE == EW_CN16_START) {
      u32x2 w0, w1;
      w0.x = pack_h16x2(o0[0], o0[1], P.fmt16);
      w0.y = pack_h16x2(o0[2], o0[3], P.fmt16);
      w1.x = pack_h16x2(o1[0], o1[1], P.fmt16);
      w1.y = pack_h16x2(o1[2], o1[3], P.fmt16);
      stg(reinterpret_cast<u32x2*>(P.h0 + off + 4 * i), w0);
      stg(reinterpret_cast<u32x2*>(P.h1 + off + 4 * i), w1);
    }
    if (P.out0 && MODE != EW_CN16_START) stg(reinterpret_cast<floatx4*>(P.out0 + off + 4 * i), o0);
    if (MODE == EW_NDB_START || MODE == EW_CN_START || MODE == EW_CHEBY_START)
      stg(reinterpret_cast<floatx4*>(P.out1 + off + 4 * i), o1);
    if (MODE == EW_CHEBY_START) stg(reinterpret_cast<floatx4*>(P.out2 + off + 4 * i), o2);
  }
  if (P.partials != nullptr) {
    const float t = block_sum<256>(part, red);
    if (threadIdx.x == 0) P.partials[f * P.chunks + chunk] = t;
  }
}

// Start of the bf16-input Chebyshev evaluation with its 16-bit operands, per
// 64 x 64 tile of a factor: A_s = a x + b I (a = 1/c, b = eps/c, both 0 for a
// degenerate factor) and b_{d-1} = c_{d-1} I + 2 c_d (2 A_s - I) as
// EW_CHEBY_START forms it, written in fp32, together with the bf16 copy of
// b_{d-1} and the transposed bf16 copy of A_s (the NT operand of the Clenshaw
// products); A_s itself is not stored, nor b_d = c_d I unless `bd` is given
// (the first Clenshaw step forms it).  B is a multiple of 64.  With `split`
// (the large-tile Clenshaw products, B a multiple of 256) only what they read
// is written: fp32 b_{d-1} in the 256 x 256 tiles on and below the diagonal
// (their epilogues read it at transposed positions of upper entries), its
// bf16 copy in those on and above it (an upper-only operand).
struct Cheby16StartArgs {
  const float* x;            // factors [nf][B][B]
  const shampoo_scale* sc;   // c and eps per factor
  const int32_t* status;
  float* bd;                 // b_d (optional)
  float* bd1;                // b_{d-1}
  uint16_t* bd1_16;          // bf16(b_{d-1})
  uint16_t* as_t16;          // bf16(A_s) transposed
  float cd, cd1;             // c_d, c_{d-1}
  int B;
  int tiles;                 // (B / 64)^2
  int split;                 // write fp32 b_{d-1} below, its bf16 copy above the diagonal (256 x 256 tiles)
};

__global__ void __launch_bounds__(256) cheby16_start_kernel(const Cheby16StartArgs P) {
  __shared__ float t[64][65];
  const int64_t f = blockIdx.x / P.tiles;
  const int tt = blockIdx.x - (int)(f * P.tiles);
  const int per = P.B / 64;
  const int r0 = (tt / per) * 64, c0 = (tt % per) * 64;
  const float c = safe_c(P.sc, P.status, f);
  float a = 1.f / c, b = P.sc[f].eps / c;
  if (P.status != nullptr && degenerate(P.status[f])) {
    a = 0.f;
    b = 0.f;
  }
  const int64_t base = f * (int64_t)P.B * P.B;
  const int tid = threadIdx.x;
  const int cr = tid >> 4, cc = (tid & 15) * 4;
  // this 64 x 64 tile lies in one 256 x 256 tile (tr, tc)
  const int tr = r0 / 256, tc = c0 / 256;
  const bool w32 = !P.split || tr >= tc, w16 = !P.split || tr <= tc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + cr + 16 * i, col = c0 + cc;
    const int64_t idx = base + (int64_t)row * P.B + col;
    const floatx4 xv = ldg(reinterpret_cast<const floatx4*>(P.x + idx));
    floatx4 o1, o2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = (row == col + e) ? 1.f : 0.f;
      const float y = a * xv[e] + b * d;
      o1[e] = P.cd * d;
      o2[e] = P.cd1 * d + 2.f * P.cd * (2.f * y - d);
      t[cr + 16 * i][cc + e] = y;
    }
    if (P.bd) stg(reinterpret_cast<floatx4*>(P.bd + idx), o1);
    if (w32) stg(reinterpret_cast<floatx4*>(P.bd1 + idx), o2);
    if (w16) stg4_h16(P.bd1_16 + idx, o2, H16_BF16);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = cr + 16 * i;
    const floatx4 y = {t[cc][lr], t[cc + 1][lr], t[cc + 2][lr], t[cc + 3][lr]};
    stg4_h16(P.as_t16 + base + (int64_t)(c0 + lr) * P.B + r0 + cc, y, H16_BF16);
  }
}

// resid[f][col] = sqrt(sum of partials[f][:count]); NONFINITE if not finite.
// Residual of one iteration per factor from the epilogue's per-tile partial
// sums of squares (fixed order).  rmin[f] tracks the smallest residual of the
// current pass (reset when `first`): a residual above twice it sets
// RESID_GROWTH -- in exact arithmetic the residuals of a pass never increase
// for spectra inside the convergence region, so such a rise is rounding
// error being amplified.
__global__ void __launch_bounds__(64) resid_kernel(const float* __restrict__ partials, int count,
                                                  float* __restrict__ resid, int ncols, int col,
                                                  float* __restrict__ rmin, int first,
                                                  int32_t* __restrict__ status) {
  const int64_t f = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i < count; i += 64) s += partials[f * count + i];
  s = wave_sum(s);
  if (threadIdx.x == 0) {
    const float r = sqrtf(s);
    if (resid != nullptr) resid[f * ncols + col] = r;
    const float lo = first ? r : rmin[f];
    if (status != nullptr && !degenerate(status[f])) {
      int bits = isfinite(r) ? 0 : SHAMPOO_BLK_NONFINITE;
      if (!first && r > 2.f * lo) bits |= SHAMPOO_BLK_RESID_GROWTH;
      if (bits) status[f] |= bits;
    }
    rmin[f] = fminf(lo, r);
  }
}

}  // namespace shp

namespace shp {

// ---------------------------------------------------------------------------
// Grafting with Adam's magnitude, per block: m, v <- Adam moments of g;
// P = (m bc1) / (sqrt(v bc2) + eps); s = ||P||_F / ||U||_F (0 if U = 0);
// theta <- theta - lr s U.  Pass 1 updates m, v and writes per-chunk partial
// sums of P^2 and U^2; pass 2 forms s in a fixed order and applies it.  A
// chunk is a range of block rows; all five descriptor tables describe blocks
// of the same shape (the gradient's rows x cols).
// ---------------------------------------------------------------------------
struct GraftArgs {
  const shampoo_block* g;
  const shampoo_block* u;
  const shampoo_block* theta;
  const shampoo_block* m;
  const shampoo_block* v;
  float beta1, beta2, eps, bc1, bc2, lr;
  float* partials;   // [nblocks][chunks][2]
  float* scale_out;  // [nblocks] or null
  int B;
  int chunks;
};

__device__ __forceinline__ bool graft_block_ok(const shampoo_block& d, int B) {
  return d.ptr != nullptr && d.rows >= 0 && d.cols >= 0 && d.rows <= B && d.cols <= B && d.ld >= d.cols;
}

__global__ void __launch_bounds__(256) graft_moments_kernel(const GraftArgs P) {
  __shared__ float red[4];
  const int64_t blk = blockIdx.x / P.chunks;
  const int chunk = blockIdx.x - (int)(blk * P.chunks);
  const shampoo_block g = P.g[blk], u = P.u[blk], m = P.m[blk], v = P.v[blk];
  const bool ok = graft_block_ok(g, P.B) && graft_block_ok(u, P.B) && graft_block_ok(m, P.B) &&
                  graft_block_ok(v, P.B) && u.rows >= g.rows && u.cols >= g.cols && m.rows >= g.rows &&
                  m.cols >= g.cols && v.rows >= g.rows && v.cols >= g.cols;
  const int rows = ok ? g.rows : 0, cols = ok ? g.cols : 0;
  const int per = (P.B + P.chunks - 1) / P.chunks;
  const int r0 = chunk * per, r1 = min(rows, r0 + per);
  float sp = 0.f, su = 0.f;
  for (int r = r0; r < r1; ++r) {
    for (int c = threadIdx.x; c < cols; c += 256) {
      const float gg = ldg(g.ptr + (int64_t)r * g.ld + c);
      float* mp = m.ptr + (int64_t)r * m.ld + c;
      float* vp = v.ptr + (int64_t)r * v.ld + c;
      const float mm = P.beta1 * ldg(mp) + (1.f - P.beta1) * gg;
      const float vv = P.beta2 * ldg(vp) + (1.f - P.beta2) * gg * gg;
      stg(mp, mm);
      stg(vp, vv);
      const float p = (mm * P.bc1) / (sqrtf(vv * P.bc2) + P.eps);
      const float uu = ldg(u.ptr + (int64_t)r * u.ld + c);
      sp += p * p;
      su += uu * uu;
    }
  }
  const float tp = block_sum<256>(sp, red);
  const float tu = block_sum<256>(su, red);
  if (threadIdx.x == 0) {
    stg(P.partials + (blk * P.chunks + chunk) * 2, tp);
    stg(P.partials + (blk * P.chunks + chunk) * 2 + 1, tu);
  }
}

__global__ void __launch_bounds__(256) graft_apply_kernel(const GraftArgs P) {
  __shared__ float s_sh;
  const int64_t blk = blockIdx.x / P.chunks;
  const int chunk = blockIdx.x - (int)(blk * P.chunks);
  if (threadIdx.x == 0) {
    float np2 = 0.f, nu2 = 0.f;
    for (int c = 0; c < P.chunks; ++c) {
      np2 += P.partials[(blk * P.chunks + c) * 2];
      nu2 += P.partials[(blk * P.chunks + c) * 2 + 1];
    }
    const float s = (nu2 > 0.f) ? sqrtf(np2) / sqrtf(nu2) : 0.f;
    s_sh = s;
    if (chunk == 0 && P.scale_out != nullptr) stg(P.scale_out + blk, s);
  }
  __syncthreads();
  const float step = P.lr * s_sh;
  const shampoo_block g = P.g[blk], u = P.u[blk], th = P.theta[blk];
  const bool ok = graft_block_ok(g, P.B) && graft_block_ok(u, P.B) && graft_block_ok(th, P.B) &&
                  u.rows >= g.rows && u.cols >= g.cols && th.rows >= g.rows && th.cols >= g.cols;
  const int rows = ok ? g.rows : 0, cols = ok ? g.cols : 0;
  const int per = (P.B + P.chunks - 1) / P.chunks;
  const int r0 = chunk * per, r1 = min(rows, r0 + per);
  for (int r = r0; r < r1; ++r) {
    for (int c = threadIdx.x; c < cols; c += 256) {
      float* tp = th.ptr + (int64_t)r * th.ld + c;
      stg(tp, ldg(tp) - step * ldg(u.ptr + (int64_t)r * u.ld + c));
    }
  }
}

}  // namespace shp
