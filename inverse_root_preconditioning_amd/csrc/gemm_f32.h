// Batched fp32 MFMA matrix product for gfx950 with fused epilogues.
//
// One launch computes C_i = A_i * B_i for every item i of up to two jobs (the
// Newton-DB update Y E and E Z, for instance, run as two jobs of one launch).
// Each workgroup of 256 threads (4 waves, 2 x 2) owns one (64 TM) x (64 TN)
// output tile of one item; each wave owns (32 TM) x (32 TN) of it as TM x TN
// blocks of V_MFMA_F32_32X32X2_F32.  Operand tiles of kBK k-values are staged
// through LDS (double-buffered, one barrier per stage) from either a dense
// stack of B x B row-major matrices or a table of block descriptors (zero
// outside the block).  The epilogue turns the fp32 accumulators into the
// output of the step (E = (3I - P)/2, an EMA, a Clenshaw term, ...) so that
// no separate elementwise pass over HBM is needed.
//
// k-order within a group of 8: for MFMA j (0..3) lane (r, h) supplies
// element k = 8 g + 4 h + j of its row of A and column of B, so every lane
// reads 4 consecutive k values at once; the sum over j and h covers all 8.
#pragma once

#include "common.h"

namespace shp {

enum { KCONTIG = 0, MNCONTIG = 1 };

constexpr int kGemmThreads = 256;
// k-depth of one LDS stage.  16 keeps a 128 x 128 tile's double-buffered
// stages at 37 KB, so four workgroups fit a CU (measured faster than 32 with
// two workgroups per CU at B = 1024).
constexpr int kBK = 16;

// One operand of a job: a dense stack (desc == nullptr) or descriptors.
struct Operand {
  const float* base;
  const shampoo_block* desc;
};

// Storage view of one item of an operand.
struct OperandView {
  const float* p;
  int64_t ld;
  int rows, cols;  // valid storage extent
  bool vec;        // 16-byte vector loads allowed
};

__device__ __forceinline__ OperandView operand_view(const Operand& op, int64_t item, int B) {
  OperandView v;
  if (op.desc == nullptr) {
    v.p = op.base + item * (int64_t)B * B;
    v.ld = B;
    v.rows = B;
    v.cols = B;
    v.vec = true;
  } else {
    const shampoo_block d = op.desc[item];
    const bool ok = d.ptr != nullptr && d.rows >= 0 && d.cols >= 0 && d.rows <= B && d.cols <= B &&
                    d.ld >= d.cols;
    v.p = d.ptr;
    v.ld = d.ld;
    v.rows = ok ? d.rows : 0;
    v.cols = ok ? d.cols : 0;
    v.vec = ((reinterpret_cast<uintptr_t>(d.ptr) & 15u) == 0) && ((d.ld & 3) == 0);
  }
  return v;
}

// Tile staging for one operand: MN x BK values (MN rows of the product).
template <int MN, int LAYOUT, bool DESC, int BK = kBK>
struct Stager {
  static constexpr int kLoads = MN * BK / 4 / kGemmThreads;  // float4 per thread per stage
  static constexpr int kStride = (LAYOUT == KCONTIG) ? (BK + 4) : (MN + 4);
  static constexpr int kFloats = (LAYOUT == KCONTIG) ? MN * (BK + 4) : BK * (MN + 4);
  static_assert(kLoads >= 1, "tile too small for one float4 per thread");
  floatx4 r[kLoads];

  __device__ __forceinline__ void load(const OperandView& v, int mn0, int k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int idx = tid + kGemmThreads * it;
      int srow, scol;
      if (LAYOUT == KCONTIG) {
        srow = mn0 + idx / (BK / 4);
        scol = k0 + (idx % (BK / 4)) * 4;
      } else {
        srow = k0 + idx / (MN / 4);
        scol = mn0 + (idx % (MN / 4)) * 4;
      }
      if (!DESC) {
        r[it] = ldg(reinterpret_cast<const floatx4*>(v.p + (int64_t)srow * v.ld + scol));
      } else {
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
        if (srow < v.rows) {
          const float* src = v.p + (int64_t)srow * v.ld + scol;
          if (v.vec && scol + 3 < v.cols) {
            x = ldg(reinterpret_cast<const floatx4*>(src));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (scol + e < v.cols) x[e] = ldg(src + e);
          }
        }
        r[it] = x;
      }
    }
  }

  __device__ __forceinline__ void store(float* lds) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int idx = tid + kGemmThreads * it;
      int off;
      if (LAYOUT == KCONTIG)
        off = (idx / (BK / 4)) * kStride + (idx % (BK / 4)) * 4;
      else
        off = (idx / (MN / 4)) * kStride + (idx % (MN / 4)) * 4;
      *reinterpret_cast<floatx4*>(lds + off) = r[it];
    }
  }

  // Fragment of 4 consecutive k (8 g + 4 h + j, j = 0..3) at row mb + r.
  __device__ __forceinline__ static floatx4 frag(const float* lds, int mb, int g, int lane) {
    const int rr = lane & 31, h = lane >> 5;
    if (LAYOUT == KCONTIG) {
      return *reinterpret_cast<const floatx4*>(lds + (mb + rr) * kStride + g * 8 + h * 4);
    } else {
      floatx4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = lds[(g * 8 + h * 4 + j) * kStride + mb + rr];
      return x;
    }
  }
};

// Launch parameters; Epi::Job carries the epilogue's per-job arguments.
template <class Epi>
struct GemmLaunch {
  using EpiT = Epi;
  Operand a[2];
  Operand b[2];
  typename Epi::Job e[2];
  int64_t nitems;      // items per job
  int B;
  int tiles_n;         // B / BN
  int tiles_per_item;  // tiles_m * tiles_n, or T (T + 1) / 2 for a symmetric product (upper tiles only)
  uint32_t total;      // njobs * nitems * tiles_per_item
};

// Epilogue of a symmetric product (only tiles with tm <= tn are computed).
// Each lane forms its outputs o = tile.value(...) at their own positions and
// writes them there (on a diagonal tile only the upper triangle).  The
// mirrored half is written coalesced through an LDS transpose in PH phases
// of BM / PH tile rows; a wave's rows (32 TM of them, from wm) fall in one
// phase, in which it stages them.  `lds` needs (BM / PH) x (BN + 1) floats
// and must be free when this is called (the main loop has ended with a
// barrier).  The accumulator layout is that of the 32 x 32 MFMA blocks; NT
// threads take part.
//
// With RED, returns this thread's share of the tile's reduction of
// tile.contrib(...) over the symmetric result: on a diagonal tile entries
// above the diagonal count twice, diagonal entries once and entries below
// not at all; an off-diagonal tile counts once and stands for its mirror too.
template <int TM, int TN, int BM, int BN, int NT, int PH, bool RED = false, class Tile>
__device__ __forceinline__ float sym_epilogue(Tile& tile, floatx16 (&acc)[TM][TN], float* lds, int m0, int n0,
                                              int wm, int wn, int lane, bool diag) {
  constexpr int LD = BN + 1, RH = BM / PH;  // tile rows per phase
  static_assert(RH % (32 * TM) == 0, "a wave's rows must fall in one phase");
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int cl = wn + 32 * j + (lane & 31);
        if constexpr (RED) {
          const float w = !diag ? 1.f : (rl < cl ? 2.f : (rl == cl ? 1.f : 0.f));
          part += w * tile.contrib(m0 + rl, n0 + cl, acc[i][j][e]);
        }
        const float o = tile.value(m0 + rl, n0 + cl, acc[i][j][e]);
        if (!diag || rl <= cl) tile.write(m0 + rl, n0 + cl, o);
        acc[i][j][e] = o;
      }
      // one 32 x 32 block at a time, so that the epilogue's own loads in
      // flight need few registers beyond the accumulators
      if constexpr (TM * TN > 4 || RED) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
  for (int h = 0; h < PH; ++h) {
    if (PH == 1 || wm / RH == h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int cl = wn + 32 * j + (lane & 31);
            lds[(rl - h * RH) * LD + cl] = acc[i][j][e];
          }
    }
    __syncthreads();
    // o[h RH + b][a] goes to (n0 + a, m0 + h RH + b); on a diagonal tile only below the diagonal.
    for (int idx = threadIdx.x; idx < RH * BN; idx += NT) {
      const int a = idx / RH, b = idx - (idx / RH) * RH;
      if (!diag || a > h * RH + b) tile.write(n0 + a, m0 + h * RH + b, lds[b * LD + a]);
    }
    if (h + 1 < PH) __syncthreads();
  }
  return part;
}

// Epilogue through LDS for workgroups with many accumulators: in each of PH
// phases the waves whose rows fall in it stage their raw accumulators, then
// all NT threads apply the epilogue in row-major order (consecutive threads,
// consecutive columns), so no accumulator register is live while the
// epilogue's own loads are in flight.  For a symmetric product (`sym`) the
// value formed at each computed position is written there (on a diagonal
// tile only on and above the diagonal), kept in LDS, and written mirrored
// through a transposed pass, and the reduction is weighted as in
// sym_epilogue.  `lds` needs (BM / PH) x (BN + 4) floats and must be free.
// Returns this thread's share of the tile's reduction.
//
// V8 (full products only, for tiles with store8): each thread takes 8
// consecutive columns of a staged row, read with two 16-byte LDS loads (rows
// BN + 4 floats apart) and written with 16- or 32-byte stores, an eighth of
// the store instructions of one entry per thread (16-bit coupled-Newton
// C^p M at B = 1024: 2.02 -> 1.69 ms; the fp32 kernel's epilogue measured
// 2% slower with it and keeps one entry per thread).
template <class T, class = void>
struct has_store8 : std::false_type {};
template <class T>
struct has_store8<T, std::void_t<decltype(&T::store8)>> : std::true_type {};

template <int TM, int TN, int BM, int BN, int NT, int PH, class Epi, bool V8 = false>
__device__ __forceinline__ float staged_epilogue(typename Epi::Tile& tile, floatx16 (&acc)[TM][TN], float* lds,
                                                 int m0, int n0, int wm, int wn, int lane, bool sym, bool diag) {
  constexpr bool kV8 = V8 && has_store8<typename Epi::Tile>::value;
  static_assert(BN % 8 == 0, "whole groups of 8 columns");
  constexpr int LD = kV8 ? BN + 4 : BN + 1, RH = BM / PH;
  static_assert(RH % (32 * TM) == 0, "a wave's rows must fall in one phase");
  float part = 0.f;
#pragma unroll
  for (int h = 0; h < PH; ++h) {
    if (PH == 1 || wm / RH == h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int cl = wn + 32 * j + (lane & 31);
            lds[(rl - h * RH) * LD + cl] = acc[i][j][e];
          }
    }
    __syncthreads();
    const int r0 = m0 + h * RH;
    if constexpr (Epi::kSym) {
      if (sym) {
        for (int idx = threadIdx.x; idx < RH * BN; idx += NT) {
          const int b = idx / BN, a = idx - (idx / BN) * BN;
          if constexpr (Epi::kReduce) {  // weights as in sym_epilogue
            const int rg = r0 + b, cg = n0 + a;
            const float w = !diag ? 1.f : (rg < cg ? 2.f : (rg == cg ? 1.f : 0.f));
            part += w * tile.contrib(rg, cg, lds[b * LD + a]);
          }
          const float o = tile.value(r0 + b, n0 + a, lds[b * LD + a]);
          if (!diag || r0 + b <= n0 + a) tile.write(r0 + b, n0 + a, o);
          lds[b * LD + a] = o;
        }
        __syncthreads();
        // o[b][a] goes to (n0 + a, r0 + b); on a diagonal tile only from above the diagonal.
        for (int idx = threadIdx.x; idx < RH * BN; idx += NT) {
          const int a = idx / RH, b = idx - (idx / RH) * RH;
          if (!diag || n0 + a > r0 + b) tile.write(n0 + a, r0 + b, lds[b * LD + a]);
        }
        if (h + 1 < PH) __syncthreads();
        continue;
      }
    }
    if constexpr (kV8) {
      for (int idx = threadIdx.x; idx < RH * BN / 8; idx += NT) {
        const int b = idx / (BN / 8), a = 8 * (idx - b * (BN / 8));
        const floatx4 lo = *reinterpret_cast<const floatx4*>(lds + b * LD + a);
        const floatx4 hi = *reinterpret_cast<const floatx4*>(lds + b * LD + a + 4);
        part += tile.store8(r0 + b, n0 + a, lo, hi);
      }
    } else {
      for (int idx = threadIdx.x; idx < RH * BN; idx += NT) {
        const int b = idx / BN, a = idx - (idx / BN) * BN;
        part += tile.store(r0 + b, n0 + a, lds[b * LD + a]);
      }
    }
    if (h + 1 < PH) __syncthreads();
  }
  return part;
}

// Epilogue of a symmetric product from registers (kDirect epilogues).  For
// each group of four accumulators a lane holds rows r..r+3 of one column c:
// it writes them there (on a diagonal tile only on and above the diagonal)
// and, with SP = 0, writes the mirrored entries, columns r..r+3 of row c,
// with one vector store (on a diagonal tile only those strictly below the
// diagonal).  Only the 32 x 32 blocks (i, j) with bit i TN + j of `mask`
// set are written.
// KPRE bounds how many groups' epilogue inputs are loaded ahead (registers).
//
// SP > 0: both halves go through `stage`, this wave's 32 x (32 SP + 4) floats
// of LDS; entry (x, y) sits at x (32 SP + 4) + (y ^ 8 SP) for x >= 16, else at
// x (32 SP + 4) + y: unswizzled, staged rows x and x + 16 start on the same
// bank, and the column-wise reads of the upper half below went two lanes to a
// bank.  For SP = 1 each 16-lane pass of the row-wise reads takes two rows 8
// apart, whose 32 floats fill complementary halves of the 64 banks (rows 1
// apart overlap on 4).  Each group is first written there at its transposed place; once
// the SP vertically adjacent blocks of one column are in, the wave reads them
// back along the mirrored rows, each store instruction covering 32 SP
// consecutive columns of 64 / (8 SP) rows (whole 128-byte lines, where a
// register-direct mirrored store covers 32 bytes of 32 rows), and along the
// upper rows, 4 or 8 columns per lane (where group-wise upper stores take one
// instruction per 1 or 2 bytes of 32 columns of 2 rows).  On a diagonal tile
// only entries of computed blocks on (upper) or strictly below (mirrored) the
// diagonal go out.
// Groups are then taken column of blocks by column of blocks (j-major).
// Mirrored entries of an off-diagonal tile: write4t_mirror where the tile has
// one (an output kept partly on and above the diagonal only), else write4t.
template <class T, class = void>
struct has_write4t_mirror : std::false_type {};
template <class T>
struct has_write4t_mirror<T, std::void_t<decltype(&T::write4t_mirror)>> : std::true_type {};
template <class Tile>
__device__ __forceinline__ void write4t_offdiag(Tile& t, int c, int r, const floatx4& o) {
  if constexpr (has_write4t_mirror<Tile>::value)
    t.write4t_mirror(c, r, o);
  else
    t.write4t(c, r, o);
}
// Whether an off-diagonal tile writes anything at its mirrored place (a tile
// without the `mirrored` query always does).
template <class T, class = void>
struct has_mirrored_query : std::false_type {};
template <class T>
struct has_mirrored_query<T, std::void_t<decltype(&T::mirrored)>> : std::true_type {};
template <class Tile>
__device__ __forceinline__ bool writes_mirror(const Tile& t) {
  if constexpr (has_mirrored_query<Tile>::value)
    return t.mirrored();
  else
    return true;
}

template <int TM, int TN, int KPRE, int SP = 0, class Tile>
__device__ __forceinline__ void sym_epilogue_direct(Tile& tile, floatx16 (&acc)[TM][TN], int m0, int n0, int wm,
                                                    int wn, int lane, bool diag, int mask, float* stage = nullptr) {
  static_assert(SP == 0 || (TM % SP == 0 && SP <= 2), "staged blocks per column");
  constexpr int LDT = 32 * SP + 4;  // staged row pitch in floats: the group writes of 16 lanes hit 64 banks
  constexpr int SWZ = 8 * SP;       // column swizzle of staged rows 16..31
  const int h = lane >> 5, cl = lane & 31;
  // staged-row base of this lane's group writes (row cl), for columns with the swizzle bit clear or set
  const int sw_w = (cl & 16) ? SWZ : 0;
  const int st_plus = cl * LDT + 4 * h + sw_w, st_minus = cl * LDT + 4 * h - sw_w;
  // group G -> block (i, j), accumulators 4 q .. 4 q + 3
  auto gi_ = [](int g) { return SP ? (g / 4) % TM : g / (TN * 4); };
  auto gj_ = [](int g) { return SP ? g / (TM * 4) : (g / 4) % TN; };
  // Forms and writes group G.
  auto emit = [&](auto G, const auto& o) __attribute__((always_inline)) {
    constexpr int i = gi_(decltype(G)::value), j = gj_(decltype(G)::value), q = decltype(G)::value % 4;
    const int r = m0 + wm + 32 * i + 8 * q + 4 * h;
    const int c = n0 + wn + 32 * j + cl;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (!diag || r + e <= c) tile.write_upper(r + e, c, o[e]);
    if (!diag || r + 3 < c) {
      tile.write4t(c, r, o);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (r + e < c) tile.write(c, r + e, o[e]);
    }
  };
  // Staged: the group goes into `stage` at its transposed place; both halves
  // are written from there.  DG: a diagonal tile (compile-time, so that
  // off-diagonal tiles carry no tests).
  auto emit_staged = [&](auto DG, auto G, const auto& o) __attribute__((always_inline)) {
    if constexpr (SP > 0) {
      constexpr int g = decltype(G)::value;
      constexpr int i = gi_(g), q = g % 4;
      constexpr int y = 32 * (i % SP) + 8 * q;  // y ^ sw = y + sw or y - sw by the bit y holds
      *reinterpret_cast<floatx4*>(stage + ((y & SWZ) ? st_minus : st_plus) + y) = o;
    }
  };
  // After the last group of the SP blocks of one column, computed or not: the
  // staged (32 SP) x 32 block goes out along its mirrored rows.
  auto flush = [&](auto DG, auto G) __attribute__((always_inline)) {
    if constexpr (SP > 0) {
      constexpr int g = decltype(G)::value;
      constexpr int i = gi_(g), j = gj_(g), q = g % 4;
      if constexpr (q == 3 && i % SP == SP - 1) {
        constexpr int i0 = i - (SP - 1);
        constexpr int kUnit = SP == 2 ? (1 | (1 << TN)) : 1;  // blocks (i0, 0) .. (i, 0) as mask bits
        if (decltype(DG)::value && (mask & (kUnit << (i0 * TN + j))) == 0) return;  // none computed here
        __builtin_amdgcn_wave_barrier();
        constexpr int LPR = 8 * SP;    // lanes per staged row
        constexpr int RPI = 64 / LPR;  // rows per instruction
        const int rr = lane / LPR, cc = 4 * (lane % LPR), cc_sw = cc ^ SWZ;
        // row of instruction t: RPI t + rr, or for SP = 1 rows 8 apart in each pass of 16 lanes
        const int rrow = SP == 1 ? 8 * (rr & 1) + (rr >> 1) : rr;
        const int c0 = n0 + wn + 32 * j, r0 = m0 + wm + 32 * i0;
        // on a diagonal tile: whether this lane's source block was computed by this wave
        const bool src = !decltype(DG)::value || ((mask >> ((i0 + cc / 32) * TN + j)) & 1);
        if (decltype(DG)::value || writes_mirror(tile)) {
#pragma unroll
          for (int t = 0; t < 32 / RPI; ++t) {
            const int tb = SP == 1 ? 4 * (t & 1) + 16 * (t >> 1) : RPI * t;  // >= 16 exactly for swizzled rows
            const int row = tb + rrow;
            const floatx4 v = *reinterpret_cast<const floatx4*>(stage + row * LDT + (tb >= 16 ? cc_sw : cc));
            if constexpr (!decltype(DG)::value) {
              write4t_offdiag(tile, c0 + row, r0 + cc, v);
            } else if (src) {
              if (r0 + cc + 3 < c0 + row) {
                tile.write4t(c0 + row, r0 + cc, v);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (r0 + cc + e < c0 + row) tile.write(c0 + row, r0 + cc + e, v[e]);
              }
            }
          }
        }
        // The upper half along its own rows, CU columns per lane: 8 for block
        // pairs (16-byte stores of the 16-bit copy), 4 for single blocks (a
        // quarter or an eighth of the store instructions of writing it group
        // by group; 8 measured slower for the fp32 kernel).
        constexpr int CU = SP == 2 ? 8 : 4, LPU = 32 / CU, RPU = 64 / LPU;
        const int ru = lane / LPU, cu = CU * (lane % LPU);
        const int sw_u = (cu & 16) ? SWZ : 0;  // the staged rows cu .. cu + CU - 1 share bit 4
        constexpr int NU = 32 * SP / RPU;  // iterations
        auto upper = [&](int t) __attribute__((always_inline)) {
          const int rl = RPU * t + ru, rs = rl ^ sw_u;
          floatx4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) lo[e] = stage[(cu + e) * LDT + rs];
          if constexpr (CU == 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) hi[e] = stage[(cu + 4 + e) * LDT + rs];
          }
          const int r = r0 + rl, c = c0 + cu;
          const bool whole = !decltype(DG)::value || r <= c;
          const bool src = !decltype(DG)::value || ((mask >> ((i0 + rl / 32) * TN + j)) & 1);
          if (src && whole) {
            if constexpr (CU == 8)
              tile.write_upper8(r, c, lo, hi);
            else
              tile.write_upper4(r, c, lo);
          } else if (src) {
#pragma unroll
            for (int e = 0; e < CU; ++e)
              if (r <= c + e) tile.write_upper(r, c + e, e < 4 ? lo[e & 3] : hi[e & 3]);
          }
        };
        // one row group at a time for 8 columns, two for 4 (as measured fastest; more spills)
        if constexpr (CU == 8) {
#pragma unroll 1
          for (int t = 0; t < NU; ++t) upper(t);
        } else {
#pragma unroll 2
          for (int t = 0; t < NU; ++t) upper(t);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  };
  auto rc = [&](auto G, int& r, int& c) __attribute__((always_inline)) {
    constexpr int i = gi_(decltype(G)::value), j = gj_(decltype(G)::value), q = decltype(G)::value % 4;
    r = m0 + wm + 32 * i + 8 * q + 4 * h;
    c = n0 + wn + 32 * j + cl;
  };
  auto acc4 = [&](auto G) __attribute__((always_inline)) {
    constexpr int i = gi_(decltype(G)::value), j = gj_(decltype(G)::value), q = decltype(G)::value % 4;
    return floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
  };
  auto computed = [&](auto G) __attribute__((always_inline)) {
    constexpr int i = gi_(decltype(G)::value), j = gj_(decltype(G)::value);
    return ((mask >> (i * TN + j)) & 1) != 0;  // a block this wave computed
  };
  // groups prefetched together: at most the epilogue's wish, the caller's register budget and the groups there are
  constexpr int K0 = Tile::kPrefetch < KPRE ? Tile::kPrefetch : KPRE;
  constexpr int K = K0 < TM * TN * 4 ? K0 : TM * TN * 4;
  auto body = [&](auto&& out, auto&& after) __attribute__((always_inline)) {
    if constexpr (K == 0) {
      static_for<TM * TN * 4>([&](auto G) __attribute__((always_inline)) {
        if (computed(G)) {
          int r, c;
          rc(G, r, c);
          out(G, tile.value4(r, c, acc4(G)));
        }
        after(G);
      });
    } else {
      // The epilogue's own inputs are requested a chunk of K groups at a time,
      // one chunk ahead of the groups being formed and written (stores in
      // between would otherwise keep each load behind the previous group's
      // stores, one memory latency per group).
      constexpr int NC = TM * TN * 4 / K;
      static_assert(NC * K == TM * TN * 4, "whole chunks");
      typename Tile::Pre pre[2][K];
      auto fetch = [&](auto C) __attribute__((always_inline)) {
        static_for<K>([&](auto G) __attribute__((always_inline)) {
          constexpr int g = decltype(C)::value * K + decltype(G)::value;
          if (!computed(std::integral_constant<int, g>{})) return;
          int r, c;
          rc(std::integral_constant<int, g>{}, r, c);
          pre[decltype(C)::value & 1][decltype(G)::value] = tile.prefetch4(r, c);
        });
      };
      fetch(std::integral_constant<int, 0>{});
      static_for<NC>([&](auto C) __attribute__((always_inline)) {
        if constexpr (decltype(C)::value + 1 < NC) fetch(std::integral_constant<int, decltype(C)::value + 1>{});
        static_for<K>([&](auto G) __attribute__((always_inline)) {
          constexpr int g = decltype(C)::value * K + decltype(G)::value;
          const std::integral_constant<int, g> gi{};
          if (computed(gi)) {
            int r, c;
            rc(gi, r, c);
            out(gi, tile.value4p(r, c, acc4(gi), pre[decltype(C)::value & 1][decltype(G)::value]));
          }
          after(gi);
        });
      });
    }
  };
  if constexpr (SP > 0) {
    auto staged = [&](auto DG) __attribute__((always_inline)) {
      body([&](auto G, const auto& o) __attribute__((always_inline)) { emit_staged(DG, G, o); },
           [&](auto G) __attribute__((always_inline)) { flush(DG, G); });
    };
    if (diag)
      staged(std::true_type{});
    else
      staged(std::false_type{});
  } else {
    body(emit, [](auto) {});
  }
}

// Workgroup lid -> (job, item, tile row tm, tile column tn), item-major: the
// tiles of both jobs of one item are neighbours, so that the workgroups that
// run together share that item's operands (E in Y E and E Z) through L2.  A
// symmetric product enumerates only its upper tiles (tm <= tn).
template <bool SYM, class L>
__device__ __forceinline__ void decode_tile(const L& P, uint32_t lid, int& job, int64_t& item, int& tm,
                                            int& tn) {
  const uint32_t tpi = (uint32_t)P.tiles_per_item;
  const uint32_t njobs = P.total / ((uint32_t)P.nitems * tpi);
  item = lid / (njobs * tpi);
  const uint32_t rem = lid - (uint32_t)item * njobs * tpi;
  if constexpr (!SYM) {
    job = rem / tpi;
    const int t = rem - job * tpi;
    tm = t / P.tiles_n;
    tn = t - tm * P.tiles_n;
  } else {
    // the off-diagonal tiles of every job row by row, then the diagonal ones,
    // which are shorter (about 0.65 of a tile; measured 4% faster for the
    // Newton-DB pair than row order; the diagonal tiles of all factors at the
    // end of the launch lose the operands' L2 reuse and measured 23% slower)
    const uint32_t noff = (uint32_t)(P.tiles_n * (P.tiles_n - 1) / 2);
    if (rem < njobs * noff) {
      job = rem / noff;
      int t = rem - job * noff;
      tm = 0;
      int rowlen = P.tiles_n - 1;
      while (t >= rowlen) {
        t -= rowlen;
        ++tm;
        --rowlen;
      }
      tn = tm + 1 + t;
    } else {
      const uint32_t r2 = rem - njobs * noff;
      job = r2 / P.tiles_n;
      tm = tn = r2 - job * P.tiles_n;
    }
  }
}

// Epilogue of one output tile.  Accumulator e of block (i, j) sits at
// row = 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, col = 32 j + lane % 32 of the
// wave's (32 TM) x (32 TN) part, at (wm, wn) in the tile at (m0, n0).  `lds`
// must hold (BM / PH) x (BN + 1) floats and be free; `red` NT / 64 floats.
// `mask` (the blocks this wave computed) is honoured by the register-direct
// symmetric epilogue; the other paths need every block computed.  SP > 0
// stages that epilogue's mirrored half (see sym_epilogue_direct): `lds` must
// then also hold NT / 64 x 32 x (32 SP + 4) floats.
template <int TM, int TN, int BM, int BN, int NT, int PH, bool SYM, int KPRE = (NT == kGemmThreads ? 2 : 1),
          int SP = 0, class L>
__device__ __forceinline__ void gemm_epilogue(const L& P, int job, int64_t item, int tm, int tn,
                                              floatx16 (&acc)[TM][TN], float* lds, float* red, int m0, int n0,
                                              int wm, int wn, int lane, int mask = (1 << (TM * TN)) - 1) {
  using Epi = typename L::EpiT;
  typename Epi::Tile tile(*(job == 0 ? &P.e[0] : &P.e[1]), item, P.B);
  float part = 0.f;
  bool done = false;
  if constexpr (Epi::kSym && SYM) {
    if constexpr (Epi::kDirect && !Epi::kReduce) {
      // waves of 1024-thread workgroups (128 VGPRs) have no room for staging beside loads ahead
      constexpr int kSP = (NT >= 1024 && Epi::Tile::kPrefetch > 0) ? 0 : SP;
      sym_epilogue_direct<TM, TN, KPRE, kSP>(tile, acc, m0, n0, wm, wn, lane, tm == tn, mask,
                                             lds + (threadIdx.x / kWave) * 32 * (32 * kSP + 4));
    }
    else
      part = sym_epilogue<TM, TN, BM, BN, NT, PH, Epi::kReduce>(tile, acc, lds, m0, n0, wm, wn, lane, tm == tn);
    done = true;
  }
  if (!done) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int col = n0 + wn + 32 * j + (lane & 31);
          part += tile.store(row, col, acc[i][j][e]);
        }
        // one 32 x 32 block at a time: the epilogue's own loads need few registers
        if constexpr (NT > kGemmThreads) __builtin_amdgcn_sched_barrier(0);
      }
  }
  if constexpr (Epi::kReduce) {
    const float tot = block_sum<NT>(part, red);
    if (threadIdx.x == 0) {
      tile.partial(tm * P.tiles_n + tn, tot);
      if (SYM && tm != tn) tile.partial(tn * P.tiles_n + tm, tot);  // the mirrored tile
    }
  }
}

// SYM: the product is symmetric (upper tiles only, see GemmLaunch::sym); a
// template parameter so that each kernel carries only the epilogue it runs.
template <int TM, int TN, int LA, int LB, bool DA, bool DB, class Epi, bool SYM, int BK = kBK, int MINW = 2>
__global__ void __launch_bounds__(kGemmThreads, MINW) gemm_f32_kernel(const GemmLaunch<Epi> P) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  using SA = Stager<BM, LA, DA, BK>;
  using SB = Stager<BN, LB, DB, BK>;
  constexpr int kPipe = 2 * (SA::kFloats + SB::kFloats);
  constexpr int kTrans = Epi::kSym ? (BM / 2) * (BN + 1) : 0;  // the symmetric epilogue's transpose
  __shared__ __attribute__((aligned(16))) float lds[kPipe > kTrans ? kPipe : kTrans];
  __shared__ float red[kGemmThreads / kWave];

  int job, tm, tn;
  int64_t item;
  decode_tile<SYM>(P, xcd_remap(blockIdx.x, P.total), job, item, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const OperandView va = operand_view(P.a[job], item, P.B);
  const OperandView vb = operand_view(P.b[job], item, P.B);

  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; readfirstlane lets the compiler
  // see that, so tests on it become scalar branches rather than exec masking.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave >> 1) * 32 * TM;  // wave's row offset inside the tile
  const int wn = (wave & 1) * 32 * TN;
  // On a diagonal tile of a symmetric product the wave below the diagonal
  // (rows 32 TM.., columns ..32 TN) holds only entries that are never
  // written: it skips its fragment reads and MFMAs (it still stages operands
  // and meets every barrier), which frees its SIMD for other workgroups.
  const bool active = !(SYM && tm == tn && wm > wn);
  // ... and a wave on the diagonal (wm == wn; the wave tiles are square) skips
  // its 32 x 32 blocks (i, j), i > j, which lie wholly below it.  The k-loop
  // body is instantiated for both cases, so the MFMA stream has no branches.
  static_assert(TM == TN, "square wave tiles");
  const bool skip_low = SYM && tm == tn && wm == wn;

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  SA sa;
  SB sb;
  constexpr int kStage = SA::kFloats + SB::kFloats;

  const int nstages = P.B / BK;
  sa.load(va, m0, 0);
  sb.load(vb, n0, 0);
  sa.store(lds);
  sb.store(lds + SA::kFloats);
  __syncthreads();

  // The whole stage loop is instantiated for both block-skip cases, so the
  // MFMA stream carries no branches and the accumulators stay in place.
  auto mainloop = [&](auto skip) __attribute__((always_inline)) {
    constexpr bool kSkip = decltype(skip)::value;
    for (int s = 0; s < nstages; ++s) {
      const int cur = s & 1;
      const float* bufA = lds + cur * kStage;
      const float* bufB = bufA + SA::kFloats;
      if (s + 1 < nstages) {
        sa.load(va, m0, (s + 1) * BK);
        sb.load(vb, n0, (s + 1) * BK);
      }
      // Fragments are double-buffered in registers: the reads for k-group
      // g+1 are issued before the MFMAs of group g, so LDS latency hides
      // behind them.
      if (active) {
        floatx4 fa[2][TM], fb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[0][i] = SA::frag(bufA, wm + 32 * i, 0, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[0][j] = SB::frag(bufB, wn + 32 * j, 0, lane);
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
          const int c = g & 1;
          if (g + 1 < BK / 8) {
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[c ^ 1][i] = SA::frag(bufA, wm + 32 * i, g + 1, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[c ^ 1][j] = SB::frag(bufB, wn + 32 * j, g + 1, lane);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                if (!kSkip || i <= j)
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[c][i][q], fb[c][j][q], acc[i][j], 0, 0, 0);
        }
      }
      if (s + 1 < nstages) {
        float* nxt = lds + (cur ^ 1) * kStage;
        sa.store(nxt);
        sb.store(nxt + SA::kFloats);
      }
      __syncthreads();
    }
  };
  if (SYM && skip_low)
    mainloop(std::true_type{});
  else
    mainloop(std::false_type{});

  gemm_epilogue<TM, TN, BM, BN, kGemmThreads, kPipe >= BM * (BN + 1) ? 1 : 2, SYM>(P, job, item, tm, tn, acc, lds,
                                                                                    red, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Large tiles for dense operands (A with k contiguous, B with n contiguous,
// B a multiple of 256): 256 x 256 output tiles, 16 waves of 64 x 64 each, one
// workgroup per CU.  Each thread moves one 16-byte piece of A and one of B
// per k-stage straight into LDS (global_load_lds_dwordx4: lane l of a wave
// writes 16 bytes at the wave's LDS base + 16 l), through a ring of three
// stages: the loads for stage s + 2 leave at the start of stage s, and a
// stage ends with a wait for the next stage's loads only, then one barrier.
// Twice the tile edge halves the operand traffic per flop of the 128 x 128
// kernel.
//
// LDS layout of a stage: A as [row][4 quads of 4 k], the quad index XOR-ed
// with big_swz(row) so that the 16-byte fragment reads hit every bank once;
// B as [k][256] with rows 4..7 of each group of 8 rotated by 32 columns, so
// that a fragment read (lanes 0..31 along row k, lanes 32..63 along row
// k + 4) covers all 64 banks.  Every stage issues its loads, past the last stage again
// the last one into the free buffer, so the count of loads in flight, and
// hence each wait, is the same on every path.
//
// Waves are placed on the 4 x 4 grid of 64 x 64 blocks so that on a diagonal
// tile of a symmetric product (6 blocks idle below the diagonal, 4 on it at
// three quarters of the work) the waves of each SIMD (w, w + 4, w + 8, w + 12
// share one, as HW_ID shows) carry 2 or 2.5 blocks of work instead of up to
// 3.75; two 32 x 32 blocks handed to idle waves even that out to 2.25.
// ---------------------------------------------------------------------------
constexpr int kBigThreads = 1024;
constexpr int kBigTile = 256;
// block (row, col) of wave w: 4 bits r * 4 + c per wave, w = 0 in the low bits
constexpr uint64_t kBigPlace = 0x9CDEF584A07B6321ull;
// XOR swizzle of the 16-byte k-quads of A's rows (4 per row): the fragment
// reads of 16 consecutive rows then cover all 64 banks (256 bytes) of LDS,
// and so do those of each 8 consecutive rows within 128 bytes.
__device__ __forceinline__ int big_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// The 64 x 64 block (wm, wn) of wave `wave` of a 256 x 256 tile and which of
// its four 32 x 32 blocks (bit 2 i + j) it computes.  Off-diagonal tiles:
// all four.  On a diagonal tile of a symmetric product: none below the
// diagonal, all but (1, 0) on it; and waves 2 and 3 (blocks (0, 3) and
// (1, 2)) hand their block (1, 1) to waves 8 and 9, idle below the diagonal
// on the SIMDs with less work, so that each SIMD computes 9 of the tile's 36
// upper 32 x 32 blocks.  Without `share` (epilogues that stage whole wave
// blocks through LDS) waves 2 and 3 keep their block (1, 1) and 8 and 9 idle.
__device__ __forceinline__ void big_wave_role(bool dtile, int wave, int& wm, int& wn, int& mask, bool share = true) {
  const bool helper = share && dtile && (wave == 8 || wave == 9);
  const int place = (int)((kBigPlace >> (4 * (helper ? wave - 6 : wave))) & 15);
  wm = (place >> 2) * 64;
  wn = (place & 3) * 64;
  mask = 0xF;
  if (dtile) {
    mask = wm > wn ? 0 : (wm == wn ? 0xB : 0xF);
    if (share && (wave == 2 || wave == 3)) mask = 0x7;
    if (helper) mask = 0x8;
  }
}

template <class Epi, bool SYM>
__global__ void __launch_bounds__(kBigThreads, 1) gemm_f32_big_kernel(const GemmLaunch<Epi> P) {
  constexpr int TM = 2, TN = 2, BM = kBigTile, BN = kBigTile, BK = 16, NT = kBigThreads;
  constexpr int kA = BM * BK, kStage = kA + BK * BN;  // floats
  constexpr int PH = 4;                                // phases of the symmetric epilogue's transpose
  static_assert((BM / PH) * (BN + 4) + NT / kWave <= 3 * kStage, "staging and reduction fit the ring");
  static_assert(BM * BK / 4 == NT && BK * BN / 4 == NT, "one 16-byte piece of A and of B per thread");
  // One LDS object only: with a second one (a separate reduction array) the
  // compiler no longer tells the ring's buffers apart and waits for every
  // load in flight before each LDS read.
  __shared__ __attribute__((aligned(16))) float lds[3 * kStage];
  float* const red = lds + 3 * kStage - NT / kWave;  // past the epilogue's transpose

  int job, tm, tn;
  int64_t item;
  decode_tile<SYM>(P, xcd_remap(blockIdx.x, P.total), job, item, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int B = P.B;
  const float* pa = P.a[job].base + item * (int64_t)B * B;
  const float* pb = P.b[job].base + item * (int64_t)B * B;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // diagonal blocks shared between waves only with the register-direct symmetric epilogue
  constexpr bool kShare = [] {
    if constexpr (Epi::kSym) return Epi::kDirect && !Epi::kReduce;
    return true;
  }();
  int wm, wn, mask;
  big_wave_role(SYM && tm == tn, wave, wm, wn, mask, kShare);

  // this thread's pieces: A row r, quad q (stored at quad q ^ swz); B row k, columns 4 nq..
  const float* srcA;
  const float* srcB;
  {
    const int r = tid >> 2, qs = tid & 3, qg = qs ^ big_swz(r);
    srcA = pa + (int64_t)(m0 + r) * B + 4 * qg;
    const int k = tid >> 6, nq = (tid & 63) ^ (((k >> 2) & 1) << 3);  // rows 4..7 of each 8 shifted by 128 B
    srcB = pb + (int64_t)k * B + n0 + 4 * nq;
  }
  const int nstages = B / BK;
  const int wbase = wave * 64 * 4;  // this wave's 1 KB of each operand region
  auto issue = [&](float* __restrict__ buf, int s) __attribute__((always_inline)) {
    const int k0 = min(s, nstages - 1) * BK;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcA + k0),
                                     (__attribute__((address_space(3))) void*)(buf + wbase), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(srcB + (int64_t)k0 * B),
                                     (__attribute__((address_space(3))) void*)(buf + kA + wbase), 16, 0, 0);
  };
  // s_waitcnt immediates: vmcnt(2) (the newest stage's two loads stay in flight) or vmcnt(0), with lgkmcnt(0)
  constexpr int kWaitAhead = 2 | (7 << 4);
  constexpr int kWaitAll = 0 | (7 << 4);

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  float* const b0 = lds;
  float* const b1 = lds + kStage;
  float* const b2 = lds + 2 * kStage;
  issue(b0, 0);
  issue(b1, 1);
  __builtin_amdgcn_s_waitcnt(kWaitAhead);
  __builtin_amdgcn_s_barrier();

  auto mainloop = [&](auto M) __attribute__((always_inline)) {
    constexpr int kMask = decltype(M)::value;
    // One stage: the loads for stage s + 2 into `wr` (pinned at the head of
    // the stage), then the MFMAs on `rd` (stage s).  The compiler lets the
    // LDS reads of `rd` pass the pending loads only because it can tell the
    // ring's buffers apart (restrict pointers into the kernel's one LDS
    // array); otherwise it would wait for every load before each read.
    auto step = [&](const float* __restrict__ rd, float* __restrict__ wr, int s) __attribute__((always_inline)) {
      issue(wr, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kMask != 0) {
        constexpr int kRows = ((kMask & 3) ? 1 : 0) | ((kMask & 12) ? 2 : 0);  // block rows i in use
        constexpr int kCols = ((kMask & 5) ? 1 : 0) | ((kMask & 10) ? 2 : 0);  // block columns j in use
        auto fragA = [&](int i, int g) __attribute__((always_inline)) {
          const int row = wm + 32 * i + (lane & 31), quad = 2 * g + (lane >> 5);
          return *reinterpret_cast<const floatx4*>(rd + 4 * (row * 4 + (quad ^ big_swz(row))));
        };
        auto fragB = [&](int j, int g) __attribute__((always_inline)) {
          // lanes 32..63 read rows 4..7 of the group, stored 32 columns over
          const float* q = rd + kA + (g * 8 + (lane >> 5) * 4) * BN + ((wn + 32 * j + (lane & 31)) ^ ((lane >> 5) << 5));
          floatx4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = q[e * BN];
          return x;
        };
        floatx4 fa[2][TM], fb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if ((kRows >> i) & 1) fa[0][i] = fragA(i, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if ((kCols >> j) & 1) fb[0][j] = fragB(j, 0);
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
          const int c = g & 1;
          if (g + 1 < BK / 8) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
              if ((kRows >> i) & 1) fa[c ^ 1][i] = fragA(i, g + 1);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              if ((kCols >> j) & 1) fb[c ^ 1][j] = fragB(j, g + 1);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                if ((kMask >> (2 * i + j)) & 1)
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[c][i][q], fb[c][j][q], acc[i][j], 0, 0, 0);
        }
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
  };
  if constexpr (SYM) {
    switch (mask) {
      case 0xF: mainloop(std::integral_constant<int, 0xF>{}); break;
      case 0xB: mainloop(std::integral_constant<int, 0xB>{}); break;
      case 0x7: mainloop(std::integral_constant<int, 0x7>{}); break;
      case 0x8: mainloop(std::integral_constant<int, 0x8>{}); break;
      default: mainloop(std::integral_constant<int, 0>{}); break;
    }
  } else {
    mainloop(std::integral_constant<int, 0xF>{});
  }
  // drain the loads issued past the last stage before the epilogue reuses LDS
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();

  // Through LDS (accumulators staged in PH phases): full products of epilogues
  // that ask for it, and symmetric products with a reduction (their epilogue
  // spills in registers; waves idle below the diagonal hold zeros, which that
  // path neither writes nor counts).
  constexpr bool kStaged = [] {
    if constexpr (Epi::kSym && SYM) return Epi::kReduce;
    return Epi::kBigStaged && !SYM;
  }();
  if constexpr (kStaged) {
    typename Epi::Tile tile(*(job == 0 ? &P.e[0] : &P.e[1]), item, P.B);
    const float part =
        staged_epilogue<TM, TN, BM, BN, NT, PH, Epi>(tile, acc, lds, m0, n0, wm, wn, lane, SYM, tm == tn);
    if constexpr (Epi::kReduce) {
      const float tot = block_sum<NT>(part, red);
      if (threadIdx.x == 0) {
        tile.partial(tm * P.tiles_n + tn, tot);
        if (SYM && tm != tn) tile.partial(tn * P.tiles_n + tm, tot);  // the mirrored tile
      }
    }
  } else {
    // mirrored half of symmetric tiles staged per 32 x 32 block (16 waves x 4.5 KB of the stage buffers)
    static_assert(NT / kWave * 32 * 36 + NT / kWave <= 3 * kStage, "staging and reduction fit the buffers");
    gemm_epilogue<TM, TN, BM, BN, NT, PH, SYM, 1, 1>(P, job, item, tm, tn, acc, lds, red, m0, n0, wm, wn, lane,
                                                     mask);
  }
}

// ---------------------------------------------------------------------------
// Epilogues.  Tile(job, item, B) is built once per workgroup; store(row, col,
// v) writes the output for one accumulator and returns its contribution to
// the tile's reduction (if any); partial(t, sum) stores that reduction.
// Epilogues with kSym also split store into value(row, col, v) -> o and
// write(row, col, o) for symmetric products; there the output at a mirrored
// position is the value formed at the computed one, which assumes the other
// inputs of the epilogue (an EMA state, Clenshaw terms) are symmetric too.
// Those with kDirect also provide value4(r, c, v) for rows r..r+3 of column c,
// write4t(c, r, o), which writes o to row c, columns r..r+3 (the mirrored
// entries) with vector stores, and write_upper(row, col, o),
// write_upper4(row, col, o) and write_upper8(row, col, lo, hi) (columns
// col..col+3 or col..col+7) for the computed entries themselves.
// ---------------------------------------------------------------------------

// out = mult * acc + beta * cin (cin may alias out); X = I for a degenerate
// factor when `status` is given.  mult = alpha * extra * c_f^pexp when
// `scale` is given, else alpha.
struct EpiStore {
  static constexpr bool kReduce = false;
  static constexpr bool kSym = true;
  static constexpr bool kDirect = true;
  // gemm_f32_big_kernel fits 128 VGPRs without spilling (symmetric / full);
  // kH16Big*: the same for gemm_h16_big_kernel, where it also has to pay off
  static constexpr bool kBigSym = true, kBigFull = false;
  static constexpr bool kBigStaged = false;  // full products of the large kernel: register-direct epilogue
  static constexpr bool kH16BigSym = true, kH16BigFull = false;
  static constexpr int kH16BigWaves = 16;
  static constexpr bool kH16Upper = true;  // operands and 16-bit copy may be kept on and above the diagonal only
  struct Job {
    float* out;          // fp32 output (may be null when only the 16-bit copy is needed)
    const float* cin;
    float alpha, beta;
    const shampoo_scale* scale;
    const int32_t* status;
    float pexp, extra;
    uint16_t* out16;     // optional 16-bit copy of the output (operand of a later product)
    int fmt16;           // H16_BF16 or H16_F16
    // symmetric products on the large 16-bit kernel: the 16-bit copy only in
    // tiles on and above the diagonal (the mirrored half is not written; the
    // other kernels write it in full)
    int upper16;
  };
  struct Tile {
    static constexpr int kPrefetch = 0;
    float* out;
    const float* cin;
    uint16_t* o16;
    uint16_t* o16m;      // the 16-bit copy's mirrored half of an off-diagonal tile (null: not written)
    int fmt;
    float mult, beta;
    bool ident;
    int B;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : B(B_) {
      const int64_t off = item * (int64_t)B_ * B_;
      out = j.out ? j.out + off : nullptr;
      cin = j.cin ? j.cin + off : nullptr;
      o16 = j.out16 ? j.out16 + off : nullptr;
      o16m = j.upper16 ? nullptr : o16;
      fmt = j.fmt16;
      beta = j.beta;
      mult = j.alpha;
      if (j.scale) mult *= j.extra * powf(safe_c(j.scale, j.status, item), j.pexp);
      ident = j.status && degenerate(j.status[item]);
    }
    __device__ __forceinline__ float value(int row, int col, float v) const {
      float o = mult * v;
      if (cin) o += beta * ldg(cin + (int64_t)row * B + col);
      if (ident) o = (row == col) ? 1.f : 0.f;
      return o;
    }
    __device__ __forceinline__ void write(int row, int col, float o) {
      const int64_t idx = (int64_t)row * B + col;
      if (out) stg(out + idx, o);
      if (o16) stg(o16 + idx, to_h16(o, fmt));
    }
    __device__ __forceinline__ floatx4 value4(int r, int c, const floatx4& v) const {
      floatx4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = value(r + e, c, v[e]);
      return o;
    }
    __device__ __forceinline__ void write4t(int c, int r, const floatx4& o) {
      const int64_t idx = (int64_t)c * B + r;
      if (out) stg(reinterpret_cast<floatx4*>(out + idx), o);
      if (o16) stg4_h16(o16 + idx, o, fmt);
    }
    // the mirrored entries of an off-diagonal tile
    __device__ __forceinline__ void write4t_mirror(int c, int r, const floatx4& o) {
      const int64_t idx = (int64_t)c * B + r;
      if (out) stg(reinterpret_cast<floatx4*>(out + idx), o);
      if (o16m) stg4_h16(o16m + idx, o, fmt);
    }
    __device__ __forceinline__ bool mirrored() const { return out != nullptr || o16m != nullptr; }
    __device__ __forceinline__ void write_upper(int row, int col, float o) { write(row, col, o); }
    // row `row`, columns col..col+3 (col..col+7), on or above the diagonal
    __device__ __forceinline__ void write_upper4(int row, int col, const floatx4& o) { write4t(row, col, o); }
    __device__ __forceinline__ void write_upper8(int row, int col, const floatx4& lo, const floatx4& hi) {
      const int64_t idx = (int64_t)row * B + col;
      if (out) {
        stg(reinterpret_cast<floatx4*>(out + idx), lo);
        stg(reinterpret_cast<floatx4*>(out + idx + 4), hi);
      }
      if (o16) stg8_h16(o16 + idx, lo, hi, fmt);
    }
    __device__ __forceinline__ float store(int row, int col, float v) {
      write(row, col, value(row, col, v));
      return 0.f;
    }
    __device__ void partial(int, float) {}
  };
};

// The two updates Y <- Y E and Z <- E Z of a Newton-DB iteration, launched
// together; a type of its own so that profiles list this launch separately.
struct EpiPair : EpiStore {};

// Output through a block descriptor: only rows x cols of the block is written.
struct EpiStoreDesc {
  static constexpr bool kBigSym = false, kBigFull = true;
  static constexpr bool kBigStaged = false;
  static constexpr bool kH16BigSym = false, kH16BigFull = true;
  static constexpr int kH16BigWaves = 16;
  static constexpr bool kSym = false;
  static constexpr bool kReduce = false;
  struct Job {
    const shampoo_block* out;
  };
  struct Tile {
    float* p;
    int64_t ld;
    int rows, cols;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B) {
      const shampoo_block d = j.out[item];
      const bool ok = d.ptr != nullptr && d.rows >= 0 && d.cols >= 0 && d.rows <= B && d.cols <= B &&
                      d.ld >= d.cols;
      p = d.ptr;
      ld = d.ld;
      rows = ok ? d.rows : 0;
      cols = ok ? d.cols : 0;
    }
    __device__ __forceinline__ float store(int row, int col, float v) {
      if (row < rows && col < cols) stg(p + (int64_t)row * ld + col, v);
      return 0.f;
    }
    __device__ void partial(int, float) {}
  };
};

// Newton-DB: P = Z Y -> E = (3 I - P) / 2, reduction ||I - P||_F^2.  Z and
// Y are polynomials in A_s, so P is symmetric and may be formed from upper
// tiles.
struct EpiNdbE {
  static constexpr bool kSym = true;
  static constexpr bool kDirect = false;
  static constexpr bool kBigSym = true, kBigFull = true;
  static constexpr bool kBigStaged = false;
  static constexpr bool kH16BigSym = false, kH16BigFull = false;
  static constexpr int kH16BigWaves = 16;
  static constexpr bool kReduce = true;
  struct Job {
    float* e;
    float* partials;  // [nitems][tiles]
    int tiles;
  };
  struct Tile {
    float* e;
    float* part;
    int B;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : B(B_) {
      e = j.e + item * (int64_t)B_ * B_;
      part = j.partials + item * j.tiles;
    }
    __device__ __forceinline__ float value(int row, int col, float v) const {
      return 1.5f * ((row == col) ? 1.f : 0.f) - 0.5f * v;
    }
    __device__ __forceinline__ void write(int row, int col, float o) { stg(e + (int64_t)row * B + col, o); }
    __device__ __forceinline__ float contrib(int row, int col, float v) const {
      const float r = ((row == col) ? 1.f : 0.f) - v;
      return r * r;
    }
    __device__ __forceinline__ float store(int row, int col, float v) {
      write(row, col, value(row, col, v));
      return contrib(row, col, v);
    }
    __device__ void partial(int t, float s) { stg(part + t, s); }
  };
};

// Coupled Newton: M' = C^p M -> store M' and C' = ((p+1) I - M') / p,
// reduction ||I - M'||_F^2.  C^p and M are polynomials in A_s, so M' is
// symmetric and may be formed from upper tiles.
struct EpiCnM {
  static constexpr bool kSym = true;
  static constexpr bool kDirect = false;
  // on the large fp32 kernel with the epilogue through LDS, full and
  // symmetric products alike (in registers it spills there)
  static constexpr bool kBigSym = true, kBigFull = true;
  static constexpr bool kBigStaged = true;
  // 16-bit: the 8-wave layout with its epilogue through LDS
  static constexpr bool kH16BigSym = true, kH16BigFull = true;
  static constexpr int kH16BigWaves = 8;
  static constexpr bool kH16Upper = true;  // operands may be kept on and above the diagonal only
  static constexpr bool kReduce = true;
  struct Job {
    float* m;            // fp32 outputs (null: not written)
    float* c;
    uint16_t* m16;       // 16-bit copies (null: not written)
    uint16_t* c16;
    int fmt16;
    float* partials;
    int tiles;
    float p;
  };
  struct Tile {
    float* m;
    float* c;
    uint16_t* m16;
    uint16_t* c16;
    int fmt;
    float* part;
    float p1, pinv;
    int B;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : B(B_) {
      const int64_t off = item * (int64_t)B_ * B_;
      m = j.m ? j.m + off : nullptr;
      c = j.c ? j.c + off : nullptr;
      m16 = j.m16 ? j.m16 + off : nullptr;
      c16 = j.c16 ? j.c16 + off : nullptr;
      fmt = j.fmt16;
      part = j.partials + item * j.tiles;
      p1 = j.p + 1.f;
      pinv = 1.f / j.p;
    }
    __device__ __forceinline__ float value(int, int, float v) const { return v; }
    // M' = o at (row, col) and the matching entry of C'
    __device__ __forceinline__ void write(int row, int col, float o) {
      const int64_t idx = (int64_t)row * B + col;
      const float cv = (p1 * ((row == col) ? 1.f : 0.f) - o) * pinv;
      if (m) stg(m + idx, o);
      if (c) stg(c + idx, cv);
      if (m16) stg(m16 + idx, to_h16(o, fmt));
      if (c16) stg(c16 + idx, to_h16(cv, fmt));
    }
    __device__ __forceinline__ float contrib(int row, int col, float v) const {
      const float r = ((row == col) ? 1.f : 0.f) - v;
      return r * r;
    }
    __device__ __forceinline__ float store(int row, int col, float v) {
      write(row, col, v);
      return contrib(row, col, v);
    }
    // store for columns col..col+7 of row `row` (col a multiple of 8), with
    // vector stores; returns the 8 entries' share of the reduction
    __device__ __forceinline__ float store8(int row, int col, const floatx4& lo, const floatx4& hi) {
      const int64_t idx = (int64_t)row * B + col;
      floatx4 clo, chi;
      float r = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dl = (row == col + e) ? 1.f : 0.f, dh = (row == col + 4 + e) ? 1.f : 0.f;
        clo[e] = (p1 * dl - lo[e]) * pinv;
        chi[e] = (p1 * dh - hi[e]) * pinv;
        r += (dl - lo[e]) * (dl - lo[e]);
        r += (dh - hi[e]) * (dh - hi[e]);
      }
      if (m) {
        stg(reinterpret_cast<floatx4*>(m + idx), lo);
        stg(reinterpret_cast<floatx4*>(m + idx + 4), hi);
      }
      if (c) {
        stg(reinterpret_cast<floatx4*>(c + idx), clo);
        stg(reinterpret_cast<floatx4*>(c + idx + 4), chi);
      }
      if (m16) stg8_h16(m16 + idx, lo, hi, fmt);
      if (c16) stg8_h16(c16 + idx, clo, chi, fmt);
      return r;
    }
    __device__ void partial(int t, float s) { stg(part + t, s); }
  };
};

// Clenshaw step with T = 2 A_s - I applied in the epilogue (acc = A_s b1):
//   b = cj I + 4 acc - 2 b1 - b2                        (final == 0)
//   X = mult (cj I + 2 acc - b1 - b2), I if degenerate   (final == 1, cj = c_0)
// An optional 16-bit copy of b is written for the next half-width product.
struct EpiClenshaw {
  static constexpr bool kH16Upper = true;  // operands and 16-bit copy may be kept on and above the diagonal only
  static constexpr bool kReduce = false;
  static constexpr bool kSym = true;
  static constexpr bool kDirect = true;
  static constexpr bool kBigSym = true, kBigFull = false;
  static constexpr bool kBigStaged = false;
  // 16-bit: the 8-wave layout, whose registers let the epilogue load 4
  // groups of b1/b2 ahead (the 16-wave one, with 1, measured slower)
  static constexpr bool kH16BigSym = true, kH16BigFull = false;
  static constexpr int kH16BigWaves = 8;
  struct Job {
    float* out;
    uint16_t* out16;     // optional 16-bit copy of b (operand of the next product)
    int fmt16;
    const float* b1;
    const float* b2;     // null: b2 = c2 I, formed here (the loads for it then read b1's lines)
    float cj;
    float c2;
    int final;
    const shampoo_scale* scale;
    const int32_t* status;
    float pexp;
    int upper16;         // the 16-bit copy only in tiles on and above the diagonal (mirrored half not written)
  };
  struct Tile {
    static constexpr int kPrefetch = 4;  // groups whose b1, b2 are loaded per chunk
    struct Pre {
      floatx4 x1, x2;
    };
    float* out;
    uint16_t* obf;
    int fmt;
    const float* b1;
    const float* b2;
    float cj, mult, k1, k2, c2;
    bool ident, is_final, b2_diag, upper16;
    int B;
    __device__ __forceinline__ Tile(const Job& j, int64_t item, int B_) : B(B_) {
      upper16 = j.upper16 != 0;
      const int64_t off = item * (int64_t)B_ * B_;
      out = j.out + off;
      obf = j.out16 ? j.out16 + off : nullptr;
      fmt = j.fmt16;
      b1 = j.b1 + off;
      b2_diag = j.b2 == nullptr;
      b2 = b2_diag ? b1 : j.b2 + off;
      c2 = j.c2;
      cj = j.cj;
      is_final = j.final != 0;
      if (j.final) {
        k1 = 2.f;
        k2 = 1.f;
        mult = powf(safe_c(j.scale, j.status, item), j.pexp);
        ident = j.status && degenerate(j.status[item]);
      } else {
        k1 = 4.f;
        k2 = 2.f;
        mult = 1.f;
        ident = false;
      }
    }
    __device__ __forceinline__ float value(int row, int col, float v) const {
      const int64_t idx = (int64_t)row * B + col;
      const float d = (row == col) ? cj : 0.f;
      const float x2 = b2_diag ? ((row == col) ? c2 : 0.f) : ldg(b2 + idx);
      float o = mult * (d + k1 * v - k2 * ldg(b1 + idx) - x2);
      if (ident) o = (row == col) ? 1.f : 0.f;
      return o;
    }
    __device__ __forceinline__ void write(int row, int col, float o) {
      const int64_t idx = (int64_t)row * B + col;
      stg(out + idx, o);
      if (obf) stg(obf + idx, to_h16(o, fmt));
    }
    // b1 and b2 come from symmetric steps (mirrored writes), so they are read
    // at the transposed position: row c, columns r..r+3, one vector load each.
    __device__ __forceinline__ Pre prefetch4(int r, int c) const {
      const int64_t idx = (int64_t)c * B + r;
      return Pre{ldg(reinterpret_cast<const floatx4*>(b1 + idx)), ldg(reinterpret_cast<const floatx4*>(b2 + idx))};
    }
    __device__ __forceinline__ floatx4 value4p(int r, int c, const floatx4& v, const Pre& p) const {
      floatx4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool dg = (r + e == c);
        const float x2 = b2_diag ? (dg ? c2 : 0.f) : p.x2[e];
        o[e] = ident ? (dg ? 1.f : 0.f) : mult * ((dg ? cj : 0.f) + k1 * v[e] - k2 * p.x1[e] - x2);
      }
      return o;
    }
    __device__ __forceinline__ floatx4 value4(int r, int c, const floatx4& v) const {
      return value4p(r, c, v, prefetch4(r, c));
    }
    __device__ __forceinline__ void write4t(int c, int r, const floatx4& o) {
      const int64_t idx = (int64_t)c * B + r;
      stg(reinterpret_cast<floatx4*>(out + idx), o);
      if (obf) stg4_h16(obf + idx, o, fmt);
    }
    // the mirrored entries of an off-diagonal tile: the 16-bit copy there only
    // when it is kept in full (upper16 clear); fp32 b is read back there
    __device__ __forceinline__ void write4t_mirror(int c, int r, const floatx4& o) {
      const int64_t idx = (int64_t)c * B + r;
      stg(reinterpret_cast<floatx4*>(out + idx), o);
      if (obf && !upper16) stg4_h16(obf + idx, o, fmt);
    }
    // When the next product takes its operand from the 16-bit copy, an
    // intermediate fp32 b is read back only at transposed positions (value4),
    // i.e. on and below the diagonal, which the mirrored writes cover: its
    // fp32 value above the diagonal is then not stored.  Without a 16-bit
    // copy the fp32 b is the next product's operand and is stored in full,
    // and so is the final X.
    __device__ __forceinline__ void write_upper(int row, int col, float o) {
      const int64_t idx = (int64_t)row * B + col;
      if (obf == nullptr || is_final || row == col) stg(out + idx, o);
      if (obf) stg(obf + idx, to_h16(o, fmt));
    }
    // row `row`, columns col..col+3 (col..col+7), on or above the diagonal
    __device__ __forceinline__ void write_upper4(int row, int col, const floatx4& o) {
      const int64_t idx = (int64_t)row * B + col;
      if (obf == nullptr || is_final)
        stg(reinterpret_cast<floatx4*>(out + idx), o);
      else if (row >= col && row < col + 4)
        stg(out + (int64_t)row * B + row, o[row - col]);
      if (obf) stg4_h16(obf + idx, o, fmt);
    }
    __device__ __forceinline__ void write_upper8(int row, int col, const floatx4& lo, const floatx4& hi) {
      const int64_t idx = (int64_t)row * B + col;
      if (obf == nullptr || is_final) {
        stg(reinterpret_cast<floatx4*>(out + idx), lo);
        stg(reinterpret_cast<floatx4*>(out + idx + 4), hi);
      } else if (row >= col && row < col + 8) {
        const int e = row - col;
        stg(out + (int64_t)row * B + row, e < 4 ? lo[e & 3] : hi[e & 3]);
      }
      if (obf) stg8_h16(obf + idx, lo, hi, fmt);
    }
    __device__ __forceinline__ float store(int row, int col, float v) {
      write(row, col, value(row, col, v));
      return 0.f;
    }
    __device__ void partial(int, float) {}
  };
};

}  // namespace shp
