// C entry points of the Shampoo block-preconditioner library (gfx950).
//
// Every call validates its arguments on the host, carves its scratch buffers
// out of the caller's workspace and enqueues kernels on the caller's stream;
// nothing is allocated and nothing synchronises.
#include <cmath>
#include <cstring>
#include <mutex>

#include "gemm_bf16.h"
#include "kernels_misc.h"

using namespace shp;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxB = 16384;
constexpr size_t kScratchBytes = SHAMPOO_NOALLOC_SCRATCH_BYTES;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_B(int B) { return B >= 64 && B <= kMaxB && (B % 64) == 0; }

int check_launch() { return hipGetLastError() == hipSuccess ? SHAMPOO_OK : SHAMPOO_EHIP; }

// Timing hook (shampoo_timing_hook): events recorded around launches of one
// kernel family on the launch's own stream.
struct TimingHook {
  int families = 0;
  hipEvent_t* events = nullptr;
  int32_t* fam_out = nullptr;
  int capacity = 0;
  int count = 0;
} g_timing;

bool timing_on(int fam) {
  return (g_timing.families & fam) != 0 && g_timing.count < g_timing.capacity;
}
void timing_before(int fam, hipStream_t st) {
  if (timing_on(fam)) (void)hipEventRecord(g_timing.events[2 * g_timing.count], st);
}
void timing_after(int fam, hipStream_t st) {
  if (timing_on(fam)) {
    (void)hipEventRecord(g_timing.events[2 * g_timing.count + 1], st);
    if (g_timing.fam_out != nullptr) g_timing.fam_out[g_timing.count] = fam;
    ++g_timing.count;
  }
}

// Sequential carving of a workspace; `base == nullptr` only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

size_t stack_elems(int64_t n, int B) { return (size_t)n * (size_t)B * (size_t)B; }

int ew_chunks(int B) {
  const int64_t n4 = (int64_t)B * B / 4;
  int64_t c = n4 / 4096;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  return (int)c;
}

// Output tile edge of an fp32 launch covering `items` products (jobs x
// factors): gemm_f32_big_kernel's 256 x 256 tiles for dense operands when B is
// a multiple of 256 and the epilogue fits that kernel's register budget, else
// gemm_f32_kernel's 128 x 128 (B a multiple of 128) or 64 x 64 tiles -- the
// largest of these whose grid still gives every compute unit a workgroup,
// and the 64 x 64 tiles when none does (a small batch is bound by how many
// compute units it occupies, not by the per-tile efficiency of larger tiles).
// The large tiles run one workgroup per compute unit, so their grid is also
// taken only when it fills whole rounds of the GPU or at least four rounds
// (a grid of 1.5 rounds leaves half the GPU idle in its second round; the
// 128 x 128 kernel runs several workgroups per unit and balances there).
constexpr int64_t kComputeUnits = 256;

template <class Epi>
int f32_tile_edge(int B, bool sym, bool dense, int64_t items) {
  auto grid = [&](int T) {
    const int64_t t = B / T;
    return items * (sym ? t * (t + 1) / 2 : t * t);
  };
  const bool fits = sym ? Epi::kBigSym : Epi::kBigFull;
  const bool mid = B % 128 == 0 && grid(128) >= kComputeUnits;
  if (dense && fits && B % kBigTile == 0 && grid(kBigTile) >= kComputeUnits) {
    const int64_t g = grid(kBigTile);
    if (g % kComputeUnits == 0 || g >= 4 * kComputeUnits || !mid) return kBigTile;
  }
  if (mid) return 128;
  return 64;
}

// Tile count (reduction partials per item) of a product of dense stacks.
template <class Epi>
int f32_tiles(int B, bool sym, int64_t items) {
  const int t = B / f32_tile_edge<Epi>(B, sym, true, items);
  return t * t;
}

// The most tiles any fp32 product of size B uses (workspace sizing).
int gemm_tiles_max(int B) {
  const int t = B / 64;
  return t * t;
}

// ---------------------------------------------------------------------------
// Batched product launch.
// ---------------------------------------------------------------------------
template <int LA, int LB, bool DA, bool DB, class Epi>
int run_gemm(const Operand* a, const Operand* b, const typename Epi::Job* e, int njobs, int64_t nitems,
             int B, bool sym, hipStream_t st, int fam = 0) {
  if (!Epi::kSym && sym) return SHAMPOO_EINVAL;  // no symmetric epilogue
  GemmLaunch<Epi> P;
  memset(&P, 0, sizeof(P));
  for (int j = 0; j < njobs; ++j) {
    P.a[j] = a[j];
    P.b[j] = b[j];
    P.e[j] = e[j];
  }
  const int T = f32_tile_edge<Epi>(B, sym, LA == KCONTIG && LB == MNCONTIG && !DA && !DB, (int64_t)njobs * nitems);
  const bool big = T == kBigTile;
  P.nitems = nitems;
  P.B = B;
  P.tiles_n = B / T;
  P.tiles_per_item = sym ? P.tiles_n * (P.tiles_n + 1) / 2 : P.tiles_n * P.tiles_n;
  const uint64_t total = (uint64_t)njobs * (uint64_t)nitems * (uint64_t)P.tiles_per_item;
  if (total == 0) return SHAMPOO_OK;
  if (total > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  P.total = (uint32_t)total;
  timing_before(fam, st);
  bool launched = false;
  if constexpr (LA == KCONTIG && LB == MNCONTIG && !DA && !DB) {
    if (big) {
      if constexpr (Epi::kSym && Epi::kBigSym) {
        if (sym) {
          hipLaunchKernelGGL((gemm_f32_big_kernel<Epi, true>), dim3(P.total), dim3(kBigThreads), 0, st, P);
          launched = true;
        }
      }
      if constexpr (Epi::kBigFull) {
        if (!sym) {
          hipLaunchKernelGGL((gemm_f32_big_kernel<Epi, false>), dim3(P.total), dim3(kBigThreads), 0, st, P);
          launched = true;
        }
      }
      if (!launched) return SHAMPOO_EUNSUPPORTED;  // unreachable: f32_tile_edge chose this kernel
    }
  }
  if constexpr (Epi::kSym) {
    if (sym && !launched) {
      if (T == 128)
        hipLaunchKernelGGL((gemm_f32_kernel<2, 2, LA, LB, DA, DB, Epi, true>), dim3(P.total), dim3(kGemmThreads), 0,
                           st, P);
      else
        hipLaunchKernelGGL((gemm_f32_kernel<1, 1, LA, LB, DA, DB, Epi, true>), dim3(P.total), dim3(kGemmThreads), 0,
                           st, P);
      launched = true;
    }
  }
  if (!launched) {
    if (T == 128)
      hipLaunchKernelGGL((gemm_f32_kernel<2, 2, LA, LB, DA, DB, Epi, false>), dim3(P.total), dim3(kGemmThreads), 0,
                         st, P);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<1, 1, LA, LB, DA, DB, Epi, false>), dim3(P.total), dim3(kGemmThreads), 0,
                         st, P);
  }
  timing_after(fam, st);
  return check_launch();
}

Operand dense(const float* p) { return Operand{p, nullptr}; }
Operand blocks(const shampoo_block* d) { return Operand{nullptr, d}; }

// Plain product of two dense stacks, C = A B, with the given epilogue.
// With `sym`, the product is known to be symmetric (in exact arithmetic):
// only the upper-triangular tiles are computed and mirrored.
template <class Epi>
int gemm_nn(const float* const* A, const float* const* Bm, const typename Epi::Job* e, int njobs, int64_t n,
            int B, hipStream_t st, bool sym = false, int fam = 0) {
  Operand oa[2], ob[2];
  for (int j = 0; j < njobs; ++j) {
    oa[j] = dense(A[j]);
    ob[j] = dense(Bm[j]);
  }
  return run_gemm<KCONTIG, MNCONTIG, false, false, Epi>(oa, ob, e, njobs, n, B, sym, st, fam);
}

template <int MODE>
int run_ew(const EwArgs& a, int64_t nf, hipStream_t st) {
  const uint64_t grid = (uint64_t)nf * a.chunks;
  if (grid == 0) return SHAMPOO_OK;
  if (grid > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  hipLaunchKernelGGL(ew_kernel<MODE>, dim3((uint32_t)grid), dim3(256), 0, st, a);
  return check_launch();
}

// `first`: the residual opens a pass (its running minimum restarts there).
int run_resid(const float* partials, int count, float* resid, int ncols, int col, float* rmin, bool first,
              int32_t* status, int64_t nf, hipStream_t st) {
  hipLaunchKernelGGL(resid_kernel, dim3((uint32_t)nf), dim3(64), 0, st, partials, count, resid, ncols, col, rmin,
                     first ? 1 : 0, status);
  return check_launch();
}

#define SHP_TRY(x)                \
  do {                            \
    const int rc_ = (x);          \
    if (rc_ != SHAMPOO_OK) return rc_; \
  } while (0)

// A small pool of equally sized stacks for the iterations.
struct Pool {
  float* buf[8];
  bool used[8];
  int n = 0;
  float* get() {
    for (int i = 0; i < n; ++i)
      if (!used[i]) {
        used[i] = true;
        return buf[i];
      }
    return nullptr;
  }
  void put(float* p) {
    for (int i = 0; i < n; ++i)
      if (buf[i] == p) used[i] = false;
  }
};

// ---------------------------------------------------------------------------
// Workspace layouts.
// ---------------------------------------------------------------------------
struct NewtonWs {
  Pool pool;
  float* partials;
  float* rmin;  // smallest residual of the current pass, per factor
};

// A pool of 16-bit stacks for the half-width coupled Newton.
struct Pool16 {
  uint16_t* buf[8];
  bool used[8];
  int n = 0;
  uint16_t* get() {
    for (int i = 0; i < n; ++i)
      if (!used[i]) {
        used[i] = true;
        return buf[i];
      }
    return nullptr;
  }
  void put(uint16_t* p) {
    for (int i = 0; i < n; ++i)
      if (buf[i] == p) used[i] = false;
  }
};

struct Cn16Ws {
  Pool16 pool;
  float* c32;       // fp32 C_0 (one iteration only)
  float* partials;
  float* rmin;      // smallest residual so far, per factor
};

size_t cn16_layout(Carver& c, int64_t nf, int B, Cn16Ws* out) {
  Cn16Ws w;
  w.c32 = c.take<float>(stack_elems(nf, B));
  w.pool.n = 7;
  for (int i = 0; i < 7; ++i) {
    w.pool.buf[i] = c.take<uint16_t>(stack_elems(nf, B));
    w.pool.used[i] = false;
  }
  const int cnt = gemm_tiles_max(B) > ew_chunks(B) ? gemm_tiles_max(B) : ew_chunks(B);
  w.partials = c.take<float>((size_t)nf * cnt);
  w.rmin = c.take<float>((size_t)nf);
  if (out) *out = w;
  return c.off;
}

size_t newton_layout(Carver& c, int64_t nf, int B, int variant, NewtonWs* out) {
  if (variant == SHAMPOO_CN_F16) return cn16_layout(c, nf, B, nullptr);
  const int nbuf = (variant == SHAMPOO_CN) ? 7 : 5;
  NewtonWs w;
  w.pool.n = nbuf;
  for (int i = 0; i < nbuf; ++i) {
    w.pool.buf[i] = c.take<float>(stack_elems(nf, B));
    w.pool.used[i] = false;
  }
  const int cnt = gemm_tiles_max(B) > ew_chunks(B) ? gemm_tiles_max(B) : ew_chunks(B);
  w.partials = c.take<float>((size_t)nf * cnt);
  w.rmin = c.take<float>((size_t)nf);
  if (out) *out = w;
  return c.off;
}

struct ScaleWs {
  float* w[2];
  float* norm[2];
  float* rq;
  float* sumsq;
};

int pi_panel(int B) { return (B % 128 == 0) ? 128 : 64; }

size_t scale_layout(Carver& c, int64_t nf, int B, ScaleWs* out) {
  ScaleWs w;
  const int np = B / pi_panel(B);
  w.w[0] = c.take<float>((size_t)nf * B * kPiCols);
  w.w[1] = c.take<float>((size_t)nf * B * kPiCols);
  w.norm[0] = c.take<float>((size_t)nf * np * kPiCols);
  w.norm[1] = c.take<float>((size_t)nf * np * kPiCols);
  w.rq = c.take<float>((size_t)nf * np * kPiCols);
  w.sumsq = c.take<float>((size_t)nf * ew_chunks(B));
  if (out) *out = w;
  return c.off;
}

struct ChebyWs {
  float* as;
  float* b[3];
  uint16_t* as_t16;    // bf16 copy of A_s^T
  uint16_t* b16[2];    // bf16 copies of the Clenshaw terms
};

size_t cheby_layout(Carver& c, int64_t nf, int B, int prec, ChebyWs* out) {
  ChebyWs w;
  // the bf16-input path keeps A_s only as its transposed bf16 copy
  w.as = (prec == SHAMPOO_BF16_IN) ? nullptr : c.take<float>(stack_elems(nf, B));
  for (int i = 0; i < 3; ++i) w.b[i] = c.take<float>(stack_elems(nf, B));
  w.as_t16 = nullptr;
  w.b16[0] = w.b16[1] = nullptr;
  if (prec == SHAMPOO_BF16_IN) {
    w.as_t16 = c.take<uint16_t>(stack_elems(nf, B));
    w.b16[0] = c.take<uint16_t>(stack_elems(nf, B));
    w.b16[1] = c.take<uint16_t>(stack_elems(nf, B));
  }
  if (out) *out = w;
  return c.off;
}

struct PrecondWs {
  float* t1;
  uint16_t* a16;   // bf16 X_L
  uint16_t* b16;   // bf16 G^T (as rows), then X_R^T
  uint16_t* t16;   // bf16 T1
};

size_t precond_layout(Carver& c, int64_t n, int B, int prec, PrecondWs* out) {
  PrecondWs w;
  w.t1 = nullptr;
  w.a16 = w.b16 = w.t16 = nullptr;
  if (prec == SHAMPOO_BF16_IN) {
    w.a16 = c.take<uint16_t>(stack_elems(n, B));
    w.b16 = c.take<uint16_t>(stack_elems(n, B));
    w.t16 = c.take<uint16_t>(stack_elems(n, B));
  } else {
    w.t1 = c.take<float>(stack_elems(n, B));
  }
  if (out) *out = w;
  return c.off;
}

int graft_chunks(int B) {
  int c = B / 64;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  return c;
}

size_t graft_layout(Carver& c, int64_t n, int B, float** partials) {
  float* p = c.take<float>((size_t)n * graft_chunks(B) * 2);
  if (partials) *partials = p;
  return c.off;
}

struct AccumWs {
  uint16_t* g16;   // bf16 G
  uint16_t* gt16;  // bf16 G^T
};

size_t accum_layout(Carver& c, int64_t n, int B, int prec, AccumWs* out) {
  AccumWs w;
  w.g16 = w.gt16 = nullptr;
  if (prec == SHAMPOO_BF16_IN) {
    w.g16 = c.take<uint16_t>(stack_elems(n, B));
    w.gt16 = c.take<uint16_t>(stack_elems(n, B));
  }
  if (out) *out = w;
  return c.off;
}

// ---------------------------------------------------------------------------
// Newton-DB.
// ---------------------------------------------------------------------------

// Where the last product of a pass goes.
struct FinalOut {
  float* x;                   // x_out, or nullptr: keep the result in a pool buffer
  const shampoo_scale* sc;
  const int32_t* status;
  float pexp, extra;
};

EpiStore::Job final_job(const FinalOut& fo) {
  EpiStore::Job j;
  j.out16 = nullptr;
  j.fmt16 = H16_BF16;
  j.out = fo.x;
  j.cin = nullptr;
  j.alpha = 1.f;
  j.beta = 0.f;
  j.scale = fo.sc;
  j.status = fo.status;
  j.pexp = fo.pexp;
  j.extra = fo.extra;
  j.upper16 = 0;
  return j;
}

EpiStore::Job plain_job(float* out, uint16_t* out16 = nullptr, int fmt16 = H16_BF16) {
  EpiStore::Job j;
  j.out16 = out16;
  j.fmt16 = fmt16;
  j.out = out;
  j.cin = nullptr;
  j.alpha = 1.f;
  j.beta = 0.f;
  j.scale = nullptr;
  j.status = nullptr;
  j.pexp = 0.f;
  j.extra = 1.f;
  j.upper16 = 0;
  return j;
}

struct NdbCtx {
  int64_t nf;
  int B;
  int iters;
  float* resid;
  int ncols;
  int32_t* status;
  NewtonWs* ws;
  hipStream_t st;
  bool sym;    // the updates Y E and E Z are symmetric: upper tiles only
  bool sym_p;  // P = Z Y from upper tiles too (opt-in, see SHAMPOO_SYM_COUPLING)
};

// One Newton-DB pass.  The prologue reads `src` and forms Y0 = a src + b I
// (a, b per factor from `sc` when given, else ua/ub).  If `y0_in_src`, Y0 is
// `src` itself (a = 1, b = 0) and is not copied.  A `src` that is a pool
// buffer is owned by the pass and returned to the pool once it is dead.
// `want_y` selects which iterate is the pass's result (Y if true, else Z).
// With fo.x set the result is written to fo.x through the final epilogue;
// else *result receives the pool buffer holding it.
int ndb_pass(const NdbCtx& c, const float* src, bool y0_in_src, const shampoo_scale* sc, float ua, float ub,
             bool want_y, int pass, const FinalOut& fo, float** result) {
  Pool& pool = c.ws->pool;
  const int B = c.B;
  const int64_t nf = c.nf;
  float* Y = y0_in_src ? const_cast<float*>(src) : pool.get();
  float* E = pool.get();
  if (Y == nullptr || E == nullptr) return SHAMPOO_EWORKSPACE;
  if (E == nullptr) return SHAMPOO_EWORKSPACE;
  if (!y0_in_src) pool.put(const_cast<float*>(src));  // no-op for the caller's factors

  EwArgs a;
  memset(&a, 0, sizeof(a));
  a.x = src;
  a.out0 = y0_in_src ? nullptr : Y;
  a.out1 = E;
  a.partials = c.ws->partials;
  a.sc = sc;
  a.status = c.status;
  a.ua = ua;
  a.ub = ub;
  a.p = 2.f;
  a.B = B;
  a.chunks = ew_chunks(B);
  SHP_TRY(run_ew<EW_NDB_START>(a, nf, c.st));
  SHP_TRY(run_resid(c.ws->partials, a.chunks, c.resid, c.ncols, pass * c.iters, c.ws->rmin, true, c.status, nf,
                    c.st));

  const int tiles = f32_tiles<EpiNdbE>(B, c.sym_p, nf);
  float* Z = E;  // Z_1 = E_0 (Z_0 = I)
  // Iteration 1: Y_1 = Y_0 E_0.
  if (c.iters == 1) {
    if (want_y) {
      if (fo.x) {
        EpiStore::Job j = final_job(fo);
        const float* A[1] = {Y};
        const float* Bm[1] = {E};
        SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, c.st, c.sym));
        *result = nullptr;
      } else {
        float* Yn = pool.get();
        if (Yn == nullptr) return SHAMPOO_EWORKSPACE;
        EpiStore::Job j = plain_job(Yn);
        const float* A[1] = {Y};
        const float* Bm[1] = {E};
        SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, c.st, c.sym));
        *result = Yn;
      }
      pool.put(Y);
      pool.put(E);
    } else {
      if (fo.x) {
        EwArgs s;
        memset(&s, 0, sizeof(s));
        s.x = E;
        s.out0 = fo.x;
        s.sc = fo.sc;
        s.status = fo.status;
        s.pexp = fo.pexp;
        s.extra = fo.extra;
        s.p = 1.f;
        s.B = B;
        s.chunks = ew_chunks(B);
        SHP_TRY(run_ew<EW_SCALE_COPY>(s, nf, c.st));
        pool.put(E);
        *result = nullptr;
      } else {
        *result = E;
      }
      pool.put(Y);
    }
    return SHAMPOO_OK;
  }
  {
    float* Yn = pool.get();
    if (Yn == nullptr) return SHAMPOO_EWORKSPACE;
    EpiStore::Job j = plain_job(Yn);
    const float* A[1] = {Y};
    const float* Bm[1] = {E};
    SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, c.st, c.sym));
    pool.put(Y);
    Y = Yn;
  }
  for (int it = 1; it < c.iters; ++it) {
    // P = Z Y -> E = (3I - P)/2 and ||I - P||^2 partials.
    float* En = pool.get();
    if (En == nullptr) return SHAMPOO_EWORKSPACE;
    {
      EpiNdbE::Job j;
      j.e = En;
      j.partials = c.ws->partials;
      j.tiles = tiles;
      const float* A[1] = {Z};
      const float* Bm[1] = {Y};
      SHP_TRY(gemm_nn<EpiNdbE>(A, Bm, &j, 1, nf, B, c.st, c.sym_p, SHAMPOO_TIME_NDB_P));
      SHP_TRY(run_resid(c.ws->partials, tiles, c.resid, c.ncols, pass * c.iters + it, c.ws->rmin, false, c.status,
                        nf, c.st));
    }
    const bool last = (it == c.iters - 1);
    if (!last) {
      float* Yn = pool.get();
      if (Yn == nullptr) return SHAMPOO_EWORKSPACE;
      float* Zn = pool.get();
      if (Zn == nullptr) return SHAMPOO_EWORKSPACE;
      EpiPair::Job j[2] = {plain_job(Yn), plain_job(Zn)};
      const float* A[2] = {Y, En};
      const float* Bm[2] = {En, Z};
      SHP_TRY(gemm_nn<EpiPair>(A, Bm, j, 2, nf, B, c.st, c.sym, SHAMPOO_TIME_NDB_PAIR));
      pool.put(Y);
      pool.put(Z);
      pool.put(En);
      Y = Yn;
      Z = Zn;
    } else {
      float* dst = fo.x ? nullptr : pool.get();
      if (!fo.x && dst == nullptr) return SHAMPOO_EWORKSPACE;
      EpiStore::Job j = fo.x ? final_job(fo) : plain_job(dst);
      const float* A[1] = {want_y ? Y : En};
      const float* Bm[1] = {want_y ? En : Z};
      SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, c.st, c.sym));
      pool.put(Y);
      pool.put(Z);
      pool.put(En);
      *result = dst;
    }
  }
  return SHAMPOO_OK;
}

int newton_db(const float* F, const shampoo_scale* sc, int64_t nf, int B, int p, bool zchain, int iters,
              float* x, float* resid, int32_t* status, NewtonWs* ws, hipStream_t st, bool sym, bool sym_c) {
  NdbCtx c{nf, B, iters, resid, (p == 2 ? 1 : 2) * iters, status, ws, st, sym, sym_c};
  FinalOut fo{x, sc, status, -1.f / (float)p, 1.f};
  float* r1 = nullptr;
  if (p == 2) return ndb_pass(c, F, false, sc, 0.f, 0.f, false, 0, fo, &r1);
  FinalOut keep{nullptr, nullptr, nullptr, 0.f, 1.f};
  if (!zchain) {
    SHP_TRY(ndb_pass(c, F, false, sc, 0.f, 0.f, true, 0, keep, &r1));      // Y_1 ~ A_s^{1/2}
    float* r2 = nullptr;
    return ndb_pass(c, r1, true, nullptr, 1.f, 0.f, false, 1, fo, &r2);  // Z_2 ~ Y_1^{-1/2}
  }
  const double s2 = std::pow(1.5, (double)iters);
  SHP_TRY(ndb_pass(c, F, false, sc, 0.f, 0.f, false, 0, keep, &r1));  // Z_1 ~ A_s^{-1/2}
  FinalOut fz{x, sc, status, -0.25f, (float)std::sqrt(s2)};
  float* r2 = nullptr;
  return ndb_pass(c, r1, false, nullptr, (float)(1.0 / s2), 0.f, true, 1, fz, &r2);
}

// ---------------------------------------------------------------------------
// Coupled Newton.
// ---------------------------------------------------------------------------
int coupled_newton(const float* F, const shampoo_scale* sc, int64_t nf, int B, int p, int iters, float* x,
                   float* resid, int32_t* status, NewtonWs* ws, hipStream_t st, bool sym, bool sym_c) {
  Pool& pool = ws->pool;
  float* M = pool.get();
  if (M == nullptr) return SHAMPOO_EWORKSPACE;
  float* C = pool.get();
  if (C == nullptr) return SHAMPOO_EWORKSPACE;
  EwArgs a;
  memset(&a, 0, sizeof(a));
  a.x = F;
  a.out0 = M;
  a.out1 = C;
  a.partials = ws->partials;
  a.sc = sc;
  a.status = status;
  a.p = (float)p;
  a.B = B;
  a.chunks = ew_chunks(B);
  SHP_TRY(run_ew<EW_CN_START>(a, nf, st));
  SHP_TRY(run_resid(ws->partials, a.chunks, resid, iters, 0, ws->rmin, true, status, nf, st));
  const float pexp = -1.f / (float)p;
  if (iters == 1) {
    EwArgs s;
    memset(&s, 0, sizeof(s));
    s.x = C;
    s.out0 = x;
    s.sc = sc;
    s.status = status;
    s.pexp = pexp;
    s.extra = 1.f;
    s.p = 1.f;
    s.B = B;
    s.chunks = ew_chunks(B);
    return run_ew<EW_SCALE_COPY>(s, nf, st);
  }
  const int tiles = f32_tiles<EpiCnM>(B, sym_c, nf);
  float* X = nullptr;  // X_1 = C_0 (X_0 = I): first iteration has no X product
  for (int it = 0; it < iters; ++it) {
    const bool last = (it == iters - 1);
    if (last) {
      FinalOut fo{x, sc, status, pexp, 1.f};
      EpiStore::Job j = final_job(fo);
      const float* A[1] = {X};
      const float* Bm[1] = {C};
      return gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, st, sym);
    }
    // C^p by squaring, with X C in the same launch as the first square.
    float* Cp = C;
    float* Xn = nullptr;
    if (it == 0) {
      X = C;  // X_1 = C_0; C_0 stays alive as X
    }
    if (p >= 2) {
      float* C2 = pool.get();
      if (C2 == nullptr) return SHAMPOO_EWORKSPACE;
      if (it > 0) {
        Xn = pool.get();
        if (Xn == nullptr) return SHAMPOO_EWORKSPACE;
        EpiStore::Job j[2] = {plain_job(Xn), plain_job(C2)};
        const float* A[2] = {X, C};
        const float* Bm[2] = {C, C};
        SHP_TRY(gemm_nn<EpiStore>(A, Bm, j, 2, nf, B, st, sym));
      } else {
        EpiStore::Job j = plain_job(C2);
        const float* A[1] = {C};
        const float* Bm[1] = {C};
        SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, st, sym));
      }
      Cp = C2;
      for (int q = 4; q <= p; q *= 2) {
        float* Cq = pool.get();
        if (Cq == nullptr) return SHAMPOO_EWORKSPACE;
        EpiStore::Job j = plain_job(Cq);
        const float* A[1] = {Cp};
        const float* Bm[1] = {Cp};
        SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, st, sym));
        pool.put(Cp);
        Cp = Cq;
      }
    } else if (it > 0) {
      Xn = pool.get();
      if (Xn == nullptr) return SHAMPOO_EWORKSPACE;
      EpiStore::Job j = plain_job(Xn);
      const float* A[1] = {X};
      const float* Bm[1] = {C};
      SHP_TRY(gemm_nn<EpiStore>(A, Bm, &j, 1, nf, B, st, sym));
    }
    // M_{k+1} = C^p M_k, C_{k+1} = ((p+1) I - M_{k+1}) / p.
    float* Mn = pool.get();
    if (Mn == nullptr) return SHAMPOO_EWORKSPACE;
    float* Cn = pool.get();
    if (Cn == nullptr) return SHAMPOO_EWORKSPACE;
    {
      EpiCnM::Job j;
      j.m = Mn;
      j.c = Cn;
      j.m16 = nullptr;
      j.c16 = nullptr;
      j.fmt16 = H16_BF16;
      j.partials = ws->partials;
      j.tiles = tiles;
      j.p = (float)p;
      const float* A[1] = {Cp};
      const float* Bm[1] = {M};
      SHP_TRY(gemm_nn<EpiCnM>(A, Bm, &j, 1, nf, B, st, sym_c, SHAMPOO_TIME_CN_M));
      SHP_TRY(run_resid(ws->partials, tiles, resid, iters, it + 1, ws->rmin, false, status, nf, st));
    }
    if (Cp != C) pool.put(Cp);
    pool.put(M);
    if (it > 0) {
      pool.put(X);
      pool.put(C);
      X = Xn;
    }
    M = Mn;
    C = Cn;
  }
  return SHAMPOO_OK;
}

// ---------------------------------------------------------------------------
// Coupled Newton on fp16 operands (fp32 accumulate).  Only 16-bit copies of
// the iterates are kept; the final product writes X in fp32.  Every product
// is in NT form with the row-major fp16 copy of the right operand standing
// for its transpose: C, C^2, C^4 and M are polynomials in A_s, symmetric in
// exact arithmetic, and their rounding asymmetry is far below fp16 precision.
// With B a multiple of 256 the symmetric products (X C, C^2, C^4) keep their
// fp16 result only in the tiles on and above the diagonal, and the products
// that take it read the rest of each panel from there, transposed.
// ---------------------------------------------------------------------------
int coupled_newton_h16(const float* F, const shampoo_scale* sc, int64_t nf, int B, int p, int iters, float* x,
                       float* resid, int32_t* status, Cn16Ws* ws, hipStream_t st, bool sym, bool sym_c) {
  const float pexp = -1.f / (float)p;
  if (iters == 1) {  // X_1 = C_0: no product
    EwArgs a;
    memset(&a, 0, sizeof(a));
    a.x = F;
    a.out1 = ws->c32;
    a.partials = ws->partials;
    a.sc = sc;
    a.status = status;
    a.p = (float)p;
    a.B = B;
    a.chunks = ew_chunks(B);
    SHP_TRY(run_ew<EW_CN_START>(a, nf, st));
    SHP_TRY(run_resid(ws->partials, a.chunks, resid, 1, 0, ws->rmin, true, status, nf, st));
    EwArgs s2;
    memset(&s2, 0, sizeof(s2));
    s2.x = ws->c32;
    s2.out0 = x;
    s2.sc = sc;
    s2.status = status;
    s2.pexp = pexp;
    s2.extra = 1.f;
    s2.p = 1.f;
    s2.B = B;
    s2.chunks = ew_chunks(B);
    return run_ew<EW_SCALE_COPY>(s2, nf, st);
  }
  Pool16& pool = ws->pool;
  uint16_t* M = pool.get();
  uint16_t* C = pool.get();
  if (M == nullptr || C == nullptr) return SHAMPOO_EWORKSPACE;
  {
    EwArgs a;
    memset(&a, 0, sizeof(a));
    a.x = F;
    a.h0 = M;
    a.h1 = C;
    a.fmt16 = H16_F16;
    a.partials = ws->partials;
    a.sc = sc;
    a.status = status;
    a.p = (float)p;
    a.B = B;
    a.chunks = ew_chunks(B);
    SHP_TRY(run_ew<EW_CN16_START>(a, nf, st));
    SHP_TRY(run_resid(ws->partials, a.chunks, resid, iters, 0, ws->rmin, true, status, nf, st));
  }
  const int tiles = (B / h16_tile_of(B, sym_c)) * (B / h16_tile_of(B, sym_c));  // reduction partials of C^p M
  // symmetric products write their fp16 result on and above the diagonal only
  // (the large-tile kernel, which the products reading it also take)
  const int up = (sym && B % kBigTile == 0) ? 1 : 0;
  auto upper_job = [up](uint16_t* out16) {
    EpiStore::Job j = plain_job(nullptr, out16, H16_F16);
    j.upper16 = up;
    return j;
  };
  uint16_t* X = nullptr;
  bool x_up = false;  // X holds only its upper tiles
  for (int it = 0; it < iters; ++it) {
    if (it == iters - 1) {
      FinalOut fo{x, sc, status, pexp, 1.f};
      EpiStore::Job j = final_job(fo);
      const uint16_t* A[1] = {X};
      const uint16_t* Bt[1] = {C};
      return h16_gemm_nt<EpiStore>(A, Bt, &j, 1, nf, B, sym, H16_F16, st, x_up ? H16_UPPER_A : 0);
    }
    if (it == 0) X = C;  // X_1 = C_0; the buffer now belongs to X
    uint16_t* Cp = C;
    bool cp_up = false;
    uint16_t* Xn = nullptr;
    if (p >= 2) {
      uint16_t* C2 = pool.get();
      if (C2 == nullptr) return SHAMPOO_EWORKSPACE;
      if (it > 0) {
        Xn = pool.get();
        if (Xn == nullptr) return SHAMPOO_EWORKSPACE;
        EpiStore::Job j[2] = {upper_job(Xn), upper_job(C2)};
        const uint16_t* A[2] = {X, C};
        const uint16_t* Bt[2] = {C, C};
        SHP_TRY(h16_gemm_nt<EpiStore>(A, Bt, j, 2, nf, B, sym, H16_F16, st, x_up ? H16_UPPER_A : 0));
      } else {
        EpiStore::Job j = upper_job(C2);
        const uint16_t* A[1] = {C};
        const uint16_t* Bt[1] = {C};
        SHP_TRY(h16_gemm_nt<EpiStore>(A, Bt, &j, 1, nf, B, sym, H16_F16, st));
      }
      Cp = C2;
      cp_up = up;
      for (int q = 4; q <= p; q *= 2) {
        uint16_t* Cq = pool.get();
        if (Cq == nullptr) return SHAMPOO_EWORKSPACE;
        EpiStore::Job j = upper_job(Cq);
        const uint16_t* A[1] = {Cp};
        const uint16_t* Bt[1] = {Cp};
        SHP_TRY(h16_gemm_nt<EpiStore>(A, Bt, &j, 1, nf, B, sym, H16_F16, st,
                                      cp_up ? (H16_UPPER_A | H16_UPPER_B) : 0));
        pool.put(Cp);
        Cp = Cq;
      }
    } else if (it > 0) {
      Xn = pool.get();
      if (Xn == nullptr) return SHAMPOO_EWORKSPACE;
      EpiStore::Job j = upper_job(Xn);
      const uint16_t* A[1] = {X};
      const uint16_t* Bt[1] = {C};
      SHP_TRY(h16_gemm_nt<EpiStore>(A, Bt, &j, 1, nf, B, sym, H16_F16, st, x_up ? H16_UPPER_A : 0));
    }
    uint16_t* Mn = pool.get();
    uint16_t* Cn = pool.get();
    if (Mn == nullptr || Cn == nullptr) return SHAMPOO_EWORKSPACE;
    {
      EpiCnM::Job j;
      j.m = nullptr;
      j.c = nullptr;
      j.m16 = Mn;
      j.c16 = Cn;
      j.fmt16 = H16_F16;
      j.partials = ws->partials;
      j.tiles = tiles;
      j.p = (float)p;
      const uint16_t* A[1] = {Cp};
      const uint16_t* Bt[1] = {M};
      timing_before(SHAMPOO_TIME_CN_M, st);
      const int rc = h16_gemm_nt<EpiCnM>(A, Bt, &j, 1, nf, B, sym_c, H16_F16, st, cp_up ? H16_UPPER_A : 0);
      timing_after(SHAMPOO_TIME_CN_M, st);
      SHP_TRY(rc);
      SHP_TRY(run_resid(ws->partials, tiles, resid, iters, it + 1, ws->rmin, false, status, nf, st));
    }
    if (Cp != C) pool.put(Cp);
    pool.put(M);
    if (it > 0) {
      pool.put(X);
      pool.put(C);
      X = Xn;
      x_up = up;
    }
    M = Mn;
    C = Cn;
  }
  return SHAMPOO_OK;
}

// ---------------------------------------------------------------------------
// Chebyshev.
// ---------------------------------------------------------------------------

// Interpolant of x^{-1/p} at the degree+1 first-kind Chebyshev nodes of
// [delta, 1 + delta], as coefficients of T_j(2 (x - delta) - 1), c_0 halved.
void cheby_fit(int degree, int p, double delta, double* c) {
  const int n = degree + 1;
  const double pi = 3.14159265358979323846;
  for (int j = 0; j < n; ++j) c[j] = 0.0;
  for (int m = 0; m < n; ++m) {
    const double th = pi * (m + 0.5) / n;
    const double x = delta + 0.5 * (1.0 + std::cos(th));
    const double fx = std::pow(x, -1.0 / p);
    for (int j = 0; j < n; ++j) c[j] += fx * std::cos(j * th);
  }
  for (int j = 0; j < n; ++j) c[j] *= 2.0 / n;
  c[0] *= 0.5;
}

int chebyshev(const float* F, const shampoo_scale* sc, int64_t nf, int B, int p, int degree, double delta,
              int prec, float* x, int32_t* status, ChebyWs* ws, hipStream_t st, bool sym) {
  double c[257];
  cheby_fit(degree, p, delta, c);
  const float pexp = -1.f / (float)p;
  EwArgs a;
  memset(&a, 0, sizeof(a));
  a.x = F;
  a.sc = sc;
  a.status = status;
  a.p = (float)p;
  a.B = B;
  a.chunks = ew_chunks(B);
  if (degree == 1) {
    a.out0 = x;
    a.c0 = (float)c[0];
    a.c1 = (float)c[1];
    a.pexp = pexp;
    a.extra = 1.f;
    return run_ew<EW_CHEBY_LINEAR>(a, nf, st);
  }
  const bool bf = (prec == SHAMPOO_BF16_IN);
  int i2 = 0, i1 = 1, i0 = 2;  // ring slots of b_{j+2}, b_{j+1}, b_j
  int s1 = 0;                  // bf16 slot holding b_{j+1}
  // bf16 terms on the large-tile kernel keep their 16-bit copy only in the tiles
  // on and above the diagonal; the next product reads the rest transposed
  const bool up = bf && sym && (B % kBigTile) == 0;
  if (bf) {
    // b_{d-1} and the 16-bit operands in one pass: A_s is needed only as bf16,
    // and b_d = c_d I is formed by the first Clenshaw step
    Cheby16StartArgs s;
    s.x = F;
    s.sc = sc;
    s.status = status;
    s.bd = nullptr;  // b_d = c_d I: the first Clenshaw step forms it
    s.bd1 = ws->b[i1];
    s.bd1_16 = ws->b16[s1];
    s.as_t16 = ws->as_t16;
    s.cd = (float)c[degree];
    s.cd1 = (float)c[degree - 1];
    s.B = B;
    s.tiles = (B / 64) * (B / 64);
    s.split = up ? 1 : 0;
    const uint64_t grid = (uint64_t)nf * s.tiles;
    if (grid > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
    if (grid > 0) hipLaunchKernelGGL(cheby16_start_kernel, dim3((uint32_t)grid), dim3(256), 0, st, s);
    SHP_TRY(check_launch());
  } else {
    a.out0 = ws->as;
    a.out1 = ws->b[i2];  // b_d
    a.out2 = ws->b[i1];  // b_{d-1}
    a.c0 = (float)c[degree];
    a.c1 = (float)c[degree - 1];
    SHP_TRY(run_ew<EW_CHEBY_START>(a, nf, st));
  }
  for (int j = degree - 2; j >= 0; --j) {
    EpiClenshaw::Job e;
    e.upper16 = up ? 1 : 0;
    e.out = (j == 0) ? x : ws->b[i0];
    e.out16 = (bf && j > 0) ? ws->b16[s1 ^ 1] : nullptr;
    e.fmt16 = H16_BF16;
    e.b1 = ws->b[i1];
    e.b2 = (bf && j == degree - 2) ? nullptr : ws->b[i2];  // bf16 path: b_d not stored
    e.c2 = (float)c[degree];
    e.cj = (float)c[j];
    e.final = (j == 0) ? 1 : 0;
    e.scale = sc;
    e.status = status;
    e.pexp = pexp;
    if (bf) {
      timing_before(SHAMPOO_TIME_CLENSHAW, st);
      const int rc = bf16_gemm_nt_clenshaw(ws->b16[s1], ws->as_t16, e, nf, B, sym, up, st);
      timing_after(SHAMPOO_TIME_CLENSHAW, st);
      SHP_TRY(rc);
      s1 ^= 1;
    } else {
      const float* A[1] = {ws->as};
      const float* Bm[1] = {ws->b[i1]};
      SHP_TRY(gemm_nn<EpiClenshaw>(A, Bm, &e, 1, nf, B, st, sym, SHAMPOO_TIME_CLENSHAW));
    }
    const int t = i2;
    i2 = i1;
    i1 = i0;
    i0 = t;
  }
  return SHAMPOO_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int shampoo_abi_version(void) { return SHAMPOO_ABI_VERSION; }

int shampoo_timing_hook(int families, hipEvent_t* events, int32_t* fam_out, int capacity) {
  if ((families & ~SHAMPOO_TIME_ALL) != 0 || capacity < 0) return SHAMPOO_EINVAL;
  if (families != 0 && (events == nullptr || capacity == 0)) return SHAMPOO_EINVAL;
  g_timing.families = families;
  g_timing.events = families ? events : nullptr;
  g_timing.fam_out = families ? fam_out : nullptr;
  g_timing.capacity = families ? capacity : 0;
  g_timing.count = 0;
  return SHAMPOO_OK;
}

int shampoo_timing_count(void) { return g_timing.count; }

const char* shampoo_strerror(int code) {
  switch (code) {
    case SHAMPOO_OK: return "success";
    case SHAMPOO_EINVAL: return "invalid argument (null pointer, negative count or parameter out of range)";
    case SHAMPOO_EUNSUPPORTED: return "unsupported configuration (B must be a multiple of 64 in [64, 16384])";
    case SHAMPOO_EWORKSPACE: return "workspace missing or smaller than shampoo_workspace_bytes";
    case SHAMPOO_EHIP: return "HIP runtime error while launching a kernel";
    case SHAMPOO_ESCRATCH:
      return "problem too large for the static scratch of the allocation-free entry point "
             "(SHAMPOO_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown shampoo error code";
  }
}

size_t shampoo_workspace_bytes(int op, int64_t count, int B, int variant_or_degree, int prec) {
  prec &= ~SHAMPOO_FULL_PRODUCTS;
  if (op == SHAMPOO_OP_NEWTON) variant_or_degree &= ~(SHAMPOO_FULL_PRODUCTS | SHAMPOO_SYM_COUPLING);
  if (count < 0 || !valid_B(B)) return 0;
  if (prec != SHAMPOO_F32 && prec != SHAMPOO_BF16_IN) return 0;
  Carver c(nullptr);
  switch (op) {
    case SHAMPOO_OP_ACCUMULATE: return accum_layout(c, count, B, prec, nullptr);
    case SHAMPOO_OP_SCALE: return scale_layout(c, count, B, nullptr);
    case SHAMPOO_OP_NEWTON:
      if (variant_or_degree < SHAMPOO_NDB || variant_or_degree > SHAMPOO_CN_F16) return 0;
      return newton_layout(c, count, B, variant_or_degree, nullptr);
    case SHAMPOO_OP_CHEBY: return cheby_layout(c, count, B, prec, nullptr);
    case SHAMPOO_OP_PRECONDITION: return precond_layout(c, count, B, prec, nullptr);
    case SHAMPOO_OP_GRAFT: return graft_layout(c, count, B, nullptr);
    default: return 0;
  }
}

int shampoo_accumulate(const shampoo_block* g_blocks, int64_t nblocks, int B, float* factors, float alpha,
                       float gamma, int prec, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nblocks < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (prec != SHAMPOO_F32 && prec != SHAMPOO_BF16_IN) return SHAMPOO_EUNSUPPORTED;
  if (prec == SHAMPOO_BF16_IN && (B % 128) != 0) return SHAMPOO_EUNSUPPORTED;
  if (!std::isfinite(alpha) || !std::isfinite(gamma)) return SHAMPOO_EINVAL;
  if (nblocks == 0) return SHAMPOO_OK;
  if (g_blocks == nullptr || factors == nullptr) return SHAMPOO_EINVAL;
  Carver cm(nullptr);
  const size_t need = accum_layout(cm, nblocks, B, prec, nullptr);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return SHAMPOO_EWORKSPACE;
  Carver c(ws);
  AccumWs w;
  accum_layout(c, nblocks, B, prec, &w);

  EpiStore::Job jl;
  jl.out16 = nullptr;
  jl.fmt16 = H16_BF16;
  jl.out = factors;
  jl.cin = factors;
  jl.alpha = gamma;
  jl.beta = alpha;
  jl.scale = nullptr;
  jl.status = nullptr;
  jl.pexp = 0.f;
  jl.extra = 1.f;
  jl.upper16 = 0;
  EpiStore::Job jr = jl;
  jr.out = factors + stack_elems(nblocks, B);
  jr.cin = jr.out;
  if (prec == SHAMPOO_BF16_IN) {
    SHP_TRY(bf16_gather(g_blocks, nblocks, B, w.g16, w.gt16, stream));
    SHP_TRY(bf16_gemm_nt_store(w.g16, w.g16, jl, nblocks, B, true, stream));
    return bf16_gemm_nt_store(w.gt16, w.gt16, jr, nblocks, B, true, stream);
  }
  const Operand g = blocks(g_blocks);
  // L = G G^T: A(m,k) = G[m][k], B(n,k) = G[n][k] -- both k-contiguous.
  SHP_TRY((run_gemm<KCONTIG, KCONTIG, true, true, EpiStore>(&g, &g, &jl, 1, nblocks, B, true, stream)));
  // R = G^T G: A(m,k) = G[k][m], B(n,k) = G[k][n] -- both mn-contiguous.
  return run_gemm<MNCONTIG, MNCONTIG, true, true, EpiStore>(&g, &g, &jr, 1, nblocks, B, true, stream);
}

int shampoo_scale_power(const float* factors, int64_t nfactors, int B, float eps_rel, int mode, const float* v0,
                        int r, int steps, float safety, shampoo_scale* scale_out, int32_t* status, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (nfactors < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (!(eps_rel >= 0.f) || !std::isfinite(eps_rel)) return SHAMPOO_EINVAL;
  if (mode != SHAMPOO_SCALE_POWER && mode != SHAMPOO_SCALE_FROBENIUS) return SHAMPOO_EINVAL;
  if (mode == SHAMPOO_SCALE_POWER) {
    if (r < 1 || r > kPiCols || steps < 1 || steps > 10000) return SHAMPOO_EINVAL;
    if (!(safety > 0.f) || !std::isfinite(safety)) return SHAMPOO_EINVAL;
  }
  if (nfactors == 0) return SHAMPOO_OK;
  if (factors == nullptr || scale_out == nullptr || status == nullptr) return SHAMPOO_EINVAL;
  if (mode == SHAMPOO_SCALE_POWER && v0 == nullptr) return SHAMPOO_EINVAL;
  Carver cm(nullptr);
  const size_t need = scale_layout(cm, nfactors, B, nullptr);
  if (ws == nullptr || ws_bytes < need) return SHAMPOO_EWORKSPACE;
  if ((uint64_t)nfactors > 0x7fffffffull / (uint64_t)(B / 64)) return SHAMPOO_EUNSUPPORTED;
  Carver c(ws);
  ScaleWs w;
  scale_layout(c, nfactors, B, &w);

  hipLaunchKernelGGL(trace_kernel, dim3((uint32_t)nfactors), dim3(256), 0, stream, factors, B, eps_rel, scale_out);
  SHP_TRY(check_launch());
  if (mode == SHAMPOO_SCALE_FROBENIUS) {
    const int chunks = ew_chunks(B);
    hipLaunchKernelGGL(sumsq_kernel, dim3((uint32_t)(nfactors * chunks)), dim3(256), 0, stream, factors, B, chunks,
                       scale_out, w.sumsq);
    SHP_TRY(check_launch());
    hipLaunchKernelGGL(frob_finalize_kernel, dim3((uint32_t)nfactors), dim3(64), 0, stream, w.sumsq, chunks, B,
                       scale_out, status);
    return check_launch();
  }
  const int panel = pi_panel(B);
  PiArgs P;
  memset(&P, 0, sizeof(P));
  P.F = factors;
  P.sc = scale_out;
  P.B = B;
  P.rq_out = w.rq;
  for (int t = 0; t <= steps; ++t) {
    P.vin = (t == 0) ? v0 : w.w[(t - 1) & 1];
    P.ldv = (t == 0) ? r : kPiCols;
    P.r = r;
    P.wout = w.w[t & 1];
    P.norm_in = (t == 0) ? nullptr : w.norm[(t - 1) & 1];
    P.norm_out = w.norm[t & 1];
    P.last = (t == steps) ? 1 : 0;
    // after the first step (V then has 32 columns per row): 256-column panels
    // read by columns when B allows, else the row-panel kernels
    const bool col = (B % 256 == 0) && P.ldv == kPiCols;
    P.npanels_in = P.npanels;  // the previous step's panels (unused on the first)
    P.npanels = col ? B / 256 : B / panel;
    P.total = (uint32_t)(nfactors * P.npanels);
    if (col)
      hipLaunchKernelGGL(pi_step_col_kernel, dim3(P.total), dim3(512), 0, stream, P);
    else if (panel == 128 && P.ldv == kPiCols)
      hipLaunchKernelGGL(pi_step_dma_kernel, dim3(P.total), dim3(256), 0, stream, P);
    else if (panel == 128)
      hipLaunchKernelGGL(pi_step_kernel<128>, dim3(P.total), dim3(256), 0, stream, P);
    else
      hipLaunchKernelGGL(pi_step_kernel<64>, dim3(P.total), dim3(256), 0, stream, P);
    SHP_TRY(check_launch());
  }
  hipLaunchKernelGGL(pi_finalize_kernel, dim3((uint32_t)nfactors), dim3(64), 0, stream, w.rq, P.npanels, r, B,
                     safety, scale_out, status);
  return check_launch();
}

int shampoo_invroot_newton(const float* factors, const shampoo_scale* scale, int64_t nfactors, int B, int p,
                           int variant, int iters, float* x_out, float* resid_out, int32_t* status, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const bool sym = (variant & SHAMPOO_FULL_PRODUCTS) == 0;
  const bool sym_c = sym && (variant & SHAMPOO_SYM_COUPLING) != 0;
  variant &= ~(SHAMPOO_FULL_PRODUCTS | SHAMPOO_SYM_COUPLING);
  if (nfactors < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (variant < SHAMPOO_NDB || variant > SHAMPOO_CN_F16) return SHAMPOO_EINVAL;
  if (iters < 1 || iters > 100) return SHAMPOO_EINVAL;
  if (variant == SHAMPOO_CN || variant == SHAMPOO_CN_F16) {
    if (p != 1 && p != 2 && p != 4 && p != 8) return SHAMPOO_EUNSUPPORTED;
  } else if (p != 2 && p != 4) {
    return SHAMPOO_EUNSUPPORTED;
  }
  if (variant == SHAMPOO_CN_F16 && (B % 128) != 0) return SHAMPOO_EUNSUPPORTED;
  if (nfactors == 0) return SHAMPOO_OK;
  if (factors == nullptr || scale == nullptr || x_out == nullptr || status == nullptr) return SHAMPOO_EINVAL;
  Carver cm(nullptr);
  const size_t need = newton_layout(cm, nfactors, B, variant, nullptr);
  if (ws == nullptr || ws_bytes < need) return SHAMPOO_EWORKSPACE;
  Carver c(ws);
  if (variant == SHAMPOO_CN_F16) {
    Cn16Ws w16;
    cn16_layout(c, nfactors, B, &w16);
    return coupled_newton_h16(factors, scale, nfactors, B, p, iters, x_out, resid_out, status, &w16, stream, sym,
                              sym_c);
  }
  NewtonWs w;
  newton_layout(c, nfactors, B, variant, &w);
  if (variant == SHAMPOO_CN)
    return coupled_newton(factors, scale, nfactors, B, p, iters, x_out, resid_out, status, &w, stream, sym, sym_c);
  return newton_db(factors, scale, nfactors, B, p, variant == SHAMPOO_NDB_Z, iters, x_out, resid_out, status, &w,
                   stream, sym, sym_c);
}

int shampoo_invroot_cheby(const float* factors, const shampoo_scale* scale, int64_t nfactors, int B, int p,
                          int degree, double interval_eps, int prec, float* x_out, int32_t* status, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  const bool sym = (prec & SHAMPOO_FULL_PRODUCTS) == 0;
  prec &= ~SHAMPOO_FULL_PRODUCTS;
  if (nfactors < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (p < 1 || p > 64) return SHAMPOO_EINVAL;
  if (degree < 1 || degree > 256) return SHAMPOO_EINVAL;
  if (!(interval_eps >= 0.0) || !std::isfinite(interval_eps)) return SHAMPOO_EINVAL;
  if (prec != SHAMPOO_F32 && prec != SHAMPOO_BF16_IN) return SHAMPOO_EUNSUPPORTED;
  if (prec == SHAMPOO_BF16_IN && (B % 128) != 0) return SHAMPOO_EUNSUPPORTED;
  if (nfactors == 0) return SHAMPOO_OK;
  if (factors == nullptr || scale == nullptr || x_out == nullptr || status == nullptr) return SHAMPOO_EINVAL;
  Carver cm(nullptr);
  const size_t need = cheby_layout(cm, nfactors, B, prec, nullptr);
  if (ws == nullptr || ws_bytes < need) return SHAMPOO_EWORKSPACE;
  Carver c(ws);
  ChebyWs w;
  cheby_layout(c, nfactors, B, prec, &w);
  return chebyshev(factors, scale, nfactors, B, p, degree, interval_eps, prec, x_out, status, &w, stream, sym);
}

int shampoo_precondition(const float* x_roots, const shampoo_block* g_blocks, int64_t nblocks, int B,
                         const shampoo_block* u_blocks, int prec, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nblocks < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (prec != SHAMPOO_F32 && prec != SHAMPOO_BF16_IN) return SHAMPOO_EUNSUPPORTED;
  if (prec == SHAMPOO_BF16_IN && (B % 128) != 0) return SHAMPOO_EUNSUPPORTED;
  if (nblocks == 0) return SHAMPOO_OK;
  if (x_roots == nullptr || g_blocks == nullptr || u_blocks == nullptr) return SHAMPOO_EINVAL;
  Carver cm(nullptr);
  const size_t need = precond_layout(cm, nblocks, B, prec, nullptr);
  if (ws == nullptr || ws_bytes < need) return SHAMPOO_EWORKSPACE;
  Carver c(ws);
  PrecondWs w;
  precond_layout(c, nblocks, B, prec, &w);
  const float* XL = x_roots;
  const float* XR = x_roots + stack_elems(nblocks, B);
  if (prec == SHAMPOO_BF16_IN) {
    // T1 = X_L G: NT form with rows of G^T; U = T1 X_R: NT form with rows of X_R^T.
    SHP_TRY(bf16_cast(XL, w.a16, nblocks, B, false, stream));
    SHP_TRY(bf16_gather(g_blocks, nblocks, B, nullptr, w.b16, stream));
    SHP_TRY(bf16_gemm_nt_bf16out(w.a16, w.b16, w.t16, nblocks, B, stream));
    SHP_TRY(bf16_cast(XR, w.b16, nblocks, B, true, stream));
    return bf16_gemm_nt_desc(w.t16, w.b16, u_blocks, nblocks, B, stream);
  }
  // T1 = X_L G: B(n,k) = G[k][n] -- mn-contiguous through descriptors.
  EpiStore::Job j = plain_job(w.t1);
  const Operand a = dense(XL);
  const Operand g = blocks(g_blocks);
  SHP_TRY((run_gemm<KCONTIG, MNCONTIG, false, true, EpiStore>(&a, &g, &j, 1, nblocks, B, false, stream)));
  // U = T1 X_R, written through the output descriptors.
  EpiStoreDesc::Job ju{u_blocks};
  const Operand t = dense(w.t1);
  const Operand xr = dense(XR);
  return run_gemm<KCONTIG, MNCONTIG, false, false, EpiStoreDesc>(&t, &xr, &ju, 1, nblocks, B, false, stream);
}

}  // extern "C"

namespace {

// Validation and launch shared by the two grafting entry points; `partials`
// is null only while validating.
int graft_check(const shampoo_block* g_blocks, const shampoo_block* u_blocks, const shampoo_block* param_blocks,
                const shampoo_block* m_blocks, const shampoo_block* v_blocks, int64_t nblocks, int B, float lr,
                float beta1, float beta2, float eps, int step) {
  if (nblocks < 0) return SHAMPOO_EINVAL;
  if (!valid_B(B)) return SHAMPOO_EUNSUPPORTED;
  if (!std::isfinite(lr) || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f) ||
      !std::isfinite(eps) || step < 1)
    return SHAMPOO_EINVAL;
  if (nblocks == 0) return SHAMPOO_OK;
  if (!g_blocks || !u_blocks || !param_blocks || !m_blocks || !v_blocks) return SHAMPOO_EINVAL;
  if ((uint64_t)nblocks * graft_chunks(B) > 0x7fffffffull) return SHAMPOO_EUNSUPPORTED;
  return SHAMPOO_OK;
}

int graft_launch(const shampoo_block* g_blocks, const shampoo_block* u_blocks, const shampoo_block* param_blocks,
                 const shampoo_block* m_blocks, const shampoo_block* v_blocks, int64_t nblocks, int B, float lr,
                 float beta1, float beta2, float eps, int step, float* scale_out, float* partials,
                 hipStream_t stream) {
  const int chunks = graft_chunks(B);
  GraftArgs a;
  memset(&a, 0, sizeof(a));
  a.partials = partials;
  a.g = g_blocks;
  a.u = u_blocks;
  a.theta = param_blocks;
  a.m = m_blocks;
  a.v = v_blocks;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.bc1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)step)));
  a.bc2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)step)));
  a.lr = lr;
  a.scale_out = scale_out;
  a.B = B;
  a.chunks = chunks;
  const dim3 grid((uint32_t)(nblocks * chunks));
  hipLaunchKernelGGL(graft_moments_kernel, grid, dim3(256), 0, stream, a);
  SHP_TRY(check_launch());
  hipLaunchKernelGGL(graft_apply_kernel, grid, dim3(256), 0, stream, a);
  return check_launch();
}

constexpr size_t kScratchFloats = kScratchBytes / sizeof(float);

}  // namespace

// Scratch of shampoo_graft_update_noalloc: the per-chunk partial sums of the
// grafting norms, 2 floats per (block, chunk).  Every GPU the library runs on
// holds its own copy until the process ends.  Host code never uses this name
// as an address: it takes the device address from g_scratch_ptr.
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up once per device.
int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SHAMPOO_EHIP;
  if (dev >= kMaxDevices) return SHAMPOO_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SHAMPOO_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return SHAMPOO_OK;
}

}  // namespace

extern "C" int shampoo_graft_update(const shampoo_block* g_blocks, const shampoo_block* u_blocks,
                                    const shampoo_block* param_blocks, const shampoo_block* m_blocks,
                                    const shampoo_block* v_blocks, int64_t nblocks, int B, float lr, float beta1,
                                    float beta2, float eps, int step, float* scale_out, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  SHP_TRY(graft_check(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1, beta2, eps,
                      step));
  if (nblocks == 0) return SHAMPOO_OK;
  Carver cm(nullptr);
  const size_t need = graft_layout(cm, nblocks, B, nullptr);
  if (ws == nullptr || ws_bytes < need) return SHAMPOO_EWORKSPACE;
  Carver c(ws);
  float* partials = nullptr;
  graft_layout(c, nblocks, B, &partials);
  return graft_launch(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1, beta2, eps, step,
                      scale_out, partials, stream);
}

extern "C" int shampoo_graft_update_noalloc(const shampoo_block* g_blocks, const shampoo_block* u_blocks,
                                            const shampoo_block* param_blocks, const shampoo_block* m_blocks,
                                            const shampoo_block* v_blocks, int64_t nblocks, int B, float lr,
                                            float beta1, float beta2, float eps, int step, float* scale_out,
                                            hipStream_t stream) {
  SHP_TRY(graft_check(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1, beta2, eps,
                      step));
  if (nblocks == 0) return SHAMPOO_OK;
  Carver cm(nullptr);
  if (graft_layout(cm, nblocks, B, nullptr) > kScratchBytes) return SHAMPOO_ESCRATCH;
  float* partials = nullptr;
  SHP_TRY(scratch_address(&partials));
  return graft_launch(g_blocks, u_blocks, param_blocks, m_blocks, v_blocks, nblocks, B, lr, beta1, beta2, eps, step,
                      scale_out, partials, stream);
}
