/*
 * shampoo.h -- C ABI of the MI355X (gfx950) Shampoo block-preconditioner library.
 *
 * One optimizer step of Shampoo's block preconditioner, for a stack of
 * B x B blocks, in five calls:
 *
 *   shampoo_accumulate       L <- alpha L + gamma G G^T,  R <- alpha R + gamma G^T G
 *   shampoo_scale_power      trace, damping eps and scale c (power iteration or Frobenius)
 *   shampoo_invroot_newton   X ~ c^{-1/p} ((F + eps I)/c)^{-1/p} by Newton-DB or coupled Newton
 *   shampoo_invroot_cheby    the same by a Chebyshev polynomial evaluated with Clenshaw
 *   shampoo_precondition     U = X_L G X_R
 *   shampoo_graft_update     theta <- theta - lr (||P||/||U||) U with P Adam's direction
 *
 * Sources (cited by page title and section): "DASH: Faster Shampoo via Batched
 * Block Preconditioning and Efficient Inverse-Root Solvers", the howistudyai.com
 * explainer of the paper ([DASH] below; its sections "Building blocks",
 * "High-level flow" and "Step-by-step"), and the arXiv 2602.02016 abstract.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All matrix pointers are DEVICE pointers owned by the caller.  Matrices are
 *    fp32, row-major.  A factor stack is float[nfactors][B][B], contiguous; the
 *    stack of a step holds the n left factors first, then the n right factors
 *    (nfactors = 2 n; block i owns factors i and n + i).
 *  - B must be a multiple of 64 with 64 <= B <= 16384 (SHAMPOO_EUNSUPPORTED).
 *  - A call only validates its arguments, enqueues kernels on `stream` and
 *    returns; it never synchronises and never allocates device memory.  Scratch
 *    memory comes from the caller's workspace `ws` of `ws_bytes` bytes (size from
 *    shampoo_workspace_bytes); it must stay allocated until the stream has
 *    executed the call, and one workspace must not be shared by calls that may
 *    run concurrently.  (shampoo_graft_update_noalloc takes no workspace: it
 *    uses a static device array of the library instead.)
 *  - Argument errors are returned synchronously as negative codes and nothing is
 *    enqueued.  A count of 0 (no blocks / factors) is a valid no-op.
 *  - Numerical trouble is reported per factor in a caller int32 status array on
 *    the device (bits below); shampoo_scale_power writes it, the inverse-root
 *    calls OR further bits into it.  Results are deterministic: no floating-point
 *    atomics are used, so a call repeated on the same inputs gives the same bits.
 *  - No C++ exception crosses this interface.
 */
#ifndef SHAMPOO_MI355X_H
#define SHAMPOO_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHAMPOO_ABI_VERSION 2

/* Return codes. */
enum {
  SHAMPOO_OK = 0,
  SHAMPOO_EINVAL = -1,        /* a null pointer, a negative count, a parameter out of range */
  SHAMPOO_EUNSUPPORTED = -2,  /* a valid value this library does not implement (B, p, prec) */
  SHAMPOO_EWORKSPACE = -3,    /* workspace missing or smaller than shampoo_workspace_bytes */
  SHAMPOO_EHIP = -4,          /* the HIP runtime refused a launch */
  SHAMPOO_ESCRATCH = -5       /* larger than the static scratch of shampoo_graft_update_noalloc */
};

/* Per-factor status bits (int32 status[nfactors] on the device). */
enum {
  SHAMPOO_BLK_NONFINITE = 1,  /* trace, spectral estimate or an iterate is not finite; values propagate */
  SHAMPOO_BLK_ZERO = 2,       /* tr(F) == 0 (all-zero history): X = I is returned */
  SHAMPOO_BLK_NONPOS_RQ = 4,  /* spectral estimate <= 0: X = I is returned */
  SHAMPOO_BLK_RESID_GROWTH = 8 /* a Newton residual rose above twice the smallest earlier residual of its
                                  pass: rounding errors are growing (the iteration diverges in this
                                  precision); X is still returned.  [DASH] "Limitations" and
                                  "Scoreboard with context" name unstable low-precision and
                                  Frobenius-scaled Newton runs; the pages give no detector */
};

/* Operand precision of the matrix products. */
enum {
  SHAMPOO_F32 = 0,            /* fp32 in, fp32 MFMA, fp32 accumulate */
  SHAMPOO_BF16_IN = 1         /* operands rounded to bf16 (RNE), bf16 MFMA, fp32 accumulate */
};

/* Scaling modes of shampoo_scale_power. */
enum {
  SHAMPOO_SCALE_POWER = 0,
  SHAMPOO_SCALE_FROBENIUS = 1
};

/* Iterations of shampoo_invroot_newton. */
enum {
  SHAMPOO_NDB = 0,            /* Newton-DB, second pass on Y (the pages' chaining) */
  SHAMPOO_NDB_Z = 1,          /* Newton-DB, second pass on Z_1 / (3/2)^iters (a variant) */
  SHAMPOO_CN = 2,             /* coupled Newton */
  SHAMPOO_CN_F16 = 3          /* coupled Newton on fp16 operands, fp32 accumulate (B % 128 == 0) */
};

/* Modifier bit, OR-ed into `variant` (shampoo_invroot_newton) or `prec`
 * (shampoo_invroot_cheby).  By default every product whose result is a
 * polynomial in the factor -- Newton-DB's Y E and E Z, coupled Newton's X C
 * and powers of C, Clenshaw's A_s b -- is symmetric in exact arithmetic, so
 * only its upper-triangular tiles are computed and mirrored (the outputs are
 * exactly symmetric).  The coupling products Z Y and C^p M are computed in
 * full by default.  With this bit set every product is computed in full. */
#define SHAMPOO_FULL_PRODUCTS 0x100

/* Opt-in modifier bit for shampoo_invroot_newton: form the coupling products
 * (Newton-DB's P = Z Y, coupled Newton's C^p M) from upper tiles as well,
 * which saves about 40% of their MFMA work.  They are symmetric in exact
 * arithmetic, but with the full product the coupled iterations stay
 * self-correcting: measured in fp32 on factors with a condition number of
 * 1e8, the mirrored coupling product matches the full one while the
 * iteration converges and then lets rounding errors grow until the iterates
 * overflow (Newton-DB by k = 15 per pass, where the full product stays
 * accurate); coupled Newton on fp16 operands loses accuracy the same way
 * over many iterations.  Use only for well-conditioned factors or few
 * iterations.  Ignored together with SHAMPOO_FULL_PRODUCTS. */
#define SHAMPOO_SYM_COUPLING 0x200

/* Operation ids of shampoo_workspace_bytes. */
enum {
  SHAMPOO_OP_ACCUMULATE = 1,
  SHAMPOO_OP_SCALE = 2,
  SHAMPOO_OP_NEWTON = 3,
  SHAMPOO_OP_CHEBY = 4,
  SHAMPOO_OP_PRECONDITION = 5,
  SHAMPOO_OP_GRAFT = 6
};

/* A B x B block inside a larger row-major fp32 matrix (a layer gradient or
 * the update).  `ptr` is the device address of the block's element (0,0), `ld`
 * the row stride in elements.  A partial edge block has rows < B or cols < B;
 * its missing entries read as zero and are never written.  Valid descriptors
 * have 0 <= rows, cols <= B and ld >= cols; the table itself lives in device
 * memory.  A descriptor that fails these checks on the device is treated as
 * an all-zero block (an invalid output descriptor is not written).  Vector
 * loads are used when ptr is 16-byte aligned and ld % 4 == 0, scalar loads
 * otherwise.  SHAMPOO_BF16_IN products need B % 128 == 0. */
typedef struct shampoo_block {
  float* ptr;
  int64_t ld;
  int32_t rows;
  int32_t cols;
} shampoo_block;

/* Per-factor scale record written by shampoo_scale_power (device memory). */
typedef struct shampoo_scale {
  float c;       /* scale constant: A_s = (F + eps I) / c */
  float eps;     /* damping: eps = eps_rel * tr(F) / B */
  float lambda;  /* spectral estimate (power) or ||F + eps I||_F (Frobenius) */
  float trace;   /* tr(F) */
} shampoo_scale;

/*
 * shampoo_accumulate -- EMA of the Kronecker factors of every block.
 * [DASH] "Step-by-step", building the preconditioners (an EMA of G G^T and
 * G^T G per block) and stacking the blocks into one 3D tensor.
 *
 *   g_blocks  device array [nblocks] of gradient block descriptors (read only)
 *   factors   device float[2 nblocks][B][B], updated in place:
 *               factors[i]          <- alpha factors[i]          + gamma G_i G_i^T
 *               factors[nblocks+i]  <- alpha factors[nblocks+i]  + gamma G_i^T G_i
 *             (alpha = beta, gamma = 1 - beta for the EMA; start from zeros)
 *   prec      SHAMPOO_F32 or SHAMPOO_BF16_IN (G rounded to bf16 before the product)
 *   ws        workspace of shampoo_workspace_bytes(SHAMPOO_OP_ACCUMULATE, nblocks, B, 0, prec)
 *             (0 bytes for SHAMPOO_F32; ws may then be NULL)
 */
int shampoo_accumulate(const shampoo_block* g_blocks, int64_t nblocks, int B,
                       float* factors, float alpha, float gamma, int prec,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_scale_power -- trace, damping and scale of every factor.
 * [DASH] "Building blocks" (multi-power-iteration; Frobenius versus spectral
 * scaling) and "Step-by-step", scaling each block.
 *
 *   factors    device float[nfactors][B][B] (not modified); A = F + eps I.
 *              F is taken to be symmetric, as a factor formed by
 *              shampoo_accumulate is: when B is a multiple of 256, rounds
 *              after the first form W = A^T V (reading F by columns).  For
 *              an F that is not symmetric that is the same iteration on A^T,
 *              which has A's eigenvalues.
 *   eps_rel    eps = eps_rel * tr(F) / B (>= 0)
 *   mode       SHAMPOO_SCALE_POWER: r start vectors v0, `steps` rounds of
 *                W = A V, columns normalised; then q_j = v_j^T A v_j,
 *                lambda = max_j q_j, c = safety * lambda
 *              SHAMPOO_SCALE_FROBENIUS: lambda = c = ||A||_F (v0 may be NULL)
 *   v0         device float[nfactors][B][r], 1 <= r <= 32, steps >= 1
 *   safety     > 0 (the pages divide by about twice the estimate: 2.0)
 *   scale_out  device shampoo_scale[nfactors]
 *   status     device int32[nfactors], overwritten: ZERO if tr(F) == 0,
 *              NONPOS_RQ if lambda <= 0, NONFINITE if trace or lambda is not finite
 */
int shampoo_scale_power(const float* factors, int64_t nfactors, int B, float eps_rel,
                        int mode, const float* v0, int r, int steps, float safety,
                        shampoo_scale* scale_out, int32_t* status,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_invroot_newton -- inverse p-th roots by inverse-free Newton iterations.
 * [DASH] "Building blocks" (Newton-DB) and "Step-by-step", solvers (a) Newton-DB
 * and (b) coupled Newton.
 *
 *   A_s = (F + eps I) / c with (c, eps) from `scale`; x_out = c^{-1/p} g(A_s).
 *   variant SHAMPOO_NDB:   pass(Y0): Z = I; iters times { E = (3I - Z Y)/2;
 *                          Y <- Y E; Z <- E Z }.  p = 2: X = pass(A_s).Z;
 *                          p = 4: X = pass(pass(A_s).Y).Z.
 *           SHAMPOO_NDB_Z: p = 4: s = (3/2)^iters, X = sqrt(s) pass(pass(A_s).Z / s).Y
 *           SHAMPOO_CN:    X = I, M = A_s; iters times { C = ((p+1) I - M)/p;
 *                          X <- X C; M <- C^p M };  p in {1, 2, 4, 8}
 *           SHAMPOO_CN_F16: the same iteration with every product on fp16
 *                          operands (RNE) and fp32 accumulation; only fp16
 *                          copies of the iterates are kept, X is written in fp32
 *                          ([DASH] Scoreboard: coupled Newton in FP16)
 *   iters      iterations per pass, 1..100
 *   x_out      device float[nfactors][B][B]
 *   resid_out  NULL or device float[nfactors][passes * iters]: ||I - Z Y||_F before
 *              each Newton-DB iteration (passes = 1 for p = 2, else 2), or
 *              ||I - M||_F before each coupled-Newton iteration (passes = 1)
 *   status     device int32[nfactors]; factors flagged ZERO or NONPOS_RQ get
 *              X = I; NONFINITE is added when a residual is not finite, and
 *              RESID_GROWTH when a residual exceeds twice the smallest earlier
 *              residual of the same pass (in exact arithmetic the residuals of a
 *              pass never increase for a spectrum inside the iteration's
 *              convergence region, (0, 3) for Newton-DB and (0, p + 1) for
 *              coupled Newton).  The residuals are computed whether or not
 *              resid_out is given.
 *   ws         shampoo_workspace_bytes(SHAMPOO_OP_NEWTON, nfactors, B, variant, SHAMPOO_F32)
 */
int shampoo_invroot_newton(const float* factors, const shampoo_scale* scale,
                           int64_t nfactors, int B, int p, int variant, int iters,
                           float* x_out, float* resid_out, int32_t* status,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_invroot_cheby -- inverse p-th roots by a Chebyshev polynomial.
 * [DASH] "Building blocks" (Chebyshev) and "Step-by-step", solver (d).
 *
 *   The polynomial interpolates f(x) = x^{-1/p} at the degree+1 first-kind
 *   Chebyshev nodes of [interval_eps, 1 + interval_eps] (fitted on the host in
 *   double precision).  With T = 2 A_s - I it is evaluated by Clenshaw's
 *   recurrence b_j = c_j I + 2 T b_{j+1} - b_{j+2}, X = c_0 I + T b_1 - b_2,
 *   i.e. degree - 1 matrix products; x_out = c^{-1/p} X.
 *   degree     1..256;  p >= 1;  interval_eps >= 0
 *   prec       SHAMPOO_F32, or SHAMPOO_BF16_IN (products on bf16 operands,
 *              the recurrence itself in fp32)
 *   status     as for shampoo_invroot_newton (ZERO / NONPOS_RQ give X = I)
 *   ws         shampoo_workspace_bytes(SHAMPOO_OP_CHEBY, nfactors, B, degree, prec)
 */
int shampoo_invroot_cheby(const float* factors, const shampoo_scale* scale,
                          int64_t nfactors, int B, int p, int degree, double interval_eps,
                          int prec, float* x_out, int32_t* status,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_precondition -- U_i = X_L,i G_i X_R,i for every block.
 * [DASH] "High-level flow" and "Step-by-step" (the preconditioned direction).
 *
 *   x_roots   device float[2 nblocks][B][B]: X_L of block i at i, X_R at nblocks + i
 *   g_blocks  device array [nblocks] of gradient block descriptors (read only)
 *   u_blocks  device array [nblocks] of output descriptors; only the rows x cols
 *             part of each output block is written.  Output blocks must not overlap
 *             the gradient blocks or each other.
 *   prec      SHAMPOO_F32 or SHAMPOO_BF16_IN
 *   ws        shampoo_workspace_bytes(SHAMPOO_OP_PRECONDITION, nblocks, B, 0, prec)
 */
int shampoo_precondition(const float* x_roots, const shampoo_block* g_blocks,
                         int64_t nblocks, int B, const shampoo_block* u_blocks, int prec,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_graft_update -- grafted parameter update of every block.
 * [DASH] "Step-by-step", grafting: the update keeps the Shampoo direction U
 * and takes its length from an Adam-like direction P.
 *
 *   Per block (elementwise over the block's rows x cols, taken from g_blocks):
 *     m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2          (in place)
 *     P = (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 *     s = ||P||_F / ||U||_F  (0 when ||U||_F = 0)
 *     theta <- theta - lr s U                                              (in place)
 *   g_blocks, u_blocks (U from shampoo_precondition), param_blocks, m_blocks,
 *   v_blocks   device arrays [nblocks] of descriptors of blocks of the same shape;
 *              the m and v blocks hold Adam's state (zeros before step 1)
 *   step       1-based step count for the bias corrections;  0 <= beta1, beta2 < 1;  eps >= 0
 *   scale_out  NULL or device float[nblocks]: s of every block
 *   ws         shampoo_workspace_bytes(SHAMPOO_OP_GRAFT, nblocks, B, 0, SHAMPOO_F32)
 */
int shampoo_graft_update(const shampoo_block* g_blocks, const shampoo_block* u_blocks,
                         const shampoo_block* param_blocks, const shampoo_block* m_blocks,
                         const shampoo_block* v_blocks, int64_t nblocks, int B, float lr, float beta1,
                         float beta2, float eps, int step, float* scale_out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * shampoo_graft_update_noalloc -- shampoo_graft_update without a workspace.
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * per-block partial norms live in a static device array of
 * SHAMPOO_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; this call allocates nothing and frees nothing.
 * Arguments, results and errors are those of shampoo_graft_update, plus
 * SHAMPOO_ESCRATCH (nothing enqueued) when the partial norms need more than
 * the static array: nblocks * min(max(B / 64, 1), 64) * 8 bytes, rounded up to
 * 256, must not exceed SHAMPOO_NOALLOC_SCRATCH_BYTES (e.g. up to 8192 blocks
 * at B = 1024).  The array starts with no meaningful contents and every call
 * overwrites all of the part it reads before reading it.  All calls on one
 * GPU share that GPU's array: calls that may overlap in time on the same GPU
 * (different streams, or different host threads without ordering) race and
 * must not be issued.  The first call on a device looks up the array's
 * address there (SHAMPOO_EHIP if that fails).
 */
#define SHAMPOO_NOALLOC_SCRATCH_BYTES (1u << 20)
int shampoo_graft_update_noalloc(const shampoo_block* g_blocks, const shampoo_block* u_blocks,
                                 const shampoo_block* param_blocks, const shampoo_block* m_blocks,
                                 const shampoo_block* v_blocks, int64_t nblocks, int B, float lr, float beta1,
                                 float beta2, float eps, int step, float* scale_out, hipStream_t stream);

/* Workspace size in bytes for an operation (op = SHAMPOO_OP_*).  `count` is
 * nfactors for SCALE/NEWTON/CHEBY and nblocks for ACCUMULATE/PRECONDITION;
 * `variant_or_degree` is the Newton variant or the Chebyshev degree (else 0);
 * `count` is nblocks for GRAFT too.
 * Returns 0 for invalid arguments as well as for operations that need none. */
size_t shampoo_workspace_bytes(int op, int64_t count, int B, int variant_or_degree, int prec);

/* Static English text for a return code (never NULL). */
const char* shampoo_strerror(int code);

/* SHAMPOO_ABI_VERSION of the built library. */
int shampoo_abi_version(void);

/* Kernel families for shampoo_timing_hook (bits, OR-able). */
enum {
  SHAMPOO_TIME_OFF = 0,
  SHAMPOO_TIME_NDB_PAIR = 1,   /* Newton-DB updates Y E and E Z, launched together (2 products) */
  SHAMPOO_TIME_NDB_P = 2,      /* Newton-DB product Z Y with the E = (3I - P)/2 epilogue */
  SHAMPOO_TIME_CLENSHAW = 4,   /* one Clenshaw product A_s b (fp32 or bf16) */
  SHAMPOO_TIME_CN_M = 8,       /* coupled Newton's product C^p M (fp32 or fp16) */
  SHAMPOO_TIME_ALL = 15
};

/*
 * shampoo_timing_hook -- measurement instrumentation (not part of the method).
 * While enabled, each launch of a kernel family in the bit set `families`
 * made by any later call records events[2 i] just before and events[2 i + 1]
 * just after the launch on that call's stream, and (when fam_out is not NULL)
 * writes the launch's family bit to fam_out[i], a HOST array, for
 * i < capacity; further launches are not recorded.  `events` are
 * caller-created HIP events (2 * capacity of them) that must outlive the
 * recorded launches.  families = SHAMPOO_TIME_OFF disables the hook.  The hook
 * is process-wide and not thread-safe; enabling it resets the count.
 * shampoo_timing_count returns how many launches have been recorded.
 */
int shampoo_timing_hook(int families, hipEvent_t* events, int32_t* fam_out, int capacity);
int shampoo_timing_count(void);

#ifdef __cplusplus
}
#endif

#endif /* SHAMPOO_MI355X_H */
