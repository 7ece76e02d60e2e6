/* externd.h -- C ABI of the MI355X (gfx950) ExTernD decomposition engine.
 *
 * The engine factors a real matrix A (m x n) as A ~= B diag(D) C with ternary B (m x k) and
 * C (k x n), real D and an expanded inner rank k = floor(mu * min(m, n)) (the pages' abstract;
 * ExTernD review, Method).  Components are fitted greedily by alternating least squares against
 * the current residual, each with the closed-form scale d = u^T R v / (|u|^2 |v|^2), and the
 * residual is deflated before the next component (review, Method and Key idea; pith.science
 * referee report, "What carries the argument").  With block >= 2 the components are fitted b at
 * a time by block-ALS with the decorrelated least-squares target of Eq. 3 (pith.science, minor
 * comment 1); with importance weights the residual is measured in the column-weighted norm and
 * the V-step uses the corrected weighted projection (review, Method; pith.science, imatrix
 * assumption).
 *
 * Conventions for every entry point:
 *  - Array pointers are HIP device pointers on the current device unless marked (host).
 *  - Matrices are dense row-major fp32 with leading dimension equal to their column count.
 *  - The caller owns and allocates every argument buffer; inputs must not alias outputs.
 *  - Calls are synchronous: they return after all work issued on `stream` has completed.
 *  - On a nonzero status the output contents are unspecified; externd_last_error() returns a
 *    thread-local message describing the failure.  No C++ exception crosses the ABI.
 *  - Packed ternary vectors: element t sits in bits 2(t%16)..2(t%16)+1 of 32-bit word t/16;
 *    00 = 0, 01 = +1, 11 = -1, 10 never written; tail bits are zero.  This is the mask+sign
 *    storage model behind the pages' "2 - sparsity bits per element" accounting
 *    (pith.science free parameters, Eq. 5).
 */
#ifndef EXTERND_H
#define EXTERND_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXTERND_OK 0
#define EXTERND_EINVAL (-1)     /* bad size, mu, tau, iteration count, block, null pointer, weight <= 0 */
#define EXTERND_ENOMEM (-2)     /* workspace allocation failed */
#define EXTERND_EDEVICE (-3)    /* HIP runtime error or device-side failure (see externd_last_error) */
#define EXTERND_ENONFINITE (-4) /* NaN or Inf in A or in the importance weights */

/* (host) optional diagnostics filled by externd_decompose. */
typedef struct {
  int64_t k;                    /* components emitted */
  int64_t passes;               /* residual matvec passes performed (V- and U-steps) */
  int64_t early_exits;          /* components whose ALS reached an exact fixed point early */
  int64_t fallback_inits;       /* components started from the largest-entry row */
  int64_t zero_components;      /* components emitted as zero because the residual was zero */
  int64_t block;                /* resolved block size (1 = sequential) */
  double energy_final_explicit; /* 1 - |R|_H^2 / |A|_H^2 recomputed from the final residual */
  double seconds;               /* host wall time of the call */
  double kernel_ms;             /* device time of the decomposition kernels (HIP events) */
  double bytes_algorithmic;     /* residual bytes the method must move (sequential path) */
  double flops_algorithmic;     /* contraction flops of the block path */
  int64_t components_used;      /* components fitted before an energy-target stop (k without one) */
  int64_t safeguard_activations;/* components replaced by the best single entry (Prop. 2) */
  int64_t sweep_reverts;        /* refits discarded for the old component (block), see sweeps */
  int64_t residual_lds;         /* sequential path: 1 if each workgroup kept its rows of R in LDS */
} externd_stats;

/* (host) optional behaviour of externd_decompose_ex; all-zero = externd_decompose.
 *   energy_target  0 = off; in (0, 1]: per-matrix rank by energy (pith.science, free parameters:
 *                  mu is the accuracy dial, chosen per matrix to reach a target energy).  The
 *                  greedy components do not depend on k, so fitting stops after the first
 *                  component i with energy[i] >= energy_target (a zero component of a vanished
 *                  residual counts, its energy is 1); components i+1 .. k-1 are written as zero
 *                  codes with D = 0 and energy[i] repeated.  On the block path the stop can fall
 *                  inside a block: the block's later components are dropped (not applied to the
 *                  residual, written as zero).  stats->components_used = i + 1.
 *   safeguard      0 or 1: Prop. 2's convergence safeguard (pith.science, major comment 1 on
 *                  Appendix A): after the ALS of each component, if the largest h_j R_ij^2 over
 *                  the residual (smallest row-major index on ties) exceeds the ALS component's
 *                  p^2 / q, the component becomes u = e_i, v = sign(R_ij) e_j, d = |R_ij|.
 *                  Sequential path only (block >= 2 after resolution is EXTERND_EINVAL).  Costs
 *                  one extra read of the residual and one grid-wide exchange per component.
 *   sweeps         0..64 refinement sweeps after the greedy pass (review, Results: sweeps add
 *                  energy and lower the rank a target needs; read as backfitting).  Each sweep
 *                  walks the fitted components in order: the component's contribution is added
 *                  back to the residual (one fp32 rounding per entry), it is refitted by ALS
 *                  starting from its previous u, and the new fit is deflated unless it leaves
 *                  the residual larger than before the add-back by more than 1e-9 |A|^2_H, in
 *                  which case the old component is deflated again (keeping whichever removes
 *                  more, as Prop. 2 does; block-ALS from a warm start is not monotone).  The energy
 *                  bookkeeping continues through the add-backs; energy[i] is then the value
 *                  right after component i's refit in the last sweep, so energy[k-1] is the
 *                  final energy.  Components past an energy-target stop are not refitted.  On
 *                  the block path each block is added back (fp64 sum over its components, one
 *                  rounding) and refitted by block-ALS from its previous U.  With a target on the
 *                  block path the stop can fall inside a block; that block is then refitted as
 *                  a smaller block of its kept components.
 *   ablation       0 for the method; bits switching parts of it off for the pages' ablation
 *                  study (review, Validation): 1 = block path only, the batched targets without
 *                  Eq. 3's decorrelation (V from U^T R, U from R H V directly); 2 = the V-step
 *                  projection ignores the importance weights (the scales and the energy stay
 *                  weighted; inert without weights).  Joint fitting is block = k (b <= 256).
 *                  Other bits, or bit 1 on the sequential path, are EXTERND_EINVAL.
 *   residual_hbm   0 or 1: the sequential path keeps both residual copies in HBM even where each
 *                  workgroup's rows of R would fit in its LDS (the default then holds them there
 *                  for the whole decomposition); results are identical, only the time differs.
 *                  Inert on the block path. */
typedef struct {
  double energy_target;
  int safeguard;
  int sweeps;
  int ablation;
  int residual_hbm;
} externd_options;

/* k = floor(mu * min(m, n) + 1e-9); -1 if m < 1, n < 1, mu not finite or > 0, or k < 1. */
int64_t externd_rank(int64_t m, int64_t n, float mu);

/* ceil(len / 16): 32-bit words per packed ternary vector of length len. */
int64_t externd_packed_words(int64_t len);

/* Decompose A (m x n, device, fp32 row-major) into packed ternary B and C, scales D and the
 * energy-preserved curve.
 *   mu                 rank multiplier, finite, > 0, with k = externd_rank(m, n, mu) >= 1
 *   tau                sparsity threshold in [0, 1]: only |x| >= tau * max|x| may be selected
 *   importance_weights n per-column weights (> 0, finite), or NULL for uniform weights
 *   als_iters          >= 1 alternations (V-step then U-step) per component or block
 *   block              0 or 1: sequential deflation; b >= 2: block-ALS with blocks of b
 *                      (clamped to k); -1: b = min(256, min(m, n) / 8), at least 1
 *   B_packed           k x packed_words(m) uint32: row i = column i of B
 *   C_packed           k x packed_words(n) uint32: row i = row i of C
 *   D                  k fp32 scales
 *   energy             k fp64: energy[i] = 1 - |R_i|_H^2 / |A|_H^2 after component i
 *   stream             hipStream_t, or NULL for the default stream
 *   stats              (host) nullable diagnostics
 * Sizes: 1 <= m, n; max(m, n) <= 16384 for the ternary projection; the sequential path keeps
 * two fp32 copies of the residual (R and its transpose), the block path one.  A = 0 is valid:
 * every factor is 0, D = 0 and energy = 1.  The library allocates its own workspace on the
 * call's stream and frees it before returning. */
int externd_decompose(const float* A, int64_t m, int64_t n, float mu, float tau,
                      const float* importance_weights, int als_iters, int block,
                      uint32_t* B_packed, uint32_t* C_packed, float* D, double* energy,
                      void* stream, externd_stats* stats);

/* externd_decompose with options (host pointer, nullable = all off).  energy_target must be 0 or
 * in (0, 1] and safeguard 0 or 1, else EXTERND_EINVAL.  With a target on the block path the host
 * reads one flag after each block (a stream synchronisation per block). */
int externd_decompose_ex(const float* A, int64_t m, int64_t n, float mu, float tau,
                         const float* importance_weights, int als_iters, int block,
                         uint32_t* B_packed, uint32_t* C_packed, float* D, double* energy,
                         const externd_options* options, void* stream, externd_stats* stats);

/* Ternary projection T_tau(x; h) of `count` independent vectors, the operator every V- and
 * U-step applies (reading of the adaptive ternarization operator, review Method; pith.science
 * free parameters, tau / Eq. 2): among |x_i| >= tau max|x|, the top-j set by |x| maximising
 * (sum h|x|)^2 / (sum h), smallest j on ties, with the signs of x.
 *   X   count x L fp32 (device), rows are the vectors
 *   h   L fp32 weights shared by all rows, or NULL
 *   V   count x L int8 output in {-1, 0, 1}
 *   PHC count x 3 fp64 output: P = sum h|x| over the support, H = sum h, support size
 * 1 <= L <= 16384, count >= 1, 0 <= tau <= 1. */
int externd_project(const float* X, int64_t count, int64_t L, float tau, const float* h,
                    int8_t* V, double* PHC, void* stream);

/* The residual matvecs of the V- and U-steps with fp64 accumulation:
 *   transpose = 1: out (n) = R^T t, t (m) ternary int8
 *   transpose = 0: out (m) = R (h .* t), t (n) ternary int8, h nullable (uniform)
 * R is m x n fp32 row-major (device).  Same device routine as the decomposition kernel. */
int externd_matvec(const float* R, int64_t m, int64_t n, const int8_t* t, const float* h,
                   int transpose, double* out, void* stream);

/* Inference straight from the packed factors (ExTernD review, Significance: ternary additions
 * and subtractions plus one scale per component; pith.science report, the mask+sign storage of
 * Eq. 5):  Y[b] = B diag(D) C X[b] for each of `batch` vectors, i.e.
 *   t_i = sum_j C_ij X[b][j],   s_i = D_i t_i,   Y[b][r] = sum_i B_ri s_i.
 * Both sums are exact integer sums over fixed-point images: X[b] scaled by a power of two per
 * vector and rounded to integers of at most 50 bits (and n |image| <= 2^62), likewise s (k |image|
 * <= 2^62); each image is within 2^-50 of the vector's max |x| (max |s|) per element.  The result
 * is deterministic and independent of the launch shape; each output is rounded once to fp32.
 *   B_packed k x packed_words(m) uint32 (device): row i = column i of B, as externd_decompose
 *   C_packed k x packed_words(n) uint32 (device): row i = row i of C
 *   D        k fp32 (device)
 *   X        batch x n fp32 row-major (device), read only
 *   Y        batch x m fp32 row-major (device), written
 * 1 <= k, m, n < 2^31, 1 <= batch <= 65535.  Inputs are not checked for NaN/Inf (a non-finite x
 * gives meaningless outputs for its vector).  The workspace (8 batch (k + m) bytes plus
 * 4 batch ceil(k / 32) and 4 ceil(batch / 2) ceil(m / 256)) is a library buffer per (device, stream), allocated on the first call and
 * grown when a call needs more (after waiting for the stream), held until the process ends; a
 * call that fits it allocates nothing.  Calls on one stream use its buffer in stream order (calls
 * from several threads on one stream are serialised); calls on different streams use different
 * buffers.  The call only enqueues its kernels on `stream` and returns without waiting; the caller
 * synchronises the stream before reading Y.  EXTERND_EINVAL / ENOMEM / EDEVICE as for
 * externd_decompose. */
int externd_apply_factors(const uint32_t* B_packed, const uint32_t* C_packed, const float* D, int64_t k,
                          int64_t m, int64_t n, const float* X, int64_t batch, float* Y, void* stream);

/* externd_apply_factors for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, arithmetic and
 * results (bit for bit) as externd_apply_factors, but the workspace is a fixed 16 MiB device
 * array inside the library, one per GPU, held until the process ends; the call allocates and frees
 * nothing.  Limit: 8 batch (k + m) + 4 batch ceil(k / 32) + 4 ceil(batch / 2) ceil(m / 256) bytes
 * (each part rounded up to 256) must fit in the 16 MiB, else EXTERND_EINVAL (batch 1: k + m up to
 * about 2 million; k = 7680, m = 2560: batch up to 202).  The call only enqueues its kernels on
 * `stream` and returns without waiting; the caller synchronises the stream before reading Y.
 * Every call on one GPU uses that GPU's array (the kernels clear what must start at zero), so
 * calls that may overlap on one GPU (different streams, threads) race: serialise them on one
 * stream.  EXTERND_EINVAL for bad sizes or null pointers,
 * EXTERND_EDEVICE for HIP errors. */
int externd_apply_factors_static(const uint32_t* B_packed, const uint32_t* C_packed, const float* D, int64_t k,
                                 int64_t m, int64_t n, const float* X, int64_t batch, float* Y, void* stream);

/* Human-readable name of a status code (static string). */
const char* externd_status_string(int status);

/* Thread-local description of the last failure on the calling thread ("" if none). */
const char* externd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXTERND_H */
