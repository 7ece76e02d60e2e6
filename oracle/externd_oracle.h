/* Plain CPU oracle for the ExTernD decomposition engine.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the product path
 * never does.  It shares no source with the GPU library.
 *
 * Method (pages: "ExTernD: Expanded-Rank Ternary Decomposition" review, sections Method and
 * Key idea; pith.science referee report, "What carries the argument" and minor comment 1 on
 * Eq. 3; abstract): A (m x n) ~= B diag(D) C with ternary B (m x k), C (k x n), real D,
 * k = floor(mu * min(m,n)), fitted greedily by alternating least squares with residual
 * deflation, or in blocks of b components with the decorrelated least-squares target of Eq. 3.
 *
 * Numeric conventions (a reading, the pages fix no precision): the residual R is stored in
 * fp32, every sum is accumulated in fp64 in ascending index order, selection inputs are rounded
 * to fp32 first, each scale d is computed in fp64 and rounded to fp32, and the deflation
 * R_ij <- fl32(R_ij - d u_i v_j) is a single fp32 operation.
 *
 * Packed ternary vectors: element t sits in bits 2(t%16)..2(t%16)+1 of word t/16;
 * 00 = 0, 01 = +1, 11 = -1; tail bits zero.
 */
#ifndef EXTERND_ORACLE_H
#define EXTERND_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int threads;              /* OpenMP threads; <= 0 = runtime default */
  int safeguard;            /* 1 = Prop. 2 best single-entry safeguard on */
  int64_t k_limit;          /* > 0: stop after this many components (sequential) */
  double* gaps;             /* nullable, k: smallest selection gap of each component */
  int64_t* counters;        /* nullable, 4: fallbacks, safeguard activations, ALS passes, zero components */
  double* energy_explicit;  /* nullable, 1: 1 - ||R||^2_H / ||A||^2_H recomputed from R at the end */
  int residual_fp64;        /* 1 = keep the residual in fp64 instead of fp32 (precision study only) */
  int block_engine;         /* 1 = run the block engine even when b == 1 (invariant test) */
  double energy_target;     /* in (0, 1]: stop after the first component whose energy >= target;
                               later components are zero with the energy held; <= 0: off */
  int64_t* used;            /* nullable, 1: components fitted before the stop (all when none) */
  int sweeps;               /* >= 1: refinement sweeps (backfitting) after the greedy pass */
  int64_t* reverts;         /* nullable, 1: refits discarded for the old component (block) */
  int ablation;             /* block engine: 1 = targets without Eq. 3's decorrelation,
                               2 = V-step projection without the weights (both: 3) */
} externd_oracle_opts;

int64_t externd_oracle_rank(int64_t m, int64_t n, float mu);
int64_t externd_oracle_words(int64_t len);
// splitmix64 (S. Vigna): the first output of the generator started from state `key`; and the
// block sketch's entry Omega[j][c] of block s (reading of the review's block-ALS initialisation:
// column 0 all ones, the rest Rademacher signs from the top bit of splitmix64 at key
// ((s 2^16 + c) 2^32 + j)).  Exposed so that tests can pin the generator to its published outputs.
uint64_t externd_oracle_splitmix64(uint64_t key);
double externd_oracle_sketch_sign(int64_t s, int64_t c, int64_t j);
// The block engine's least-squares targets for given ternary U (bs x m) and V (bs x n),
// component-major (pith.science minor comment 1, Eq. 3, and its mirror for U): X = (U^T U +
// eps I)^-1 U^T A (bs x n) and Ft = (V^T H V + eps I)^-1 (A H V)^T (bs x m), eps = 1e-6 trace of
// the Gram / bs; naive != 0 drops the inverse (the ablation).  The same routines the decomposition
// uses; exposed so that tests can pin them to a library solve.
int externd_oracle_block_targets(const float* A, int64_t m, int64_t n, const float* h, const int8_t* U,
                                 const int8_t* V, int64_t bs, int naive, double* X, double* Ft);

/* T_tau(x; h): v (int8, L), out[0..2] = P, H, S, *jstar = support size, *gap = selection gap. */
int externd_oracle_project(const float* x, int64_t L, float tau, const float* h,
                           int8_t* v, double* out, int64_t* jstar, double* gap);

/* Free-running decomposition.  block <= 1: sequential deflation; block >= 2: block-ALS;
 * block == -1: b = min(256, min(m,n)/8) (at least 1).
 * Energy target (pith.science free parameters: mu is the accuracy dial, set per matrix to reach
 * a target energy): the greedy components do not depend on k, so fitting until the energy
 * first reaches the target gives the per-matrix rank directly.  After the first component i
 * with energy[i] >= target (a zero component of a vanished residual counts, its energy is 1),
 * components i+1.. are zero with energy[i] repeated and gap +inf; on the block path the stop
 * can fall inside a block, whose later components are then dropped (zero scale, not applied).
 * The safeguard (Prop. 2) applies to the sequential engine only. */
int externd_oracle_decompose(const float* A, int64_t m, int64_t n, float mu, float tau,
                             const float* h, int als_iters, int block,
                             uint32_t* B, uint32_t* C, float* D, double* energy,
                             const externd_oracle_opts* opts);

/* Replay: walk the components (or blocks) of a finished decomposition (B, C, D given), applying
 * each with the oracle's deflation rule.  Before applying component (block) s listed in
 * `sample` (ascending), fit it afresh from the replayed residual and write the oracle's own
 * result to Bo/Co/Do/gap_o (one slot per sample; a block slot holds b components), and to
 * dec_o the refit's energy decrease in units of |A|^2_H (2 d p - d^2 q per component; for a block
 * the steps of its own energy walk on the replayed residual), so that a given component (block)
 * that differs from the refit can be compared by what it removes.
 * energy_replay[i] = energy after applying the given component i, from the oracle's own exact
 * p, q of that component on the replayed residual.  With opts->k_limit > 0 the walk stops
 * after that many components (entries beyond it are left untouched). */
int externd_oracle_replay(const float* A, int64_t m, int64_t n, float mu, float tau,
                          const float* h, int als_iters, int block,
                          const uint32_t* B, const uint32_t* C, const float* D,
                          const int64_t* sample, int64_t nsample,
                          uint32_t* Bo, uint32_t* Co, float* Do, double* gap_o,
                          double* dec_o, double* energy_replay, const externd_oracle_opts* opts);

/* Inference from the packed factors: Y (batch x m) = (B diag(D) C X^T)^T for X (batch x n),
 * fp64 sums in index order, one fp32 rounding.  B: k x words(m), C: k x words(n). */
int externd_oracle_apply(const uint32_t* B, const uint32_t* C, const float* D, int64_t k, int64_t m,
                         int64_t n, const float* X, int64_t batch, float* Y, int threads);

/* Energy preserved by given factors, recomputed from its definition: the residual
 * A - sum_{c <= i} D_c b_c c_c^T is formed in fp64 one component at a time and, after each
 * component i listed in `at` (ascending, < k), out[t] = 1 - |residual|^2_h / |A|^2_h
 * (column weights h, NULL = uniform).  B: k x words(m), C: k x words(n). */
int externd_oracle_explicit_energy(const float* A, int64_t m, int64_t n, const float* h,
                                   const uint32_t* B, const uint32_t* C, const float* D, int64_t k,
                                   const int64_t* at, int64_t nat, double* out, int threads);

/* Plain matvecs used by kernel-level parity tests: out = R^T u (transpose = 1) or R (h .* v). */
int externd_oracle_matvec(const float* R, int64_t m, int64_t n, const int8_t* t, const float* h,
                          int transpose, double* out, int threads);

#ifdef __cplusplus
}
#endif
#endif
