// Internal declarations shared by the host API and the HIP kernels of libexternd.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace externd {

// ---- sequential persistent kernel (seq.hip)
struct SeqLaunch {
  float* R;
  float* RT;
  const float* h;
  const double* rs0;
  const double* rowE;
  double* xz;
  double* xw;
  double* xf;
  double* rsg;  // grid x m private row-sum copies
  unsigned* bar;
  uint32_t* Bp;
  uint32_t* Cp;
  float* D;
  double* energy;
  u64* stats;
  double* bytes;
  int m, n, ldr, ldt, k, T, EHm, grid;
  bool rl;  // R slab resident in LDS
  bool keys = true;  // LDS key array of the unweighted selections (seq_plan)
  float tau;
  unsigned spin_limit;
  double target = 0.0;  // > 0: stop once the energy reaches it
  int safeguard = 0;    // 1: Prop. 2 best single-entry safeguard
  int sweeps = 0;       // refinement sweeps after the greedy pass
  int ablation = 0;     // 2: the V-step projection ignores the weights
};
size_t seq_smem_bytes(int m, int n, bool weighted, int G, bool rl, bool keys);
// Grid size (one workgroup per CU at most), whether the R slab is held in LDS (only where it fits
// and allow_rl) and whether the LDS key array of the unweighted selections fits beside the rest
// (else they take the general selection); 0 if the problem does not fit the kernel's on-chip state.
int seq_plan(int m, int n, bool weighted, int ncu, bool allow_rl, int* grid, bool* rl, bool* keys);
hipError_t seq_launch(const SeqLaunch& L, hipStream_t st);
// out[r] = R_r . (t .* h) for rows of a padded row-major matrix; t (and h, nullable) padded to
// len4 * 4 entries.  Same slab routine as the sequential kernel.
hipError_t matvec_rows(float* Rp, int rows, int len4, int ld, const int8_t* t, const float* h, double* out,
                       hipStream_t st);

// ---- staging and checks (stage.hip)
// flags[0]: bit0 non-finite A, bit1 non-finite h, bit2 h <= 0; flags[1]: bits of max h
hipError_t check_inputs(const float* A, int m, int n, const float* h, unsigned* flags, hipStream_t st);
// R (m x ldr) = A with zero padding; rs = A 1 (fp64); rowE = sum_j h_j A_ij^2 (fp64)
hipError_t stage_rows(const float* A, int m, int n, const float* h, float* R, int ldr, double* rs,
                      double* rowE, hipStream_t st);
// RT (n x ldt) = A^T with zero padding
hipError_t stage_transpose(const float* A, int m, int n, float* RT, int ldt, hipStream_t st);
// rowE = sum_j h_j R_ij^2 (fp64) on an m x ldr residual
hipError_t row_energy(const float* R, int m, int n, int ldr, const float* h, double* rowE, hipStream_t st);
// ternary vectors (int8) of a matrix of `count` rows -> scratch for projection tests
hipError_t project_rows(const float* X, int count, int L, float tau, const float* h, int EHm, int8_t* V,
                        double* PHC, hipStream_t st);

// ---- block-ALS (block.hip)
struct BlockLaunch {
  float* R;            // m x ldr residual
  float* RT;           // n x ldt: its transpose, kept alongside
  int m, n, ldr, ldt, k, b, T, EHm;
  float tau;
  const float* h;
  const double* rowE;  // m
  uint32_t* Bp;
  uint32_t* Cp;
  float* D;
  double* energy;
  u64* stats;
  void* ws;            // workspace (block_workspace_bytes)
  double target = 0.0; // > 0: stop once the energy reaches it
  int sweeps = 0;      // refinement sweeps after the greedy pass
  int ablation = 0;    // 1: targets without Eq. 3's decorrelation, 2: V-step projection unweighted
};
size_t block_workspace_bytes(int m, int n, int b, bool weighted);
// flops: multiply-adds of the residual by ternary operands x 2; bytes: residual bytes that the
// contractions read and the updates read and write (4 m n per pass)
hipError_t block_run(const BlockLaunch& L, hipStream_t st, double* flops, double* bytes);

// Inference from the packed factors (apply.hip)
size_t infer_workspace_bytes(int k, int m, int batch);
// size of the file-scope inference workspace of each GPU (allocation-free entry point)
constexpr size_t kInferStaticBytes = (size_t)16 << 20;
// device address of this GPU's file-scope inference workspace (kInferStaticBytes bytes)
hipError_t infer_static_scratch(void** ptr);
hipError_t infer_run(const uint32_t* B, const uint32_t* C, const float* D, int k, int m, int n, const float* X,
                     int batch, float* Y, void* ws, hipStream_t st);

}  // namespace externd
