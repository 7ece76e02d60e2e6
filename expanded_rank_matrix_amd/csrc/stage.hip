// Staging kernels: input checks, residual copies, row sums and energies.
// E0 = |A|_H^2 and the initial row sums A 1 are fp64 sums in a fixed order per row.
#include "externd_internal.hpp"

namespace externd {

__global__ void __launch_bounds__(256) check_kernel(const float* A, size_t total, const float* h, int n,
                                                   unsigned* flags) {
  unsigned bad = 0u;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const float x = A[i];
    if (!isfinite(x)) bad |= 1u;
  }
  unsigned hmax = 0u;
  if (h) {
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
      const float x = h[j];
      if (!isfinite(x)) bad |= 2u;
      else if (!(x > 0.0f)) bad |= 4u;
      else {
        const unsigned k = __float_as_uint(x);
        hmax = k > hmax ? k : hmax;
      }
    }
  }
  if (bad) atomicOr(&flags[0], bad);
  if (hmax) atomicMax(&flags[1], hmax);
}

hipError_t check_inputs(const float* A, int m, int n, const float* h, unsigned* flags, hipStream_t st) {
  const size_t total = (size_t)m * n;
  int grid = (int)((total + 255) / 256);
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(check_kernel, dim3(grid), dim3(256), 0, st, A, total, h, n, flags);
  return hipGetLastError();
}

// one wave per row: copy with zero padding, fp64 row sum and weighted energy
__global__ void __launch_bounds__(256) stage_rows_kernel(const float* A, int m, int n, const float* h, float* R,
                                                        int ldr, double* rs, double* rowE) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const float* a = A + (size_t)i * n;
  float* r = R + (size_t)i * ldr;
  double s = 0.0, e = 0.0;
  for (int j = lane; j < ldr; j += 64) {
    const float x = j < n ? a[j] : 0.0f;
    r[j] = x;
    if (j < n) {
      s += (double)x;
      e += (h ? (double)h[j] : 1.0) * (double)x * (double)x;
    }
  }
  s = wave_sum_f64(s);
  e = wave_sum_f64(e);
  if (lane == 0) {
    rs[i] = s;
    rowE[i] = e;
  }
}

hipError_t stage_rows(const float* A, int m, int n, const float* h, float* R, int ldr, double* rs, double* rowE,
                      hipStream_t st) {
  hipLaunchKernelGGL(stage_rows_kernel, dim3((m + 3) / 4), dim3(256), 0, st, A, m, n, h, R, ldr, rs, rowE);
  return hipGetLastError();
}

// 64 x 64 tiles through LDS
__global__ void __launch_bounds__(256) transpose_kernel(const float* A, int m, int n, float* RT, int ldt) {
  __shared__ float tile[64][65];
  const int bi = blockIdx.y * 64, bj = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int i = bi + r, j = bj + tx;
    tile[r][tx] = (i < m && j < n) ? A[(size_t)i * n + j] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int j = bj + r, i = bi + tx;
    if (j < n && i < ldt) RT[(size_t)j * ldt + i] = tile[tx][r];
  }
}

hipError_t stage_transpose(const float* A, int m, int n, float* RT, int ldt, hipStream_t st) {
  dim3 grid((n + 63) / 64, (ldt + 63) / 64);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, A, m, n, RT, ldt);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) row_energy_kernel(const float* R, int m, int n, int ldr, const float* h,
                                                        double* rowE) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const float* r = R + (size_t)i * ldr;
  double e = 0.0;
  for (int j = lane; j < n; j += 64) {
    const double x = (double)r[j];
    e += (h ? (double)h[j] : 1.0) * x * x;
  }
  e = wave_sum_f64(e);
  if (lane == 0) rowE[i] = e;
}

hipError_t row_energy(const float* R, int m, int n, int ldr, const float* h, double* rowE, hipStream_t st) {
  hipLaunchKernelGGL(row_energy_kernel, dim3((m + 3) / 4), dim3(256), 0, st, R, m, n, ldr, h, rowE);
  return hipGetLastError();
}

}  // namespace externd

