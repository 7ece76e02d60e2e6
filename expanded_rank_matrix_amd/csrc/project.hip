// Batched ternary projection: one workgroup per vector, the same device routine the
// decomposition kernels use for every V- and U-step selection.
#include "externd_internal.hpp"
#include "select.hpp"

namespace externd {

template <int kPNT, int E>
__global__ void __launch_bounds__(kPNT) project_kernel(const float* X, int L, float tau, const float* h, int EHm,
                                                       int8_t* V, double* PHC) {
  __shared__ SelScratch s;
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = X + (size_t)row * L;
  float av[E], hw[E];
  int sg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid + e * kPNT;
    const float v = j < L ? x[j] : 0.0f;
    av[e] = fabsf(v);
    sg[e] = v > 0.0f ? 1 : (v < 0.0f ? -1 : 0);
    hw[e] = (h && j < L) ? h[j] : 1.0f;
  }
  const SelResult r = h ? ternary_select<kPNT, E, true>(av, hw, tau, EHm, s) : ternary_select<kPNT, E, false>(av, hw, tau, 0, s);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid + e * kPNT;
    if (j < L) {
      const unsigned k = __float_as_uint(av[e]);
      const bool on = r.count > 0u && k != 0u && k >= r.ekey && k >= r.tkey;
      V[(size_t)row * L + j] = on ? (int8_t)sg[e] : (int8_t)0;
    }
  }
  if (tid == 0) {
    PHC[3 * (size_t)row + 0] = r.P;
    PHC[3 * (size_t)row + 1] = r.H;
    PHC[3 * (size_t)row + 2] = (double)r.count;
  }
}

hipError_t project_rows(const float* X, int count, int L, float tau, const float* h, int EHm, int8_t* V,
                        double* PHC, hipStream_t st) {
  // 512 threads (256 VGPRs per lane) up to 8192 elements, 1024 threads beyond
  const int E = (L + 511) / 512;
  dim3 grid(count);
  if (E <= 1) hipLaunchKernelGGL((project_kernel<512, 1>), grid, dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else if (E <= 2) hipLaunchKernelGGL((project_kernel<512, 2>), grid, dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else if (E <= 4) hipLaunchKernelGGL((project_kernel<512, 4>), grid, dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else if (E <= 8) hipLaunchKernelGGL((project_kernel<512, 8>), grid, dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else if (E <= 16) hipLaunchKernelGGL((project_kernel<512, 16>), grid, dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else if (L <= 16384) hipLaunchKernelGGL((project_kernel<1024, 16>), grid, dim3(1024), 0, st, X, L, tau, h, EHm, V, PHC);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace externd
