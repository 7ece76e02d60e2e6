// Batched ternary projection: one workgroup per vector, the same device routine the
// decomposition kernels use for every V- and U-step selection.
#include "externd_internal.hpp"
#include "select.hpp"

namespace externd {

template <bool W>
__global__ void __launch_bounds__(512) project_kernel(const float* X, int L, float tau, const float* h, int EHm,
                                                      int8_t* V, double* PHC) {
  __shared__ SelScratchT<W> s;
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = X + (size_t)row * L;
  const SelResult r = ternary_select<512, W>(x, h, L, tau, EHm, s);
  for (int j = tid; j < L; j += 512) {
    const float xv = x[j];
    V[(size_t)row * L + j] = selected(xv, r) ? (xv > 0.0f ? (int8_t)1 : (int8_t)-1) : (int8_t)0;
  }
  if (tid == 0) {
    PHC[3 * (size_t)row + 0] = r.P;
    PHC[3 * (size_t)row + 1] = r.H;
    PHC[3 * (size_t)row + 2] = (double)r.count;
  }
}

hipError_t project_rows(const float* X, int count, int L, float tau, const float* h, int EHm, int8_t* V,
                        double* PHC, hipStream_t st) {
  if (h) hipLaunchKernelGGL(project_kernel<true>, dim3(count), dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  else hipLaunchKernelGGL(project_kernel<false>, dim3(count), dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  return hipGetLastError();
}

}  // namespace externd
