// Batched ternary projection: one workgroup per vector, the same device routine the
// decomposition kernels use for every V- and U-step selection.
#include "externd_internal.hpp"
#include "select.hpp"

namespace externd {

// Unweighted vectors go through the key-array selection the sequential kernel uses (the row's
// fp32 bit patterns staged in LDS), with the same fallback to the general selection.
template <bool W>
__global__ void __launch_bounds__(512) project_kernel(const float* X, int L, float tau, const float* h, int EHm,
                                                      int8_t* V, double* PHC) {
  __shared__ SelScratchT<W> s;
  extern __shared__ unsigned keys[];  // L values, unweighted only
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = X + (size_t)row * L;
  SelResult r;
  if (W) {
    r = ternary_select<512, W>(x, h, L, tau, EHm, s);
  } else {
    unsigned kx = 0u;
    for (int j = tid; j < L; j += 512) {
      const unsigned kb = __float_as_uint(x[j]);
      keys[j] = kb;
      kx = (kb & 0x7FFFFFFFu) > kx ? (kb & 0x7FFFFFFFu) : kx;
    }
    select_prepare<512>(s, kx);
    unsigned km = 0u;
    for (int w = 0; w < 8; ++w) km = s.red_u[w] > km ? s.red_u[w] : km;
    bool ok = true;
    r = ternary_select_keys<512>(keys, L, tau, km, s, &ok);
    if (!ok) {
      select_prepare<512>(s, km);
      r = ternary_select<512, false, float, W, true>(x, nullptr, L, tau, 0, s);
    }
  }
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
  if (h) {
    hipLaunchKernelGGL(project_kernel<true>, dim3(count), dim3(512), 0, st, X, L, tau, h, EHm, V, PHC);
  } else {
    static bool attr[64] = {};  // once per device: up to 64 KB of staged keys
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!attr[dev]) {
      e = hipFuncSetAttribute((const void*)project_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              64 * 1024);
      if (e != hipSuccess) return e;
      attr[dev] = true;
    }
    hipLaunchKernelGGL(project_kernel<false>, dim3(count), dim3(512), sizeof(unsigned) * (size_t)L, st, X, L, tau,
                       h, EHm, V, PHC);
  }
  return hipGetLastError();
}

}  // namespace externd
