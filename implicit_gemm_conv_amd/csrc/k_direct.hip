// k_direct.hip -- the simplest path: one thread per output element.
//
// Each thread walks its window tap by tap and channel by channel with fp32
// FMAs, skipping taps that fall in the zero padding.  It accepts every problem
// the descriptor can express (any filter size, any channel count, groups,
// dilation, all three dtypes) and serves as the always-available fallback and
// as a layout-free cross-check of the MFMA paths.
#include "conv_device.h"

namespace convfwd {

template <typename T>
__global__ __launch_bounds__(256) void conv_direct_kernel(ConvParams p, const T* __restrict__ x,
                                                          const T* __restrict__ w,
                                                          T* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.M * p.cout) return;
  const int co = (int)(idx % p.cout);
  const int m = (int)(idx / p.cout);
  const int xo = m % p.ow;
  int t = m / p.ow;
  const int yo = t % p.oh;
  t /= p.oh;
  const int zo = t % p.od;
  const int n = t / p.od;
  const T* wrow = w + (int64_t)co * p.K;
  const int c0 = (co / p.cout_g) * p.cin_g;   // first input channel of this output's group
  float acc = 0.f;
  for (int a = 0; a < p.kd; ++a) {
    const int zi = zo * p.sd - p.pd + a * p.ed;
    if (zi < 0 || zi >= p.d) continue;
    for (int b = 0; b < p.kh; ++b) {
      const int yi = yo * p.sh - p.ph + b * p.eh;
      if (yi < 0 || yi >= p.h) continue;
      for (int e = 0; e < p.kw; ++e) {
        const int xi = xo * p.sw - p.pw + e * p.ew;
        if (xi < 0 || xi >= p.w) continue;
        const T* xp = x + (int64_t)n * p.xs_n + (int64_t)zi * p.xs_d + (int64_t)yi * p.xs_h +
                      (int64_t)xi * p.xs_w + c0;
        const T* wp = wrow + ((a * p.kh + b) * p.kw + e) * p.cin_g;
        for (int c = 0; c < p.cin_g; ++c) acc = fmaf(to_f32(xp[c]), to_f32(wp[c]), acc);
      }
    }
  }
  y[out_row(p, m) + co] = from_f32<T>(acc);
}

hipError_t launch_direct(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                         hipStream_t s) {
  const int64_t total = (int64_t)p.M * p.cout;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dtype == kF32)
    hipLaunchKernelGGL(conv_direct_kernel<float>, dim3(blocks), dim3(256), 0, s, p,
                       (const float*)x, (const float*)w, (float*)y);
  else if (dtype == kF16)
    hipLaunchKernelGGL(conv_direct_kernel<_Float16>, dim3(blocks), dim3(256), 0, s, p,
                       (const _Float16*)x, (const _Float16*)w, (_Float16*)y);
  else
    hipLaunchKernelGGL(conv_direct_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, p,
                       (const __bf16*)x, (const __bf16*)w, (__bf16*)y);
  return hipGetLastError();
}

}  // namespace convfwd
