// k_bwd.hip -- the filter rearrangement behind backward-data (the transposed
// convolution of the tutorial's variant list, "Convolution variants worth
// knowing").
//
// Backward-data sends dy[o] * w[k] back to dx[i] for i = o*s - p + k*e.  Split
// dx positions by their stride phase r (i = j*s + r, per dimension): the taps
// that reach phase r are those with k*e = r + p (mod s), an arithmetic run
// k = k0 + t*s' (s' = s / gcd(e, s)), and over them o = j + q0 - t*e'
// (e' = e / gcd(e, s)).  With the run reversed (t' = T-1-t) each phase is an
// ordinary forward convolution of dy at unit stride, dilation e' and low pad
// (T-1)*e' - q0, whose output rows are every s-th position of dx -- so the
// forward kernels compute it, reading a filter whose rows are dx channels and
// whose depth is (t'_d, t'_h, t'_w, dy channel of the group), the forward
// layout of the exchanged problem.  This kernel writes those per-phase filters
// from w, phase after phase (phases in (r_d, r_h, r_w) order), each tap of w
// landing in exactly one phase, so the result has w's size.
#include "conv_device.h"

namespace convfwd {

namespace {

// Phase of tap k along one dimension and its reversed index in that phase.
__device__ __forceinline__ void tap_phase(const BwdGeom& g, int dim, int k, int* r, int* tr) {
  const int s = g.s[dim];
  const int ph = ((k * g.e[dim] - g.p[dim]) % s + s) % s;
  int gcd = g.e[dim], b = s;
  while (b) {
    const int t = gcd % b;
    gcd = b;
    b = t;
  }
  const int t = (k - g.k0[dim][ph]) / (s / gcd);
  *r = ph;
  *tr = g.t[dim][ph] - 1 - t;
}

template <typename T>
__global__ __launch_bounds__(256) void conv_bwd_filter_kernel(BwdGeom g, const T* __restrict__ w,
                                                              T* __restrict__ wt) {
  const int cin_g = g.cin / g.groups, og = g.cout / g.groups;
  const int64_t total = (int64_t)g.cout * g.k[0] * g.k[1] * g.k[2] * cin_g;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  // w index = (((co*K_d + kd)*K_h + kh)*K_w + kw)*cin_g + cl
  int64_t r = idx;
  const int cl = (int)(r % cin_g);
  r /= cin_g;
  const int kw = (int)(r % g.k[2]);
  r /= g.k[2];
  const int kh = (int)(r % g.k[1]);
  r /= g.k[1];
  const int kd = (int)(r % g.k[0]);
  const int co = (int)(r / g.k[0]);
  int rd, rh, rw, td, th, tw;
  tap_phase(g, 0, kd, &rd, &td);
  tap_phase(g, 1, kh, &rh, &th);
  tap_phase(g, 2, kw, &rw, &tw);
  const int Td = g.t[0][rd], Th = g.t[1][rh], Tw = g.t[2][rw];
  // start of the phase's block: all taps of earlier phases, C_in * og values each
  const int64_t off = (int64_t)og * g.cin *
                      ((int64_t)g.pre[0][rd] * g.k[1] * g.k[2] + (int64_t)Td * g.pre[1][rh] * g.k[2] +
                       (int64_t)Td * Th * g.pre[2][rw]);
  const int grp = co / og;
  const int c = grp * cin_g + cl;   // dx channel: the row of the phase filter
  const int64_t within = ((((int64_t)c * Td + td) * Th + th) * Tw + tw) * og + (co - grp * og);
  wt[off + within] = w[idx];
}

}  // namespace

hipError_t launch_bwd_filter(const BwdGeom& g, int dtype, const void* w, void* wt, hipStream_t s) {
  const int64_t total = (int64_t)g.cout * g.k[0] * g.k[1] * g.k[2] * (g.cin / g.groups);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dtype == kF32)
    hipLaunchKernelGGL(conv_bwd_filter_kernel<float>, dim3(blocks), dim3(256), 0, s, g, (const float*)w,
                       (float*)wt);
  else if (dtype == kF16)
    hipLaunchKernelGGL(conv_bwd_filter_kernel<_Float16>, dim3(blocks), dim3(256), 0, s, g,
                       (const _Float16*)w, (_Float16*)wt);
  else
    hipLaunchKernelGGL(conv_bwd_filter_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, g, (const __bf16*)w,
                       (__bf16*)wt);
  return hipGetLastError();
}

}  // namespace convfwd
