// k_grouped.hip -- grouped convolutions with few channels per group, down to
// depthwise (one input and one output channel per group).
//
// The tutorial page ("Convolution variants worth knowing") notes that
// depthwise convolutions do very little arithmetic per byte and are bound by
// memory, not by the matrix unit; the same holds for grouped layers with a few
// channels per group (ResNeXt).  A per-group GEMM would be a few columns wide,
// so this path skips the GEMM form and runs on the vector ALU with fp32 FMAs.
//
// Two kernels.  The tiled one takes groups with as many output as input
// channels (C_out/G == C_in/G, depthwise included) when 16 bytes of channels
// hold whole groups, filters up to 7 wide, stride 1 or 2 and no dilation
// along w.  A thread owns one 16-byte slice of channels (8 fp16/bf16 or 4
// fp32, whole groups, so the slice's outputs need only the slice's inputs) and
// a run of TW consecutive outputs along w.  For each (kd, kh) it loads the
// (TW-1)*s + K_w input positions its outputs' windows cover, each one 16-byte
// load, all in flight together, and reuses every load across the K_w taps that
// read it.  The filter is staged once per workgroup in LDS as fp32, reordered
// to (tap, C_out, C_in/G) so that one tap's weights for a slice are adjacent.
// Consecutive threads take consecutive slices of one output position, so a
// wave's loads and stores cover whole rows of channels.
//
// The general kernel takes everything else the path accepts (other channel
// ratios, dilation along w, odd channel counts, unaligned tensors): one
// thread per (output position, group), the filter in LDS in its own layout,
// and a window row's loads gathered before its FMAs.
#include "conv_device.h"

namespace convfwd {

namespace {

constexpr int kMaxOG = 16;              // output channels per group in the general kernel
constexpr int kLdsElems = 16 * 1024;    // filter elements staged (at most 64 KB as fp32)
constexpr int kMaxKW = 7;               // widest filter of the tiled kernel
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Element j of a 16-byte slice as fp32.
template <typename T> __device__ __forceinline__ float slice_elem(const u4& v, int j);
template <> __device__ __forceinline__ float slice_elem<float>(const u4& v, int j) {
  // through a scalar: clang's bit_cast of a vector-element subscript reads element 0
  const uint32_t d = v[j];
  return __builtin_bit_cast(float, d);
}
template <> __device__ __forceinline__ float slice_elem<_Float16>(const u4& v, int j) {
  const uint32_t d = v[j >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (d >> 16) : (d & 0xffffu)));
}
template <> __device__ __forceinline__ float slice_elem<__bf16>(const u4& v, int j) {
  const uint32_t d = v[j >> 1];
  return __builtin_bit_cast(float, (j & 1) ? (d & 0xffff0000u) : (d << 16));
}

// ---- tiled kernel: C_out/G == C_in/G = CG, 16-byte slices, K_w = KW, stride SW ----
template <typename T, int CG, int KW, int SW>
__global__ __launch_bounds__(256) void conv_grouped_tiled_kernel(ConvParams p, const T* __restrict__ x,
                                                                 const T* __restrict__ w,
                                                                 T* __restrict__ y, int tiles_w) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int VE = 16 / (int)sizeof(T);      // channels per slice
  constexpr int TW = CG >= 8 ? 4 : 8;          // outputs along w per thread
  constexpr int NP = (TW - 1) * SW + KW;       // input positions per window row
  constexpr int NW = VE * CG;                  // one tap's weights for a slice
  extern __shared__ float wls[];               // [tap][C_out][CG], fp32

  const int ntaps = p.kd * p.kh * KW;
  const int wtotal = p.cout * p.K;
  for (int i = threadIdx.x; i < wtotal; i += 256) {
    const int c = i % CG, r = i / CG;
    const int tap = r % ntaps, co = r / ntaps;
    wls[(tap * p.cout + co) * CG + c] = to_f32(w[i]);
  }
  __syncthreads();

  const int U = p.cin / VE;                    // slices per position
  const int64_t units = (int64_t)p.n * p.od * p.oh * tiles_w * U;
  const int64_t idx = (int64_t)xcd_tile(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (idx >= units) return;
  const int u = (int)(idx % U);
  int64_t r = idx / U;
  const int twi = (int)(r % tiles_w);
  r /= tiles_w;
  const int yo = (int)(r % p.oh);
  r /= p.oh;
  const int zo = (int)(r % p.od);
  const int n = (int)(r / p.od);
  const int ow0 = twi * TW;
  const int xi0 = ow0 * SW - p.pw;

  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, (short)0, (int)((int64_t)p.n * p.xs_n * (int)sizeof(T)), kRawBufferFlags);

  float acc[TW][VE];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int j = 0; j < VE; ++j) acc[t][j] = 0.f;

  for (int a = 0; a < p.kd; ++a) {
    const int zi = zo * p.sd - p.pd + a * p.ed;
    if (zi < 0 || zi >= p.d) continue;
    for (int b = 0; b < p.kh; ++b) {
      const int yi = yo * p.sh - p.ph + b * p.eh;
      if (yi < 0 || yi >= p.h) continue;
      const int row = n * p.xs_n + zi * p.xs_d + yi * p.xs_h + u * VE;
      u4 xv[NP];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int xi = xi0 + j;
        const bool ok = xi >= 0 && xi < p.w;
        xv[j] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, ok ? (uint32_t)((row + xi * p.xs_w) * (int)sizeof(T)) : kOutOfRange, 0, 0);
      }
      const float* wrow = wls + ((a * p.kh + b) * KW * p.cout + u * VE) * CG;
#pragma unroll
      for (int e = 0; e < KW; ++e) {
        float wv[NW];
        const f32x4_t* wp = (const f32x4_t*)(wrow + e * p.cout * CG);
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
          const f32x4_t v = wp[q];
          wv[4 * q] = v[0]; wv[4 * q + 1] = v[1]; wv[4 * q + 2] = v[2]; wv[4 * q + 3] = v[3];
        }
        // channel outermost: consecutive FMAs update different accumulators
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int o = 0; o < VE; ++o)   // (o / CG) * CG is the first channel of o's group
              acc[t][o] = fmaf(slice_elem<T>(xv[t * SW + e], (o / CG) * CG + c), wv[o * CG + c], acc[t][o]);
      }
    }
  }

  T* yrow = y + ((((int64_t)n * p.od + zo) * p.oh + yo) * p.ow) * p.cout + u * VE;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    if (ow0 + t < p.ow) {
      T out[VE];
#pragma unroll
      for (int j = 0; j < VE; ++j) out[j] = from_f32<T>(acc[t][j]);
      *(u4*)(yrow + (int64_t)(ow0 + t) * p.cout) = __builtin_bit_cast(u4, out);
    }
  }
#endif
}

// ---- general kernel: one thread per (output position, group) ----
template <typename T, int CG>
__global__ __launch_bounds__(256) void conv_grouped_kernel(ConvParams p, const T* __restrict__ x,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ y) {
  constexpr int kBatch = 8;                    // window positions gathered before their FMAs
  __shared__ T wl[kLdsElems];
  const int og = p.cout_g;
  const int wtotal = p.cout * p.K;
  for (int i = threadIdx.x; i < wtotal; i += 256) wl[i] = w[i];
  __syncthreads();

  const int64_t pairs = (int64_t)p.M * p.groups;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < pairs; idx += stride) {
    const int g = (int)(idx % p.groups);
    const int m = (int)(idx / p.groups);
    const int xo = m % p.ow;
    int t = m / p.ow;
    const int yo = t % p.oh;
    t /= p.oh;
    const int zo = t % p.od;
    const int n = t / p.od;
    float acc[kMaxOG];
#pragma unroll
    for (int o = 0; o < kMaxOG; ++o) acc[o] = 0.f;
    const T* wg = wl + (size_t)g * og * p.K;
    const T* xg = x + (int64_t)n * p.xs_n + g * CG;
    for (int a = 0; a < p.kd; ++a) {
      const int zi = zo * p.sd - p.pd + a * p.ed;
      if (zi < 0 || zi >= p.d) continue;
      for (int b = 0; b < p.kh; ++b) {
        const int yi = yo * p.sh - p.ph + b * p.eh;
        if (yi < 0 || yi >= p.h) continue;
        const T* xrow = xg + (int64_t)zi * p.xs_d + (int64_t)yi * p.xs_h;
        for (int e0 = 0; e0 < p.kw; e0 += kBatch) {
          float xv[kBatch][CG];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const int xi = xo * p.sw - p.pw + (e0 + k) * p.ew;
            const bool ok = e0 + k < p.kw && xi >= 0 && xi < p.w;
#pragma unroll
            for (int c = 0; c < CG; ++c) xv[k][c] = ok ? to_f32(xrow[(int64_t)xi * p.xs_w + c]) : 0.f;
          }
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            if (e0 + k >= p.kw) break;
            const T* wt = wg + ((a * p.kh + b) * p.kw + e0 + k) * CG;
#pragma unroll
            for (int o = 0; o < kMaxOG; ++o) {
              if (o < og) {
#pragma unroll
                for (int c = 0; c < CG; ++c) acc[o] = fmaf(xv[k][c], to_f32(wt[o * p.K + c]), acc[o]);
              }
            }
          }
        }
      }
    }
    T* yp = y + (int64_t)m * p.cout + g * og;
#pragma unroll
    for (int o = 0; o < kMaxOG; ++o)
      if (o < og) yp[o] = from_f32<T>(acc[o]);
  }
}

template <typename T, int CG, int KW>
hipError_t launch_tiled_kw(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int TW = CG >= 8 ? 4 : 8;
  const int tiles_w = (p.ow + TW - 1) / TW;
  const int64_t units = (int64_t)p.n * p.od * p.oh * tiles_w * (p.cin / VE);
  const unsigned blocks = (unsigned)((units + 255) / 256);
  const size_t lds = (size_t)p.cout * p.K * sizeof(float);
  if (p.sw == 1)
    hipLaunchKernelGGL((conv_grouped_tiled_kernel<T, CG, KW, 1>), dim3(blocks), dim3(256), lds, s, p,
                       (const T*)x, (const T*)w, (T*)y, tiles_w);
  else
    hipLaunchKernelGGL((conv_grouped_tiled_kernel<T, CG, KW, 2>), dim3(blocks), dim3(256), lds, s, p,
                       (const T*)x, (const T*)w, (T*)y, tiles_w);
  return hipGetLastError();
}

template <typename T, int CG>
hipError_t launch_tiled_cg(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  switch (p.kw) {
    case 1: return launch_tiled_kw<T, CG, 1>(p, x, w, y, s);
    case 3: return launch_tiled_kw<T, CG, 3>(p, x, w, y, s);
    case 5: return launch_tiled_kw<T, CG, 5>(p, x, w, y, s);
    default: return launch_tiled_kw<T, CG, 7>(p, x, w, y, s);
  }
}

template <typename T>
bool tiled_takes(const ConvParams& p, const void* x, const void* y) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int cg = p.cin_g;
  return p.cout_g == cg && VE % cg == 0 && p.cin % VE == 0 &&
         (p.kw == 1 || p.kw == 3 || p.kw == 5 || p.kw == kMaxKW) && (p.sw == 1 || p.sw == 2) &&
         p.ew == 1 && (((uintptr_t)x | (uintptr_t)y) & 15) == 0 &&
         (int64_t)p.n * p.xs_n * (int64_t)sizeof(T) < ((int64_t)1 << 31);
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (tiled_takes<T>(p, x, y)) {
    switch (p.cin_g) {
      case 1: return launch_tiled_cg<T, 1>(p, x, w, y, s);
      case 2: return launch_tiled_cg<T, 2>(p, x, w, y, s);
      case 4: return launch_tiled_cg<T, 4>(p, x, w, y, s);
      default:
        if constexpr (sizeof(T) == 2) return launch_tiled_cg<T, 8>(p, x, w, y, s);
        return hipErrorInvalidValue;
    }
  }
  const int64_t pairs = (int64_t)p.M * p.groups;
  // persistent: at most eight workgroups per CU, each staging the filter once
  int64_t blocks = (pairs + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  switch (p.cin_g) {
    case 1: hipLaunchKernelGGL((conv_grouped_kernel<T, 1>), dim3((unsigned)blocks), dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y); break;
    case 2: hipLaunchKernelGGL((conv_grouped_kernel<T, 2>), dim3((unsigned)blocks), dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y); break;
    case 4: hipLaunchKernelGGL((conv_grouped_kernel<T, 4>), dim3((unsigned)blocks), dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y); break;
    case 8: hipLaunchKernelGGL((conv_grouped_kernel<T, 8>), dim3((unsigned)blocks), dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y); break;
    default: hipLaunchKernelGGL((conv_grouped_kernel<T, 16>), dim3((unsigned)blocks), dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y); break;
  }
  return hipGetLastError();
}

}  // namespace

bool grouped_accepts(const ConvParams& p, int dtype) {
  (void)dtype;
  const int cg = p.cin_g;
  return p.groups > 1 && (cg == 1 || cg == 2 || cg == 4 || cg == 8 || cg == 16) &&
         p.cout_g <= kMaxOG && (int64_t)p.cout * p.K <= kLdsElems;
}

hipError_t launch_grouped(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                          hipStream_t s) {
  if (dtype == kF32) return launch_typed<float>(p, x, w, y, s);
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
