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
// hold whole groups, filters 1, 3, 5 or 7 wide, stride 1 or 2 and no dilation
// along w.  A thread owns one 16-byte slice of channels (8 fp16/bf16 or 4
// fp32, whole groups, so the slice's outputs need only the slice's inputs) and
// a run of TW consecutive outputs along w.  For each (kd, kh) it loads the
// (TW-1)*s + K_w input positions its outputs' windows cover, each one 16-byte
// load, all in flight together, and reuses every load across the K_w taps that
// read it.  Groups of two or more 16-bit channels use two-channel dot products
// with fp32 accumulation (v_dot2_f32_f16 / v_dot2_f32_bf16), halving the
// instruction count; depthwise layers use one fp32 FMA per product (fp16
// operands feed v_fma_mix_f32 directly).  The filter is staged once per
// workgroup in LDS, reordered to (tap, C_out, C_in/G) so that one tap's weights
// for a slice are adjacent.  The grid is persistent, sized to what the chip
// holds at the kernel's occupancy (three or four waves per SIMD).  Consecutive
// threads take consecutive slices of one output position, so a wave's loads
// and stores cover whole rows of channels.
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

// Outputs along w per thread of the tiled kernel: as many as fit in the
// register budget of its occupancy (accumulators, the window row's loads and
// one tap's weights); with two output rows per thread (TH = 2) four.
template <int CG, int KW, int SW, int TH>
constexpr int tiled_tw() {
  return TH == 2 ? 4 : (CG <= 2 && KW * SW <= 3) ? 8 : (CG <= 4 ? 4 : 2);
}

// Workgroups per CU the tiled kernel is built for: depthwise slices keep 8
// outputs x 8 channels of fp32 accumulators and 10 input slices live, which
// spill at four workgroups per CU (128 registers) but fit at three (170);
// three runs depthwise 3x3x3 16% faster, while the narrower groups are 8%
// faster at four.
template <int CG, int TH>
constexpr int tiled_occ() {
  return CG == 1 ? 3 : 4;   // (TH = 2, depthwise only, holds 2 x 4 x 8 accumulators)
}

// Dot products of pairs of channels (v_dot2_f32_{f16,bf16}: two products
// and an fp32 accumulate in one instruction) for 16-bit groups of two or more
// channels; fp32 FMAs otherwise.
template <typename T> struct Pair;
template <> struct Pair<_Float16> { typedef _Float16 type __attribute__((ext_vector_type(2))); };
template <> struct Pair<__bf16> { typedef __bf16 type __attribute__((ext_vector_type(2))); };

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, _Float16*) {
  typedef Pair<_Float16>::type P;
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(P, a), __builtin_bit_cast(P, b), c, false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, __bf16*) {
  typedef Pair<__bf16>::type P;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(P, a), __builtin_bit_cast(P, b), c, false);
}

template <typename T, int CG>
constexpr bool use_dot2() { return sizeof(T) == 2 && CG >= 2; }

// ---- tiled kernel: C_out/G == C_in/G = CG, 16-byte slices, K_w = KW, stride SW ----
// Persistent: the grid is at most what the chip holds at the kernel's
// occupancy, and each thread strides over (slice, TH output rows x TW outputs)
// units.
template <typename T, int CG, int KW, int SW, int TH>
__global__ __launch_bounds__(256, (tiled_occ<CG, TH>())) void conv_grouped_tiled_kernel(
    ConvParams p, const T* __restrict__ x, const T* __restrict__ w, T* __restrict__ y, int tiles_w) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int VE = 16 / (int)sizeof(T);      // channels per slice
  constexpr int TW = tiled_tw<CG, KW, SW, TH>();   // outputs along w per unit
  static_assert(TH == 1 || TH == 2, "output rows per unit");
  constexpr int NP = (TW - 1) * SW + KW;       // input positions per window row
  constexpr bool D2 = use_dot2<T, CG>();
  // one tap's weights for a slice: VE * CG values, as fp32 or as channel pairs
  constexpr int NWD = D2 ? VE * CG / 2 : VE * CG;
  extern __shared__ uint32_t wls[];            // [tap][C_out][CG]: fp32, or T pairs

  // Filter element i = co * K + k (k = tap * CG + c) moves to (tap, co, c).
  // The workgroup reads consecutive elements; each thread steps (co, k) by
  // 256 elements incrementally instead of dividing by K per element.
  {
    const int wtotal = p.cout * p.K;
    const int dq = 256 / p.K, dr = 256 % p.K;
    int co = threadIdx.x / p.K, k = threadIdx.x % p.K;
    for (int i = threadIdx.x; i < wtotal; i += 256) {
      const int dst = ((k / CG) * p.cout + co) * CG + (k % CG);   // CG is a power of two
      if constexpr (D2) ((T*)wls)[dst] = w[i];
      else ((float*)wls)[dst] = to_f32(w[i]);
      co += dq;
      k += dr;
      if (k >= p.K) { k -= p.K; ++co; }
    }
  }
  __syncthreads();

  // Unit counts stay below 2^31: x and y are below 2^31 bytes.
  const int U = p.cin / VE;                    // slices per position
  const int ohu = (p.oh + TH - 1) / TH;       // units along h
  const int units = p.n * p.od * ohu * tiles_w * U;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, (short)0, (int)((int64_t)p.n * p.xs_n * (int)sizeof(T)), kRawBufferFlags);

  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < units; idx += gridDim.x * 256) {
    const int u = idx % U;
    int r = idx / U;
    const int twi = r % tiles_w;
    r /= tiles_w;
    const int yo = (r % ohu) * TH;              // first output row of the unit
    r /= ohu;
    const int zo = r % p.od;
    const int n = r / p.od;
    const int ow0 = twi * TW;
    const int xi0 = ow0 * SW - p.pw;

    float acc[TH][TW][VE];
#pragma unroll
    for (int h = 0; h < TH; ++h)
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int j = 0; j < VE; ++j) acc[h][t][j] = 0.f;

    for (int a = 0; a < p.kd; ++a) {
      const int zi = zo * p.sd - p.pd + a * p.ed;
      if (zi < 0 || zi >= p.d) continue;
      // TH = 1: input row b of the window (any stride and dilation along h).
      // TH = 2 (unit stride, undilated): input row b serves output row h with
      // tap b - h, so each of the K_h + 1 rows is loaded once for both.
      for (int b = 0; b < p.kh + TH - 1; ++b) {
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
#pragma unroll
        for (int h = 0; h < TH; ++h) {
        const int tb = b - h;                    // the tap this row is for output row h
        if (tb < 0 || tb >= p.kh) continue;
        // this slice's weights of tap (a, tb, 0), in dwords
        const uint32_t* wrow = wls + ((a * p.kh + tb) * KW * p.cout + u * VE) * CG / (D2 ? 2 : 1);
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          uint32_t wv[NWD];
          const u4* wp = (const u4*)(wrow + e * p.cout * CG / (D2 ? 2 : 1));
#pragma unroll
          for (int q = 0; q < NWD / 4; ++q) {
            const u4 v = wp[q];
            wv[4 * q] = v[0]; wv[4 * q + 1] = v[1]; wv[4 * q + 2] = v[2]; wv[4 * q + 3] = v[3];
          }
          if constexpr (D2) {
            // output o (group o / CG) takes the CG / 2 channel pairs of its group
#pragma unroll
            for (int c2 = 0; c2 < CG / 2; ++c2)
#pragma unroll
              for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int o = 0; o < VE; ++o)
                  acc[h][t][o] = dot2(xv[t * SW + e][(o / CG) * (CG / 2) + c2], wv[o * (CG / 2) + c2],
                                      acc[h][t][o], (T*)nullptr);
          } else {
            // channel outermost: consecutive FMAs update different accumulators
#pragma unroll
            for (int c = 0; c < CG; ++c)
#pragma unroll
              for (int t = 0; t < TW; ++t)
#pragma unroll
                for (int o = 0; o < VE; ++o)   // (o / CG) * CG is the first channel of o's group
                  acc[h][t][o] = fmaf(slice_elem<T>(xv[t * SW + e], (o / CG) * CG + c),
                                      __builtin_bit_cast(float, wv[o * CG + c]), acc[h][t][o]);
          }
        }
        }
      }
    }

#pragma unroll
    for (int h = 0; h < TH; ++h) {
      if (yo + h >= p.oh) continue;
      T* yrow = y + ((((int64_t)n * p.od + zo) * p.oh + yo + h) * p.ow) * p.cout + u * VE;
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (ow0 + t < p.ow) {
          T out[VE];
#pragma unroll
          for (int j = 0; j < VE; ++j) out[j] = from_f32<T>(acc[h][t][j]);
          store16_nt(yrow + (int64_t)(ow0 + t) * p.cout, __builtin_bit_cast(u32x4_t, out));
        }
      }
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

template <typename T, int CG, int KW, int SW, int TH>
hipError_t launch_tiled_th(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int TW = tiled_tw<CG, KW, SW, TH>();
  const int tiles_w = (p.ow + TW - 1) / TW;
  const int64_t units = (int64_t)p.n * p.od * ((p.oh + TH - 1) / TH) * tiles_w * (p.cin / VE);
  int64_t blocks = (units + 255) / 256;
  // persistent: as many workgroups as the chip holds at the kernel's occupancy
  const int cap = tiled_occ<CG, TH>() * device_cus();
  if (blocks > cap) blocks = cap;
  const size_t lds = (size_t)p.cout * p.K * (use_dot2<T, CG>() ? sizeof(T) : sizeof(float));
  hipLaunchKernelGGL((conv_grouped_tiled_kernel<T, CG, KW, SW, TH>), dim3((unsigned)blocks), dim3(256), lds, s,
                     p, (const T*)x, (const T*)w, (T*)y, tiles_w);
  return hipGetLastError();
}

// Depthwise at unit stride and no dilation along h, filters up to 3 wide: two
// output rows per thread, each input row loaded once for both.
template <typename T, int CG, int KW, int SW>
hipError_t launch_tiled_sw(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if constexpr (CG == 1 && SW == 1 && KW <= 3) {
    if (p.sh == 1 && p.eh == 1) return launch_tiled_th<T, CG, KW, SW, 2>(p, x, w, y, s);
  }
  return launch_tiled_th<T, CG, KW, SW, 1>(p, x, w, y, s);
}

template <typename T, int CG, int KW>
hipError_t launch_tiled_kw(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.sw == 1) return launch_tiled_sw<T, CG, KW, 1>(p, x, w, y, s);
  return launch_tiled_sw<T, CG, KW, 2>(p, x, w, y, s);
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
