// conv_device.h -- device helpers shared by the gfx950 convolution kernels:
// element conversions, output-row decoding, per-dimension tap masks, MFMA
// wrappers and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv_params.h"

namespace convfwd {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---- element conversions (fp32 accumulation; one RNE rounding on output) ----
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// v_cvt_f16_f32 rounds to nearest even in the default mode.
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }
// gfx950 converts with v_cvt_pk_bf16_f32, round to nearest even.
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// ---- output-row decoding ----
// Output position m = ((n*od + z)*oh + y)*ow + x.  Gives the input origin of
// its window (the position of tap (0,0,0), possibly in the padding) as an
// element offset into x, and the per-dimension validity masks: bit t of md is
// set iff input depth z*sd - pd + t*ed lies inside [0, d), likewise mh and mw.
struct RowInfo {
  int base;      // element offset of the window origin (may be negative or past the end)
  uint32_t md, mh, mw;
};

// Bits t with 0 <= i0 + t*e < size set, t < k <= 16 (so every shift is < 32):
// the taps t in [ceil(-i0 / e), floor((size - 1 - i0) / e)] of a filter whose
// taps are e positions apart.
// Undilated filters (e == 1, a value every workgroup shares, so the branch is
// uniform) need no division.
__device__ __forceinline__ uint32_t dim_mask(int i0, int k, int size, int e = 1) {
  int lo, hi;
  if (e == 1) {
    lo = max(0, -i0);
    hi = min(k, size - i0);
  } else {
    lo = i0 >= 0 ? 0 : (-i0 + e - 1) / e;
    hi = i0 > size - 1 ? 0 : min(k, (size - 1 - i0) / e + 1);
  }
  if (hi <= lo) return 0u;
  return ((1u << hi) - 1u) & ~((1u << lo) - 1u);
}

__device__ __forceinline__ RowInfo decode_row(const ConvParams& p, int m) {
  RowInfo r;
  if (m >= p.M) {
    r.base = 0; r.md = r.mh = r.mw = 0u;
    return r;
  }
  const int xo = m % p.ow;
  int t = m / p.ow;
  const int yo = t % p.oh;
  t /= p.oh;
  const int zo = t % p.od;
  const int n = t / p.od;
  const int z0 = zo * p.sd - p.pd;
  const int y0 = yo * p.sh - p.ph;
  const int x0 = xo * p.sw - p.pw;
  r.base = n * p.xs_n + z0 * p.xs_d + y0 * p.xs_h + x0 * p.xs_w;
  r.md = dim_mask(z0, p.kd, p.d, p.ed);
  r.mh = dim_mask(y0, p.kh, p.h, p.eh);
  r.mw = dim_mask(x0, p.kw, p.w, p.ew);
  return r;
}

// Element offset in y of output row m (its channel 0): m * cout for a dense y,
// else through the row strides of a stride phase of backward-data.
__device__ __forceinline__ int64_t out_row(const ConvParams& p, int m) {
  if (!p.remap) return (int64_t)m * p.cout;
  const int xo = m % p.ow;
  int t = m / p.ow;
  const int yo = t % p.oh;
  t /= p.oh;
  const int zo = t % p.od;
  const int n = t / p.od;
  return (int64_t)p.y_off + (int64_t)n * p.ys_n + (int64_t)zo * p.ys_d + (int64_t)yo * p.ys_h +
         (int64_t)xo * p.ys_w;
}

__device__ __forceinline__ bool tap_valid(const RowInfo& r, int kd, int kh, int kw) {
  return ((r.md >> kd) & (r.mh >> kh) & (r.mw >> kw) & 1u) != 0u;
}

// ---- output stores ----
// A 16-byte non-temporal store: output tiles are written once and not read
// back by the kernel, and a whole grid storing its tiles at once writes
// faster this way than through the ordinary write-allocate path (1-9% per
// launch on the measured shapes).
__device__ __forceinline__ void store16_nt(void* dst, u32x4_t v) {
  __builtin_nontemporal_store(v, (u32x4_t*)dst);
}
__device__ __forceinline__ void store16_nt(void* dst, uint4 v) {
  const u32x4_t vv = {v.x, v.y, v.z, v.w};
  store16_nt(dst, vv);
}

// ---- tile decode and small divisions without division sequences ----
// The per-tile and per-lane set-up runs before a workgroup's first loads, and
// with one or two waves per SIMD every instruction of it is exposed; a
// division by a run-time value costs ~30 instructions, a quarter-rate 32-bit
// multiply four times a full-rate one.

// Tile grid of the staged kernels and, for each divisor of the tile decode,
// m = ceil(2^32 / d) (0 for d = 1), computed on the host.
struct TileArgs {
  int tiles_n, wblocks, hblocks;
  uint32_t m_tn, m_wb, m_hb, m_od;
  uint32_t x_bytes, w_bytes;
};

inline uint32_t div_magic(int d) { return d <= 1 ? 0u : (uint32_t)(((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d); }

// floor(n / d) for 0 <= n < 2^24 with m = div_magic(d): n * m / 2^32 exceeds
// n / d by less than 2^-8, so it is the quotient or one more.
__device__ __forceinline__ int fast_div(int n, int d, uint32_t m) {
  if (m == 0u) return n;
  const int q = (int)__umulhi((uint32_t)n, m);
  return q * d > n ? q - 1 : q;
}

// floor(x / D) for 0 <= x < 1024 with one full-rate 24-bit multiply: the
// reciprocal rounded up errs by less than x * D / 2^16 / D < 1/64 of a unit,
// while x / D lies at least 1/D below the next whole number.
template <int D>
__device__ __forceinline__ int div_small(int x) {
  static_assert(D >= 1 && D <= 64, "small divisor");
  return (int)(__umul24((unsigned)x, (65536u + D - 1) / D) >> 16);
}

// Depth taps t < k with 0 <= z0 + t * e < d, as dim_mask, without a division
// when e == 1.
__device__ __forceinline__ uint32_t depth_mask(int z0, int k, int d, int e) {
  if (e == 1) return ((1u << min(k, max(0, d - z0))) - 1u) & ~((1u << max(0, -z0)) - 1u);
  return dim_mask(z0, k, d, e);
}

// ---- XCD-aware tile order ----
// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Give each XCD one contiguous run of tile ids so that the tiles resident on
// an XCD at the same time are spatial neighbours sharing that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int nblocks) {
  const int q = nblocks >> 3, rem = nblocks & 7;
  const int xcd = b & 7, local = b >> 3;
  return xcd * q + min(xcd, rem) + local;
}

// ---- MFMA wrappers: D(16x16, fp32) += A(16x32) * B(32x16) ----
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as the 8
// consecutive k in group l / 16; it receives D rows 4*(l/16) .. +3 of column
// l % 16.
__device__ __forceinline__ f32x4_t mfma16x16x32(half8_t a, half8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(bf168_t a, bf168_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16) * B(16x32).  Lane l supplies row (l % 32) of A
// and column (l % 32) of B, each as the 8 consecutive k of group l / 32; it
// receives column l % 32 of D, rows 8q + 4*(l/32) + i in element 4q + i.
__device__ __forceinline__ f32x16_t mfma32x32x16(half8_t a, half8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16(bf168_t a, bf168_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef half8_t type; };
template <> struct Vec8<__bf16> { typedef bf168_t type; };

}  // namespace convfwd
