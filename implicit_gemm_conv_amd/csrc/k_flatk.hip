// k_flatk.hip -- implicit GEMM over the flattened (tap, channel) axis, any C_in.
//
// This is the tail path for channel counts that the 64-channel steps of the
// main path cannot take (C_in = 21, 65, 3, ...) and the fp32 path.  The GEMM
// depth K = taps * C_in is walked in steps of 32 consecutive k, with no
// per-tap padding: a step may straddle taps.  Column k of the virtual im2col
// matrix is tap k / C_in, channel k % C_in, which is also the filter's own
// flat index, so filter rows are read as they lie in memory.
//
// Each thread owns one k column of the step and tracks its (kd, kh, kw, c)
// incrementally (no division in the loop).  Gathers are element-granular
// (rows of odd channel counts are only 2-byte aligned), go through registers
// and are written to a double-buffered LDS tile whose rows are padded by 16
// bytes so that 16-byte fragment reads of 8 consecutive rows hit distinct
// banks.  The next step's gathers are issued before the current step's
// MFMAs.  fp16/bf16 use v_mfma_f32_16x16x32_*; fp32 uses v_mfma_f32_16x16x4_f32
// (eight per step), all with fp32 accumulators and one rounding at the store.
#include "conv_device.h"

namespace convfwd {

namespace {

template <typename T> struct Frag;
template <> struct Frag<_Float16> { typedef half8_t type; };
template <> struct Frag<__bf16> { typedef bf168_t type; };
template <> struct Frag<float> { typedef struct { f32x4_t lo, hi; } type; };

// One 32-deep step of D(16x16) += Wfrag * Xfrag^T for one block.
__device__ __forceinline__ f32x4_t step_mfma(half8_t a, half8_t b, f32x4_t c) {
  return mfma16x16x32(a, b, c);
}
__device__ __forceinline__ f32x4_t step_mfma(bf168_t a, bf168_t b, f32x4_t c) {
  return mfma16x16x32(a, b, c);
}
// Lane group g supplies k = 8g + e to the e-th 16x16x4 product; over e < 8
// and g < 4 that covers the 32 k of the step once each.
template <typename F>
__device__ __forceinline__ f32x4_t step_mfma(const F& a, const F& b, f32x4_t c) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
  return c;
}

template <typename T, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void conv_flatk_kernel(ConvParams p, const T* __restrict__ x,
                                                         const T* __restrict__ w,
                                                         T* __restrict__ y, int tiles_n) {
  typedef typename Frag<T>::type F;
  constexpr int BK = 32;
  constexpr int EB = sizeof(T);
  constexpr int ROWB = BK * EB + 16;      // padded LDS row
  constexpr int A_PER = BM / 8;           // rows gathered per thread per step
  constexpr int B_PER = BN / 8;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static_assert(WM * WN == 4, "4 waves");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  const int kk = tid & 31;   // this thread's k column within a step
  const int rsub = tid >> 5; // first row it gathers; then every 8th

  RowInfo ri[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) ri[i] = decode_row(p, m0 + rsub + 8 * i);
  const T* wrow[B_PER];
#pragma unroll
  for (int j = 0; j < B_PER; ++j) {
    const int n = n0 + rsub + 8 * j;
    wrow[j] = n < p.cout ? w + (int64_t)n * p.K : nullptr;
  }

  // (kd, kh, kw, c) of column k = kk of the first step.
  int k = kk;
  int c = kk % p.cin;
  int tap = kk / p.cin;
  int kw_ = tap % p.kw;
  tap /= p.kw;
  int kh_ = tap % p.kh;
  int kd_ = tap / p.kh;

  T ra[A_PER], rb[B_PER];
  auto gather = [&]() {
    const bool kin = k < p.K;
    const int off = kd_ * p.xs_d + kh_ * p.xs_h + kw_ * p.xs_w + c;
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      ra[i] = (kin && tap_valid(ri[i], kd_, kh_, kw_)) ? x[ri[i].base + off] : (T)0.f;
#pragma unroll
    for (int j = 0; j < B_PER; ++j) rb[j] = (kin && wrow[j]) ? wrow[j][k] : (T)0.f;
  };
  auto advance = [&]() {
    k += BK;
    c += BK;
    while (c >= p.cin) {
      c -= p.cin;
      if (++kw_ == p.kw) {
        kw_ = 0;
        if (++kh_ == p.kh) {
          kh_ = 0;
          ++kd_;
        }
      }
    }
  };
  auto stash = [&](int stage) {
    char* sa = smem + stage * STAGE_BYTES;
    char* sb = sa + BM * ROWB;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) *(T*)(sa + (rsub + 8 * i) * ROWB + kk * EB) = ra[i];
#pragma unroll
    for (int j = 0; j < B_PER; ++j) *(T*)(sb + (rsub + 8 * j) * ROWB + kk * EB) = rb[j];
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 15, fg = lane >> 4;
  const int S = (p.K + BK - 1) / BK;

  gather();
  stash(0);
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    if (s + 1 < S) {
      advance();
      gather();
    }
    const char* sa = smem + (s & 1) * STAGE_BYTES;
    const char* sb = sa + BM * ROWB;
    F af[FM], bfr[FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
      af[a] = *(const F*)(sa + (wm * TM + a * 16 + fr) * ROWB + fg * 8 * EB);
#pragma unroll
    for (int b = 0; b < FN; ++b)
      bfr[b] = *(const F*)(sb + (wn * TN + b * 16 + fr) * ROWB + fg * 8 * EB);
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = step_mfma(bfr[b], af[a], acc[a][b]);
    if (s + 1 < S) stash((s + 1) & 1);
    __syncthreads();
  }

  // Epilogue: lane holds D[n = 4*fg + i][m = fr] of each 16x16 block.
  const bool vec_ok = (p.cout & 3) == 0;
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = m0 + wm * TM + a * 16 + fr;
    if (m >= p.M) continue;
    T* yrow = y + (int64_t)m * p.cout;
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int n = n0 + wn * TN + b * 16 + fg * 4;
      if (vec_ok && n + 3 < p.cout) {
        if constexpr (sizeof(T) == 2) {
          union { T h[4]; uint2 u; } pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][i]);
          *(uint2*)(yrow + n) = pk.u;
        } else {
          *(f32x4_t*)(yrow + n) = acc[a][b];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < p.cout) yrow[n + i] = from_f32<T>(acc[a][b][i]);
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.cout + BN - 1) / BN;
  hipLaunchKernelGGL((conv_flatk_kernel<T, BM, BN, WM, WN>), dim3(tiles_m * tiles_n), dim3(256),
                     0, s, p, (const T*)x, (const T*)w, (T*)y, tiles_n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.cout <= 32) return launch_cfg<T, 128, 32, 4, 1>(p, x, w, y, s);
  return launch_cfg<T, 128, 64, 2, 2>(p, x, w, y, s);
}

}  // namespace

bool flatk_accepts(const ConvParams& p, int dtype) {
  (void)dtype;
  return plain(p) && p.kd <= 16 && p.kh <= 16 && p.kw <= 16;
}

hipError_t launch_flatk(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s) {
  if (dtype == kF32) return launch_typed<float>(p, x, w, y, s);
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
