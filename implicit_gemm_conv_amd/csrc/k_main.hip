// k_main.hip -- the main implicit-GEMM path for fp16/bf16 with C_in % 64 == 0.
//
// GEMM view ("Convolutions" tutorial, section 5, implicit GEMM): row m of the
// virtual im2col matrix is output position m, column k = (tap, c).  A K step
// covers 64 channels of one tap, so every A row segment is 128 contiguous
// bytes of the channels-last input and every B row segment 128 contiguous
// bytes of the filter.
//
// Per workgroup (256 threads = 4 waves of 64):
//  * tile BM x BN of the output; tile ids follow the XCD-aware order;
//  * once per tile, each loader thread decodes its output rows into a window
//    origin plus three per-dimension validity masks (the precomputed pad and
//    stride masks); per K step a row's tap is valid iff one bit of each mask
//    is set, else the lane reads a 16-byte zero block instead of the input;
//  * operands move global -> LDS with 16-byte direct-to-LDS loads
//    (global_load_lds_dwordx4), STAGES buffers deep, so the loads of the next
//    steps are in flight while the current one is multiplied;
//  * LDS rows hold 64 channels (8 chunks of 16 B) with the chunk index XORed
//    by (row & 7), so the 16-byte fragment reads of 8 consecutive rows hit
//    distinct banks;
//  * each wave multiplies a (BM/WM) x (BN/WN) sub-tile with
//    v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators.  The filter fragment
//    is the MFMA's first operand, so a lane ends up holding 4 consecutive
//    output channels of one output row and stores them as one 8-byte write.
// The K loop runs channel chunks in the outer position and taps in the inner
// one, so consecutive steps re-read input rows shifted by one tap, which the
// caches still hold.
#include "conv_device.h"

namespace convfwd {

namespace {

__device__ __attribute__((aligned(64))) uint32_t g_zero_block[16];  // 64 zero bytes

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Waits until at most N of this thread's vector-memory operations are
// outstanding, then joins the workgroup barrier.  One asm block (with a
// memory clobber) so that the compiler neither moves LDS accesses across it
// nor adds a blanket vmcnt(0) for the direct-to-LDS loads still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <typename T, int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(256) void conv_main_kernel(ConvParams p, const T* __restrict__ x,
                                                        const T* __restrict__ w,
                                                        T* __restrict__ y, int tiles_n) {
  typedef typename Vec8<T>::type V8;
  constexpr int BK = 64;                // channels per K step
  constexpr int ROWB = BK * 2;          // LDS bytes per tile row
  constexpr int A_LOADS = BM / 32;      // 16-byte loads per thread per step
  constexpr int B_LOADS = BN / 32;
  constexpr int NL = A_LOADS + B_LOADS;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(NL * (STAGES - 2) < 64, "vmcnt");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  // Loader geometry: a wave's load instruction fills 8 consecutive tile rows
  // (1 KB of LDS); lane l writes row l/8, physical chunk l%8, which holds the
  // logical chunk (l%8) ^ (row & 7) = (l%8) ^ (l/8).
  const int lrow = wave * 8 + (lane >> 3);
  const int lchunk = (lane & 7) ^ (lane >> 3);

  RowInfo ri[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) ri[i] = decode_row(p, m0 + i * 32 + lrow);
  const T* bsrc[B_LOADS];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int n = n0 + j * 32 + lrow;
    bsrc[j] = n < p.cout ? w + (int64_t)n * p.K + lchunk * 8 : nullptr;
  }
  const char* zero = (const char*)g_zero_block;

  const int S = (p.cin / BK) * p.ntaps;
  int ic = 0, ikd = 0, ikh = 0, ikw = 0;  // (channel chunk, tap) of the next step to issue

  auto issue = [&](int stage) {
    char* sa = smem + stage * STAGE_BYTES;
    char* sb = sa + BM * ROWB;
    const int xoff = ikd * p.xs_d + ikh * p.xs_h + ikw * p.xs_w + ic * BK + lchunk * 8;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const void* src =
          tap_valid(ri[i], ikd, ikh, ikw) ? (const void*)(x + ri[i].base + xoff) : (const void*)zero;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(sa + (i * 32 + wave * 8) * ROWB), 16, 0, 0);
    }
    const int woff = ((ikd * p.kh + ikh) * p.kw + ikw) * p.cin + ic * BK;
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      const void* src = bsrc[j] ? (const void*)(bsrc[j] + woff) : (const void*)zero;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(sb + (j * 32 + wave * 8) * ROWB), 16, 0, 0);
    }
    if (++ikw == p.kw) {
      ikw = 0;
      if (++ikh == p.kh) {
        ikh = 0;
        if (++ikd == p.kd) {
          ikd = 0;
          ++ic;
        }
      }
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 15, fg = lane >> 4;

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < S) issue(s);

  for (int s = 0; s < S; ++s) {
    // Loads of step s must have landed; later steps may still be in flight.
    const int newer = min(STAGES - 2, S - 1 - s);
    if (STAGES >= 4 && newer >= 2) wait_vmcnt_barrier<NL * 2 * (STAGES >= 4)>();
    else if (STAGES >= 3 && newer >= 1) wait_vmcnt_barrier<NL * (STAGES >= 3)>();
    else wait_vmcnt_barrier<0>();
    if (s + STAGES - 1 < S) issue((s + STAGES - 1) % STAGES);

    const char* sa = smem + (s % STAGES) * STAGE_BYTES;
    const char* sb = sa + BM * ROWB;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ((ks * 4 + fg) ^ (fr & 7)) * 16;
      V8 af[FM], bfr[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a)
        af[a] = *(const V8*)(sa + (wm * TM + a * 16 + fr) * ROWB + chunk);
#pragma unroll
      for (int b = 0; b < FN; ++b)
        bfr[b] = *(const V8*)(sb + (wn * TN + b * 16 + fr) * ROWB + chunk);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = mfma16x16x32(bfr[b], af[a], acc[a][b]);
    }
  }

  // Epilogue: lane holds D[n = 4*fg + i][m = fr] of each 16x16 block.
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = m0 + wm * TM + a * 16 + fr;
    if (m >= p.M) continue;
    T* yrow = y + (int64_t)m * p.cout;
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int n = n0 + wn * TN + b * 16 + fg * 4;
      if (n + 3 < p.cout) {
        union { T h[4]; uint2 u; } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][i]);
        *(uint2*)(yrow + n) = pk.u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < p.cout) yrow[n + i] = from_f32<T>(acc[a][b][i]);
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_cfg(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.cout + BN - 1) / BN;
  hipLaunchKernelGGL((conv_main_kernel<T, BM, BN, WM, WN, STAGES>), dim3(tiles_m * tiles_n),
                     dim3(256), 0, s, p, (const T*)x, (const T*)w, (T*)y, tiles_n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  // Enough 256-row tiles to fill 256 CUs: big tiles; otherwise smaller ones.
  const long tiles_256 = (long)((p.M + 255) / 256) * ((p.cout + 127) / 128);
  if (tiles_256 >= 256) return launch_cfg<T, 256, 128, 4, 1, 3>(p, x, w, y, s);
  return launch_cfg<T, 128, 64, 2, 2, 3>(p, x, w, y, s);
}

}  // namespace

bool main_accepts(const ConvParams& p, int dtype) {
  return (dtype == kF16 || dtype == kBF16) && p.cin % 64 == 0 && p.cout % 4 == 0 && p.kd <= 16 &&
         p.kh <= 16 && p.kw <= 16;
}

hipError_t launch_main(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
