// k_main.hip -- the main implicit-GEMM path for fp16/bf16 with C_in % BK == 0.
//
// GEMM view ("Convolutions" tutorial, section 5, implicit GEMM): row m of the
// virtual im2col matrix is output position m, column k = (tap, c).  A K step
// covers BK (32 or 64) channels of one tap, so every A row segment is BK*2
// contiguous bytes of the channels-last input and every B row segment BK*2
// contiguous bytes of the filter.
//
// Per workgroup (256 threads = 4 waves of 64):
//  * tile BM x BN of the output; tile ids follow the XCD-aware order;
//  * once per tile, each loader thread decodes its output rows into a window
//    origin plus three per-dimension validity masks (the precomputed pad and
//    stride masks); per K step a row's tap is valid iff one bit of each mask
//    is set;
//  * operands move global -> LDS with 16-byte buffer loads that write LDS
//    directly (buffer_load_dwordx4 ... lds), STAGES buffers deep, so the
//    loads of the next steps are in flight while the current one is
//    multiplied.  A lane whose tap falls in the padding gets an offset past
//    the end of the buffer, and the hardware's range check returns zeros;
//  * LDS rows hold BK channels in 16-byte chunks whose index is XORed with a
//    function of the row (chosen per row width and fragment size), so that
//    the 16-byte fragment reads run at the full LDS rate;
//  * each wave multiplies a (BM/WM) x (BN/WN) sub-tile in MF x MF blocks,
//    v_mfma_f32_32x32x16 (MF = 32) or v_mfma_f32_16x16x32 (MF = 16), fp32
//    accumulators.  On gfx950 one wave can keep the matrix unit busy with
//    independent 32x32x16 MFMAs, while 16x16x32 needs two waves per SIMD.
//    The filter fragment is the MFMA's first operand, so a lane ends up
//    holding runs of 4 consecutive output channels of one output row and
//    stores each run as one 8-byte write.
// The K loop runs channel chunks in the outer position and taps in the inner
// one, so consecutive steps re-read input rows shifted by one tap, which the
// caches still hold.
#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Offset that fails the buffer range check (every tensor is < 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Buffer resource word 3 for raw (untyped, unswizzled) buffers on gfx9 parts.
constexpr int kRawBufferFlags = 0x00020000;

// Waits until at most N of this thread's vector-memory operations are
// outstanding, then joins the workgroup barrier.  One asm block (with a
// memory clobber) so that the compiler neither moves LDS accesses across it
// nor adds a blanket vmcnt(0) for the direct-to-LDS loads still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Physical 16-byte chunk of logical chunk `lc` in LDS row `r` (rows of CPR
// chunks) for fragments of MF rows.  In a fragment read, lanes 0..MF-1 take
// one chunk of MF consecutive rows and the next lane groups other chunks of
// the same rows; timed with a read-only probe, these XOR patterns serve that
// read at the full LDS rate (~190-210 B/clk per CU) where the others measured
// reach 60-125: for 64-byte rows bits 1..2 of r with 16-row fragments, bits
// 2..3 with 32-row ones; for 128-byte rows bits 1..3 with either.
template <int CPR, int MF>
__device__ __forceinline__ int swz(int r, int lc) {
  if constexpr (CPR == 8) return lc ^ ((r >> 1) & 7);
  else if constexpr (MF == 32) return lc ^ ((r >> 2) & 3);
  else return lc ^ ((r >> 1) & 3);
}

template <int MF> struct Acc;
template <> struct Acc<16> { typedef f32x4_t type; };
template <> struct Acc<32> { typedef f32x16_t type; };

template <typename V8, typename A>
__device__ __forceinline__ A mfma_block(V8 a, V8 b, A c) {
  if constexpr (sizeof(A) == 16) return mfma16x16x32(a, b, c);
  else return mfma32x32x16(a, b, c);
}

// One BM x BN output tile `tile` of problem p (the kernels below pick the tile
// and the problem).
template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int MF>
__device__ __forceinline__ void main_tile(const ConvParams& p, const T* __restrict__ x,
                                          const T* __restrict__ w, T* __restrict__ y, int tile,
                                          int tiles_n, uint32_t x_bytes, uint32_t w_bytes) {
  // The body uses buffer-resource builtins that exist only for the GPU; the
  // host pass needs nothing but the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  typedef typename Acc<MF>::type AccT;
  constexpr int ROWB = BK * 2;          // LDS bytes per tile row
  constexpr int CPR = BK / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows one wave instruction fills
  constexpr int RPR = 4 * RPI;          // rows the workgroup fills per load round
  constexpr int A_LOADS = BM / RPR;     // 16-byte loads per thread per step
  constexpr int B_LOADS = BN / RPR;
  constexpr int NL = A_LOADS + B_LOADS;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / MF, FN = TN / MF;
  constexpr int KSUB = MF == 32 ? 16 : 32;   // k per MFMA
  constexpr int LG = 64 / MF;                 // lane groups along k (2 or 4)
  constexpr int NQ = MF == 32 ? 4 : 1;        // runs of 4 channels per lane per block
  constexpr int NACC = MF == 32 ? 16 : 4;
  constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(BM % RPR == 0 && BN % RPR == 0, "loader rounds");
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM % MF == 0 && TN % MF == 0, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert(NL * (STAGES - 2) < 64, "vmcnt");

  constexpr int OUT_ROWB = BN * 2;      // one output row of the tile in LDS
  constexpr int OCH = BN / 8;           // its 16-byte pieces
  constexpr int SMEM = STAGES * STAGE_BYTES > BM * OUT_ROWB ? STAGES * STAGE_BYTES : BM * OUT_ROWB;
  static_assert(OCH == 8 || OCH == 16, "output row pieces");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = (tile / tiles_n) * BM;
  // Column tiles never straddle a channel group: tile tn covers output
  // channels n0 .. of group g = tn / tpg, which reads input channels
  // g*cin_g .. (g+1)*cin_g - 1; columns stop at the group's end n_end.
  const int tpg = (p.cout_g + BN - 1) / BN;   // column tiles per group
  const int tn = tile % tiles_n;
  const int grp = tn / tpg;
  const int n0 = grp * p.cout_g + (tn - grp * tpg) * BN;
  const int n_end = (grp + 1) * p.cout_g;
  const int c_grp = grp * p.cin_g;

  // Loader geometry: a wave's load instruction fills RPI consecutive tile
  // rows (1 KB of LDS); lane l writes row l / CPR of them, physical chunk
  // l % CPR, so it fetches the logical chunk that the swizzle puts there (its
  // own inverse, being an XOR).  Load rounds are RPR >= 32 rows apart, so the
  // row bits the swizzle reads are those of lrow in every round.
  const int lrow = wave * RPI + lane / CPR;
  const int lchunk = swz<CPR, MF>(lrow, lane % CPR);

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)w_bytes, kRawBufferFlags);

  RowInfo ri[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    ri[i] = decode_row(p, m0 + i * RPR + lrow);
    ri[i].base = (ri[i].base + c_grp + lchunk * 8) * 2;   // byte offset of this lane's chunk at tap 0
  }
  uint32_t boff[B_LOADS];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int n = n0 + j * RPR + lrow;
    boff[j] = n < n_end ? (uint32_t)((n * p.K + lchunk * 8) * 2) : kOutOfRange;
  }

  const int S = (p.cin_g / BK) * p.ntaps;
  int ic = 0, ikd = 0, ikh = 0, ikw = 0;  // (channel chunk, tap) of the next step to issue

  auto issue = [&](int stage) {
    char* sa = smem + stage * STAGE_BYTES;
    char* sb = sa + BM * ROWB;
    const int xoff = (ikd * p.ed * p.xs_d + ikh * p.eh * p.xs_h + ikw * p.ew * p.xs_w + ic * BK) * 2;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const uint32_t off =
          tap_valid(ri[i], ikd, ikh, ikw) ? (uint32_t)(ri[i].base + xoff) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(sa + (i * RPR + wave * RPI) * ROWB), 16, off, 0, 0, 0);
    }
    const uint32_t woff = (uint32_t)((((ikd * p.kh + ikh) * p.kw + ikw) * p.cin_g + ic * BK) * 2);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_ptr_t)(sb + (j * RPR + wave * RPI) * ROWB), 16, boff[j] + woff, 0, 0, 0);
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

  AccT acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < NACC; ++e) acc[a][b][e] = 0.f;

  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane % MF, fg = lane / MF;   // fragment row, k group

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
    for (int ks = 0; ks < BK / KSUB; ++ks) {
      const int chunk = swz<CPR, MF>(fr, ks * LG + fg) * 16;
      V8 af[FM], bfr[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a)
        af[a] = *(const V8*)(sa + (wm * TM + a * MF + fr) * ROWB + chunk);
#pragma unroll
      for (int b = 0; b < FN; ++b)
        bfr[b] = *(const V8*)(sb + (wn * TN + b * MF + fr) * ROWB + chunk);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = mfma_block(bfr[b], af[a], acc[a][b]);
    }
  }

  // Epilogue.  For output row m = its fragment row, a lane holds runs of 4
  // consecutive output channels: channel 16*b' + 4*fg + i (MF = 16) or
  // 32*b' + 8*q + 4*fg + i (MF = 32, q = 0..3) in accumulator element 4*q + i.
  // The tile goes through LDS (row-major, 16-byte piece k of row r at slot
  // k ^ (r % OCH)) so that each store writes whole 16-byte pieces of rows.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int row = wm * TM + a * MF + fr;
#pragma unroll
    for (int b = 0; b < FN; ++b) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int ch = wn * TN + b * MF + 8 * q + 4 * fg;
        union { T h[4]; uint2 u; } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][4 * q + i]);
        *(uint2*)(smem + row * OUT_ROWB + (((ch >> 3) ^ (row % OCH)) * 16) + ((ch >> 2) & 1) * 8) = pk.u;
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int ORPI = 64 / OCH;        // output rows per wave instruction
  const bool whole16 = (p.cout & 7) == 0 && (p.cout_g & 7) == 0;   // 16-byte stores stay aligned
#pragma unroll 4
  for (int i = 0; i < BM / (4 * ORPI); ++i) {
    const int row = (4 * i + wave) * ORPI + lane / OCH, k = lane % OCH;
    const uint4 v = *(const uint4*)(smem + row * OUT_ROWB + ((k ^ (row % OCH)) * 16));
    const int m = m0 + row;
    const int n = n0 + k * 8;
    if (m < p.M) {
      T* dst = y + out_row(p, m) + n;
      if (n + 8 <= n_end) {
        if (whole16) {
          store16_nt(dst, v);
        } else {
          *(uint2*)dst = make_uint2(v.x, v.y);
          *(uint2*)(dst + 4) = make_uint2(v.z, v.w);
        }
      } else if (n + 4 <= n_end) {
        *(uint2*)dst = make_uint2(v.x, v.y);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int MF>
__global__ __launch_bounds__(256, OCC) void conv_main_kernel(ConvParams p, const T* __restrict__ x,
                                                             const T* __restrict__ w,
                                                             T* __restrict__ y, int tiles_n,
                                                             uint32_t x_bytes, uint32_t w_bytes) {
  main_tile<T, BM, BN, BK, WM, WN, STAGES, MF>(p, x, w, y, xcd_tile(blockIdx.x, gridDim.x), tiles_n,
                                               x_bytes, w_bytes);
}

// Several problems that share x and y (the stride phases of backward-data,
// each writing its own rows of y) in one launch: workgroups [begin[i],
// begin[i+1]) take the tiles of problem i, whose filter starts w_off[i] bytes
// into w.  One launch lets the phases' start-up and tail overlap.
constexpr int kMaxPhases = 8;
struct MainPhases {
  int count;
  int begin[kMaxPhases + 1];
  int tiles_n[kMaxPhases];
  uint32_t w_off[kMaxPhases], w_bytes[kMaxPhases];
  ConvParams p[kMaxPhases];
};

template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int MF>
__global__ __launch_bounds__(256, OCC) void conv_main_phased_kernel(MainPhases ph, const T* __restrict__ x,
                                                                    const T* __restrict__ w,
                                                                    T* __restrict__ y, uint32_t x_bytes) {
  // Tiles in launch order, not in per-XCD runs: the phases come heaviest
  // first (most taps), and workgroups are dealt round-robin to the 8 XCDs, so
  // every XCD takes an equal share of every phase, heaviest first.  Runs of
  // tile ids per XCD would hand the whole heaviest phase to one XCD (stride-2
  // 3x3x3 backward-data: phases of 8, 4, 2 and 1 taps; 36.4 us against 25.7).
  const int b = blockIdx.x;
  int i = 0;
  while (i + 1 < ph.count && b >= ph.begin[i + 1]) ++i;
  main_tile<T, BM, BN, BK, WM, WN, STAGES, MF>(ph.p[i], x, (const T*)((const char*)w + ph.w_off[i]), y,
                                               b - ph.begin[i], ph.tiles_n[i], x_bytes, ph.w_bytes[i]);
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int MF>
hipError_t launch_cfg(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = p.groups * ((p.cout_g + BN - 1) / BN);
  const uint32_t xb = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  const uint32_t wb = (uint32_t)((int64_t)p.cout * p.K * 2);
  hipLaunchKernelGGL((conv_main_kernel<T, BM, BN, BK, WM, WN, STAGES, OCC, MF>),
                     dim3(tiles_m * tiles_n), dim3(256), 0, s, p, (const T*)x, (const T*)w,
                     (T*)y, tiles_n, xb, wb);
  return hipGetLastError();
}

// Tile configurations.  CONVFWD_MAIN_VARIANT (a build-time define) forces one
// of them for every problem, for tile-size sweeps; by default the choice below
// depends on the problem size and channel alignment.
constexpr int variant_bk(int v) {
  return (v == 1 || v == 4 || v == 7 || v == 9 || v == 10 || v == 12 || v == 13 || v == 14 || v == 41 || v == 43 ||
          v == 45 || v == 47)
             ? 64
             : 32;
}

template <typename T>
hipError_t launch_variant(int v, const ConvParams& p, const void* x, const void* w, void* y,
                          hipStream_t s) {
  switch (v) {
    // 16x16x32 MFMA blocks
    case 1: return launch_cfg<T, 256, 128, 64, 4, 1, 3, 1, 16>(p, x, w, y, s);
    case 3: return launch_cfg<T, 256, 128, 32, 4, 1, 2, 2, 16>(p, x, w, y, s);
    case 4: return launch_cfg<T, 128, 128, 64, 2, 2, 2, 2, 16>(p, x, w, y, s);
    case 7: return launch_cfg<T, 64, 128, 64, 1, 4, 3, 2, 16>(p, x, w, y, s);
    case 8: return launch_cfg<T, 128, 64, 32, 2, 2, 3, 2, 16>(p, x, w, y, s);
    case 9: return launch_cfg<T, 64, 64, 64, 2, 2, 4, 2, 16>(p, x, w, y, s);
    case 10: return launch_cfg<T, 64, 128, 64, 1, 4, 4, 1, 16>(p, x, w, y, s);
    case 11: return launch_cfg<T, 64, 64, 32, 2, 2, 4, 3, 16>(p, x, w, y, s);
    case 12: return launch_cfg<T, 32, 128, 64, 1, 4, 4, 2, 16>(p, x, w, y, s);
    case 13: return launch_cfg<T, 64, 64, 64, 2, 2, 3, 3, 16>(p, x, w, y, s);
    case 14: return launch_cfg<T, 128, 64, 64, 2, 2, 3, 2, 16>(p, x, w, y, s);
    // 32x32x16 MFMA blocks
    case 41: return launch_cfg<T, 256, 128, 64, 4, 1, 2, 1, 32>(p, x, w, y, s);
    case 42: return launch_cfg<T, 256, 128, 32, 4, 1, 2, 2, 32>(p, x, w, y, s);
    case 43: return launch_cfg<T, 128, 128, 64, 2, 2, 2, 2, 32>(p, x, w, y, s);
    case 44: return launch_cfg<T, 256, 128, 32, 4, 1, 3, 2, 32>(p, x, w, y, s);
    case 45: return launch_cfg<T, 256, 128, 64, 4, 1, 3, 1, 32>(p, x, w, y, s);
    case 46: return launch_cfg<T, 256, 128, 32, 2, 2, 2, 2, 32>(p, x, w, y, s);
    case 47: return launch_cfg<T, 128, 128, 64, 2, 2, 3, 1, 32>(p, x, w, y, s);
    case 48: return launch_cfg<T, 128, 128, 32, 2, 2, 3, 2, 32>(p, x, w, y, s);
    case 49: return launch_cfg<T, 128, 64, 32, 2, 2, 3, 2, 32>(p, x, w, y, s);
    case 50: return launch_cfg<T, 128, 128, 32, 2, 2, 2, 3, 32>(p, x, w, y, s);
    default: return launch_cfg<T, 128, 64, 32, 2, 2, 3, 2, 16>(p, x, w, y, s);
  }
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
#ifdef CONVFWD_MAIN_VARIANT
  if (p.cin_g % variant_bk(CONVFWD_MAIN_VARIANT) == 0)
    return launch_variant<T>(CONVFWD_MAIN_VARIANT, p, x, w, y, s);
#endif
  const bool bk64 = p.cin_g % 64 == 0;
  const long tiles_256 = (long)((p.M + 255) / 256) * p.groups * ((p.cout_g + 127) / 128);
  const long tiles_128 = (long)((p.M + 127) / 128) * p.groups * ((p.cout_g + 127) / 128);
  // A short GEMM depth (a few K steps per tile: 3x1x1 or 1x1 filters) leaves
  // each tile's first loads and last stores exposed; 128x128 tiles with BK = 32
  // and 32x32x16 MFMAs fit three workgroups per CU, which overlap more of them
  // (3x1x1 (4,32^3,64->128): 17 us against 21 us on the 128x128, BK = 64 tile).
  if (p.K <= 192 && p.cout_g > 64 && tiles_128 >= 512) return launch_variant<T>(50, p, x, w, y, s);
  // groups of at most 64 output channels: a 64-wide column tile (a 128-wide one
  // would leave half its columns idle)
  if (p.cout_g <= 64 && bk64 && tiles_256 >= 256) return launch_variant<T>(14, p, x, w, y, s);
  if (tiles_256 >= 256) return launch_variant<T>(bk64 ? 4 : 3, p, x, w, y, s);
  return launch_variant<T>(bk64 ? 9 : 8, p, x, w, y, s);
}

}  // namespace

bool main_accepts(const ConvParams& p, int dtype) {
  return (dtype == kF16 || dtype == kBF16) && p.cin_g % 32 == 0 && p.cout_g % 4 == 0 && p.kd <= 16 &&
         p.kh <= 16 && p.kw <= 16;
}

hipError_t launch_main(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

const int* main_tile_configs(int* count) {
  static const int kConfigs[] = {9, 14, 4, 3, 8, 13, 11, 10, 7, 12, 1, 43, 47, 49, 50};
  *count = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
  return kConfigs;
}

bool main_config_accepts(const ConvParams& p, int dtype, int config) {
  return main_accepts(p, dtype) && (config == 0 || p.cin_g % variant_bk(config) == 0);
}

hipError_t launch_main_config(const ConvParams& p, int dtype, int config, const void* x, const void* w,
                              void* y, hipStream_t s) {
  if (config == 0) return launch_main(p, dtype, x, w, y, s);
  if (dtype == kF16) return launch_variant<_Float16>(config, p, x, w, y, s);
  return launch_variant<__bf16>(config, p, x, w, y, s);
}

namespace {

template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int MF>
hipError_t launch_phased_cfg(const ConvParams* ps, const uint32_t* w_off, int count, const void* x,
                             const void* w, void* y, hipStream_t s) {
  const uint32_t xb = (uint32_t)((int64_t)ps[0].n * ps[0].xs_n * 2);
  for (int base = 0; base < count; base += kMaxPhases) {
    MainPhases ph;
    ph.count = count - base < kMaxPhases ? count - base : kMaxPhases;
    int total = 0;
    for (int i = 0; i < ph.count; ++i) {
      const ConvParams& p = ps[base + i];
      const int tiles_n = p.groups * ((p.cout_g + BN - 1) / BN);
      ph.begin[i] = total;
      total += ((p.M + BM - 1) / BM) * tiles_n;
      ph.tiles_n[i] = tiles_n;
      ph.w_off[i] = w_off[base + i];
      ph.w_bytes[i] = (uint32_t)((int64_t)p.cout * p.K * 2);
      ph.p[i] = p;
    }
    ph.begin[ph.count] = total;
    hipLaunchKernelGGL((conv_main_phased_kernel<T, BM, BN, BK, WM, WN, STAGES, OCC, MF>), dim3(total),
                       dim3(256), 0, s, ph, (const T*)x, (const T*)w, (T*)y, xb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The tile choice of launch_typed, made for the phases' rows together.
template <typename T>
hipError_t launch_phased_typed(const ConvParams* ps, const uint32_t* w_off, int count, const void* x,
                               const void* w, void* y, hipStream_t s) {
  const ConvParams& p = ps[0];
  const bool bk64 = p.cin_g % 64 == 0;
  long rows = 0;
  for (int i = 0; i < count; ++i) rows += ps[i].M;
  const long tiles_256 = ((rows + 255) / 256) * p.groups * ((p.cout_g + 127) / 128);
  if (p.cout_g <= 64 && bk64 && tiles_256 >= 256)
    return launch_phased_cfg<T, 128, 64, 64, 2, 2, 3, 2, 16>(ps, w_off, count, x, w, y, s);
  if (tiles_256 >= 256) {
    if (bk64) return launch_phased_cfg<T, 128, 128, 64, 2, 2, 2, 2, 16>(ps, w_off, count, x, w, y, s);
    return launch_phased_cfg<T, 256, 128, 32, 4, 1, 2, 2, 16>(ps, w_off, count, x, w, y, s);
  }
  if (bk64) return launch_phased_cfg<T, 64, 64, 64, 2, 2, 4, 2, 16>(ps, w_off, count, x, w, y, s);
  return launch_phased_cfg<T, 128, 64, 32, 2, 2, 3, 2, 16>(ps, w_off, count, x, w, y, s);
}

}  // namespace

hipError_t launch_main_phased(const ConvParams* ps, const uint32_t* w_off, int count, int dtype,
                              const void* x, const void* w, void* y, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (dtype == kF16) return launch_phased_typed<_Float16>(ps, w_off, count, x, w, y, s);
  return launch_phased_typed<__bf16>(ps, w_off, count, x, w, y, s);
}

}  // namespace convfwd
