// k_runs.hip -- implicit GEMM for any C_in (the unaligned-channel tail path)
// and fp32, reading the im2col matrix as contiguous runs; also the grouped and
// dilated variants.
//
// With K ordered (kd, kh, kw, c), the K_w * C_in columns of one (kd, kh) form
// a run that is contiguous in memory on both sides of the product: in x the
// K_w window positions of an output are adjacent along w with all their
// channels ("Convolutions" tutorial, section 5: the im2col row of an output
// is its window, flattened), and in the filter (C_out, K_d, K_h, K_w, C_in)
// the same run is one slice of a filter row.  The GEMM depth is walked run by
// run, each run cut into steps of 32 columns (the last one zero-padded), so a
// step of an output row is 32 consecutive input elements.  Rows of odd
// channel counts are only 2-byte aligned: a step is fetched as 16-byte pieces
// with unaligned buffer loads, and the columns of window positions that fall
// in the padding (or past the run) are zeroed with branch-free masks.  A
// piece that would start before x or reach past the end of a tensor (only on
// its first and last lines; the buffer range check would drop its dwords
// whole, and a 2-byte element can share a dword with bytes past the end) is
// loaded from the nearest 16 bytes inside the tensor and moved into place
// with byte-align instructions when it is consumed.  (Fetching those pieces
// element by element made the waves holding them wait for every load in
// flight at each such step: 3-4.5 us on the C_in = 21 and fp32 layers.)
// Grouped or w-dilated problems use shorter runs: the C_in/G channels of one
// tap, a group's slice of one window position.
//
// Pipeline: the pieces of DEPTH steps are in flight in registers at once; each
// step's pieces are masked and written to a double-buffered LDS tile (rows
// padded by 16 bytes so that fragment reads of 16 rows hit distinct banks),
// then read as MFMA fragments: v_mfma_f32_16x16x32_{f16,bf16}, or for fp32
// eight v_mfma_f32_16x16x4_f32 per step.  Four waves split the tile along M.
#include "conv_device.h"

namespace convfwd {

namespace {

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kBK = 32;     // GEMM columns per step

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <typename T> struct RunFrag;
template <> struct RunFrag<_Float16> { typedef half8_t type; };
template <> struct RunFrag<__bf16> { typedef bf168_t type; };
template <> struct RunFrag<float> { struct type { f32x4_t lo, hi; }; };

__device__ __forceinline__ f32x4_t run_mfma(half8_t a, half8_t b, f32x4_t c) { return mfma16x16x32(a, b, c); }
__device__ __forceinline__ f32x4_t run_mfma(bf168_t a, bf168_t b, f32x4_t c) { return mfma16x16x32(a, b, c); }
// Lane group g supplies column 8g + e to the e-th 16x16x4 product; over e < 8
// and g < 4 that covers the 32 columns of the step once each.
template <typename F>
__device__ __forceinline__ f32x4_t run_mfma(const F& a, const F& b, f32x4_t c) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
  return c;
}

// Keep the elements j of a 16-byte piece with jl <= j < jh, zero the others.
template <int EB>
__device__ __forceinline__ u4 keep_range(u4 v, int jl, int jh) {
  u4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (EB == 4) {
      r[d] = (d >= jl && d < jh) ? v[d] : 0u;
    } else {
      const uint32_t lo = (2 * d >= jl && 2 * d < jh) ? 0x0000ffffu : 0u;
      const uint32_t hi = (2 * d + 1 >= jl && 2 * d + 1 < jh) ? 0xffff0000u : 0u;
      r[d] = v[d] & (lo | hi);
    }
  }
  return r;
}

// The 16 bytes at element offset e of a tensor of `bytes` >= 16 bytes.  A
// piece that starts before the tensor or runs past its end (only on its first
// and last lines) is loaded from the nearest 16 bytes inside it instead, and
// *shift = (piece start - load start) in bytes, -15 .. 15, tells the consumer
// to move it into place (shift_piece) once it has arrived; 0 for a piece
// wholly inside.  One load per piece either way and no wait at issue: the
// consumer's wait is the pipeline's own.
template <int EB>
__device__ __forceinline__ u4 load_piece(__amdgpu_buffer_rsrc_t rsrc, int e, bool ok, int bytes, int* shift) {
  const int bo = e * EB;
  const int c = min(max(bo, 0), bytes - 16);
  *shift = ok ? bo - c : 0;
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? (uint32_t)c : kOutOfRange, 0, 0);
}

// Byte j of the result is byte j + s of v (-16 < s < 16), zero where that lies
// outside v: v placed in a zero-padded 48-byte window, four dwords taken at
// byte 16 + s with v_alignbyte.
__device__ __forceinline__ u4 shift_piece(u4 v, int s) {
  const int t = 16 + s;
  const int dw = t >> 2, b = t & 3;
  auto z = [&](int k) -> uint32_t { return k == 4 ? v[0] : k == 5 ? v[1] : k == 6 ? v[2] : k == 7 ? v[3] : 0u; };
  u4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(z(dw + i + 1), z(dw + i), (uint32_t)b);
  return r;
}

template <typename T, int BM, int BN, int DEPTH>
__global__ __launch_bounds__(256, 2) void conv_runs_kernel(ConvParams p, const T* __restrict__ x,
                                                           const T* __restrict__ w, T* __restrict__ y,
                                                           int tiles_n, int x_bytes, int w_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename RunFrag<T>::type F;
  constexpr int EB = sizeof(T);
  constexpr int EPC = 16 / EB;                 // elements per 16-byte piece
  constexpr int CPR = kBK / EPC;               // pieces per row per step
  constexpr int ROWB = kBK * EB + 16;          // padded LDS row
  constexpr int A_PER = BM * CPR / 256;        // A pieces per thread per step
  constexpr int B_PIECES = BN * CPR;
  constexpr int B_PER = (B_PIECES + 255) / 256;
  constexpr int TM = BM / 4;                   // rows per wave
  constexpr int FM = TM / 16, FN = BN / 16;
  constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(BM * CPR % 256 == 0 && TM % 16 == 0 && BN % 16 == 0, "tile");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM;
  // column tiles never straddle a channel group (see launch_cfg)
  const int tpg = (p.cout_g + BN - 1) / BN;
  const int tn = tile % tiles_n;
  const int grp = tn / tpg;
  const int n0 = grp * p.cout_g + (tn - grp * tpg) * BN;
  const int n_end = (grp + 1) * p.cout_g;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, w_bytes, kRawBufferFlags);

  // A run is the K_w * C_in columns of one (kd, kh) when the whole window row
  // is contiguous (one group, undilated along w); otherwise the C_in/G
  // columns of one tap (kd, kh, kw).
  const bool wide = p.groups == 1 && p.ew == 1;
  const int run = wide ? p.kw * p.cin : p.cin_g;
  const int nkw = wide ? 1 : p.kw;             // runs per (kd, kh)
  const int sps = (run + kBK - 1) / kBK;       // steps per run
  const int S = p.kd * p.kh * nkw * sps;

  // A pieces: thread piece i -> tile row, piece q; the run of that output row
  // at (kd, kh) = (0, 0) starts at element a_e[i] - q * EPC, and its columns
  // [a_lo, a_hi) (relative to this piece's first column at step column 0) lie
  // inside the input along w.
  int a_e[A_PER], a_lo[A_PER], a_hi[A_PER];
  uint32_t a_dh[A_PER];   // depth-tap bits | height-tap bits << 16
  uint32_t a_w[A_PER];    // width-tap bits (per-tap runs) or all ones (whole window rows)
  int a_ldsoff[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int c = tid + 256 * i, row = c / CPR, q = c % CPR;
    const RowInfo ri = decode_row(p, m0 + row);
    const int lo_w = ri.mw ? __builtin_ctz(ri.mw) : 0;
    const int hi_w = ri.mw ? 32 - __builtin_clz(ri.mw) : 0;
    a_e[i] = ri.base + grp * p.cin_g + q * EPC;
    a_lo[i] = (wide ? lo_w * p.cin : 0) - q * EPC;
    a_hi[i] = (wide ? hi_w * p.cin : p.cin_g) - q * EPC;
    a_dh[i] = ri.md | (ri.mh << 16);
    a_w[i] = wide ? 0xffffffffu : ri.mw;
    a_ldsoff[i] = row * ROWB + q * 16;
  }
  // B pieces: filter row n0 + brow, piece bq; columns past the run are zero.
  int b_e[B_PER], b_hi[B_PER], b_ldsoff[B_PER];
  bool b_ok[B_PER];
#pragma unroll
  for (int j = 0; j < B_PER; ++j) {
    const int c = tid + 256 * j, brow = c / CPR, bq = c % CPR;
    const int co = n0 + brow;
    b_ok[j] = c < B_PIECES && co < n_end;
    b_e[j] = co * p.K + bq * EPC;
    b_hi[j] = run - bq * EPC;
    b_ldsoff[j] = BM * ROWB + brow * ROWB + bq * 16;
  }

  // Loads of the step (kd, kh, k0) into register slot `slot`; steps past the
  // end load nothing.
  u4 ra[DEPTH][A_PER], rb[DEPTH][B_PER];
  // shift_piece amounts of a slot's pieces (0 almost always), 5-bit two's
  // complement fields: A piece i at bit 5 i, B piece j at bit 5 (A_PER + j)
  static_assert(A_PER + B_PER <= 6, "shift fields");
  uint32_t sh_packed[DEPTH];
  int l_kd = 0, l_kh = 0, l_kw = 0, l_k0 = 0, l_step = 0;
  int s_k0[DEPTH];   // column offset of the step in each slot (for the masks)
  auto load_step = [&](int slot) {
    const bool live = l_step < S;
    const int xo = l_kd * p.ed * p.xs_d + l_kh * p.eh * p.xs_h + l_kw * p.ew * p.xs_w + l_k0;
    const int wo = ((l_kd * p.kh + l_kh) * nkw + l_kw) * run + l_k0;
    uint32_t packed = 0u;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      // a piece wholly outside the row's valid columns is not loaded (reads as zero)
      const bool ok = live && ((a_dh[i] >> l_kd) & (a_dh[i] >> (16 + l_kh)) & (a_w[i] >> l_kw) & 1u) &&
                      a_lo[i] - l_k0 < EPC && a_hi[i] - l_k0 > 0;
      int sh;
      ra[slot][i] = load_piece<EB>(xr, a_e[i] + xo, ok, x_bytes, &sh);
      packed |= ((uint32_t)sh & 31u) << (5 * i);
    }
#pragma unroll
    for (int j = 0; j < B_PER; ++j) {
      int sh;
      rb[slot][j] = load_piece<EB>(wr, b_e[j] + wo, live && b_ok[j] && b_hi[j] - l_k0 > 0, w_bytes, &sh);
      packed |= ((uint32_t)sh & 31u) << (5 * (A_PER + j));
    }
    sh_packed[slot] = packed;
    s_k0[slot] = l_k0;
    l_k0 += kBK;
    if (l_k0 >= run) {
      l_k0 = 0;
      if (++l_kw == nkw) {
        l_kw = 0;
        if (++l_kh == p.kh) {
          l_kh = 0;
          ++l_kd;
        }
      }
    }
    ++l_step;
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fg = lane >> 4;

#pragma unroll
  for (int t = 0; t < DEPTH; ++t) load_step(t);

  // One step on register slot `slot`: mask its pieces into LDS stage
  // (step & 1), then the MFMAs; the slot is refilled with the step DEPTH on.
  auto run_step = [&](int step, int slot) {
    char* st = smem + (step & 1) * STAGE;
    const int k0 = s_k0[slot];
    // pieces loaded from a clamped offset at a tensor's first or last line:
    // moved into place now that they have arrived (a wave-uniform branch)
    if (__builtin_amdgcn_ballot_w64(sh_packed[slot] != 0u) != 0) {
      const uint32_t pk = sh_packed[slot];
      // field f, sign-extended from 5 bits
      auto field = [&](int f) { return (int)(pk << (27 - 5 * f)) >> 27; };
#pragma unroll
      for (int i = 0; i < A_PER; ++i) ra[slot][i] = shift_piece(ra[slot][i], field(i));
#pragma unroll
      for (int j = 0; j < B_PER; ++j) rb[slot][j] = shift_piece(rb[slot][j], field(A_PER + j));
    }
    // Only a piece that a valid-column boundary cuts needs masking (pieces
    // wholly outside were not loaded); most steps of most waves have none, so
    // the masks are skipped for the whole wave then.
    bool cut = false;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int jl = a_lo[i] - k0, jh = a_hi[i] - k0;
      cut |= (jl > 0 && jl < EPC) || (jh > 0 && jh < EPC);
    }
#pragma unroll
    for (int j = 0; j < B_PER; ++j) {
      const int jh = b_hi[j] - k0;
      cut |= jh > 0 && jh < EPC;
    }
    if (__builtin_amdgcn_ballot_w64(cut) != 0) {
#pragma unroll
      for (int i = 0; i < A_PER; ++i)
        *(u4*)(st + a_ldsoff[i]) = keep_range<EB>(ra[slot][i], a_lo[i] - k0, a_hi[i] - k0);
#pragma unroll
      for (int j = 0; j < B_PER; ++j)
        if (tid + 256 * j < B_PIECES) *(u4*)(st + b_ldsoff[j]) = keep_range<EB>(rb[slot][j], 0, b_hi[j] - k0);
    } else {
#pragma unroll
      for (int i = 0; i < A_PER; ++i) *(u4*)(st + a_ldsoff[i]) = ra[slot][i];
#pragma unroll
      for (int j = 0; j < B_PER; ++j)
        if (tid + 256 * j < B_PIECES) *(u4*)(st + b_ldsoff[j]) = rb[slot][j];
    }
    // The step's pieces are visible to every wave; the LDS stage written two
    // steps from now is no longer being read.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_step(slot);
    if (step < S) {
      F af[FM], bf[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) af[a] = *(const F*)(st + (wave * TM + a * 16 + fr) * ROWB + fg * 8 * EB);
#pragma unroll
      for (int b = 0; b < FN; ++b) bf[b] = *(const F*)(st + BM * ROWB + (b * 16 + fr) * ROWB + fg * 8 * EB);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = run_mfma(bf[b], af[a], acc[a][b]);
    }
  };
  for (int s = 0; s < S; s += DEPTH) {
#pragma unroll
    for (int t = 0; t < DEPTH; ++t)
      if (s + t < S) run_step(s + t, t);   // uniform: the last round stops at the last step
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads past the end

  // Epilogue: lane holds D[n = 4*fg + i][m = fr] of each 16x16 block.  Runs
  // of 4 channels go out as one store when they are aligned to its size (y
  // itself may be only element-aligned on this path).
  const bool vec_ok =
      (p.cout & 3) == 0 && (p.cout_g & 3) == 0 && (((uintptr_t)y & (uintptr_t)(4 * EB - 1)) == 0);
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = m0 + wave * TM + a * 16 + fr;
    if (m >= p.M) continue;
    T* yrow = y + out_row(p, m);
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int n = n0 + b * 16 + fg * 4;
      if (vec_ok && n + 3 < n_end) {
        if constexpr (EB == 2) {
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
          if (n + i < n_end) yrow[n + i] = from_f32<T>(acc[a][b][i]);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---- the K walk split over the waves: 16- or 32-row tiles for problems with few tiles ----
// With 64-row tiles the fp32 (1,8^3,16->32) layer makes 8 workgroups (32 busy
// SIMDs of 1024) and the C_in = 21 (4,16^3) layer one per CU, and each runs a
// serial chain of short K steps, each a barrier and an LDS round trip apart.
// Here a workgroup owns 16 FM output rows x BN columns and its four waves take
// every fourth step of the same K walk.  In a 16 x 16 MFMA fragment, lane l
// supplies row l % 16 at the 8 columns 8 (l / 16) .. + 7 of the step (for fp32
// as the two 4-column halves of the eight 16x16x4 products), which is exactly
// one 16-byte piece of the row's run (two for fp32): every lane loads its own
// fragments straight into registers, DEPTH of its wave's steps ahead, masked
// and shifted as above, with no LDS staging and no barrier in the loop.  At
// the end waves 1..3 hand their partial sums to wave 0 through LDS.
template <typename T, int FM, int BN, int DEPTH>
__global__ __launch_bounds__(256) void conv_runs_ksplit_kernel(ConvParams p, const T* __restrict__ x,
                                                               const T* __restrict__ w, T* __restrict__ y,
                                                               int tiles_n, int x_bytes, int w_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename RunFrag<T>::type F;
  constexpr int EB = sizeof(T);
  constexpr int EPC = 16 / EB;          // elements per piece
  constexpr int PPF = 8 / EPC;          // pieces per lane fragment: 1 (16-bit), 2 (fp32)
  constexpr int FN = BN / 16;
  constexpr int NP = (FM + FN) * PPF;   // pieces per lane per step: FM A fragments, then FN B fragments
  static_assert(BN % 16 == 0 && NP <= 12, "tile");
  __shared__ __attribute__((aligned(16))) f32x4_t red[3][FM][FN][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * 16 * FM;
  const int tpg = (p.cout_g + BN - 1) / BN;
  const int tn = tile % tiles_n;
  const int grp = tn / tpg;
  const int n0 = grp * p.cout_g + (tn - grp * tpg) * BN;
  const int n_end = (grp + 1) * p.cout_g;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, w_bytes, kRawBufferFlags);

  const bool wide = p.groups == 1 && p.ew == 1;
  const int run = wide ? p.kw * p.cin : p.cin_g;
  const int nkw = wide ? 1 : p.kw;
  const int sps = (run + kBK - 1) / kBK;
  const int S = p.kd * p.kh * nkw * sps;
  const int fr = lane & 15, fg = lane >> 4;
  const int c0 = 8 * fg;                // this lane's first column of a step

  // A fragment a: output row m0 + 16 a + fr; its run at (kd, kh, kw) =
  // (0, 0, 0) starts at element a_e, its valid columns are [a_lo, a_hi)
  int a_e[FM], a_lo[FM], a_hi[FM];
  uint32_t a_dh[FM], a_w[FM];
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const RowInfo ri = decode_row(p, m0 + 16 * a + fr);
    const int lo_w = ri.mw ? __builtin_ctz(ri.mw) : 0;
    const int hi_w = ri.mw ? 32 - __builtin_clz(ri.mw) : 0;
    a_e[a] = ri.base + grp * p.cin_g;
    a_lo[a] = wide ? lo_w * p.cin : 0;
    a_hi[a] = wide ? hi_w * p.cin : p.cin_g;
    a_dh[a] = ri.md | (ri.mh << 16);
    a_w[a] = wide ? 0xffffffffu : ri.mw;
  }
  // B: filter rows n0 + 16 b + fr
  int b_e[FN];
  bool b_ok[FN];
#pragma unroll
  for (int b = 0; b < FN; ++b) {
    const int co = n0 + 16 * b + fr;
    b_ok[b] = co < n_end;
    b_e[b] = co * p.K;
  }

  // this wave's steps: wave, wave + 4, ...; the walk (kd, kh, kw, k0) of the
  // next step to load, advanced four steps at a time
  int l_kd = 0, l_kh = 0, l_kw = 0, l_k0 = 0;
  auto advance = [&]() {
    l_k0 += kBK;
    if (l_k0 >= run) {
      l_k0 = 0;
      if (++l_kw == nkw) {
        l_kw = 0;
        if (++l_kh == p.kh) {
          l_kh = 0;
          ++l_kd;
        }
      }
    }
  };
  for (int i = 0; i < wave; ++i) advance();
  const int nst = S > wave ? (S - wave + 3) / 4 : 0;
  int l_step = 0;                        // index among this wave's steps

  u4 rp[DEPTH][NP];
  uint64_t sh_packed[DEPTH];            // shift_piece amounts, 5-bit fields
  int s_k0[DEPTH];
  auto load_step = [&](int slot) {
    const bool live = l_step < nst;
    const int xo = l_kd * p.ed * p.xs_d + l_kh * p.eh * p.xs_h + l_kw * p.ew * p.xs_w + l_k0;
    const int wo = ((l_kd * p.kh + l_kh) * nkw + l_kw) * run + l_k0;
    uint64_t packed = 0u;
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      const bool tap = ((a_dh[a] >> l_kd) & (a_dh[a] >> (16 + l_kh)) & (a_w[a] >> l_kw) & 1u) != 0u;
#pragma unroll
      for (int u = 0; u < PPF; ++u) {
        const int cc = l_k0 + c0 + u * EPC;     // run column of the piece's first element
        const bool ok = live && tap && a_lo[a] - cc < EPC && a_hi[a] - cc > 0;
        const int k = PPF * a + u;
        int sh;
        rp[slot][k] = load_piece<EB>(xr, a_e[a] + xo + c0 + u * EPC, ok, x_bytes, &sh);
        packed |= (uint64_t)((uint32_t)sh & 31u) << (5 * k);
      }
    }
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int u = 0; u < PPF; ++u) {
        const int cc = l_k0 + c0 + u * EPC;
        const int k = PPF * (FM + b) + u;
        int sh;
        rp[slot][k] = load_piece<EB>(wr, b_e[b] + wo + c0 + u * EPC, live && b_ok[b] && run - cc > 0, w_bytes, &sh);
        packed |= (uint64_t)((uint32_t)sh & 31u) << (5 * k);
      }
    sh_packed[slot] = packed;
    s_k0[slot] = l_k0;
    for (int i = 0; i < 4; ++i) advance();
    ++l_step;
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < DEPTH; ++t) load_step(t);

  auto run_step = [&](int slot) {
    const int k0 = s_k0[slot];
    if (__builtin_amdgcn_ballot_w64(sh_packed[slot] != 0u) != 0) {
      const uint64_t pk = sh_packed[slot];
      auto field = [&](int f) { return (int)((int64_t)(pk << (59 - 5 * f)) >> 59); };
#pragma unroll
      for (int k = 0; k < NP; ++k) rp[slot][k] = shift_piece(rp[slot][k], field(k));
    }
    // columns outside the row's valid window or past the run read as zero
    u4 pc[NP];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int u = 0; u < PPF; ++u) {
        const int cc = k0 + c0 + u * EPC;
        pc[PPF * a + u] = keep_range<EB>(rp[slot][PPF * a + u], a_lo[a] - cc, a_hi[a] - cc);
      }
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int u = 0; u < PPF; ++u) {
        const int cc = k0 + c0 + u * EPC;
        pc[PPF * (FM + b) + u] = keep_range<EB>(rp[slot][PPF * (FM + b) + u], 0, run - cc);
      }
    load_step(slot);
    // fragment f from pieces PPF f .. PPF f + PPF - 1
    auto frag = [&](int f) {
      F v;
      if constexpr (PPF == 1) {
        v = __builtin_bit_cast(F, pc[f]);
      } else {
        v.lo = __builtin_bit_cast(f32x4_t, pc[2 * f]);
        v.hi = __builtin_bit_cast(f32x4_t, pc[2 * f + 1]);
      }
      return v;
    };
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      const F af = frag(a);
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = run_mfma(frag(FM + b), af, acc[a][b]);
    }
  };
  for (int s0 = 0; s0 < nst; s0 += DEPTH) {
#pragma unroll
    for (int t = 0; t < DEPTH; ++t)
      if (s0 + t < nst) run_step(t);   // uniform
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads past the end

  // partial sums of waves 1..3 to wave 0 (same lane, same fragment layout)
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) red[wave - 1][a][b][lane] = acc[a][b];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int v = 0; v < 3; ++v) acc[a][b] += red[v][a][b][lane];

  // lane holds D[n = 4 fg + i][m = fr] of each 16 x 16 block
  const bool vec_ok =
      (p.cout & 3) == 0 && (p.cout_g & 3) == 0 && (((uintptr_t)y & (uintptr_t)(4 * EB - 1)) == 0);
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = m0 + 16 * a + fr;
    if (m >= p.M) continue;
    T* yrow = y + out_row(p, m);
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int n = n0 + b * 16 + fg * 4;
      if (vec_ok && n + 3 < n_end) {
        if constexpr (EB == 2) {
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
          if (n + i < n_end) yrow[n + i] = from_f32<T>(acc[a][b][i]);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int FM, int BN>
hipError_t launch_ksplit(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = (p.M + 16 * FM - 1) / (16 * FM);
  const int tiles_n = p.groups * ((p.cout_g + BN - 1) / BN);
  const int xb = (int)((int64_t)p.n * p.xs_n * sizeof(T));
  const int wb = (int)((int64_t)p.cout * p.K * sizeof(T));
  hipLaunchKernelGGL((conv_runs_ksplit_kernel<T, FM, BN, 4>), dim3(tiles_m * tiles_n), dim3(256), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, tiles_n, xb, wb);
  return hipGetLastError();
}

// Steps in flight in registers: 8 with 64-row tiles (the small problems they
// serve have few workgroups), else 2 (on (4,32^3,65) two steps ahead with four
// resident workgroups per CU beat four or six steps ahead with fewer: 115 us
// against 149 and 158).
template <typename T, int BM, int BN>
hipError_t launch_cfg(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  constexpr int DEPTH = BM == 64 && (sizeof(T) == 2 || BN < 128) ? 8 : 2;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = p.groups * ((p.cout_g + BN - 1) / BN);
  const int xb = (int)((int64_t)p.n * p.xs_n * sizeof(T));
  const int wb = (int)((int64_t)p.cout * p.K * sizeof(T));
  hipLaunchKernelGGL((conv_runs_kernel<T, BM, BN, DEPTH>), dim3(tiles_m * tiles_n), dim3(256), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, tiles_n, xb, wb);
  return hipGetLastError();
}

// Column tile: the smallest of 32, 48, 64, 80, 128 that holds one group's
// C_out/G (128 and several column tiles beyond that); row tile 128 when that still gives a few
// hundred tiles, else 64 (fp32 always 64).
template <typename T, int BM>
hipError_t launch_bn(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.cout_g <= 32) return launch_cfg<T, BM, 32>(p, x, w, y, s);
  if (p.cout_g <= 48) return launch_cfg<T, BM, 48>(p, x, w, y, s);
  if (p.cout_g <= 64) return launch_cfg<T, BM, 64>(p, x, w, y, s);
  if (p.cout_g <= 80) return launch_cfg<T, BM, 80>(p, x, w, y, s);
  return launch_cfg<T, BM, 128>(p, x, w, y, s);
}

// Steps of the K walk (32 columns each) and the 64-row tile count: with fewer
// 64-row tiles than two per CU and at least two steps per wave, the K walk is
// split over the waves, with column tiles of 32 or 64: 16-row tiles under half
// a tile per CU (fp32 (1,8^3,16->32), 8 tiles: 17.2 -> 8.9 us), else 32-row
// tiles, whose filter fragments each serve two row fragments (C_in = 21
// (4,16^3), 256 tiles: 14.9 -> 13.3 us; with 16-row tiles every wave fetched
// the filter for 16 rows and it ran 4% slower than the 64-row kernel).
int runs_steps(const ConvParams& p) {
  const bool wide = p.groups == 1 && p.ew == 1;
  const int run = wide ? p.kw * p.cin : p.cin_g;
  return p.kd * p.kh * (wide ? 1 : p.kw) * ((run + kBK - 1) / kBK);
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.cout_g <= 64 && runs_steps(p) >= 8) {
    const int bn = p.cout_g <= 32 ? 32 : 64;
    const int64_t tiles64 = (int64_t)(p.M + 63) / 64 * p.groups * ((p.cout_g + bn - 1) / bn);
    if (2 * tiles64 < device_cus())
      return bn == 32 ? launch_ksplit<T, 1, 32>(p, x, w, y, s) : launch_ksplit<T, 1, 64>(p, x, w, y, s);
    if (tiles64 < 2 * device_cus())
      return bn == 32 ? launch_ksplit<T, 2, 32>(p, x, w, y, s) : launch_ksplit<T, 2, 64>(p, x, w, y, s);
  }
  if constexpr (sizeof(T) == 2) {
    if ((p.M + 127) / 128 >= 512) return launch_bn<T, 128>(p, x, w, y, s);
  }
  return launch_bn<T, 64>(p, x, w, y, s);
}

}  // namespace

bool runs_accepts(const ConvParams& p, int dtype) {
  // pieces at a tensor's ends are loaded as the 16 bytes that end or start it
  const int64_t eb = dtype == kF32 ? 4 : 2;
  const bool big = p.n == 0 || ((int64_t)p.n * p.xs_n * eb >= 16 && (int64_t)p.cout * p.K * eb >= 16);
  return big && p.kd <= 16 && p.kh <= 16 && p.kw <= 16;
}

hipError_t launch_runs(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  if (dtype == kF32) return launch_typed<float>(p, x, w, y, s);
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
