// k_slab.hip -- implicit GEMM whose K steps read the w-taps and the h-taps of
// a filter plane from one staged block of input rows (fp16/bf16, C_in % 32 ==
// 0, unit stride along h and w, K_h in {2, 3}, K_w <= 3; dilation 1 along h
// and w, or 2 along both with a 3 x 3 plane).
//
// The classic implicit GEMM ("Convolutions" tutorial, section 5) gathers the
// A tile of every tap afresh, although the tiles of neighbouring taps are the
// same input values moved by one position.  Here a tile is 16 consecutive
// output rows along h times 32 consecutive outputs along w (512 GEMM rows, one
// depth plane of one image; the last tiles along h and w may hang over the
// output's end, their extra rows computed on zeros and not stored) and 128
// output channels.  For one (channel chunk of 32, kd) the workgroup stages the
// 18 input rows x 34 positions that the tile's windows cover (a "slab", zeros
// outside the input); output row g of the tile reads slab row g + kh for tap
// kh and position r + kw for tap kw, so all K_h * K_w taps of the plane come
// out of one staging.  Per (chunk, kd) the input bytes through the caches are
// 18 * 34 positions instead of K_h * 16 * 34.
//
// A K step is one (chunk, kd, kh); its filter slice (K_w taps x 128 output
// channels x 32 channels) is staged per step, two stages deep.  The slab of
// the next (chunk, kd) goes out in pieces from the MFMA blocks of the first
// K_h - 1 steps of the current one, into the second of two slab stages, and
// must land by the barrier that starts the next plane; the filter slice of
// step s + 1 goes out right after the barrier that starts step s.  A slab is
// 40 wave loads of 16 positions (612 needed), the filter slices of a step 24 KB.
// A dilated plane ("Convolution variants worth knowing": taps e positions apart)
// changes only where the taps read: at e = 2 output row g takes slab row
// g + 2 kh and position r + 2 kw, from a slab of 20 rows x 36 positions (48
// wave loads, 48 KB a stage).
//
// Eight waves, two per SIMD: wave v owns output rows 4 (v % 4) .. + 3 of the
// tile (128 GEMM rows) x channels 64 (v / 4) .. + 63 = 4 x 2 blocks of
// v_mfma_f32_32x32x16, 128 accumulator registers, so that the two waves of a
// SIMD cover each other's barrier waits and fragment-read latency (one wave
// per SIMD with a 128 x 128 block ran 5-9% slower on the same loads).  LDS: slab
// position o of row r at (34 r + o) * 64 bytes, its four 16-byte channel
// chunks XOR-swizzled by bits 2..3 of o (the same for every row), so fragment
// addresses are per-lane constants plus immediates, and one 256-byte LDS pass
// over 16 consecutive positions hits 16 distinct slots for every tap offset.
// Fragments are double-buffered in registers; the epilogue stages the tile
// through LDS so that stores write whole 16-byte pieces of output rows, as
// non-temporal stores (1-2% faster than ordinary ones: every workgroup writes
// its 128 KB at the same time, at the end).
#include <type_traits>

#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kSeg = 32;                            // outputs along w per tile row
constexpr int kRowsOut = 16;                        // output rows along h per tile
constexpr int kBM = kSeg * kRowsOut;                // 512 GEMM rows
constexpr int kMaxKW = 3;
constexpr int kMaxKH = 3;
constexpr int kRowB = 64;                           // bytes per position / filter row (32 channels)
constexpr int kLdsBytes = 160 * 1024;

// Slab extents at dilation E along h and w: positions per row (E = 1: 34,
// E = 2: 36), rows (18, 20), 16-position wave loads per wave (5, 6) and the
// bytes of one slab stage (40, 48 KB; the loads may run past the slab into a
// spare tail).
template <int E>
struct SlabGeom {
  static constexpr int SW = kSeg + (kMaxKW - 1) * E;
  static constexpr int ROWS = kRowsOut + (kMaxKH - 1) * E;
  static constexpr int LOADS = (ROWS * SW + 127) / 128;
  static constexpr int BYTES = 8 * LOADS * 16 * kRowB;
  static_assert(8 * LOADS * 16 >= ROWS * SW, "slab loads cover the slab");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time (so
// register arrays indexed by I stay in registers however large the body is)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// physical 16-byte chunk of logical chunk c at slab position o (or filter row o)
__device__ __forceinline__ int swz(int o, int c) { return c ^ ((o >> 2) & 3); }

template <typename T, int KW, int KH, int NB, int E>
__global__ __launch_bounds__(512, 1) void conv_slab_kernel(ConvParams p, const T* __restrict__ x,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ y, TileArgs ta) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  static_assert(NB == 128 || NB == 64, "channels per tile");
  static_assert(E == 1 || (E == 2 && KW == 3 && KH == 3), "dilation along h and w");
  constexpr int kSW = SlabGeom<E>::SW;
  constexpr int kA_LOADS = SlabGeom<E>::LOADS;
  constexpr int kSlabBytes = SlabGeom<E>::BYTES;
  constexpr int WR = NB == 128 ? 4 : 2;            // output rows (A fragments) per wave
  constexpr int NM = 2 * WR;                       // MFMAs per block per wave
  constexpr int B_ROWS = KW * NB;                  // filter rows per step
  constexpr int B_BYTES = B_ROWS * kRowB;
  constexpr int B_PIECES = B_ROWS * 4;             // 16-byte pieces per step (a multiple of 64)
  constexpr int B_LOADS = (B_PIECES + 511) / 512;  // per thread (the last round: the first waves)
  static_assert(KW >= 1 && KW <= kMaxKW && KH >= 2 && KH <= kMaxKH, "filter extents");
  static_assert(B_PIECES % 64 == 0, "whole waves of filter pieces");
  constexpr int B_BASE = 2 * kSlabBytes;
  constexpr int RING = B_BASE + 2 * B_BYTES;
  static_assert(RING <= kLdsBytes, "LDS");
  constexpr int OUT_ROWB = NB * 2;                 // one output row of the tile in LDS
  constexpr int OCH = NB / 8;                      // its 16-byte pieces
  constexpr int OUT_TILE = kBM * OUT_ROWB;
  constexpr int SMEM = RING > OUT_TILE ? RING : OUT_TILE;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // NB = 128: wave v owns output rows 4 (v % 4) .. + 3, channels 64 (v / 4) ..;
  // NB = 64: output rows 2 v .. 2 v + 1, all 64 channels
  const int wm = NB == 128 ? (wave & 3) : wave, wn = NB == 128 ? (wave >> 2) : 0;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  // tile: column tiles fastest, then w-block, h-block, depth, image (the
  // divisions by host-computed reciprocals)
  int t = fast_div(tile, ta.tiles_n, ta.m_tn);
  const int n0 = (tile - t * ta.tiles_n) * NB;
  // a column tile never straddles a channel group (NB divides C_out/G when
  // G > 1): the group's input channels start at cbase, its outputs end at n_end
  const int grp = p.groups == 1 ? 0 : n0 / p.cout_g;
  const int cbase = grp * p.cin_g, n_end = (grp + 1) * p.cout_g;
  int t2 = fast_div(t, ta.wblocks, ta.m_wb);
  const int ow0 = (t - t2 * ta.wblocks) * kSeg;
  t = fast_div(t2, ta.hblocks, ta.m_hb);
  const int oh0 = (t2 - t * ta.hblocks) * kRowsOut;
  const int img = fast_div(t, p.od, ta.m_od);
  const int od = t - img * p.od;
  const int z0 = od * p.sd - p.pd;
  const int y0 = oh0 - p.ph;   // unit stride along h and w
  const int x0 = ow0 - p.pw;

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)ta.x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)ta.w_bytes, kRawBufferFlags);

  // ---- slab loader: wave load i = 8 q + wave fills positions 16 i .. 16 i + 15
  // (four lanes each, one 16-byte chunk per lane); this lane's row, position
  // and chunk.  Validity along h and w is fixed per lane; along depth it is a
  // bit mask over kd. ----
  // (set-up with full-rate arithmetic only: 24-bit multiplies, a row of x and
  // a filter row being under 2^24 bytes, which slab_accepts checks; selects)
  uint32_t a_base[kA_LOADS];   // byte offset of the piece at (kd, chunk) = 0
  uint32_t a_mask[kA_LOADS];   // depth bits; 0 if the position is outside the input or the slab
  const uint32_t dmask = depth_mask(z0, p.kd, p.d, p.ed);
  const uint32_t ubase = (uint32_t)((img * p.xs_n + z0 * p.xs_d + y0 * p.xs_h + x0 * p.xs_w + cbase) * 2);
  const unsigned rowB = (unsigned)p.xs_h * 2, posB = (unsigned)p.xs_w * 2;
#pragma unroll
  for (int q = 0; q < kA_LOADS; ++q) {
    const int pos = (8 * q + wave) * 16 + (lane >> 2);
    const int r = div_small<kSW>(pos), o = pos - r * kSW;
    const int c = swz(o, lane & 3);                    // logical chunk this lane fetches
    const bool ok = r < kRowsOut + (KH - 1) * E && o < kSeg + (KW - 1) * E &&
                    (unsigned)(y0 + r) < (unsigned)p.h && (unsigned)(x0 + o) < (unsigned)p.w;
    a_base[q] = ubase + __umul24((unsigned)r, rowB) + __umul24((unsigned)o, posB) + c * 16;
    a_mask[q] = ok ? dmask : 0u;
  }
  // ---- filter loader: piece j = 512 s + tid -> (tap kw, row n, physical chunk) ----
  uint32_t b_base[B_LOADS];
  const unsigned K2 = (unsigned)p.K * 2, cin2 = (unsigned)p.cin_g * 2;
#pragma unroll
  for (int s = 0; s < B_LOADS; ++s) {
    const int j = s * 512 + tid;
    const int row = j >> 2, phys = j & 3;     // row = kw * NB + n
    const int kw = row / NB, n = row % NB;
    const int c = swz(row, phys);
    b_base[s] = j < B_PIECES && (n0 + n) < n_end
                    ? __umul24((unsigned)(n0 + n), K2) + __umul24((unsigned)kw, cin2) + c * 16
                    : kOutOfRange;
  }

  const int nchunks = p.cin_g / 32;
  const int NG = nchunks * p.kd;               // slabs: (chunk, kd), kd fastest
  // Past the last slab or step every load zero-fills (masks, not branches),
  // into a stage no step reads any more.
  int a_ic = 0, a_kd = 0, a_slot = 0;          // next slab to issue
  auto issue_a_part = [&](int q0, int q1) __attribute__((always_inline)) {
    char* sa = smem + a_slot * kSlabBytes;
    const uint32_t live = a_ic < nchunks ? ~0u : 0u;
    const uint32_t xoff = (uint32_t)((a_kd * p.ed * p.xs_d + a_ic * 32) * 2);
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      const bool ok = (((a_mask[q] & live) >> a_kd) & 1u) != 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(sa + ((8 * q + wave) * 16) * kRowB), 16, ok ? a_base[q] + xoff : kOutOfRange,
          0, 0, 0);
    }
    if (q1 == kA_LOADS) {
      const int d1 = a_kd + 1;
      const bool wrap = d1 == p.kd;
      a_kd = wrap ? 0 : d1;
      a_ic += (int)wrap;
      a_slot ^= 1;
    }
  };
  int b_ic = 0, b_kd = 0, b_kh = 0, b_slot = 0;   // next filter step to issue: kh fastest
  auto issue_b = [&]() __attribute__((always_inline)) {
    char* sb = smem + B_BASE + b_slot * B_BYTES;
    const uint32_t live = b_ic < nchunks ? ~0u : 0u;
    const uint32_t woff = (uint32_t)(((b_kd * KH + b_kh) * KW * p.cin_g + b_ic * 32) * 2);
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      // every wave loads in all but a partial last round (64-channel tiles:
      // there only the first waves, wave-uniformly); a compile-time "yes"
      // elsewhere keeps branches out of the MFMA-interleaved code
      if ((s + 1 < B_LOADS || B_PIECES % 512 == 0) || s * 512 + wave * 64 < B_PIECES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_ptr_t)(sb + (s * 512 + wave * 64) * 16), 16, (b_base[s] + woff) | (~live & kOutOfRange),
            0, 0, 0);
    const int h1 = b_kh + 1;
    const bool wh = h1 == KH;
    b_kh = wh ? 0 : h1;
    const int d1 = b_kd + (int)wh;
    const bool wd = d1 == p.kd;
    b_kd = wd ? 0 : d1;
    b_ic += (int)wd;
    b_slot ^= 1;
  };

  // ---- fragment addresses: lane (r = lane % 32, g2 = lane / 32); tile row
  // WR wm + a reads slab row WR wm + a + kh ----
  const int r = lane & 31, g2 = lane >> 5;
  int a_addr[KW][2], b_addr[2];
#pragma unroll
  for (int kw = 0; kw < KW; ++kw)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o = r + kw * E;
      a_addr[kw][ks] = (wm * WR * kSW + o) * kRowB + swz(o, 2 * ks + g2) * 16;
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) b_addr[ks] = r * kRowB + swz(r, 2 * ks + g2) * 16;

  f32x16_t acc[WR][2];
#pragma unroll
  for (int a = 0; a < WR; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // A step is 2 K_w blocks (tap kw, k-half ks) of 8 MFMAs per wave.  Block j+1's
  // fragments are read while block j's MFMAs run; the step's last block
  // passes the barrier first and reads the next step's first fragments.
  constexpr int NBLK = 2 * KW;
  constexpr int USLOTS = (KH - 1) * (NBLK - 1);   // blocks that carry slab pieces
  V8 fa[2][WR], fb[2][2];
  auto read_block = [&](V8(&af)[WR], V8(&bf)[2], const char* sa, const char* sb, int kw, int ks)
      __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < WR; ++a) af[a] = *(const V8*)(sa + a_addr[kw][ks] + a * kSW * kRowB);
#pragma unroll
    for (int b = 0; b < 2; ++b) bf[b] = *(const V8*)(sb + b_addr[ks] + (kw * NB + wn * 64 + b * 32) * kRowB);
  };
  auto mma_block = [&](const V8(&af)[WR], const V8(&bf)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < WR; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(bf[b], af[a], acc[a][b]);
  };
  // Step kh of a slab on (sa = slab stage + kh rows, sb); unless it is the
  // last, hand over to (na, nb).  At its closing barrier the filter of the
  // next step must have landed (and, at a slab's last step, the next slab);
  // the slab pieces this step issued may still be in flight.
  auto run_step = [&](const char* sa, const char* sb, const char* na, const char* nb, auto khc, auto last)
      __attribute__((always_inline)) {
    constexpr int kh = decltype(khc)::value;
    constexpr bool kLast = decltype(last)::value;
    constexpr int NWAIT = kh + 1 < KH ? ((kh + 1) * (NBLK - 1) * kA_LOADS) / USLOTS -
                                            (kh * (NBLK - 1) * kA_LOADS) / USLOTS
                                      : 0;
    static_for<0, NBLK>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      constexpr int cur = j & 1, nxt = cur ^ 1;
      if constexpr (j + 1 < NBLK) {
        read_block(fa[nxt], fb[nxt], sa, sb, (j + 1) >> 1, (j + 1) & 1);
        if constexpr (kh + 1 < KH) {
          constexpr int u = kh * (NBLK - 1) + j;
          issue_a_part((u * kA_LOADS) / USLOTS, ((u + 1) * kA_LOADS) / USLOTS);
        }
        mma_block(fa[cur], fb[cur]);
        // in the shadow of each MFMA: a fragment read (the first WR + 2), address VALU, a load
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < WR + 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!kLast) {
        // every wave's reads of this step have returned; the next step has landed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt_barrier<NWAIT>();
        read_block(fa[nxt], fb[nxt], na, nb, 0, 0);
        issue_b();                          // the step after next, into this step's filter stage
        mma_block(fa[cur], fb[cur]);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < WR + 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, (B_LOADS + NM - 1) / NM, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mma_block(fa[cur], fb[cur]);
      }
    });
  };

  if (NG > 0) {
    issue_a_part(0, kA_LOADS);            // slab 0
    issue_b();                            // filter of step 0
    wait_vmcnt_barrier<0>();
    issue_b();                            // filter of step 1
    read_block(fa[0], fb[0], smem, smem + B_BASE, 0, 0);
    int fs = 0;                           // filter stage of the step being computed
    // the K_h steps of slab g; in the final slab the last step hands over to nothing
    auto slab = [&](int g, auto final_c) __attribute__((always_inline)) {
      constexpr bool kFinal = decltype(final_c)::value;
      const char* sa = smem + (g & 1) * kSlabBytes;
      const char* sn = smem + ((g + 1) & 1) * kSlabBytes;
      auto step = [&](auto khc) __attribute__((always_inline)) {
        constexpr int kh = decltype(khc)::value;
        const char* sb = smem + B_BASE + fs * B_BYTES;
        const char* nb = smem + B_BASE + (fs ^ 1) * B_BYTES;
        const char* sak = sa + kh * E * kSW * kRowB;
        const char* nak = kh + 1 < KH ? sa + (kh + 1) * E * kSW * kRowB : sn;
        run_step(sak, sb, nak, nb, khc, std::integral_constant<bool, kFinal && kh + 1 == KH>{});
        fs ^= 1;
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      if constexpr (KH > 2) step(std::integral_constant<int, 2>{});
    };
    for (int g = 0; g + 1 < NG; ++g) slab(g, std::false_type{});
    slab(NG - 1, std::true_type{});
  }

  // ---- epilogue: the tile goes through LDS so each store writes whole
  // 16-byte pieces of output rows.  Lane (r, g2) holds tile rows
  // 32 (WR wm + a) + r and channels 64 wn + 32 b + 8 q + 4 g2 + i; in LDS a row
  // is NB * 2 bytes, its 16-byte piece k at slot k ^ (row % OCH); after a
  // barrier the workgroup stores the whole tile.  Wait for the zero-fill loads
  // past the end and for every wave's last reads first. ----
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int a = 0; a < WR; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (wm * WR + a) * 32 + r;
        const int k = wn * 8 + 4 * b + q;
        union { T h[4]; uint2 u; } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][4 * q + i]);
        *(uint2*)(smem + row * OUT_ROWB + ((k ^ (row & (OCH - 1))) * 16) + g2 * 8) = pk.u;
      }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const bool whole16 = (p.cout & 7) == 0;   // 16-byte stores stay aligned
  const int64_t plane = (int64_t)(img * p.od + od) * p.oh;
#pragma unroll 4
  for (int i = 0; i < kBM * OCH / 512; ++i) {
    const int piece = i * 512 + tid;
    const int row = piece / OCH, k = piece % OCH;
    const uint4 v = *(const uint4*)(smem + row * OUT_ROWB + ((k ^ (row & (OCH - 1))) * 16));
    const int oh = oh0 + (row >> 5);
    const int n = n0 + k * 8;
    if (oh < p.oh && ow0 + (row & 31) < p.ow) {
      const int64_t m = (plane + oh) * p.ow + ow0 + (row & 31);
      T* dst = y + m * p.cout + n;
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

template <typename T, int KW, int KH, int NB, int E>
hipError_t launch_k(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = p.n * p.od * ((p.oh + kRowsOut - 1) / kRowsOut) * ((p.ow + kSeg - 1) / kSeg);
  TileArgs ta;
  ta.tiles_n = (p.cout + NB - 1) / NB;
  ta.wblocks = (p.ow + kSeg - 1) / kSeg;
  ta.hblocks = (p.oh + kRowsOut - 1) / kRowsOut;
  ta.m_tn = div_magic(ta.tiles_n);
  ta.m_wb = div_magic(ta.wblocks);
  ta.m_hb = div_magic(ta.hblocks);
  ta.m_od = div_magic(p.od);
  ta.x_bytes = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  ta.w_bytes = (uint32_t)((int64_t)p.cout * p.K * 2);
  hipLaunchKernelGGL((conv_slab_kernel<T, KW, KH, NB, E>), dim3(tiles_m * ta.tiles_n), dim3(512), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, ta);
  return hipGetLastError();
}

// 64-channel tiles for grouped layers (a tile stays inside one group), for
// C_out <= 64 (a 128-channel tile would leave half its columns idle) and when
// 128-channel tiles would be fewer than the compute units (one workgroup fits
// a CU: (8, 64^2, 256) makes 128 of them, and 64-channel tiles run it faster
// on all 256 CUs).
template <typename T, int KW, int KH, int E = 1>
hipError_t launch_nb(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int64_t tiles_m = (int64_t)p.n * p.od * ((p.oh + kRowsOut - 1) / kRowsOut) * ((p.ow + kSeg - 1) / kSeg);
  if (p.groups > 1 || p.cout <= 64 || tiles_m * ((p.cout + 127) / 128) < device_cus())
    return launch_k<T, KW, KH, 64, E>(p, x, w, y, s);
  return launch_k<T, KW, KH, 128, E>(p, x, w, y, s);
}

template <typename T, int KH>
hipError_t launch_kh(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  switch (p.kw) {
    case 1: return launch_nb<T, 1, KH>(p, x, w, y, s);
    case 2: return launch_nb<T, 2, KH>(p, x, w, y, s);
    default: return launch_nb<T, 3, KH>(p, x, w, y, s);
  }
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.eh == 2) return launch_nb<T, 3, 3, 2>(p, x, w, y, s);   // dilated 3 x 3
  return p.kh == 2 ? launch_kh<T, 2>(p, x, w, y, s) : launch_kh<T, 3>(p, x, w, y, s);
}

}  // namespace

bool slab_accepts(const ConvParams& p, int dtype) {
  return (dtype == kF16 || dtype == kBF16) && p.remap == 0 && p.sh == 1 && p.sw == 1 &&
         p.eh == p.ew && (p.eh == 1 || (p.eh == 2 && p.kh == 3 && p.kw == 3)) && p.cin_g % 32 == 0 && p.cout % 4 == 0 &&
         (p.groups == 1 || p.cout_g % 64 == 0) &&
         p.kw <= kMaxKW && p.kh >= 2 && p.kh <= kMaxKH && p.kd <= 16 &&
         // the set-up's 24-bit multiplies and tile decode
         (int64_t)p.xs_h * 2 < (1 << 24) && (int64_t)p.K * 2 < (1 << 24) &&
         (int64_t)p.n * p.od * ((p.oh + kRowsOut - 1) / kRowsOut) * ((p.ow + kSeg - 1) / kSeg) *
                 ((p.cout + 63) / 64) < (1 << 24);
}

hipError_t launch_slab(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
