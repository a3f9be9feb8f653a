// k_phase.hip -- implicit GEMM for stride 2 along h and w: every tap reads the
// input rows staged once per (channel chunk, kd), split by stride phase
// (fp16/bf16, C_in/G % 64 == 0, K_h in {2, 3}, K_w in {2, 3}, dilation 1
// along h and w).
//
// At stride 2 the classic implicit GEMM ("Convolutions" tutorial, section 5)
// gathers each tap's A tile afresh, and neighbouring outputs read input
// positions two apart, so a block of input staged in plain order cannot serve
// a tap with consecutive reads.  Here output row oh at tap kh reads input row
// 2*oh - p_h + kh: the taps kh = 0 and 2 read the even rows of the window
// block, the tap kh = 1 the odd ones.  Likewise along w, output ow at tap kw
// reads position 2*ow - p_w + kw: kw = 0 and 2 read the even positions (kw = 2
// one further), kw = 1 the odd ones.  So per (chunk, kd) the workgroup stages
// two blocks of input rows, the even rows ("E", serving kh = 0, 2) and the odd
// rows ("O", serving kh = 1), and stores each row with its even positions
// first and its odd positions after them: the 16 outputs of a tile row then
// read 16 consecutive slots for every (kh, kw).
//
// Tile: 8 output rows x 16 outputs along w (128 GEMM rows, one depth plane of
// one image; the last tiles along h and w may hang over the output's end,
// computed on zeros and not stored) x 64 output channels (a tile stays inside
// one channel group).  A position holds 64 channels, 128 bytes: whole cache
// lines, which direct-to-LDS loads move at about twice the rate of half lines.
// E holds 9 rows x 33 positions (37 KB), O 8 rows (33 KB) for a 3 x 3 plane.
// K steps follow the stride phases: per (chunk, kd) the steps kh = 0, 2 read E
// and kh = 1 reads O, each with its K_w filter taps (64 channels x 64 output
// channels each, staged per step two stages deep).  E blocks alternate
// between two buffers and O has one: O(p) loads during the first E step of
// (chunk, kd) p, and E(p+2) during the odd step of p into the buffer E(p) has
// just left, a full period before it is read; the filter slice of step s + 2
// goes out after the barrier that ends step s.  LDS: 2 x 38 KB + 33 KB +
// 2 x 24 KB = 157 KB.
//
// Eight waves, two per SIMD: wave (mb = v % 4, kp = v / 4) owns output rows
// 2 mb, 2 mb + 1 of the tile (32 GEMM rows) x all 64 channels, on the k
// slices 2 kp, 2 kp + 1 of each 64-channel chunk (two v_mfma_f32_32x32x16
// blocks, 32 accumulators); the two waves of a row block add their partial
// sums through LDS at the end.  With one wave per SIMD the K steps were bound
// by LDS fragment reads (one wave cannot keep enough reads in flight) and by
// the per-lane set-up, which now splits over twice the waves.  Fragment reads
// run one unit (a tap's k slice) ahead of the MFMAs.  LDS positions and filter
// rows are 128 bytes; their 16-byte chunks are XOR-swizzled: a filter row R by
// bits 1..3 of R, a staged position by (s >> 1 & 3) ^ (s & 1) << 2 of its slot
// s inside its phase sub-row.  Timed with a read-only probe, the position
// swizzle serves the A reads of all three taps at the full LDS rate (~200
// B/clk per CU; with bits 1..3 of s the kw = 2 tap, which starts one slot on,
// got ~110).
#include <type_traits>

#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kTW = 16;             // outputs along w per tile
constexpr int kTH = 8;              // output rows along h per tile
constexpr int kBM = kTW * kTH;      // 128 GEMM rows
constexpr int kBN = 64;             // output channels per tile
constexpr int kCK = 64;             // input channels per chunk (one 128-byte position)
constexpr int kPosB = kCK * 2;      // bytes per staged position / filter row
constexpr int kLdsBytes = 160 * 1024;
constexpr int kWaves = 8;           // two per SIMD

// XOR applied to the 16-byte chunk index of the staged position at slot s of
// its phase sub-row
__device__ __forceinline__ int pos_swz(int s) { return ((s >> 1) & 3) ^ ((s & 1) << 2); }

template <int KH, int KW>
struct PhaseGeom {
  static constexpr int SE = kTW + (KW - 1) / 2;   // even positions per row (0, 2, .. 2(TW-1) + KW-1)
  static constexpr int SO = kTW + (KW - 2) / 2;   // odd positions per row
  static constexpr int SR = SE + SO;              // slots per staged row
  static constexpr int RE = kTH + (KH - 1) / 2;   // rows of E (input rows 0, 2, ..)
  static constexpr int RO = kTH + (KH - 2) / 2;   // rows of O (input rows 1, 3, ..)
  static constexpr int WE = (RE * SR + 7) / 8;    // 1-KB wave loads (8 positions) per E block
  static constexpr int WO = (RO * SR + 7) / 8;
  static constexpr int LE = (WE + kWaves - 1) / kWaves;   // per wave, at most
  static constexpr int LO = (WO + kWaves - 1) / kWaves;
  static constexpr int EBYTES = WE * 1024;
  static constexpr int OBYTES = WO * 1024;
  static constexpr int FLOADS = KW * kBN * 8 / 64;   // filter wave loads per step
  static constexpr int FBYTES = KW * kBN * kPosB;
  static constexpr int O_BASE = 2 * EBYTES;
  static constexpr int F_BASE = O_BASE + OBYTES;
  static constexpr int BYTES = F_BASE + 2 * FBYTES;
  static_assert(FLOADS % kWaves == 0, "whole filter rounds");
  static_assert(BYTES <= kLdsBytes, "LDS");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// The K_h steps of one (chunk, kd) in the order they run: the even taps (on
// E), then the odd ones (on O).
template <int KH>
__host__ __device__ constexpr int step_kh(int i) {
  return KH == 3 ? (i == 0 ? 0 : i == 1 ? 2 : 1) : i;
}

template <typename T, int KH, int KW>
__global__ __launch_bounds__(512, 1) void conv_phase_kernel(ConvParams p, const T* __restrict__ x,
                                                            const T* __restrict__ w,
                                                            T* __restrict__ y, TileArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  typedef PhaseGeom<KH, KW> G;
  static_assert(KH >= 2 && KH <= 3 && KW >= 2 && KW <= 3, "filter extents");
  constexpr int NE = (KH + 1) / 2;     // steps on E per (chunk, kd)
  constexpr int NU = 2 * KW;           // units per step: (tap kw, half of the row blocks)
  __shared__ __attribute__((aligned(1024))) char smem[G::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  // tile: output channels fastest, then w-block, h-block, depth, image
  int t = fast_div(tile, a.tiles_n, a.m_tn);
  const int n0 = (tile - t * a.tiles_n) * kBN;
  const int grp = p.groups == 1 ? 0 : n0 / p.cout_g;
  const int cbase = grp * p.cin_g, n_end = (grp + 1) * p.cout_g;
  int t2 = fast_div(t, a.wblocks, a.m_wb);
  const int ow0 = (t - t2 * a.wblocks) * kTW;
  t = fast_div(t2, a.hblocks, a.m_hb);
  const int oh0 = (t2 - t * a.hblocks) * kTH;
  const int img = fast_div(t, p.od, a.m_od);
  const int od = t - img * p.od;
  const int z0 = od * p.sd - p.pd;
  const int y0 = 2 * oh0 - p.ph;   // input row of staged row 0
  const int x0 = 2 * ow0 - p.pw;   // input position of even slot 0

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)a.x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)a.w_bytes, kRawBufferFlags);
  // depth taps inside the input; without depth dilation no division is needed
  const uint32_t dmask = depth_mask(z0, p.kd, p.d, p.ed);

  // ---- block loaders: wave load i = 8 l + wave fills positions 8 i .. 8 i + 7
  // of the block (eight lanes each, one 16-byte chunk per lane).  This lane's
  // byte offset at (kd, chunk) = 0 and its depth mask (0 outside the input or
  // past the block's end).  The set-up runs on every workgroup before its
  // first loads, so it uses full-rate arithmetic only (24-bit multiplies:
  // a row of x and a filter row are under 2^24 bytes, which phase_accepts
  // checks; selects instead of branches). ----
  const int rowB = p.xs_h * 2, posB = p.xs_w * 2;
  const uint32_t ubase = (uint32_t)((img * p.xs_n + z0 * p.xs_d + y0 * p.xs_h + x0 * p.xs_w + cbase) * 2);
  const int lane_pos = 8 * wave + (lane >> 3);   // this lane's position in wave load l = 0
  constexpr int kRound = 8 * kWaves;             // positions per round of wave loads
  // base[l]: byte offset at (kd, chunk) = 0; bit l of *inside: the position lies
  // inside the input along h and w (and inside the block)
  auto setup = [&](uint32_t* base, uint32_t* inside, int L, int R, int odd) __attribute__((always_inline)) {
    uint32_t bits = 0;
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int pos = lane_pos + kRound * l;
      const int b = div_small<G::SR>(pos), slot = pos - b * G::SR;
      const int ph = slot >= G::SE ? 1 : 0;
      const int s = slot - ph * G::SE;             // index inside the phase sub-row
      const int c = (lane & 7) ^ pos_swz(s);       // logical chunk this lane fetches
      const int r = 2 * b + odd, o = 2 * s + ph;   // staged row, position
      const uint32_t ok = (uint32_t)(b < R) & (uint32_t)((unsigned)(y0 + r) < (unsigned)p.h) &
                          (uint32_t)((unsigned)(x0 + o) < (unsigned)p.w);
      bits |= ok << l;
      base[l] = ubase + __umul24((unsigned)r, (unsigned)rowB) + __umul24((unsigned)o, (unsigned)posB) + c * 16;
    }
    *inside = bits;
  };
  uint32_t e_base[G::LE], o_base[G::LO], e_in, o_in;

  // ---- filter loader: wave load i = 8 l + wave fills rows R = 8 i .. 8 i + 7
  // (R = kw * 64 + n) of a stage ----
  constexpr int FL = G::FLOADS / kWaves;
  uint32_t f_base[FL];
  auto setup_filter = [&]() __attribute__((always_inline)) {
    const unsigned K2 = (unsigned)p.K * 2, cin2 = (unsigned)p.cin_g * 2;
#pragma unroll
    for (int l = 0; l < FL; ++l) {
      const int R = (kWaves * l + wave) * 8 + (lane >> 3);
      const int kw = R >> 6, n = R & 63;
      const int c = (lane & 7) ^ ((R >> 1) & 7);
      f_base[l] = n0 + n < n_end ? __umul24((unsigned)(n0 + n), K2) + __umul24((unsigned)kw, cin2) + c * 16
                                 : kOutOfRange;
    }
  };

  const int nchunks = p.cin_g / kCK;
  const int NP = nchunks * p.kd;        // (chunk, kd) periods, kd fastest
  char* const o_buf = smem + G::O_BASE;
  char* const f_buf = smem + G::F_BASE;

  // Blocks and filter slices of periods past the end zero-fill (no memory
  // traffic) into buffers no step reads any more.
  auto issue_block = [&](char* buf, const uint32_t* base, uint32_t inside, int W, int kd, int ch, bool live,
                         int l0, int l1) __attribute__((always_inline)) {
    // the plane kd is inside the input (and the period exists): uniform
    const uint32_t plane = live && ((dmask >> kd) & 1u) ? ~0u : 0u;
    const uint32_t in = inside & plane;
    const uint32_t xo = (uint32_t)((kd * p.ed * p.xs_d + ch * kCK) * 2);
#pragma unroll
    for (int l = l0; l < l1; ++l) {
      if (kWaves * l + wave < W) {   // wave-uniform: the last round may be partial
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(buf + (kWaves * l + wave) * 1024), 16,
                                                 ((in >> l) & 1u) ? base[l] + xo : kOutOfRange, 0, 0, 0);
      }
    }
  };
  // the filter slice of step (kd, kh) of chunk ch into stage st
  auto issue_filter = [&](int kd, int ch, int kh, bool live, int st) __attribute__((always_inline)) {
    const uint32_t dead = live ? 0u : kOutOfRange;
    const uint32_t wo = (uint32_t)((((kd * KH + kh) * KW) * p.cin_g + ch * kCK) * 2);
    char* fbuf = f_buf + st * G::FBYTES;
#pragma unroll
    for (int l = 0; l < FL; ++l)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(fbuf + (kWaves * l + wave) * 1024), 16,
                                               (f_base[l] + wo) | dead, 0, 0, 0);
  };

  // ---- fragment addresses: wave (mb = wave % 4, kp = wave / 4) owns tile rows
  // 32 mb .. 32 mb + 31 and the k slices 2 kp, 2 kp + 1 (channels 32 kp ..
  // 32 kp + 31 of the chunk); lane (r = lane % 32: tile row 2 mb + r / 16,
  // output j = r % 16; kg = lane / 32).  A: slot j + (kw >> 1) of the phase
  // sub-row kw & 1 of block row 2 mb + r / 16 + (kh >> 1); B: filter row
  // kw * 64 + 32 nb + r. ----
  const int mb = wave & 3, kp = wave >> 2;
  const int r32 = lane & 31, kg = lane >> 5;
  int a_off[2][2], b_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int s = (r32 & 15) + e, ks = 2 * kp + t2;
      a_off[e][t2] = ((2 * mb + (r32 >> 4)) * G::SR + s) * kPosB + (((2 * ks + kg) ^ pos_swz(s)) * 16);
    }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
    b_off[t2] = r32 * kPosB + (((2 * (2 * kp + t2) + kg) ^ ((r32 >> 1) & 7)) * 16);

  f32x16_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.f;

  // unit u = (tap kw = u / 2, the wave's k slice u % 2) of step kh on block
  // `ab`, filter stage `sb`; double-buffered by unit (an even number per step)
  V8 fa[2], fb[2][2];   // [register buffer] and [register buffer][nb]
  auto read_unit = [&](V8& A, V8(&B)[2], const char* ab, const char* sb, auto khc, auto uc)
      __attribute__((always_inline)) {
    constexpr int kh = decltype(khc)::value, u = decltype(uc)::value;
    constexpr int kw = u >> 1, t2 = u & 1;
    constexpr int imm = ((kh >> 1) * G::SR + (kw & 1) * G::SE) * kPosB;
    A = *(const V8*)(ab + a_off[kw >> 1][t2] + imm);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) B[nb] = *(const V8*)(sb + b_off[t2] + (kw * kBN + nb * 32) * kPosB);
  };
  auto mma_unit = [&](const V8& A, const V8(&B)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32x32x16(B[nb], A, acc[nb]);
  };

  // One step: kh on block ab with filter stage sb.  While unit u's MFMAs run,
  // unit u + 1's fragments are read and this step's block pieces go out
  // (pieces(u)); the last unit waits (pieces(NU): the next step's filter, and
  // the next block when a block ends, must have landed), passes the barrier,
  // reads the next step's first unit from (nab, nsb) and sends the filter of
  // the step after next into this step's stage (next2()).
  auto run_step = [&](const char* ab, const char* sb, const char* nab, const char* nsb, auto khc, auto nkhc,
                      auto lastc, auto pieces, auto next2) __attribute__((always_inline)) {
    constexpr bool kLast = decltype(lastc)::value;
    static_for<0, NU>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      constexpr int cur = u & 1, nxt = cur ^ 1;
      if constexpr (u + 1 < NU) {
        read_unit(fa[nxt], fb[nxt], ab, sb, khc, std::integral_constant<int, u + 1>{});
        pieces(uc);
        mma_unit(fa[cur], fb[cur]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!kLast) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        pieces(std::integral_constant<int, NU>{});
        read_unit(fa[nxt], fb[nxt], nab, nsb, nkhc, std::integral_constant<int, 0>{});
        next2();
        mma_unit(fa[cur], fb[cur]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mma_unit(fa[cur], fb[cur]);
      }
    });
  };

  // per-wave piece counts of E and O (the last round of wave loads may be partial)
  const bool e_full = wave < G::WE - kWaves * (G::LE - 1);
  const bool o_full = wave < G::WO - kWaves * (G::LO - 1);

  // (kd, chunk) after (kd, ch) in the walk, kd fastest
  auto advance = [&](int& kd, int& ch) __attribute__((always_inline)) {
    if (++kd == p.kd) {
      kd = 0;
      ++ch;
    }
  };

  // The first loads go out as soon as their addresses are known; the rest of
  // the set-up overlaps their latency.
  setup(e_base, &e_in, G::LE, G::RE, 0);
  if (NP > 0) issue_block(smem, e_base, e_in, G::WE, 0, 0, true, 0, G::LE);   // E of period 0
  setup_filter();
  if (NP > 0) issue_filter(0, 0, step_kh<KH>(0), true, 0);
  setup(o_base, &o_in, G::LO, G::RO, 1);

  if (NP > 0) {
    int pkd = 0, pch = 0;   // (kd, chunk) of the period
    int qkd = 0, qch = 0;   // of the next one
    advance(qkd, qch);
    if constexpr (NE == 2) {
      // E of period 1 as well: from here on E(p + 2) goes out during the odd step of p
      issue_block(smem + G::EBYTES, e_base, e_in, G::WE, qkd, qch, NP > 1, 0, G::LE);
      if (e_full) wait_vmcnt_barrier<G::LE>();
      else wait_vmcnt_barrier<G::LE - 1>();
    } else {
      wait_vmcnt_barrier<0>();
    }
    issue_filter(0, 0, step_kh<KH>(1), true, 1);
    read_unit(fa[0], fb[0], smem, f_buf, std::integral_constant<int, step_kh<KH>(0)>{},
              std::integral_constant<int, 0>{});
    int fs = 0;            // filter stage of the period's first step
    // the K_h steps of period pp; in the final period the last step hands over to nothing
    auto period = [&](int pp, auto finalc) __attribute__((always_inline)) {
      constexpr bool kFinal = decltype(finalc)::value;
      int rkd = qkd, rch = qch;       // the period after next
      advance(rkd, rch);
      const bool nlive = pp + 1 < NP;
      const char* eb = smem + (pp & 1) * G::EBYTES;
      char* en = smem + ((pp + 1) & 1) * G::EBYTES;   // E of the next period
      static_for<0, KH>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int kh = step_kh<KH>(i);
        constexpr bool on_e = i < NE, first_e = i == 0, last_e = i == NE - 1;
        constexpr int nkh = step_kh<KH>(i + 1 < KH ? i + 1 : 0);
        const int st = (fs + i) & 1;
        const char* ab = on_e ? eb : o_buf;
        const char* nab = i + 1 < KH ? (i + 1 < NE ? eb : o_buf) : en;
        const char* sb = f_buf + st * G::FBYTES;
        const char* nsb = f_buf + (st ^ 1) * G::FBYTES;
        // Block pieces.  K_h = 3: O(pp) during the first E step (needed two steps
        // later), E(pp + 2) during the odd step into the buffer E(pp) has just
        // left (needed four steps later).  K_h = 2 (one E step): O(pp) and then
        // E(pp + 1) during the E step, so that the wait below can leave exactly
        // the E pieces in flight.
        auto pieces = [&](auto uc) __attribute__((always_inline)) {
          constexpr int u = decltype(uc)::value;
          constexpr int NI = NU - 1;                               // units that issue
          constexpr bool o_here = first_e;
          constexpr bool e_here = NE == 2 ? !on_e : last_e;
          constexpr int oa = 0, ob = o_here && e_here ? NI / 2 : NI;   // O over units [oa, ob)
          constexpr int ea = o_here && e_here ? NI / 2 : 0, eb2 = NI;  // E over units [ea, eb2)
          if constexpr (u < NU) {
            if constexpr (o_here && u >= oa && u < ob)
              issue_block(o_buf, o_base, o_in, G::WO, pkd, pch, true, ((u - oa) * G::LO) / (ob - oa),
                          ((u - oa + 1) * G::LO) / (ob - oa));
            if constexpr (e_here && u >= ea && u < eb2) {
              if constexpr (NE == 2)
                issue_block((char*)eb, e_base, e_in, G::WE, rkd, rch, pp + 2 < NP, ((u - ea) * G::LE) / (eb2 - ea),
                            ((u - ea + 1) * G::LE) / (eb2 - ea));
              else
                issue_block(en, e_base, e_in, G::WE, qkd, qch, nlive, ((u - ea) * G::LE) / (eb2 - ea),
                            ((u - ea + 1) * G::LE) / (eb2 - ea));
            }
          } else if constexpr (e_here) {
            // the next block and the next filter must have landed; E may stay in flight
            if (e_full) wait_vmcnt_barrier<G::LE>();
            else wait_vmcnt_barrier<G::LE - 1>();
          } else if constexpr (o_here) {
            if (o_full) wait_vmcnt_barrier<G::LO>();
            else wait_vmcnt_barrier<G::LO - 1>();
          } else {
            wait_vmcnt_barrier<0>();
          }
        };
        // the filter of the step after next goes into this step's stage
        auto next2 = [&]() __attribute__((always_inline)) {
          if constexpr (i + 2 < KH) issue_filter(pkd, pch, step_kh<KH>(i + 2), true, st);
          else issue_filter(qkd, qch, step_kh<KH>(i + 2 - KH), nlive, st);
        };
        run_step(ab, sb, nab, nsb, std::integral_constant<int, kh>{}, std::integral_constant<int, nkh>{},
                 std::integral_constant<bool, kFinal && i + 1 == KH>{}, pieces, next2);
      });
      fs ^= (KH & 1);
      pkd = qkd;
      pch = qch;
      qkd = rkd;
      qch = rch;
    };
    for (int pp = 0; pp + 1 < NP; ++pp) period(pp, std::false_type{});
    period(NP - 1, std::true_type{});
  }

  // ---- epilogue.  The two waves of a row block hold partial sums over their
  // k slices: the upper one (kp = 1) writes its fp32 partials to LDS (32
  // rows x 64 channels, 8 KB per row block, 16-byte unit u of row r at slot
  // u ^ (r % 16)), the lower one adds them, rounds once and stages the tile
  // in LDS (128-byte rows, 16-byte piece k at slot k ^ (row % 8)) so each
  // store writes whole 16-byte pieces of output rows.  Lane (r32, kg) holds
  // row 32 mb + r32, channels 32 nb + 8 q + 4 kg + i. ----
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  char* const part = smem + mb * 8192;
  char* const tileb = smem + 4 * 8192;
  if (kp == 1) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = nb * 8 + 2 * q + kg;
        const f32x4_t v4 = {acc[nb][4 * q], acc[nb][4 * q + 1], acc[nb][4 * q + 2], acc[nb][4 * q + 3]};
        *(f32x4_t*)(part + r32 * 256 + ((u ^ (r32 & 15)) * 16)) = v4;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (kp == 0) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = nb * 8 + 2 * q + kg;
        const f32x4_t o4 = *(const f32x4_t*)(part + r32 * 256 + ((u ^ (r32 & 15)) * 16));
        const int row = mb * 32 + r32;
        const int k = nb * 4 + q;
        union { T h[4]; uint2 u; } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[nb][4 * q + i] + o4[i]);
        *(uint2*)(tileb + row * 128 + ((k ^ (row & 7)) * 16) + kg * 8) = pk.u;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const bool whole16 = (p.cout & 7) == 0;
  const int64_t plane = (int64_t)(img * p.od + od) * p.oh;
#pragma unroll
  for (int it = 0; it < kBM * 8 / (64 * kWaves); ++it) {
    const int piece = it * 64 * kWaves + tid;
    const int row = piece >> 3, k = piece & 7;
    const uint4 v = *(const uint4*)(tileb + row * 128 + ((k ^ (row & 7)) * 16));
    const int oh = oh0 + (row >> 4), ow = ow0 + (row & 15);
    const int n = n0 + k * 8;
    if (oh < p.oh && ow < p.ow) {
      T* dst = y + ((plane + oh) * p.ow + ow) * p.cout + n;
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

template <typename T, int KH, int KW>
hipError_t launch_k(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  TileArgs a;
  a.tiles_n = (p.cout + kBN - 1) / kBN;
  a.wblocks = (p.ow + kTW - 1) / kTW;
  a.hblocks = (p.oh + kTH - 1) / kTH;
  a.m_tn = div_magic(a.tiles_n);
  a.m_wb = div_magic(a.wblocks);
  a.m_hb = div_magic(a.hblocks);
  a.m_od = div_magic(p.od);
  a.x_bytes = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  a.w_bytes = (uint32_t)((int64_t)p.cout * p.K * 2);
  const int64_t tiles = (int64_t)p.n * p.od * a.hblocks * a.wblocks * a.tiles_n;
  hipLaunchKernelGGL((conv_phase_kernel<T, KH, KW>), dim3((unsigned)tiles), dim3(64 * kWaves), 0, s, p, (const T*)x,
                     (const T*)w, (T*)y, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.kh == 2) return p.kw == 2 ? launch_k<T, 2, 2>(p, x, w, y, s) : launch_k<T, 2, 3>(p, x, w, y, s);
  return p.kw == 2 ? launch_k<T, 3, 2>(p, x, w, y, s) : launch_k<T, 3, 3>(p, x, w, y, s);
}

}  // namespace

bool phase_accepts(const ConvParams& p, int dtype) {
  // rows of x and of the filter under 2^24 bytes (the set-up's 24-bit
  // multiplies) and fewer than 2^24 tiles (the tile decode's division)
  return (dtype == kF16 || dtype == kBF16) && p.remap == 0 && p.sh == 2 && p.sw == 2 && p.eh == 1 &&
         p.ew == 1 && p.kh >= 2 && p.kh <= 3 && p.kw >= 2 && p.kw <= 3 && p.kd <= 16 && p.cin_g % kCK == 0 &&
         p.cout % 4 == 0 && (p.groups == 1 || p.cout_g % kBN == 0) && (int64_t)p.xs_h * 2 < (1 << 24) &&
         (int64_t)p.K * 2 < (1 << 24) &&
         (int64_t)p.n * p.od * ((p.oh + kTH - 1) / kTH) * ((p.ow + kTW - 1) / kTW) * ((p.cout + kBN - 1) / kBN) <
             (1 << 24);
}

hipError_t launch_phase(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
