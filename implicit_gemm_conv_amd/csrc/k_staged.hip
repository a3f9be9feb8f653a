// k_staged.hip -- the slab scheme for channel counts that are not a multiple
// of 32, and for tensors that are aligned to their element size only
// (fp16/bf16, one group, unit stride and no dilation along h and w, K_h and
// K_w in {2, 3}; any C_in with (C_in mod 8) * K_d * K_h * K_w <= 32).
//
// The classic implicit GEMM ("Convolutions" tutorial, section 5) gathers each
// tap's A tile afresh, although neighbouring taps read the same input moved
// by one position; the slab kernel stages the input rows of a tile once per
// (channel chunk, kd) and serves every (kh, kw) tap from them, but it fills
// LDS with direct-to-LDS 16-byte loads, which need 16-byte aligned positions
// (C_in a multiple of 8 at least) and a whole number of 32-channel chunks.
// Here the same staging goes through registers: each 16-byte piece of a
// position is fetched with an unaligned buffer load (a position of 65 bf16
// channels starts every 130 bytes) and written to an aligned, swizzled LDS
// slot.  The GEMM depth of one output row (K ordered kd, kh, kw, c) splits in
// two parts:
//  * channels c < C_main = C_in - (C_in mod 8) in 32-channel chunks (a last
//    partial chunk holds 8, 16 or 24; its missing pieces read as zeros): the
//    slab walk, one K block of 32 per (chunk, tap);
//  * the r = C_in mod 8 channels left over, over all T = K_d K_h K_w taps:
//    T r <= 32 entries (tap-major, channel-minor, the filter's own order)
//    packed into one more K block, gathered element by element once per tile.
// On (4, 32^3, 65 -> 65) the depth is 2 x 27 chunk blocks + 1 packed block
// (1760 columns for 1755) where 32-channel padding would take 81 blocks.
//
// Tile: 16 output rows x 32 outputs along w (512 GEMM rows, one depth plane of
// one image; rows past the output's end are computed on zeros and not
// stored) x NB output channels, NB in {32, 64, 80}, so that C_out = 65 runs on
// 80 columns.  Four waves, one per SIMD: wave v owns output rows 4v .. 4v + 3
// of the tile (8 fragments of 16 outputs) x all NB channels, v_mfma_f32_
// 16x16x32 blocks with the filter as the first operand, so a lane receives 4
// consecutive channels of one output.  Per K block a wave reads 8 + NB/16
// fragments (1 KB each) for 8 NB/16 MFMAs.  (Eight waves of half the rows
// would leave 256 registers a wave, too few for the 80 accumulators, the
// double-buffered fragments and the loads in flight.)
//
// Pipeline, per K step (chunk, kd, kh) of K_w blocks: the filter slice of
// step s + 1 is fetched into registers after the barrier that starts step s
// and written to its LDS stage before the barrier that ends it; the slab of
// the next (chunk, kd) is fetched during the first step of the current one
// and written before its last step's closing barrier.  Fragments of the next
// block are read while the current block's MFMAs run.  LDS: slab position o
// of row r at (34 r + o) * 64 bytes, filter row kw NB + n at (kw NB + n) * 64,
// their four 16-byte pieces XOR-swizzled by bits 2..3 of o (of the row), so
// that 16 lanes reading 16 consecutive positions hit distinct bank groups.
//
// Epilogue: one output row of the tile (32 outputs x C_out channels when one
// column tile covers C_out) is contiguous in y.  Each wave writes its four
// rows into LDS exactly as they lie in y, shifted so that 16-byte boundaries
// of y and of LDS coincide, and stores aligned 16-byte pieces (element stores
// for the partial pieces at either end); with several column tiles the
// channels go out element by element.
#include <type_traits>

#include "conv_device.h"

namespace convfwd {

namespace {

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kSeg = 32;                            // outputs along w per tile row
constexpr int kRowsOut = 16;                        // output rows along h per tile
constexpr int kSW = kSeg + 2;                       // slab positions per row (K_w <= 3)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWave = kRowsOut / kWaves;        // output rows per wave
constexpr int kFA = 2 * kRowsWave;                  // A fragments per wave
constexpr int kBM = kSeg * kRowsOut;                // 512 GEMM rows
constexpr int kALoads = 10;                         // 16-byte slab pieces per thread: 40 wave loads of
                                                    // 16 positions cover 18 x 34
constexpr int kSlabBytes = kWaves * kALoads * 16 * 64;   // 40 KB a stage
constexpr int kLdsBytes = 160 * 1024;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

struct StagedArgs {
  TileArgs ta;
  int cmain;       // channels taken in 32-channel chunks (C_in rounded down to a multiple of 8)
  int nch;         // chunks: ceil(cmain / 32)
  int rp;          // channels past cmain (C_in mod 8)
  int npe;         // packed entries: taps * rp (at most 32)
  uint32_t m_rp;   // div_magic(rp)
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// physical 16-byte piece of logical piece c at slab position o (or filter row o)
__device__ __forceinline__ int swz(int o, int c) { return c ^ ((o >> 2) & 3); }

template <typename T, int KW, int KH, int NB>
__global__ __launch_bounds__(kThreads, 1) void conv_staged_kernel(ConvParams p, const T* __restrict__ x,
                                                             const T* __restrict__ w, T* __restrict__ y,
                                                             StagedArgs sa) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  static_assert(NB % 16 == 0 && NB >= 16 && NB <= 80, "channels per tile");
  static_assert(KW >= 2 && KW <= 3 && KH >= 2 && KH <= 3, "filter extents");
  constexpr int NF = NB / 16;                      // filter fragments per block
  constexpr int B_ROWS = KW * NB;                  // filter rows per step
  constexpr int B_BYTES = B_ROWS * 64;
  constexpr int B_PIECES = B_ROWS * 4;             // a multiple of 64
  constexpr int B_LOADS = (B_PIECES + kThreads - 1) / kThreads;
  constexpr int F_BASE = 2 * kSlabBytes;
  constexpr int PK_A = F_BASE + 2 * B_BYTES;       // the packed block: input side
  constexpr int PK_B = PK_A + kBM * 64;            //   and filter side
  constexpr int RING = PK_B + NB * 64;
  constexpr int PA_PER = kBM * 32 / kThreads;      // packed input-side entries per thread
  constexpr int PB_PER = NB * 32 / kThreads;       // packed filter-side entries per thread
  constexpr int SEGB = 64 * NB + 16;               // one output row as laid out in y, plus the lead
  constexpr int OUT = kRowsOut * SEGB;
  constexpr int SMEM = RING > OUT ? RING : OUT;
  static_assert(SMEM <= kLdsBytes, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileArgs& ta = sa.ta;
  // tile: column tiles fastest, then w-block, h-block, depth, image
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  int t = fast_div(tile, ta.tiles_n, ta.m_tn);
  const int n0 = (tile - t * ta.tiles_n) * NB;
  int t2 = fast_div(t, ta.wblocks, ta.m_wb);
  const int ow0 = (t - t2 * ta.wblocks) * kSeg;
  t = fast_div(t2, ta.hblocks, ta.m_hb);
  const int oh0 = (t2 - t * ta.hblocks) * kRowsOut;
  const int img = fast_div(t, p.od, ta.m_od);
  const int od = t - img * p.od;
  const int z0 = od * p.sd - p.pd;
  const int y0 = oh0 - p.ph;
  const int x0 = ow0 - p.pw;

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)ta.x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)ta.w_bytes, kRawBufferFlags);

  const uint32_t dmask = depth_mask(z0, p.kd, p.d, p.ed);
  const uint32_t ubase = (uint32_t)((img * p.xs_n + z0 * p.xs_d + y0 * p.xs_h + x0 * p.xs_w) * 2);
  const unsigned rowB = (unsigned)p.xs_h * 2, posB = (unsigned)p.xs_w * 2;
  const unsigned K2 = (unsigned)p.K * 2, cin2 = (unsigned)p.cin * 2;

  // ---- slab loader: wave load i = 4 q + wave covers positions 16 i .. + 15,
  // four lanes a position, one 16-byte piece each.  A piece is fetched if its
  // position lies inside the input (depth: bit kd of a_mask) and its 8
  // channels lie below cmain (its logical piece in bits 16.. of a_mask). ----
  uint32_t a_base[kALoads], a_mask[kALoads];
#pragma unroll
  for (int q = 0; q < kALoads; ++q) {
    const int pos = (kWaves * q + wave) * 16 + (lane >> 2);
    const int r = div_small<kSW>(pos), o = pos - r * kSW;
    const int c = swz(o, lane & 3);
    const bool ok = r < kRowsOut + KH - 1 && o < kSeg + KW - 1 && (unsigned)(y0 + r) < (unsigned)p.h &&
                    (unsigned)(x0 + o) < (unsigned)p.w;
    a_base[q] = ubase + __umul24((unsigned)r, rowB) + __umul24((unsigned)o, posB) + c * 16;
    a_mask[q] = (ok ? dmask : 0u) | ((uint32_t)c << 16);
  }
  // ---- filter loader: piece j = 256 s + tid -> (tap kw, row n, physical piece) ----
  uint32_t b_base[B_LOADS];
  int b_pc[B_LOADS];
#pragma unroll
  for (int s = 0; s < B_LOADS; ++s) {
    const int j = s * kThreads + tid;
    const int row = j >> 2, phys = j & 3;          // row = kw * NB + n
    const int kw = row / NB, n = row - kw * NB;
    const int c = swz(row, phys);
    const bool ok = j < B_PIECES && n0 + n < p.cout;
    b_base[s] = __umul24((unsigned)(n0 + n), K2) + __umul24((unsigned)kw, cin2) + c * 16;
    b_pc[s] = ok ? c : (1 << 20);                  // past any cmain (< 2^23): never fetched
  }

  u4 sreg[kALoads], freg[B_LOADS];
  const int NG = sa.nch * p.kd;                    // slabs (chunk, kd), kd fastest
  // Past the last slab or step the loads fetch nothing (zeros, never written).
  int a_ic = 0, a_kd = 0;
  auto issue_a = [&](int q0, int q1) __attribute__((always_inline)) {
    const int lim = sa.cmain - 32 * a_ic;
    const uint32_t xoff = (uint32_t)((a_kd * p.ed * p.xs_d + a_ic * 32) * 2);
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      // offsets of wanted pieces are below 2^31; bit 31 makes the others out of range
      const bool ok = ((a_mask[q] >> a_kd) & 1u) != 0u && (int)((a_mask[q] >> 13) & 0x18u) + 8 <= lim;
      sreg[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (a_base[q] + xoff) | ((uint32_t)!ok << 31), 0, 0);
    }
    if (q1 == kALoads) {
      const int d1 = a_kd + 1;
      const bool wrap = d1 == p.kd;
      a_kd = wrap ? 0 : d1;
      a_ic += (int)wrap;
    }
  };
  auto write_a = [&](int stage, int q0, int q1) __attribute__((always_inline)) {
    char* sa_ = smem + stage * kSlabBytes;
#pragma unroll
    for (int q = q0; q < q1; ++q) *(u4*)(sa_ + (kWaves * q + wave) * 1024 + lane * 16) = sreg[q];
  };
  int b_ic = 0, b_kd = 0, b_kh = 0;                // next filter step: kh fastest
  auto issue_b = [&]() __attribute__((always_inline)) {
    const int lim = sa.cmain - 32 * b_ic;
    const uint32_t woff = (uint32_t)((((b_kd * KH + b_kh) * KW) * p.cin + b_ic * 32) * 2);
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      if ((s + 1 < B_LOADS || B_PIECES % kThreads == 0) || s * kThreads + wave * 64 < B_PIECES)
        freg[s] = __builtin_amdgcn_raw_buffer_load_b128(
            wr, (b_base[s] + woff) | ((uint32_t)(8 * b_pc[s] + 8 > lim) << 31), 0, 0);
    const int h1 = b_kh + 1;
    const bool wh = h1 == KH;
    b_kh = wh ? 0 : h1;
    const int d1 = b_kd + (int)wh;
    const bool wd = d1 == p.kd;
    b_kd = wd ? 0 : d1;
    b_ic += (int)wd;
  };
  auto write_b = [&](int stage) __attribute__((always_inline)) {
    char* sb = smem + F_BASE + stage * B_BYTES;
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      if ((s + 1 < B_LOADS || B_PIECES % kThreads == 0) || s * kThreads + wave * 64 < B_PIECES)
        *(u4*)(sb + (s * kThreads + tid) * 16) = freg[s];
  };

  // ---- fragment addresses: lane (rr = lane % 16, g = lane / 16) reads piece g
  // of slab position 16 (a % 2) + rr + kw in slab row 4 wave + a / 2 + kh (A
  // fragment a), and of filter row kw NB + 16 b + rr (B fragment b). ----
  const int rr = lane & 15, g = lane >> 4;
  int a_addr[KW];
#pragma unroll
  for (int kw = 0; kw < KW; ++kw) a_addr[kw] = (kRowsWave * wave * kSW + rr + kw) * 64 + swz(rr + kw, g) * 16;
  const int b_addr = rr * 64 + swz(rr, g) * 16;

  f32x4_t acc[kFA][NF];
#pragma unroll
  for (int a = 0; a < kFA; ++a)
#pragma unroll
    for (int b = 0; b < NF; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mma_block = [&](const V8(&af)[kFA], const V8(&bf)[NF]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < kFA; ++a)
#pragma unroll
      for (int b = 0; b < NF; ++b) acc[a][b] = mfma16x16x32(bf[b], af[a], acc[a][b]);
  };

  // ---- prologue: the loads of slab 0 and of the filter of step 0 go out,
  // then the packed block is gathered element by element into its own LDS
  // area (the input side as 512 rows x 32 entries laid out and swizzled like
  // slab positions, the filter side as NB rows x 32 entries); its MFMAs run
  // after the K loop, so that no accumulator is live while the gathers are.
  // Thread t gathers entry t % 32 of rows t / 32 + 8 i: its tap and channel
  // are fixed. ----
  if (NG > 0) {
    issue_a(0, kALoads);
    issue_b();
  }
  const bool packed = sa.npe > 0;
  if (packed) {
    const int el = tid & 31, r0 = tid >> 5;
    const int tt = min(fast_div(el, sa.rp, sa.m_rp), p.ntaps - 1);   // entries past npe: any tap
    const int c = sa.cmain + el - tt * sa.rp;
    const int kw = tt % KW, t1 = tt / KW;
    const int kh = t1 % KH, kd = t1 / KH;
    const bool live = el < sa.npe;
    const uint32_t toff = (uint32_t)((kd * p.ed * p.xs_d + kh * p.xs_h + kw * p.xs_w + c) * 2);
    const bool dok = live && ((dmask >> kd) & 1u) != 0u;
    uint32_t hv[PA_PER], hw[PB_PER];
#pragma unroll
    for (int i = 0; i < PA_PER; ++i) {
      const int row = r0 + 8 * i, th = row >> 5, pos = row & 31;
      const bool ok = dok && (unsigned)(y0 + th + kh) < (unsigned)p.h && (unsigned)(x0 + pos + kw) < (unsigned)p.w;
      const uint32_t off = ubase + __umul24((unsigned)th, rowB) + __umul24((unsigned)pos, posB) + toff;
      hv[i] = __builtin_amdgcn_raw_buffer_load_b16(xr, off | ((uint32_t)!ok << 31), 0, 0);
    }
    const uint32_t woffe = (uint32_t)((tt * p.cin + c) * 2);
#pragma unroll
    for (int i = 0; i < PB_PER; ++i) {
      const int n = n0 + r0 + 8 * i;
      const bool ok = live && n < p.cout;
      hw[i] = __builtin_amdgcn_raw_buffer_load_b16(wr, (__umul24((unsigned)n, K2) + woffe) | ((uint32_t)!ok << 31),
                                                   0, 0);
    }
#pragma unroll
    for (int i = 0; i < PA_PER; ++i) {
      const int row = r0 + 8 * i;
      *(uint16_t*)(smem + PK_A + row * 64 + swz(row, el >> 3) * 16 + (el & 7) * 2) = (uint16_t)hv[i];
    }
#pragma unroll
    for (int i = 0; i < PB_PER; ++i) {
      const int row = r0 + 8 * i;
      *(uint16_t*)(smem + PK_B + row * 64 + swz(row, el >> 3) * 16 + (el & 7) * 2) = (uint16_t)hw[i];
    }
    if (NG == 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if (NG > 0) {
    wait_vmcnt<0>();
    write_a(0, 0, kALoads);
    write_b(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue_b();                                     // filter of step 1
    // block kw of every step computes on fragment set kw and reads the next
    // block's set meanwhile (the last block: the next step's set 0)
    V8 fa[KW][kFA], fb[KW][NF];
    auto read_block = [&](V8(&af)[kFA], V8(&bf)[NF], const char* sa_, const char* sb, int kw)
        __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < kFA; ++a) af[a] = *(const V8*)(sa_ + a_addr[kw] + ((a >> 1) * kSW + 16 * (a & 1)) * 64);
#pragma unroll
      for (int b = 0; b < NF; ++b) bf[b] = *(const V8*)(sb + b_addr + (kw * NB + 16 * b) * 64);
    };
    read_block(fa[0], fb[0], smem, smem + F_BASE, 0);
    int fs = 0;                                    // filter stage of the step being computed
    // Step kh of slab g: K_w blocks.  The step fetches its share of the next
    // slab's pieces (in the shadow of its first blocks) and the filter of the
    // next step; its last block writes both to LDS, passes the barrier and
    // reads the next step's first fragments before its MFMAs.
    auto plane = [&](int gi, auto final_c) __attribute__((always_inline)) {
      constexpr bool kFinal = decltype(final_c)::value;
      const char* sa0 = smem + (gi & 1) * kSlabBytes;
      const char* sn = smem + ((gi + 1) & 1) * kSlabBytes;
      static_for<0, KH>([&](auto khc) __attribute__((always_inline)) {
        constexpr int kh = decltype(khc)::value;
        constexpr bool kLastStep = kFinal && kh + 1 == KH;
        constexpr int q0 = kh * kALoads / KH, q1 = (kh + 1) * kALoads / KH;   // this step's slab pieces
        const char* sak = sa0 + kh * kSW * 64;
        const char* sb = smem + F_BASE + fs * B_BYTES;
        const char* nak = kh + 1 < KH ? sa0 + (kh + 1) * kSW * 64 : sn;
        const char* nb = smem + F_BASE + (fs ^ 1) * B_BYTES;
        static_for<0, KW>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          constexpr int cur = j, nxt = j + 1 < KW ? j + 1 : 0;
          if constexpr (j + 1 < KW) {
            read_block(fa[nxt], fb[nxt], sak, sb, j + 1);
            if constexpr (!kLastStep) issue_a(q0 + j * (q1 - q0) / (KW - 1), q0 + (j + 1) * (q1 - q0) / (KW - 1));
            mma_block(fa[cur], fb[cur]);
            __builtin_amdgcn_sched_barrier(0);
          } else if constexpr (!kLastStep) {
            wait_vmcnt<0>();
            write_b(fs ^ 1);
            write_a((gi + 1) & 1, q0, q1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            read_block(fa[nxt], fb[nxt], nak, nb, 0);
            issue_b();                             // the step after next
            mma_block(fa[cur], fb[cur]);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            mma_block(fa[cur], fb[cur]);
          }
        });
        fs ^= 1;
      });
    };
    for (int gi = 0; gi + 1 < NG; ++gi) plane(gi, std::false_type{});
    plane(NG - 1, std::true_type{});
  }

  // ---- the packed block (its LDS area was written before the first barrier) ----
  if (packed) {
    V8 pa[kFA], pw[NF];
#pragma unroll
    for (int a = 0; a < kFA; ++a) {
      const int row = (kRowsWave * wave + (a >> 1)) * 32 + 16 * (a & 1) + rr;
      pa[a] = *(const V8*)(smem + PK_A + row * 64 + swz(row, g) * 16);
    }
#pragma unroll
    for (int b = 0; b < NF; ++b) pw[b] = *(const V8*)(smem + PK_B + b_addr + 16 * b * 64);
    mma_block(pa, pw);
  }

  // ---- epilogue ----
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ta.tiles_n == 1) {
    // Row th of the tile: outputs ow0 .. ow0 + nv - 1 of output row oh0 + th,
    // nv * C_out contiguous elements of y starting at byte address ga; in LDS
    // at seg + lead + the same byte offset, lead = ga % 16.
    const int nv = min(kSeg, p.ow - ow0);
#pragma unroll
    for (int hi = 0; hi < kRowsWave; ++hi) {
      const int th = kRowsWave * wave + hi;
      if (oh0 + th >= p.oh) continue;
      const int64_t m = ((int64_t)(img * p.od + od) * p.oh + oh0 + th) * p.ow + ow0;
      const int lead = (int)((uintptr_t)(y + m * p.cout) & 15);
      char* seg = smem + th * SEGB + lead;
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = 2 * hi + ah;
        const int pos = 16 * ah + rr;
        if (pos < nv) {
#pragma unroll
          for (int b = 0; b < NF; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int n = 16 * b + 4 * g + i;
              if (n < p.cout) *(T*)(seg + 2 * (pos * p.cout + n)) = from_f32<T>(acc[a][b][i]);
            }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's rows, read back by this wave
#pragma unroll
    for (int hi = 0; hi < kRowsWave; ++hi) {
      const int th = kRowsWave * wave + hi;
      if (oh0 + th >= p.oh) continue;
      const int64_t m = ((int64_t)(img * p.od + od) * p.oh + oh0 + th) * p.ow + ow0;
      char* ga = (char*)(y + m * p.cout);
      const int lead = (int)((uintptr_t)ga & 15);
      char* gbase = ga - lead;
      const int span = lead + 2 * nv * p.cout;
      const char* seg = smem + th * SEGB;
      for (int k = lane; 16 * k < span; k += 64) {
        const u4 v = *(const u4*)(seg + 16 * k);
        if (16 * k >= lead && 16 * k + 16 <= span) {
          store16_nt(gbase + 16 * k, v);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int bo = 16 * k + 2 * e;
            if (bo >= lead && bo < span)
              *(uint16_t*)(gbase + bo) = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int a = 0; a < kFA; ++a) {
      const int th = kRowsWave * wave + (a >> 1), pos = 16 * (a & 1) + rr;
      if (oh0 + th >= p.oh || ow0 + pos >= p.ow) continue;
      const int64_t m = ((int64_t)(img * p.od + od) * p.oh + oh0 + th) * p.ow + ow0 + pos;
      T* yrow = y + m * p.cout;
#pragma unroll
      for (int b = 0; b < NF; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n0 + 16 * b + 4 * g + i;
          if (n < p.cout) yrow[n] = from_f32<T>(acc[a][b][i]);
        }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int KW, int KH, int NB>
hipError_t launch_k(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  StagedArgs sa;
  TileArgs& ta = sa.ta;
  ta.tiles_n = (p.cout + NB - 1) / NB;
  ta.wblocks = (p.ow + kSeg - 1) / kSeg;
  ta.hblocks = (p.oh + kRowsOut - 1) / kRowsOut;
  ta.m_tn = div_magic(ta.tiles_n);
  ta.m_wb = div_magic(ta.wblocks);
  ta.m_hb = div_magic(ta.hblocks);
  ta.m_od = div_magic(p.od);
  ta.x_bytes = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  ta.w_bytes = (uint32_t)((int64_t)p.cout * p.K * 2);
  sa.rp = p.cin % 8;
  sa.cmain = p.cin - sa.rp;
  sa.nch = (sa.cmain + 31) / 32;
  sa.npe = p.ntaps * sa.rp;
  sa.m_rp = div_magic(sa.rp);
  const int tiles_m = p.n * p.od * ta.hblocks * ta.wblocks;
  hipLaunchKernelGGL((conv_staged_kernel<T, KW, KH, NB>), dim3(tiles_m * ta.tiles_n), dim3(kThreads), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, sa);
  return hipGetLastError();
}

// Columns per tile: C_out rounded up to 32, 64 or 80 when it is at most 80;
// beyond, whichever of 64 and 80 pads C_out less.
template <typename T, int KW, int KH>
hipError_t launch_nb(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  if (p.cout <= 32) return launch_k<T, KW, KH, 32>(p, x, w, y, s);
  if (p.cout <= 64) return launch_k<T, KW, KH, 64>(p, x, w, y, s);
  if (p.cout <= 80 || (p.cout + 79) / 80 * 80 < (p.cout + 63) / 64 * 64) return launch_k<T, KW, KH, 80>(p, x, w, y, s);
  return launch_k<T, KW, KH, 64>(p, x, w, y, s);
}

template <typename T, int KH>
hipError_t launch_kh(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  return p.kw == 2 ? launch_nb<T, 2, KH>(p, x, w, y, s) : launch_nb<T, 3, KH>(p, x, w, y, s);
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  return p.kh == 2 ? launch_kh<T, 2>(p, x, w, y, s) : launch_kh<T, 3>(p, x, w, y, s);
}

}  // namespace

bool staged_accepts(const ConvParams& p, int dtype) {
  const int64_t tiles = (int64_t)p.n * p.od * ((p.oh + kRowsOut - 1) / kRowsOut) * ((p.ow + kSeg - 1) / kSeg) *
                        ((p.cout + 31) / 32);
  return (dtype == kF16 || dtype == kBF16) && p.remap == 0 && p.groups == 1 && p.sh == 1 && p.sw == 1 &&
         p.eh == 1 && p.ew == 1 && p.kh >= 2 && p.kh <= 3 && p.kw >= 2 && p.kw <= 3 && p.kd <= 16 &&
         (int64_t)p.ntaps * (p.cin % 8) <= 32 &&
         // 32-bit buffer offsets, the set-up's 24-bit multiplies and tile decode
         (int64_t)p.n * p.xs_n * 2 < ((int64_t)1 << 31) && (int64_t)p.cout * p.K * 2 < ((int64_t)1 << 31) &&
         (int64_t)p.xs_h * 2 < (1 << 24) && (int64_t)p.K * 2 < (1 << 24) && tiles < (1 << 24);
}

hipError_t launch_staged(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                         hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
