// k_staged.hip -- the slab scheme for channel counts that are not a multiple
// of 32, and for tensors that are aligned to their element size only
// (fp16/bf16, one group, unit stride and no dilation along h and w, K_h and
// K_w in {2, 3}; C_in >= 8 with (C_in mod 8) * K_d * K_h * K_w <= 32, and
// K_d <= 3 when C_in mod 8 != 0).
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
//    packed into one more K block.  Its input side comes from the 16 bytes
//    that end every slab position (fetched with the slab of each depth tap
//    of the last chunk), gathered element by element into fragments during
//    the last slab; its filter side is fetched element by element at the
//    start.
// On (4, 32^3, 65 -> 65) the depth is 2 x 27 chunk blocks + 1 packed block
// (1760 columns for 1755) where 32-channel padding would take 81 blocks.
//
// Tile: 16 output rows x 32 outputs along w (512 GEMM rows, one depth plane of
// one image; rows past the output's end are computed on zeros and not
// stored) x NB output channels, NB in {32, 64, 80}, so that C_out = 65 runs on
// 80 columns.  Eight waves, two per SIMD: wave v owns output rows 2v, 2v + 1
// of the tile (4 fragments of 16 outputs) x all NB channels, v_mfma_f32_
// 16x16x32 blocks with the filter as the first operand, so a lane receives 4
// consecutive channels of one output.  Per K block a wave reads 4 + NB/16
// fragments (1 KB each) for 4 NB/16 MFMAs.  A wave then fits in 256
// registers (249 for the 3x3x3 instance with 80 columns; the K_h = 2, K_w = 3,
// 80-column one spills two), and the second wave on each SIMD covers the
// other's waits, which one wave per SIMD left exposed: against four waves of
// four rows (one per SIMD, ~500 registers) this runs 4-21% faster on every
// shape timed, C_in = 65 (4, 32^3) 44.4 -> 38.9 us, with identical results.
// The kernel keeps the wave count as a parameter (4 or 8).
//
// Pipeline, per K step (chunk, kd, kh) of K_w blocks: the filter slice of
// step t is fetched into registers (one of K_h sets) after the barrier that
// ends step t - 3 and written to its LDS stage before the barrier that ends
// step t - 1; the pieces of the next (chunk, kd) slab are fetched during the
// steps before a slab's last and written before its closing barrier.  The
// next block's fragment reads are interleaved one after every second MFMA of
// the current block (every third with four waves; the scheduler would
// otherwise issue them in one burst).  LDS: slab position o
// of row r at (34 r + o) * 64 bytes, filter row kw NB + n at (kw NB + n) * 64,
// their four 16-byte pieces XOR-swizzled by bits 1..2 of o (of the row).  A
// 16x16x32 operand read has lanes l and l + 16 fetch other pieces of the same
// 16 positions; measured with a read-only probe, this swizzle serves that
// pattern at the full LDS rate (~200 B/clk per CU), where the bits 2..3
// swizzle that suits the 32x32x16 operand of the slab kernel gets ~125.
//
// Epilogue: one output row of the tile (32 outputs x C_out channels when one
// column tile covers C_out) is contiguous in y.  Each wave writes its
// rows into LDS exactly as they lie in y, shifted so that 16-byte boundaries
// of y and of LDS coincide, and stores aligned 16-byte pieces (element stores
// for the partial pieces at either end); with several column tiles the
// channels go out element by element.
#include <type_traits>

#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kSeg = 32;                            // outputs along w per tile row
constexpr int kRowsOut = 16;                        // output rows along h per tile
constexpr int kSW = kSeg + 2;                       // slab positions per row (K_w <= 3)
constexpr int kBM = kSeg * kRowsOut;                // 512 GEMM rows
constexpr int kSlabLoads = 40;                      // wave loads of 16 positions per slab stage
                                                    // (40 x 16 positions cover 18 x 34)
constexpr int kSlabBytes = kSlabLoads * 16 * 64;    // 40 KB a stage
constexpr int kRemLoads = 12;                       // wave loads of 64 positions per REM plane
                                                    // (768 slots, 612 used)
constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxPackKd = 3;                       // depth taps with leftover channels

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
__device__ __forceinline__ int swz(int o, int c) { return c ^ ((o >> 1) & 3); }

template <typename T, int KW, int KH, int NB, int W>
__global__ __launch_bounds__(64 * W, 1) void conv_staged_kernel(ConvParams p, const T* __restrict__ x,
                                                             const T* __restrict__ w, T* __restrict__ y,
                                                             StagedArgs sa) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  static_assert(NB % 16 == 0 && NB >= 16 && NB <= 80, "channels per tile");
  static_assert(KW >= 2 && KW <= 3 && KH >= 2 && KH <= 3, "filter extents");
  static_assert(W == 4 || W == 8, "waves");
  constexpr int kWaves = W;
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRowsWave = kRowsOut / kWaves;     // output rows per wave
  constexpr int kFA = 2 * kRowsWave;               // A fragments per wave
  constexpr int kALoads = kSlabLoads / kWaves;     // slab pieces per thread
  constexpr int NF = NB / 16;                      // filter fragments per block
  constexpr int B_ROWS = KW * NB;                  // filter rows per step
  constexpr int B_BYTES = B_ROWS * 64;
  constexpr int B_PIECES = B_ROWS * 4;             // a multiple of 64
  constexpr int B_LOADS = (B_PIECES + kThreads - 1) / kThreads;
  constexpr int F_BASE = 2 * kSlabBytes;
  // The packed block's inputs land through direct-to-LDS loads: PK_B, its
  // filter side (NB rows x 32 entries, 2-byte loads, each lane's element
  // written as a zero-extended 4-byte word), and REM, per kd plane (at most
  // 3) and slab position the 16 bytes that end the position, its last 8
  // channels, the leftover ones among them (16-byte loads, a position a lane).
  constexpr int PK_B = F_BASE + 2 * B_BYTES;
  constexpr int PB_PER = NB * 32 / kThreads;       // filter-side entries per thread
  constexpr int REM = PK_B + NB * 32 * 4;
  constexpr int REM_SLOTS = kRemLoads * 64;        // slab positions (612 used) per kd plane
  constexpr int REM_PER = (kRemLoads + kWaves - 1) / kWaves;   // REM loads per thread and plane
  // With eight waves the 12 wave loads of a plane leave 4 spare ones in the
  // last round: they load nothing (out of range) into a 1 KB dummy area, so
  // that every wave issues the same number of loads and the waits can count
  // them.
  constexpr bool REM_SPARE = REM_PER * kWaves > kRemLoads;
  constexpr int R_LOADS = PB_PER;                  // filter-side element loads per thread
  constexpr int REM_DUMMY = REM + kMaxPackKd * REM_SLOTS * 16;
  constexpr int RING = REM_DUMMY + (REM_SPARE ? 1024 : 0);
  constexpr int SEGB = 64 * NB + 16;               // one output row as laid out in y, plus the lead
  constexpr int DUMMY = kRowsOut * SEGB;            // 64 dummy element slots
  constexpr int OUT = DUMMY + 128;
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

  // The filter slice of step t goes out after the barrier that ends step
  // t - 3, into register set t % KH, and is written to LDS before the barrier
  // that ends step t - 1; the next slab's pieces go out during the steps
  // before a slab's last and are written before its closing barrier.
  // Every wave issues the same number of loads (its share, or out-of-range
  // ones past the end), so the waits can count them.
  u4 sreg[kALoads], freg[KH][B_LOADS];
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
  auto write_a = [&](int stage) __attribute__((always_inline)) {
    char* sa_ = smem + stage * kSlabBytes;
#pragma unroll
    for (int q = 0; q < kALoads; ++q) *(u4*)(sa_ + (kWaves * q + wave) * 1024 + lane * 16) = sreg[q];
  };
  int b_ic = 0, b_kd = 0, b_kh = 0;                // next filter step: kh fastest
  auto issue_b = [&](u4(&fr)[B_LOADS]) __attribute__((always_inline)) {
    const int lim = sa.cmain - 32 * b_ic;
    const uint32_t woff = (uint32_t)((((b_kd * KH + b_kh) * KW) * p.cin + b_ic * 32) * 2);
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      fr[s] = __builtin_amdgcn_raw_buffer_load_b128(wr, (b_base[s] + woff) | ((uint32_t)(8 * b_pc[s] + 8 > lim) << 31),
                                                    0, 0);
    const int h1 = b_kh + 1;
    const bool wh = h1 == KH;
    b_kh = wh ? 0 : h1;
    const int d1 = b_kd + (int)wh;
    const bool wd = d1 == p.kd;
    b_kd = wd ? 0 : d1;
    b_ic += (int)wd;
  };
  auto write_b = [&](const u4(&fr)[B_LOADS], int stage) __attribute__((always_inline)) {
    char* sb = smem + F_BASE + stage * B_BYTES;
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      if ((s + 1 < B_LOADS || B_PIECES % kThreads == 0) || s * kThreads + wave * 64 < B_PIECES)
        *(u4*)(sb + (s * kThreads + tid) * 16) = fr[s];
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

  // ---- prologue: slab 0 (with its REM plane), the filter slices of steps 0
  // and 1, the packed block's filter-side loads (PK_B entry e of filter row n
  // at 32 n + e) and the filter of step 2; slab 0 and the first filter land
  // before the first barrier. ----
  const bool packed = sa.npe > 0;
  // REM loads of the slab about to be fetched (a_ic, a_kd): live in the last
  // channel chunk (out of range otherwise, so that every slab issues them).
  const uint32_t rtail = (uint32_t)(2 * p.cin - 16);
  uint32_t r_base[REM_PER];
#pragma unroll
  for (int i = 0; i < REM_PER; ++i) {
    const int wl = i * kWaves + wave, pos = wl * 64 + lane, r = pos / kSW, o = pos - r * kSW;
    const bool ok = packed && wl < kRemLoads && r < kRowsOut + KH - 1 && o < kSeg + KW - 1 && (unsigned)(y0 + r) < (unsigned)p.h &&
                    (unsigned)(x0 + o) < (unsigned)p.w;
    r_base[i] = ok ? ubase + __umul24((unsigned)r, rowB) + __umul24((unsigned)o, posB) + rtail : kOutOfRange;
  }
  auto issue_rem = [&]() __attribute__((always_inline)) {
    const bool live = a_ic == sa.nch - 1 && ((dmask >> a_kd) & 1u) != 0u;
    const uint32_t zoff = (uint32_t)(a_kd * p.ed * p.xs_d * 2);
#pragma unroll
    for (int i = 0; i < REM_PER; ++i) {
      const int wl = i * kWaves + wave;             // wave-uniform
      char* dst = (!REM_SPARE || wl < kRemLoads)
                      ? smem + REM + (min(a_kd, kMaxPackKd - 1) * REM_SLOTS + wl * 64) * 16
                      : smem + REM_DUMMY;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, live ? r_base[i] + zoff : kOutOfRange, 0, 0,
                                               0);
    }
  };
  issue_rem();
  issue_a(0, kALoads);
  issue_b(freg[0]);
  issue_b(freg[1 % KH]);
  // The packed block's filter-side load i, out of range when not packed.
  auto issue_r = [&](int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      {
        const int el = tid & 31, n = n0 + (tid >> 5) + (kThreads / 32) * i;
        const int tt = min(fast_div(el, sa.rp, sa.m_rp), p.ntaps - 1);   // entries past npe: any tap
        const uint32_t woffe = (uint32_t)((tt * p.cin + sa.cmain + el - tt * sa.rp) * 2);
        const bool ok = packed && el < sa.npe && n < p.cout;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(smem + PK_B + (i * kThreads + wave * 64) * 4), 2,
                                                 (__umul24((unsigned)n, K2) + woffe) | ((uint32_t)!ok << 31), 0, 0, 0);
      }
    }
  };
  issue_r(0, R_LOADS);
  wait_vmcnt<B_LOADS + R_LOADS>();                 // all but the filter of step 1 and the filter-side loads
  write_a(0);
  write_b(freg[0], 0);
  issue_b(freg[2 % KH]);                           // (its set is free once step 0's is written)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  {
    // A block multiplies the fragments fa (input, one set, refilled with the
    // next block's fragment a right after fragment a's MFMAs are issued) and
    // fb[kw] (filter: block kw of every step uses set kw and reads the next
    // block's set, the last block the next step's set 0, before its MFMAs).
    V8 fa[kFA], fb[KW][NF];
    auto read_a = [&](const char* sa_, int kw, int a) __attribute__((always_inline)) {
      return *(const V8*)(sa_ + a_addr[kw] + ((a >> 1) * kSW + 16 * (a & 1)) * 64);
    };
    auto read_b = [&](V8(&bf)[NF], const char* sb, int kw) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < NF; ++b) bf[b] = *(const V8*)(sb + b_addr + (kw * NB + 16 * b) * 64);
    };
    // the MFMAs of a block on (fa, bf), fa refilled from (na, nkw); the next
    // block's fragment reads go out one after every third MFMA (left to
    // itself the scheduler issues them in one burst at the block's end, and
    // with one wave per SIMD the matrix unit then waits for LDS)
    auto mma_stream = [&](const V8(&bf)[NF], const char* na, int nkw) __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < kFA; ++a) {
#pragma unroll
        for (int b = 0; b < NF; ++b) acc[a][b] = mfma16x16x32(bf[b], fa[a], acc[a][b]);
        fa[a] = read_a(na, nkw, a);
      }
      constexpr int RI = kWaves == 8 ? 2 : 3;    // MFMAs per interleaved fragment read
#pragma unroll
      for (int i = 0; i < kFA * NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % RI == RI - 1 && i / RI < kFA + NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
#pragma unroll
    for (int a = 0; a < kFA; ++a) fa[a] = read_a(smem, 0, a);
    read_b(fb[0], smem + F_BASE, 0);
    // The packed block: its input-side fragments gathered from REM (lane
    // entries e = 8 g + j: tap e / rp, channel cmain + e % rp, element 8 - rp
    // + e % rp of the position's last 16 bytes), its filter side from PK_B.
    // Both are in LDS from the last slab on (its REM plane was fetched during
    // the slab before, PK_B in the prologue); the gathers go out in its first
    // step, the MFMAs follow its last block's.
    V8 pa[kFA], pw[NF];
    auto gather_pack = [&]() __attribute__((always_inline)) {
      int eoff[8];
      uint32_t elive = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 8 * g + j;
        const int tt = min(fast_div(e, sa.rp, sa.m_rp), p.ntaps - 1);
        const int c = e - tt * sa.rp;
        const int kw = tt % KW, t1 = tt / KW;
        const int kh = t1 % KH, kd = t1 / KH;
        eoff[j] = ((kd * REM_SLOTS + kh * kSW + kw) * 16) + (8 - sa.rp + c) * 2;
        elive |= (e < sa.npe ? 1u : 0u) << j;
      }
#pragma unroll
      for (int a = 0; a < kFA; ++a) {
        const int th = kRowsWave * wave + (a >> 1), pos = 16 * (a & 1) + rr;
        const char* base = smem + REM + (th * kSW + pos) * 16;
        u4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t lo = (elive >> (2 * d)) & 1u ? *(const uint16_t*)(base + eoff[2 * d]) : 0u;
          const uint32_t hi = (elive >> (2 * d + 1)) & 1u ? *(const uint16_t*)(base + eoff[2 * d + 1]) : 0u;
          v[d] = lo | (hi << 16);
        }
        pa[a] = __builtin_bit_cast(V8, v);
      }
#pragma unroll
      for (int b = 0; b < NF; ++b) {
        const char* row = smem + PK_B + (16 * b + rr) * 128 + g * 32;
        const u4 e0 = *(const u4*)row, e1 = *(const u4*)(row + 16);
        const u4 v = {(e0[0] & 0xffffu) | (e0[1] << 16), (e0[2] & 0xffffu) | (e0[3] << 16),
                      (e1[0] & 0xffffu) | (e1[1] << 16), (e1[2] & 0xffffu) | (e1[3] << 16)};
        pw[b] = __builtin_bit_cast(V8, v);
      }
    };
    int fs = 0;                                    // filter stage of the step being computed
    // Step kh of slab g: K_w blocks.  In the shadow of its first blocks the
    // step fetches its share of the next slab's pieces; its last block waits
    // for the next step's filter (closing a slab: and the next slab), writes
    // them to LDS, passes the barrier, reads the next step's first fragments
    // and fetches the filter three steps on before its MFMAs.
    auto plane = [&](int gi, auto final_c) __attribute__((always_inline)) {
      constexpr bool kFinal = decltype(final_c)::value;
      const char* sa0 = smem + (gi & 1) * kSlabBytes;
      const char* sn = smem + ((gi + 1) & 1) * kSlabBytes;
      static_for<0, KH>([&](auto khc) __attribute__((always_inline)) {
        constexpr int kh = decltype(khc)::value;
        constexpr bool kLastStep = kFinal && kh + 1 == KH;
        // slab pieces of this step: [q0, q1) (none in a slab's last step)
        constexpr int q0 = kh * kALoads / (KH - 1), q1 = kh + 1 < KH ? (kh + 1) * kALoads / (KH - 1) : q0;
        // loads the step issues ahead of the next slab: its pieces, and in the
        // first step the next slab's REM plane
        constexpr int nq = q1 - q0 + (kh == 0 ? REM_PER : 0);
        constexpr int qprev = kh == 0 ? 0 : q0 - (kh - 1) * kALoads / (KH - 1) + (kh == 1 ? REM_PER : 0);
        // loads newer than the next step's filter: the pieces of the step
        // before, the filter two steps on, this step's pieces; closing a slab
        // only that filter (the pieces all went out before it)
        constexpr int kNewer = kh + 1 == KH ? B_LOADS : (kFinal ? 0 : qprev + nq) + B_LOADS;
        const char* sak = sa0 + kh * kSW * 64;
        const char* sb = smem + F_BASE + fs * B_BYTES;
        const char* nak = kh + 1 < KH ? sa0 + (kh + 1) * kSW * 64 : sn;
        const char* nb = smem + F_BASE + (fs ^ 1) * B_BYTES;
        static_for<0, KW>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          constexpr int cur = j, nxt = j + 1 < KW ? j + 1 : 0;
          if constexpr (j + 1 < KW) {
            read_b(fb[nxt], sb, j + 1);
            if constexpr (!kFinal && kh == 0 && j == 0) issue_rem();
            if constexpr (kFinal && kh == 0 && j == 0) {
              if (packed) gather_pack();
            }
            if constexpr (!kFinal && q1 > q0) issue_a(q0 + j * (q1 - q0) / (KW - 1), q0 + (j + 1) * (q1 - q0) / (KW - 1));
            mma_stream(fb[cur], sak, j + 1);
            __builtin_amdgcn_sched_barrier(0);
          } else if constexpr (!kLastStep) {
            wait_vmcnt<kNewer>();
            write_b(freg[(kh + 1) % KH], fs ^ 1);
            if constexpr (kh + 1 == KH) write_a((gi + 1) & 1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            read_b(fb[nxt], nb, 0);
            issue_b(freg[(kh + 3) % KH]);          // three steps on (the set just written, for K_h = 2)
            mma_stream(fb[cur], nak, 0);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            mma_block(fa, fb[cur]);
            if (packed) mma_block(pa, pw);
          }
        });
        fs ^= 1;
      });
    };
    for (int gi = 0; gi + 1 < NG; ++gi) plane(gi, std::false_type{});
    plane(NG - 1, std::true_type{});
  }

  // ---- epilogue ----
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (ta.tiles_n == 1) {
    // Row th of the tile: outputs ow0 .. ow0 + nv - 1 of output row oh0 + th,
    // nv * C_out contiguous elements of y starting at byte address ga; in LDS
    // at seg + lead + the same byte offset, lead = ga % 16.
    // Without branches: an element that is no output (past C_out, or past
    // the output's end along w) goes to a dummy slot of its lane's own.
    const int nv = min(kSeg, p.ow - ow0);
    const bool all_pos = nv == kSeg;
#pragma unroll
    for (int hi = 0; hi < kRowsWave; ++hi) {
      const int th = kRowsWave * wave + hi;
      if (oh0 + th >= p.oh) continue;
      const int64_t m = ((int64_t)(img * p.od + od) * p.oh + oh0 + th) * p.ow + ow0;
      const int lead = (int)((uintptr_t)(y + m * p.cout) & 15);
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = 2 * hi + ah;
        const int pos = 16 * ah + rr;
        const uint32_t pbase = (uint32_t)(th * SEGB + lead + 2 * pos * p.cout + 8 * g);
        const bool pos_ok = pos < nv;
        // the lane's 4 channels start on a 4-byte boundary of LDS (and of y)
        // or 2 bytes past one: one aligned dword write and two 2-byte writes
        // either way (the dword holds channels 0-1 or 1-2 of the four)
        const bool odd = (((lead >> 1) + pos * p.cout) & 1) != 0;
#pragma unroll
        for (int b = 0; b < NF; ++b) {
          if (all_pos && 16 * b + 16 <= p.cout) {
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = __builtin_bit_cast(uint16_t, from_f32<T>(acc[a][b][i]));
            char* q = smem + pbase + 32 * b;
            *(uint32_t*)(q + (odd ? 2 : 0)) = odd ? (e[1] | (e[2] << 16)) : (e[0] | (e[1] << 16));
            *(uint16_t*)(q + (odd ? 0 : 4)) = (uint16_t)(odd ? e[0] : e[2]);
            *(uint16_t*)(q + 6) = (uint16_t)e[3];
          } else if (pos_ok && 16 * b + 4 * g < p.cout) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool ok = 16 * b + 4 * g + i < p.cout;
              *(T*)(smem + (ok ? pbase + 2 * (16 * b + i) : (uint32_t)(DUMMY + 2 * lane))) = from_f32<T>(acc[a][b][i]);
            }
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

template <typename T, int KW, int KH, int NB, int W>
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
  hipLaunchKernelGGL((conv_staged_kernel<T, KW, KH, NB, W>), dim3(tiles_m * ta.tiles_n), dim3(64 * W), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, sa);
  return hipGetLastError();
}

// Columns per tile: C_out rounded up to 32, 64 or 80 when it is at most 80;
// beyond, whichever of 64 and 80 pads C_out less.
template <typename T, int KW, int KH>
hipError_t launch_nb(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  constexpr int W = 8;   // waves per workgroup, two per SIMD
  if (p.cout <= 32) return launch_k<T, KW, KH, 32, W>(p, x, w, y, s);
  if (p.cout <= 64) return launch_k<T, KW, KH, 64, W>(p, x, w, y, s);
  if (p.cout <= 80 || (p.cout + 79) / 80 * 80 < (p.cout + 63) / 64 * 64) return launch_k<T, KW, KH, 80, W>(p, x, w, y, s);
  return launch_k<T, KW, KH, 64, W>(p, x, w, y, s);
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
         p.cin >= 8 && (int64_t)p.ntaps * (p.cin % 8) <= 32 && (p.cin % 8 == 0 || p.kd <= kMaxPackKd) &&
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
