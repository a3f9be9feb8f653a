// k_strip.hip -- implicit GEMM with the w-taps of a filter row read from one
// staged input strip (fp16/bf16, C_in % 32 == 0, unit stride along w,
// W_out % 32 == 0, K_w <= 5).
//
// In the classic implicit GEMM ("Convolutions" tutorial, section 5) the A
// tile of tap (kd, kh, kw+1) is the A tile of tap (kd, kh, kw) shifted by one
// position along w, yet each is gathered afresh.  Here a K step is one
// (channel chunk of 32, kd, kh): for each 32-output w-segment of the tile the
// workgroup stages the 32 + K_w - 1 input positions that segment needs (one
// "strip", padded to 36 positions, zeros outside the input) and forms the A
// operand of all K_w taps by reading the strip at offsets 0 .. K_w-1.  The
// filter slices of those K_w taps are staged beside it.  Input traffic through
// the caches drops K_w-fold (less the two halo positions per segment).
//
// Tile: 512 output rows = 16 w-segments of 32 (consecutive flat rows, which
// W_out % 32 == 0 makes whole segments) x 128 output channels.  Four waves,
// each owning 4 segments = 128 rows x 128 channels = 4 x 4 blocks of
// v_mfma_f32_32x32x16 (one wave per SIMD keeps the matrix unit busy with
// 32x32x16).  Per step each wave issues 96 MFMAs between barriers.
//
// LDS layout: strip position o of segment g at row (36 g + o), 64 bytes (32
// channels, four 16-byte chunks); the chunk index is XORed with bits 2..3 of o,
// so the 16 consecutive positions one 256-byte LDS pass serves land on 16
// distinct 16-byte slots for every tap offset.  Because the swizzle depends
// only on the position inside the segment, every fragment address is a
// per-lane constant (one per tap and k-half) plus an immediate.
// Loads are 16-byte buffer loads straight into LDS; a position in the padding
// gets an offset past the buffer end, which the range check turns into zeros.
//
// Pipeline (K_w <= 3, where three strip stages and two filter stages fit in
// LDS): the strip of step s+2 is issued in pieces from the MFMA blocks of step
// s and the filter slices of step s+2 right after the barrier that ends step
// s; both must land by the barrier that ends step s+1.  Spreading the strip
// loads over the step keeps their direct-to-LDS writes from arriving in one
// burst (they slow the fragment reads they overlap).  With K_w = 4, 5 there are
// two stages of each and all loads of step s+2 go out after that barrier.
// Fragments are double-buffered in registers, so a block's LDS reads run under
// the previous block's MFMAs.  The epilogue stages the tile through LDS so
// stores write whole 16-byte pieces of rows.
#include <type_traits>

#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kSeg = 32;                   // outputs per w-segment
constexpr int kSegs = 16;                  // segments per tile
constexpr int kBM = kSeg * kSegs;          // 512 rows
constexpr int kBN = 128;                   // output channels per tile
constexpr int kSW = 36;                    // strip positions per segment (32 + K_w - 1 <= 36)
constexpr int kMaxKW = kSW - kSeg + 1;     // 5
constexpr int kRowB = 64;                  // bytes per strip position / filter row (32 channels)
constexpr int kStripBytes = kSegs * kSW * kRowB;   // 36 KB
constexpr int kA_LOADS = kSegs * kSW / 16 / 4;     // 9 wave-instructions per wave per step
constexpr int kLdsBytes = 160 * 1024;              // LDS per workgroup on gfx950
constexpr int kOutRowB = kBN * 2;                  // one output row of the tile in LDS (256 bytes)
constexpr int kOutTileBytes = kBM * kOutRowB;      // 128 KB

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// physical 16-byte chunk of logical chunk c at strip position o (or filter row o)
__device__ __forceinline__ int swz(int o, int c) { return c ^ ((o >> 2) & 3); }

template <typename T, int KW>
__global__ __launch_bounds__(256, 1) void conv_strip_kernel(ConvParams p, const T* __restrict__ x,
                                                            const T* __restrict__ w,
                                                            T* __restrict__ y, int tiles_n,
                                                            uint32_t x_bytes, uint32_t w_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  constexpr int B_ROWS = KW * kBN;                 // filter rows per step
  constexpr int B_BYTES = B_ROWS * kRowB;
  constexpr int B_LOADS = B_ROWS * 4 / 256;        // 16-byte pieces per thread
  constexpr int NL = kA_LOADS + B_LOADS;
  static_assert(KW >= 1 && KW <= kMaxKW, "K_w");
  static_assert(NL < 64, "vmcnt");
  // LDS ring: A_ST strip stages, then two filter stages.  Three strip stages
  // (when they fit) give the strided input loads two steps of lead; the
  // filter slices, which every workgroup reads and the L2 keeps, get one.
  constexpr int A_ST = 3 * kStripBytes + 2 * B_BYTES <= kLdsBytes ? 3 : 2;
  constexpr int B_BASE = A_ST * kStripBytes;
  constexpr int RING = B_BASE + 2 * B_BYTES;
  static_assert(RING <= kLdsBytes, "LDS");
  constexpr int SMEM = RING > kOutTileBytes ? RING : kOutTileBytes;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * kBM;
  const int n0 = (tile % tiles_n) * kBN;

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)w_bytes, kRawBufferFlags);

  // ---- strip loader: wave instruction i = 4 q + wave fills positions
  // 16 i .. 16 i + 15 (four lanes each); this lane's position and chunk ----
  uint32_t a_base[kA_LOADS];   // byte offset of the piece at (kd, kh, chunk) = 0
  uint32_t a_mask[kA_LOADS];   // depth bits | height bits << 16; 0 if the position is empty
#pragma unroll
  for (int q = 0; q < kA_LOADS; ++q) {
    const int pos = (4 * q + wave) * 16 + (lane >> 2);
    const int g = pos / kSW, o = pos - (pos / kSW) * kSW;
    const int phys = lane & 3;
    const int c = swz(o, phys);                        // logical chunk this lane fetches
    const int m = m0 + g * kSeg;                       // first row of the segment
    uint32_t base = 0, mask = 0;
    if (o < kSeg + KW - 1 && m < p.M) {
      const int ow0 = m % p.ow;
      int t = m / p.ow;
      const int oh = t % p.oh;
      t /= p.oh;
      const int od = t % p.od;
      const int n = t / p.od;
      const int z0 = od * p.sd - p.pd, y0 = oh * p.sh - p.ph;
      const int iw = ow0 - p.pw + o;
      if (iw >= 0 && iw < p.w) {
        mask = dim_mask(z0, p.kd, p.d, p.ed) | (dim_mask(y0, p.kh, p.h, p.eh) << 16);
        base = (uint32_t)(((n * p.xs_n + z0 * p.xs_d + y0 * p.xs_h + iw * p.xs_w) + c * 8) * 2);
      }
    }
    a_base[q] = base;
    a_mask[q] = mask;
  }
  // ---- filter loader: piece j = 256 s + tid -> (tap kw, row n, physical chunk) ----
  uint32_t b_base[B_LOADS];
#pragma unroll
  for (int s = 0; s < B_LOADS; ++s) {
    const int j = s * 256 + tid;
    const int row = j >> 2, phys = j & 3;     // row = kw * 128 + n
    const int kw = row / kBN, n = row % kBN;
    const int c = swz(row, phys);
    b_base[s] = (n0 + n) < p.cout ? (uint32_t)(((n0 + n) * p.K + kw * p.cin + c * 8) * 2)
                                  : kOutOfRange;
  }

  const int nchunks = p.cin / 32;
  const int S = nchunks * p.kd * p.kh;
  // step order: kh fastest, then kd, then the channel chunk
  auto advance = [&](int& ic, int& kd, int& kh) {
    const int h1 = kh + 1;
    const bool wh = h1 == p.kh;
    kh = wh ? 0 : h1;
    const int d1 = kd + (int)wh;
    const bool wd = d1 == p.kd;
    kd = wd ? 0 : d1;
    ic += (int)wd;
  };
  // Past the last step every load zero-fills (bit masks, not branches), so the
  // issue code runs unconditionally.
  int a_ic = 0, a_kd = 0, a_kh = 0, a_slot = 0;   // next strip step to issue
  auto issue_a_part = [&](int q0, int q1) {
    char* sa = smem + a_slot * kStripBytes;
    const uint32_t live = a_ic < nchunks ? ~0u : 0u;
    const uint32_t xoff = (uint32_t)((a_kd * p.ed * p.xs_d + a_kh * p.eh * p.xs_h + a_ic * 32) * 2);
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      const bool ok = (((a_mask[q] & live) >> a_kd) & (a_mask[q] >> (16 + a_kh)) & 1u) != 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(sa + ((4 * q + wave) * 16) * kRowB), 16, ok ? a_base[q] + xoff : kOutOfRange,
          0, 0, 0);
    }
    if (q1 == kA_LOADS) {
      advance(a_ic, a_kd, a_kh);
      a_slot = a_slot + 1 == A_ST ? 0 : a_slot + 1;
    }
  };
  auto issue_a = [&]() { issue_a_part(0, kA_LOADS); };
  int b_ic = 0, b_kd = 0, b_kh = 0, b_slot = 0;   // next filter step to issue
  auto issue_b = [&]() {
    char* sb = smem + B_BASE + b_slot * B_BYTES;
    const uint32_t live = b_ic < nchunks ? ~0u : 0u;
    const uint32_t woff = (uint32_t)(((b_kd * p.kh + b_kh) * p.kw * p.cin + b_ic * 32) * 2);
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_ptr_t)(sb + (s * 256 + wave * 64) * 16), 16, (b_base[s] + woff) | (~live & kOutOfRange), 0,
          0, 0);
    advance(b_ic, b_kd, b_kh);
    b_slot ^= 1;
  };
  // loads a wave may still have in flight when it needs the next step: the
  // strip loads issued after that step's filter loads
  constexpr int WAIT_N = A_ST == 3 ? kA_LOADS : 0;
  // Loads issued at the step barrier: with three strip stages only the filter
  // slices (the strip loads are spread over the next step's blocks, which keeps
  // the direct-to-LDS writes from piling onto the fragment reads at one point).
  auto issue_ahead = [&]() {
    if constexpr (A_ST == 3) {
      issue_b();                           // filter: two steps ahead
    } else {
      issue_a();
      issue_b();
    }
  };

  // ---- fragment addresses: lane (r = lane % 32, g2 = lane / 32) ----
  const int r = lane & 31, g2 = lane >> 5;
  int a_addr[KW][2], b_addr[2];
#pragma unroll
  for (int kw = 0; kw < KW; ++kw)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o = r + kw;
      a_addr[kw][ks] = (wave * 4 * kSW + o) * kRowB + swz(o, 2 * ks + g2) * 16;
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) b_addr[ks] = r * kRowB + swz(r, 2 * ks + g2) * 16;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // A step is 2 K_w blocks (tap kw, k-half ks) of 16 MFMAs.  Fragments are
  // double-buffered in registers: block j+1 is read from LDS while block j's
  // MFMAs run.  The step's last block passes the barrier first (its own
  // fragments are already in registers), so the next step's first fragments
  // and the loads two steps ahead are issued under its MFMAs; the address
  // arithmetic of those loads is interleaved with the MFMAs.
  constexpr int NBLK = 2 * KW;
  V8 fa[2][4], fb[2][4];
  auto read_block = [&](V8(&af)[4], V8(&bf)[4], const char* sa, const char* sb, int kw, int ks) {
#pragma unroll
    for (int a = 0; a < 4; ++a) af[a] = *(const V8*)(sa + a_addr[kw][ks] + a * kSW * kRowB);
#pragma unroll
    for (int b = 0; b < 4; ++b) bf[b] = *(const V8*)(sb + b_addr[ks] + (kw * kBN + b * 32) * kRowB);
  };
  auto mma_block = [&](const V8(&af)[4], const V8(&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(bf[b], af[a], acc[a][b]);
  };
  // one step on stages (sa, sb); unless it is the last, also hand over to (na, nb)
  auto run_step = [&](const char* sa, const char* sb, const char* na, const char* nb, auto last) {
    constexpr bool kLast = decltype(last)::value;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j + 1 < NBLK) {
        read_block(fa[nxt], fb[nxt], sa, sb, (j + 1) >> 1, (j + 1) & 1);
        // part of the strip two steps ahead (its slot was freed at the last barrier)
        constexpr int NB1 = NBLK - 1;
        const int q0 = (j * kA_LOADS) / NB1, q1 = ((j + 1) * kA_LOADS) / NB1;
        if constexpr (A_ST == 3) issue_a_part(q0, q1);
        mma_block(fa[cur], fb[cur]);
        // in the shadow of each MFMA: a fragment read (first 8), load address VALU, a load
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!kLast) {
        // every wave's reads of this step have returned; the next step has landed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        wait_vmcnt_barrier<WAIT_N>();
        read_block(fa[nxt], fb[nxt], na, nb, 0, 0);
        issue_ahead();                      // into the slots this step freed
        mma_block(fa[cur], fb[cur]);
        // in the shadow of each MFMA: a fragment read (first 8), load address VALU, a load
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, (NL + 15) / 16, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mma_block(fa[cur], fb[cur]);
      }
    }
  };

  if (S > 0) {
    if constexpr (A_ST == 3) {
      issue_a();                            // strip 0
      issue_b();                            // filter 0
      issue_a();                            // strip 1
      wait_vmcnt_barrier<kA_LOADS>();       // step 0 landed
      issue_b();                            // filter 1; strip 2 goes out during step 0
    } else {
      issue_a();
      issue_b();
      wait_vmcnt_barrier<0>();              // step 0 landed
      issue_a();
      issue_b();
    }
    read_block(fa[0], fb[0], smem, smem + B_BASE, 0, 0);
    int ra = 0, rb = 0;                     // slots of the step being computed
    for (int s = 0; s + 1 < S; ++s) {
      const int ra1 = ra + 1 == A_ST ? 0 : ra + 1, rb1 = rb ^ 1;
      run_step(smem + ra * kStripBytes, smem + B_BASE + rb * B_BYTES, smem + ra1 * kStripBytes,
               smem + B_BASE + rb1 * B_BYTES, std::false_type{});
      ra = ra1;
      rb = rb1;
    }
    run_step(smem + ra * kStripBytes, smem + B_BASE + rb * B_BYTES, nullptr, nullptr, std::true_type{});
  }

  // ---- epilogue: the tile goes through LDS so that each store writes whole
  // 16-byte pieces of output rows (4 rows of 128 channels per wave
  // instruction) instead of 8 bytes in each of 32 rows.  Lane (r, g2) holds
  // rows 32 a + r of this wave and channels 32 b + 8 q + 4 g2 + i.  In LDS a
  // row is 256 bytes; its 16-byte piece k sits at slot k ^ (row % 16), so the
  // writes spread over the banks and every read of 4 rows is conflict-free.
  // Wait for the zero-fill loads past the end and for every wave's last reads.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  char* ep = smem + wave * (kOutTileBytes / 4);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = a * 32 + r;
        union { T h[4]; uint2 u; } pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][4 * q + i]);
        *(uint2*)(ep + row * kOutRowB + (((4 * b + q) ^ (row & 15)) * 16) + g2 * 8) = pk.u;
      }
  const bool whole16 = (p.cout & 7) == 0;   // 16-byte stores stay aligned
#pragma unroll 4
  for (int i = 0; i < kBM / 4 / 4; ++i) {
    const int row = 4 * i + (lane >> 4), k = lane & 15;
    const uint4 v = *(const uint4*)(ep + row * kOutRowB + ((k ^ (row & 15)) * 16));
    const int m = m0 + wave * (kBM / 4) + row;
    const int n = n0 + k * 8;
    if (m < p.M) {
      T* dst = y + (int64_t)m * p.cout + n;
      if (n + 8 <= p.cout) {
        if (whole16) {
          store16_nt(dst, v);
        } else {
          *(uint2*)dst = make_uint2(v.x, v.y);
          *(uint2*)(dst + 4) = make_uint2(v.z, v.w);
        }
      } else if (n + 4 <= p.cout) {
        *(uint2*)dst = make_uint2(v.x, v.y);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int KW>
hipError_t launch_kw(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = (p.cout + kBN - 1) / kBN;
  const uint32_t xb = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  const uint32_t wb = (uint32_t)((int64_t)p.cout * p.K * 2);
  hipLaunchKernelGGL((conv_strip_kernel<T, KW>), dim3(tiles_m * tiles_n), dim3(256), 0, s, p,
                     (const T*)x, (const T*)w, (T*)y, tiles_n, xb, wb);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y, hipStream_t s) {
  switch (p.kw) {
    case 1: return launch_kw<T, 1>(p, x, w, y, s);
    case 2: return launch_kw<T, 2>(p, x, w, y, s);
    case 3: return launch_kw<T, 3>(p, x, w, y, s);
    case 4: return launch_kw<T, 4>(p, x, w, y, s);
    default: return launch_kw<T, 5>(p, x, w, y, s);
  }
}

}  // namespace

bool strip_accepts(const ConvParams& p, int dtype) {
  return (dtype == kF16 || dtype == kBF16) && p.groups == 1 && p.ew == 1 && p.cin % 32 == 0 &&
         p.cout % 4 == 0 && p.sw == 1 &&
         p.ow % kSeg == 0 && p.kw <= kMaxKW && p.kd <= 16 && p.kh <= 16;
}

hipError_t launch_strip(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
