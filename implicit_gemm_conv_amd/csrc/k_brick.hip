// k_brick.hip -- implicit GEMM with the input brick staged in LDS (fp16/bf16,
// C_in % 16 == 0, at least 4 filter taps).
//
// The classic implicit GEMM ("Convolutions" tutorial, section 5) gathers row
// m of the virtual im2col matrix afresh for every tap, so the input is read
// through the caches K_d*K_h*K_w times.  Here a workgroup owns a box of
// output positions (TD x TH x TW of one image, up to 256 or 512 of them, and 128
// output channels).  For each chunk of 16 input channels it stages in LDS the
// input brick that box needs -- ((TD-1)*s_d + K_d) x ((TH-1)*s_h + K_h) x
// ((TW-1)*s_w + K_w) positions, zero where the brick leaves the input -- and
// then forms the A operand of every tap by reading that brick at the tap's
// shift.  Global traffic per chunk is one brick plus one 4 KB filter slice
// per tap, instead of one im2col tile per tap.
//
// Schedule (4 waves; one or two workgroups per CU):
//  * each wave owns 32*FMB output rows x 128 channels = FMB x 4 blocks of
//    v_mfma_f32_32x32x16, with fp32 accumulators;
//  * a K step is one (channel chunk, tap); the fragments of step g+1 are read
//    from LDS into a second register set while the MFMAs of step g run;
//  * filter slices travel global -> LDS with direct-to-LDS buffer loads,
//    four steps ahead, in four stages; the brick of the next chunk is
//    loaded into the other of two brick buffers, SPT 16-byte loads per
//    thread per step, spread over the current chunk's first taps;
//  * one barrier per step; every step issues the same number of loads (lanes
//    with nothing to load use an offset the range check turns into zeros),
//    so one fixed vmcnt wait covers every step.
// LDS positions hold 16 channels (32 bytes, two 16-byte halves); the half
// index is XORed with bit 3 of the position, so 16 consecutive positions read
// at the same half hit 16 distinct 16-byte bank groups.
#include "conv_device.h"

namespace convfwd {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

constexpr int kBN = 128;                   // output channels per workgroup
constexpr int kStageBytes = kBN * 32;      // one filter slice (4 KB)
constexpr int kStages = 4;
constexpr int kSinkBytes = 4096;           // target of loads that carry nothing

// Waits until at most N of this thread's vector-memory operations are
// outstanding and all its LDS reads have returned, then joins the barrier.
// (The LDS reads of the next step's fragments must be complete before any
// wave refills the stage they came from.)
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// A ds_read_b128 is served 16 lanes at a time over 256 bytes of banks; 16
// consecutive records (32 bytes each) at the same half must therefore land on
// 16 distinct 16-byte slots mod 256, which XOR-ing the half with bit 3 of the
// record index achieves for any starting record (i.e. any tap shift).
__device__ __forceinline__ int half_swz(int pos, int h) { return h ^ ((pos >> 3) & 1); }

// Exact q = a / b, r = a % b for 0 <= a < 2^24, 1 <= b < 2^24, via a float
// reciprocal and one correction each way.
__device__ __forceinline__ void divmod(int a, int b, float inv_b, int& q, int& r) {
  q = (int)((float)a * inv_b);
  r = a - q * b;
  const int lo = r < 0, hi = r >= b;
  q += hi - lo;
  r += (lo - hi) * b;
}

}  // namespace

struct BrickGeom {
  int TD, TH, TW;            // output box
  int BD, BH, BW;            // brick extents in input positions
  int npos;                  // BD * BH * BW
  int nslots;                // ceil(npos / 128): brick loads per thread per chunk
  int tiles_d, tiles_h, tiles_w, tiles_n;
  int rows;                  // TD * TH * TW
  float inv_bw, inv_bhw, inv_tw, inv_thw;
};

namespace {

// FMB: 32-row MFMA blocks per wave (rows per workgroup = 128 * FMB);
// MAXSLOTS: brick buffer size in 4 KB slots (128 positions each); OCC:
// workgroups per CU the LDS and register budget is sized for.
template <typename T, int SPT, int FMB, int MAXSLOTS, int OCC>
__global__ __launch_bounds__(256, OCC) void conv_brick_kernel(ConvParams p, BrickGeom g,
                                                            const T* __restrict__ x,
                                                            const T* __restrict__ w,
                                                            T* __restrict__ y, uint32_t x_bytes,
                                                            uint32_t w_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  constexpr int NL = 1 + SPT;                // loads per thread per step
  constexpr int kBrickBytes = MAXSLOTS * 4096;
  __shared__ __attribute__((aligned(1024)))
  char smem[2 * kBrickBytes + kStages * kStageBytes + kSinkBytes];
  char* const brick0 = smem;
  char* const stage0 = smem + 2 * kBrickBytes;
  char* const sink = stage0 + kStages * kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fg = lane >> 5;

  // ---- tile coordinates (XCD-aware order; channel tiles fastest) ----
  int t = xcd_tile(blockIdx.x, gridDim.x);
  const int tn = t % g.tiles_n; t /= g.tiles_n;
  const int tw_ = t % g.tiles_w; t /= g.tiles_w;
  const int th_ = t % g.tiles_h; t /= g.tiles_h;
  const int td_ = t % g.tiles_d;
  const int nimg = t / g.tiles_d;
  const int od0 = td_ * g.TD, oh0 = th_ * g.TH, ow0 = tw_ * g.TW;
  const int n0 = tn * kBN;
  // input origin of the brick (may lie in the padding)
  const int id0 = od0 * p.sd - p.pd, ih0 = oh0 * p.sh - p.ph, iw0 = ow0 * p.sw - p.pw;

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)w_bytes, kRawBufferFlags);

  // ---- this lane's output rows: brick position of tap (0,0,0) and flat m ----
  int rowpos[FMB], rowm[FMB];
#pragma unroll
  for (int a = 0; a < FMB; ++a) {
    const int tr = (wave * FMB + a) * 32 + fr;
    int tdd, rem, thh, tww;
    divmod(tr, g.TH * g.TW, g.inv_thw, tdd, rem);
    divmod(rem, g.TW, g.inv_tw, thh, tww);
    const bool in_box = tr < g.rows;
    const int od = od0 + tdd, oh = oh0 + thh, ow = ow0 + tww;
    const bool valid = in_box && od < p.od && oh < p.oh && ow < p.ow;
    rowpos[a] = in_box ? (tdd * p.sd * g.BH + thh * p.sh) * g.BW + tww * p.sw : 0;
    rowm[a] = valid ? ((nimg * p.od + od) * p.oh + oh) * p.ow + ow : -1;
  }

  // ---- filter loader: thread t fills row t/2, physical half t%2 ----
  const int brow = tid >> 1;
  const int bhalf = half_swz(brow, tid & 1);
  const uint32_t wrow_off = (n0 + brow) < p.cout
                                ? (uint32_t)(((n0 + brow) * p.K + bhalf * 8) * 2)
                                : kOutOfRange;

  // ---- brick loader: slot q of thread t is 16-byte piece j = 256 q + t,
  // position j / 2, physical half j % 2 ----
  const int nchunks = p.cin / 16;
  const int G = nchunks * p.ntaps;
  // Computed without branches (every lane does the same arithmetic, then a
  // select), so the load issue stays in one basic block.
  auto brick_slot_off = [&](int q, int chunk) -> uint32_t {
    const int j = q * 256 + tid;
    const int pos = j >> 1;
    int bd, rem, bh, bw;
    divmod(pos, g.BH * g.BW, g.inv_bhw, bd, rem);
    divmod(rem, g.BW, g.inv_bw, bh, bw);
    const int id = id0 + bd, ih = ih0 + bh, iw = iw0 + bw;
    const bool inside = (pos < g.npos) & (chunk < nchunks) & ((unsigned)id < (unsigned)p.d) &
                        ((unsigned)ih < (unsigned)p.h) & ((unsigned)iw < (unsigned)p.w);
    const int h = half_swz(pos, j & 1);
    const uint32_t off =
        (uint32_t)((nimg * p.xs_n + id * p.xs_d + ih * p.xs_h + iw * p.xs_w + chunk * 16 + h * 8) * 2);
    return inside ? off : kOutOfRange;
  };

  // Step iterator for the filter loads: (chunk, kd, kh, kw), branch-free.
  int bc = 0, bkd = 0, bkh = 0, bkw = 0, bn = 0;
  int bstage = 0;
  auto issue_b = [&]() {
    const uint32_t dead = bn < G ? 0u : kOutOfRange;
    const uint32_t off =
        (wrow_off + (uint32_t)(((((bkd * p.kh + bkh) * p.kw + bkw) * p.cin) + bc * 16) * 2)) | dead;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wr, (lds_ptr_t)(stage0 + bstage * kStageBytes + wave * 1024), 16, off, 0, 0, 0);
    const int w1 = bkw + 1;
    const bool ww = w1 == p.kw;
    bkw = ww ? 0 : w1;
    const int h1 = bkh + (int)ww;
    const bool wh = h1 == p.kh;
    bkh = wh ? 0 : h1;
    const int d1 = bkd + (int)wh;
    const bool wd = d1 == p.kd;
    bkd = wd ? 0 : d1;
    bc += (int)wd;
    ++bn;
    bstage = bstage + 1 == kStages ? 0 : bstage + 1;
  };
  // Brick loads issued during step (chunk c, tap u): slots u*SPT .. u*SPT+SPT-1
  // of chunk c+1, into brick buffer (c+1) % 2.
  // Slots past the brick, and all slots after the last chunk, go to the sink
  // (their offsets are out of range: brick_slot_off checks pos and chunk).
  auto issue_brick = [&](int c, int u) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int q = u * SPT + k;
      const bool live = q < g.nslots && q < MAXSLOTS && c + 1 < nchunks;
      char* dst = live ? brick0 + ((c + 1) & 1) * kBrickBytes + q * 4096 + wave * 1024
                       : sink + wave * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, brick_slot_off(q, c + 1),
                                               0, 0, 0);
    }
  };

  // ---- fragment reads for step (chunk c, tap shift `shift`, filter stage) ----
  V8 fa0[FMB], fb0[4], fa1[FMB], fb1[4];
  auto read_frags = [&](int c, int shift, int stage, V8* fa, V8* fb) {
    const char* br = brick0 + (c & 1) * kBrickBytes;
#pragma unroll
    for (int a = 0; a < FMB; ++a) {
      const int pos = rowpos[a] + shift;
      fa[a] = *(const V8*)(br + pos * 32 + half_swz(pos, fg) * 16);
    }
    const char* sb = stage0 + stage * kStageBytes;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = b * 32 + fr;
      fb[b] = *(const V8*)(sb + n * 32 + half_swz(n, fg) * 16);
    }
  };

  f32x16_t acc[FMB][4];
#pragma unroll
  for (int a = 0; a < FMB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  auto mfmas = [&](const V8* fa, const V8* fb) {
#pragma unroll
    for (int a = 0; a < FMB; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(fb[b], fa[a], acc[a][b]);
  };

  // Step iterator for the fragment reads (chunk, tap) and its brick shift.
  int rc = 0, rkd = 0, rkh = 0, rkw = 0, rstage = 0;
  auto shift_of = [&](int kd, int kh, int kw) { return (kd * g.BH + kh) * g.BW + kw; };
  auto advance_r = [&]() {
    const int w1 = rkw + 1;
    const bool ww = w1 == p.kw;
    rkw = ww ? 0 : w1;
    const int h1 = rkh + (int)ww;
    const bool wh = h1 == p.kh;
    rkh = wh ? 0 : h1;
    const int d1 = rkd + (int)wh;
    const bool wd = d1 == p.kd;
    rkd = wd ? 0 : d1;
    rc += (int)wd;
    rstage = rstage + 1 == kStages ? 0 : rstage + 1;
  };

  // ---- prologue: brick of chunk 0 (all slots), filter slices 0 and 1 ----
  for (int q = 0; q < g.nslots; ++q) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (lds_ptr_t)(brick0 + q * 4096 + wave * 1024), 16, brick_slot_off(q, 0), 0, 0, 0);
  }
  issue_b();
  issue_b();
  wait_vmcnt_barrier<0>();
  read_frags(0, 0, 0, fa0, fb0);
  advance_r();
  // Two rounds of what every step issues (the filter slice four steps ahead
  // plus SPT brick loads, here all to the sink), so the in-flight pattern
  // matches the loop's; the fragment reads of step 0 finish before any wave
  // may refill stage 0.
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    issue_b();
#pragma unroll
    for (int k = 0; k < SPT; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(sink + wave * 1024), 16,
                                               kOutOfRange, 0, 0, 0);
  }
  wait_vmcnt_barrier<2 * NL>();

  // ---- main loop: two steps per trip so the fragment sets alternate ----
  int sc = 0, su = 0;   // chunk and tap index of the step being multiplied
  // The LDS reads of the next step go out first (a scheduling fence keeps
  // them there), so their latency hides under this step's MFMAs; the brick
  // loads' address arithmetic then interleaves with the MFMAs.
  auto step = [&](V8* fa_cur, V8* fb_cur, V8* fa_nxt, V8* fb_nxt) {
    issue_b();
    read_frags(rc, shift_of(rkd, rkh, rkw), rstage, fa_nxt, fb_nxt);
    __builtin_amdgcn_sched_barrier(0);
    advance_r();
    issue_brick(sc, su);
    mfmas(fa_cur, fb_cur);
    wait_vmcnt_barrier<2 * NL>();
    if (++su == p.ntaps) { su = 0; ++sc; }
  };
  int s = 0;
  for (; s + 1 < G; s += 2) {
    step(fa0, fb0, fa1, fb1);
    step(fa1, fb1, fa0, fb0);
  }
  if (s < G) step(fa0, fb0, fa1, fb1);
  wait_vmcnt_barrier<0>();

  // ---- epilogue: 8-byte stores of 4 consecutive channels ----
#pragma unroll
  for (int a = 0; a < FMB; ++a) {
    if (rowm[a] < 0) continue;
    T* yrow = y + (int64_t)rowm[a] * p.cout;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + b * 32 + 8 * q + 4 * fg;
        if (n + 3 < p.cout) {
          union { T h[4]; uint2 u; } pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[a][b][4 * q + i]);
          *(uint2*)(yrow + n) = pk.u;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < p.cout) yrow[n + i] = from_f32<T>(acc[a][b][4 * q + i]);
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Output box for a problem: up to `max_rows` rows, brick within
// `max_slots` * 128 positions, choosing the box that minimises the MFMA rows
// issued (every tile issues max_rows, full or not) plus a charge for the
// brick positions loaded.  Returns false if no box fits.
bool choose_geom(const ConvParams& p, int max_rows, int max_slots, BrickGeom* out) {
  double best = 1e30;
  bool found = false;
  const int tw_opts[] = {p.ow, 32, 64, 16, 8};
  for (int tw : tw_opts) {
    if (tw < 1 || tw > p.ow || tw > max_rows) continue;
    for (int th = 1; th <= p.oh && th * tw <= max_rows; ++th) {
      for (int td = 1; td <= p.od && td * th * tw <= max_rows; ++td) {
        const int rows = td * th * tw;
        const int bd = (td - 1) * p.sd + p.kd, bh = (th - 1) * p.sh + p.kh,
                  bw = (tw - 1) * p.sw + p.kw;
        const long npos = (long)bd * bh * bw;
        if (npos > (long)max_slots * 128) continue;
        const long tiles = (long)p.n * ((p.od + td - 1) / td) * ((p.oh + th - 1) / th) *
                           ((p.ow + tw - 1) / tw);
        const double cost = (double)tiles * max_rows + 0.25 * (double)tiles * npos;
        if (cost < best) {
          best = cost;
          found = true;
          out->TD = td; out->TH = th; out->TW = tw;
          out->BD = bd; out->BH = bh; out->BW = bw;
          out->npos = (int)npos;
          out->nslots = (int)((npos + 127) / 128);
          out->rows = rows;
          out->tiles_d = (p.od + td - 1) / td;
          out->tiles_h = (p.oh + th - 1) / th;
          out->tiles_w = (p.ow + tw - 1) / tw;
        }
      }
    }
  }
  if (!found) return false;
  out->tiles_n = (p.cout + kBN - 1) / kBN;
  out->inv_bw = 1.0f / (float)out->BW;
  out->inv_bhw = 1.0f / (float)(out->BH * out->BW);
  out->inv_tw = 1.0f / (float)out->TW;
  out->inv_thw = 1.0f / (float)(out->TH * out->TW);
  return true;
}

// Two shapes of the kernel: 512 rows per workgroup, one workgroup per CU
// (large bricks), and 256 rows with two workgroups per CU (so one wave's
// address arithmetic overlaps the other's MFMAs).
struct BrickCfg {
  int fmb, max_slots, occ;
};
constexpr BrickCfg kCfgBig{4, 12, 1};
constexpr BrickCfg kCfgSmall{2, 7, 2};

template <typename T, int FMB, int MAXSLOTS, int OCC>
hipError_t launch_cfg(const ConvParams& p, const BrickGeom& g, const void* x, const void* w,
                      void* y, hipStream_t s) {
  const long tiles = (long)p.n * g.tiles_d * g.tiles_h * g.tiles_w * g.tiles_n;
  const uint32_t xb = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  const uint32_t wb = (uint32_t)((int64_t)p.cout * p.K * 2);
  // the next chunk's brick must be loaded within its first ntaps - 3 steps
  const int spt_needed = (g.nslots + (p.ntaps - 3) - 1) / (p.ntaps - 3);
  const dim3 grid((unsigned)tiles), block(256);
  if (spt_needed <= 1)
    hipLaunchKernelGGL((conv_brick_kernel<T, 1, FMB, MAXSLOTS, OCC>), grid, block, 0, s, p, g,
                       (const T*)x, (const T*)w, (T*)y, xb, wb);
  else if (spt_needed <= 2)
    hipLaunchKernelGGL((conv_brick_kernel<T, 2, FMB, MAXSLOTS, OCC>), grid, block, 0, s, p, g,
                       (const T*)x, (const T*)w, (T*)y, xb, wb);
  else if (spt_needed <= 4)
    hipLaunchKernelGGL((conv_brick_kernel<T, 4, FMB, MAXSLOTS, OCC>), grid, block, 0, s, p, g,
                       (const T*)x, (const T*)w, (T*)y, xb, wb);
  else
    hipLaunchKernelGGL((conv_brick_kernel<T, MAXSLOTS, FMB, MAXSLOTS, OCC>), grid, block, 0, s,
                       p, g, (const T*)x, (const T*)w, (T*)y, xb, wb);
  return hipGetLastError();
}

#ifndef CONVFWD_BRICK_CFG
#define CONVFWD_BRICK_CFG 2
#endif

template <typename T>
hipError_t launch_typed(const ConvParams& p, const void* x, const void* w, void* y,
                        hipStream_t s) {
  BrickGeom g;
  if (CONVFWD_BRICK_CFG == 2 && choose_geom(p, 128 * kCfgSmall.fmb, kCfgSmall.max_slots, &g))
    return launch_cfg<T, kCfgSmall.fmb, kCfgSmall.max_slots, kCfgSmall.occ>(p, g, x, w, y, s);
  if (!choose_geom(p, 128 * kCfgBig.fmb, kCfgBig.max_slots, &g)) return hipErrorInvalidValue;
  return launch_cfg<T, kCfgBig.fmb, kCfgBig.max_slots, kCfgBig.occ>(p, g, x, w, y, s);
}

}  // namespace

bool brick_accepts(const ConvParams& p, int dtype) {
  if (!(dtype == kF16 || dtype == kBF16) || !plain(p)) return false;
  if (p.cin % 16 != 0 || p.cout % 4 != 0 || p.ntaps < 4) return false;
  if (p.kd > 16 || p.kh > 16 || p.kw > 16) return false;
  BrickGeom g;
  return choose_geom(p, 128 * kCfgBig.fmb, kCfgBig.max_slots, &g);
}

hipError_t launch_brick(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s) {
  if (dtype == kF16) return launch_typed<_Float16>(p, x, w, y, s);
  return launch_typed<__bf16>(p, x, w, y, s);
}

}  // namespace convfwd
