// k_rows.hip -- the tiny-C_in path (fp16/bf16, C_in < 16, C_in * K_w <= 32,
// K_d * K_h * ceil(C_in * K_w / 8) <= 24, C_out <= 64): input rows staged in LDS, MFMA fragments built from runs of
// the filter window.
//
// With very few input channels the implicit-GEMM depth K = C_in*K_d*K_h*K_w
// is small (147 for the 7x7, 3-channel ResNet-50 first layer of the
// "Convolutions" tutorial, section 4) and the layer is bound by writing its
// output, not by arithmetic.  The layout of the (k_w, c) part of K matters:
// for one filter row (kd, kh) the C_in*K_w elements an output needs are one
// contiguous run of the channels-last input row.  So:
//  * K is reordered as (filter row r = (kd, kh), run position j), and each
//    run of C_in*K_w is cut into P groups of 8 (the last padded with zero
//    filter weights); a lane's 8-element MFMA operand is one such group, 8
//    consecutive halves of an LDS copy of the input row;
//  * a workgroup owns 4 consecutive output rows (one per wave) of up to 112
//    outputs each and all C_out <= 64 channels; it stages the input rows they
//    touch -- whole rows, 16-byte pieces, zeros outside the image -- in LDS;
//  * the filter, reordered and zero-padded to the group layout, is staged in
//    LDS once per workgroup; workgroups are persistent and loop over tiles;
//  * each wave computes 7 x 4 blocks of v_mfma_f32_16x16x32 (16 outputs x
//    16 channels) per output row; with C_out of 16, 32 or 64 its row of
//    outputs is one contiguous run of y, staged through LDS and stored as
//    whole 16-byte pieces (else runs of 4 channels, 8 bytes);
//  * the next tile's rows are loaded into registers while a tile computes,
//    and two workgroups share a CU, so one's stores overlap the other's work.
#include "conv_device.h"

namespace convfwd {

namespace {

constexpr int kSegBlocks = 7;              // 16-output MFMA blocks per wave row
constexpr int kSeg = 16 * kSegBlocks;      // outputs per output-row segment (112)
constexpr int kRowsPerTile = 4;            // output rows per workgroup tile (one per wave)
constexpr int kMaxGroups = 24;             // filter groups of 8 (R * P), i.e. K <= 192
constexpr int kMaxSteps = kMaxGroups / 4;  // MFMA k-steps of 32
constexpr int kNB = 4;                     // 16-channel output blocks (C_out <= 64)
constexpr int kInBytes = 24 * 1024;        // staged input rows
constexpr int kMaxPieces = 6;              // staged 16-byte pieces per thread per tile
constexpr int kBBytes = kMaxGroups * 64 * 16;   // filter table: [group][channel] x 16 B

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;

}  // namespace

// Host-computed layout of one tile's staged rows.
struct RowsGeom {
  int P;              // groups of 8 per filter row: ceil(C_in * K_w / 8)
  int R;              // filter rows: K_d * K_h
  int S;              // MFMA k-steps: ceil(R * P / 4)
  int RH;             // staged input rows per depth tap: 3 * s_h + K_h
  int nrows;          // staged rows: K_d * RH
  int lo_pix;         // first staged pixel relative to the segment's window origin (<= 0)
  int row_halves;     // halves per staged row (multiple of 8)
  int shift;          // halves the staged rows are moved by in LDS (0 or 1) so
                      // that every lane's 8-half group starts on 4 bytes
  int tiles_h, tiles_w;
  int tiles;          // n * d_out * tiles_h * tiles_w
};

namespace {

// ALIGNED: every group starts on a 4-byte LDS boundary (stride * C_in even,
// with the staging shift applied) and is read as four dwords; otherwise it is
// read as eight halves.
template <typename T, bool ALIGNED>
__global__ __launch_bounds__(256, 2) void conv_rows_kernel(ConvParams p, RowsGeom g,
                                                           const T* __restrict__ x,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ y, uint32_t x_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef typename Vec8<T>::type V8;
  __shared__ __attribute__((aligned(16))) char lds_in[kInBytes];
  __shared__ __attribute__((aligned(16))) char lds_b[kBBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fr = lane & 15, fg = lane >> 4;
  const int run = p.cin * p.kw;           // elements of one filter-row run
  const int nq = g.R * g.P;               // real groups

  // ---- filter table: entry (q, n) = 8 halves of filter row r = q / P,
  // run positions 8*(q % P) .. +7 (zero past the run or past C_out).  The
  // filter (C_out * K <= 64 * 192 halves, at most lds_in's size) is first
  // copied as it is into lds_in with consecutive threads reading consecutive
  // elements, then the table is built from that copy: reading the table's
  // entries straight from global memory touches one cache line per lane. ----
  {
    // 16-byte pieces (the hardware serves unaligned buffer loads at any
    // alignment), all six per thread in flight before any LDS write: 2-byte
    // loads took 48 instructions per thread, with every workgroup reading the
    // same lines at once at the start
    constexpr int kPieces = kMaxGroups * 8 * 64 / 8 / 256;   // 16-byte pieces per thread (6)
    static_assert(kPieces * 256 * 16 <= kInBytes, "filter copy fits lds_in");
    const int wn = p.cout * p.K;
    const int wbytes = wn * 2;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, wbytes, kRawBufferFlags);
    u32x4_t pcs[kPieces];
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int k = tid + 256 * j;
      pcs[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, k * 16 < wbytes ? (uint32_t)(k * 16) : kOutOfRange, 0, 0);
    }
    // with an odd element count the last element shares a dword with what
    // lies past the filter, which the range check drops: its piece's owner
    // copies it on its own after writing the piece
    const int k_last = (wbytes - 2) / 16;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int k = tid + 256 * j;
      if (k * 16 < wbytes) {
        *(u32x4_t*)(lds_in + k * 16) = pcs[j];
        if (k == k_last && (wn & 1)) ((T*)lds_in)[wn - 1] = w[wn - 1];
      }
    }
  }
  __syncthreads();
  {
    // all reads issued unconditionally (addresses clamped into the copy),
    // zeros selected afterwards: one LDS round trip instead of a branch per
    // element
    constexpr int kEnt = kMaxGroups * 64 / 256;   // table entries per thread (6)
    const int wn = p.cout * p.K;
    const T* wl = (const T*)lds_in;
    T hv[kEnt][8];
    bool keep[kEnt][8];
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
      const int e = tid + 256 * k;
      const int q = e >> 6, n = e & 63;
      const bool ok = q < nq && n < p.cout;
      const int r = ok ? q / g.P : 0, j0 = ok ? (q % g.P) * 8 : 0;
      const int base = n * p.K + r * run + j0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hv[k][i] = wl[min(base + i, wn - 1)];
        keep[k][i] = ok && j0 + i < run;
      }
    }
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
      union { T h[8]; uint4 u; } v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v.h[i] = keep[k][i] ? hv[k][i] : (T)0.f;
      *(uint4*)(lds_b + (tid + 256 * k) * 16) = v.u;
    }
  }

  // ---- per-lane constants ----
  // LDS byte offset of this lane's group in k-step s, relative to the wave's
  // first staged row and the output's first pixel.
  int grp_off[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    const int q = 4 * s + fg;
    const int r = q < nq ? q / g.P : 0;
    const int part = q < nq ? q % g.P : 0;
    const int kd = r / p.kh, kh = r % p.kh;
    grp_off[s] = ((kd * g.RH + kh) * g.row_halves + part * 8) * 2;
  }
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRawBufferFlags);
  const int row_pieces = g.row_halves / 8;
  const int pieces = g.nrows * row_pieces;
  const int wrow_halves = p.w * p.cin;    // one input row in global memory

  // Tile coordinates and the global byte offsets of this thread's staging
  // pieces (piece i = tid + 256 k: staged row i / row_pieces, 16-byte piece
  // i % row_pieces; out-of-range pieces read zeros).
  struct TileCoord {
    int nimg, od, oh0, ow0;
  };
  auto coords = [&](int tile) {
    TileCoord c;
    int t = tile;
    const int tw_ = t % g.tiles_w; t /= g.tiles_w;
    const int th_ = t % g.tiles_h; t /= g.tiles_h;
    c.od = t % p.od;
    c.nimg = t / p.od;
    c.oh0 = th_ * kRowsPerTile;
    c.ow0 = tw_ * kSeg;
    return c;
  };
  uint4 stage_regs[kMaxPieces];
  auto prefetch = [&](int tile) {
    const TileCoord c = coords(tile < g.tiles ? tile : 0);
    const bool live = tile < g.tiles;
    const int id0 = c.od * p.sd - p.pd, ih0 = c.oh0 * p.sh - p.ph;
    const int h_lo = (c.ow0 * p.sw - p.pw + g.lo_pix) * p.cin;   // first staged half of the row
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int i = tid + 256 * k;
      const int row = i / row_pieces, pc = i - (i / row_pieces) * row_pieces;
      const int kd = row / g.RH, rr = row - (row / g.RH) * g.RH;
      const int id = id0 + kd, ih = ih0 + rr;
      const int h0 = h_lo + pc * 8;
      const bool inside = live && i < pieces && (unsigned)id < (unsigned)p.d &&
                          (unsigned)ih < (unsigned)p.h && h0 >= 0 && h0 < wrow_halves;
      const uint32_t off =
          inside ? (uint32_t)(((int64_t)((c.nimg * p.d + id) * p.h + ih) * wrow_halves + h0) * 2)
                 : kOutOfRange;
      stage_regs[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int i = tid + 256 * k;
      if (i < pieces) {
        const int row = i / row_pieces, pc = i - (i / row_pieces) * row_pieces;
        char* dst = lds_in + (row * g.row_halves + pc * 8 + g.shift) * 2;
        const uint4 v = stage_regs[k];
        if (g.shift == 0) {
          *(uint4*)dst = v;
        } else {
          // a copy moved by one half (dst is 2 past a 16-byte boundary):
          // halves 0 and 7 alone, the six between re-paired into an aligned
          // dword and an aligned 8-byte pair (a misaligned 16-byte LDS write
          // costs several times more)
          *(uint16_t*)dst = (uint16_t)v.x;
          *(uint32_t*)(dst + 2) = __builtin_amdgcn_alignbit(v.y, v.x, 16);
          *(uint2*)(dst + 6) = make_uint2(__builtin_amdgcn_alignbit(v.z, v.y, 16),
                                          __builtin_amdgcn_alignbit(v.w, v.z, 16));
          *(uint16_t*)(dst + 14) = (uint16_t)(v.w >> 16);
        }
      }
    }
  };

  prefetch(blockIdx.x);
  for (int tile = blockIdx.x; tile < g.tiles; tile += gridDim.x) {
    const TileCoord tc = coords(tile);
    const int nimg = tc.nimg, od = tc.od, oh0 = tc.oh0, ow0 = tc.ow0;
    __syncthreads();   // the previous tile's reads of lds_in are done
    commit();
    __syncthreads();
    prefetch(tile + gridDim.x);   // next tile's rows load while this one computes

    // ---- one output row per wave ----
    const int oh = oh0 + wave;
    f32x4_t acc[kSegBlocks][kNB];
#pragma unroll
    for (int b = 0; b < kSegBlocks; ++b)
#pragma unroll
      for (int c = 0; c < kNB; ++c) acc[b][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // first element of block 0's window for this lane's output, in bytes
    const int lane_off = (wave * p.sh * g.row_halves + (fr * p.sw - g.lo_pix) * p.cin + g.shift) * 2;
    const int blk_step = 16 * p.sw * p.cin * 2;
    for (int s = 0; s < g.S; ++s) {
      V8 bfr[kNB];
#pragma unroll
      for (int c = 0; c < kNB; ++c)
        bfr[c] = *(const V8*)(lds_b + ((4 * s + fg) * 64 + c * 16 + fr) * 16);
      const char* abase = lds_in + lane_off + grp_off[s];
#pragma unroll
      for (int b = 0; b < kSegBlocks; ++b) {
        union { uint16_t h[8]; uint32_t d[4]; V8 v; } a;
        if constexpr (ALIGNED) {
          const uint32_t* src = (const uint32_t*)(abase + b * blk_step);
#pragma unroll
          for (int i = 0; i < 4; ++i) a.d[i] = src[i];
        } else {
          const uint16_t* src = (const uint16_t*)(abase + b * blk_step);
#pragma unroll
          for (int i = 0; i < 8; ++i) a.h[i] = src[i];
        }
#pragma unroll
        for (int c = 0; c < kNB; ++c) acc[b][c] = mfma16x16x32(bfr[c], a.v, acc[b][c]);
      }
    }

    // ---- store: lane holds channels 16c + 4*fg + i of output ow0 + 16b + fr ----
    // With C_out in {16, 32, 64} a wave's row of outputs is one contiguous run
    // of y: it is staged through the wave's quarter of lds_in (free once every
    // wave's reads of this tile are done), 32 outputs at a time with 16-byte
    // piece k of output o at slot k ^ (o % pieces per output), and stored as
    // whole 16-byte pieces, 1 KB of consecutive bytes per wave instruction.
    const int ppo = p.cout / 8;              // 16-byte pieces per output
    if (p.cout == 16 || p.cout == 32 || p.cout == 64) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      char* ep = lds_in + wave * (kInBytes / 4);
      const int ob = p.cout * 2;             // bytes per output
      T* yrow = y + (int64_t)((nimg * p.od + od) * p.oh + oh) * p.ow * p.cout;
#pragma unroll
      for (int bp = 0; bp < (kSegBlocks + 1) / 2; ++bp) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int b = 2 * bp + bb;
          if (b >= kSegBlocks) continue;
          const int o = 16 * bb + fr;
#pragma unroll
          for (int c = 0; c < kNB; ++c) {
            const int n = c * 16 + fg * 4;
            if (n < p.cout) {
              union { T h[4]; uint2 u; } pk;
#pragma unroll
              for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[b][c][i]);
              *(uint2*)(ep + o * ob + (((n >> 3) ^ (o & (ppo - 1))) * 16) + ((n >> 2) & 1) * 8) = pk.u;
            }
          }
        }
        const int nout = (2 * bp + 1 < kSegBlocks ? 32 : 16);
        // at most 32 outputs x 128 bytes = 4 KB per wave: four 1 KB rounds,
        // every read issued before the stores (a loop with a run-time count
        // waited on each read in turn; unrolled, the stem runs 8% faster)
        uint4 vv[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int l = lane * 16 + it * 1024;
          const int o = l / ob, k = (l - o * ob) >> 4;
          vv[it] = l < nout * ob ? *(const uint4*)(ep + o * ob + ((k ^ (o & (ppo - 1))) * 16))
                                 : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int l = lane * 16 + it * 1024;
          const int o = l / ob, k = (l - o * ob) >> 4;
          const int ow = ow0 + 32 * bp + o;
          if (l < nout * ob && oh < p.oh && ow < p.ow) store16_nt(yrow + (int64_t)ow * p.cout + k * 8, vv[it]);
        }
      }
    } else if (oh < p.oh) {
      T* yrow = y + (int64_t)((nimg * p.od + od) * p.oh + oh) * p.ow * p.cout;
#pragma unroll
      for (int b = 0; b < kSegBlocks; ++b) {
        const int ow = ow0 + b * 16 + fr;
        if (ow >= p.ow) continue;
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
          const int n = c * 16 + fg * 4;
          if (n + 3 < p.cout) {
            union { T h[4]; uint2 u; } pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) pk.h[i] = from_f32<T>(acc[b][c][i]);
            *(uint2*)(yrow + (int64_t)ow * p.cout + n) = pk.u;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < p.cout) yrow[(int64_t)ow * p.cout + n + i] = from_f32<T>(acc[b][c][i]);
          }
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

bool make_geom(const ConvParams& p, RowsGeom* g) {
  const int run = p.cin * p.kw;
  g->P = (run + 7) / 8;
  g->R = p.kd * p.kh;
  if (g->R * g->P > kMaxGroups) return false;
  g->S = (g->R * g->P + 3) / 4;
  g->RH = (kRowsPerTile - 1) * p.sh + p.kh;
  g->nrows = p.kd * g->RH;
  // staged pixels: from the segment's window origin rounded down so the row
  // starts on a 16-byte boundary of the input row, to past the last window
  const int span = (kSeg - 1) * p.sw + p.kw;            // pixels the segment's windows touch
  // window origin o = ow0*sw - pw; the staged start must be o + lo_pix with
  // (o + lo_pix) * cin a multiple of 8 for every segment: segments start at
  // multiples of kSeg, so o changes by kSeg*sw between segments.
  if ((kSeg * p.sw * p.cin) % 8 != 0) return false;
  int lo = 0;
  while (((-p.pw + lo) * p.cin) % 8 != 0) --lo;         // (o + lo) * cin == 0 mod 8 at o = -pw
  g->lo_pix = lo;
  // 8 halves of slack: a lane's last group may run up to 7 halves past the
  // window (those positions carry zero filter weights but must hold finite
  // staged values)
  const int pix = span - lo;
  const int halves = (pix * p.cin + 8 + 7) / 8 * 8;
  g->row_halves = halves;
  // A group of the lane for output column j starts at half
  // (j*sw - lo)*cin + 8*part (+ whole rows); with sw*cin even its parity is
  // the same for every lane, and a shift of one half makes it even.
  g->shift = ((p.sw * p.cin) % 2 == 0 && ((-lo) * p.cin) % 2 != 0) ? 1 : 0;
  if ((long)g->nrows * g->row_halves * 2 + 16 > kInBytes) return false;
  if (g->nrows * (g->row_halves / 8) > 256 * kMaxPieces) return false;
  g->tiles_h = (p.oh + kRowsPerTile - 1) / kRowsPerTile;
  g->tiles_w = (p.ow + kSeg - 1) / kSeg;
  g->tiles = p.n * p.od * g->tiles_h * g->tiles_w;
  return true;
}

}  // namespace

bool rows_accepts(const ConvParams& p, int dtype) {
  if (!(dtype == kF16 || dtype == kBF16) || !plain(p)) return false;
  if (p.cin >= 16 || p.cin * p.kw > 32 || p.cout > 64) return false;
  if ((p.w * p.cin) % 8 != 0) return false;       // input rows start on 16-byte boundaries
  RowsGeom g;
  return make_geom(p, &g);
}

hipError_t launch_rows(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  RowsGeom g;
  if (!make_geom(p, &g)) return hipErrorInvalidValue;
  const uint32_t xb = (uint32_t)((int64_t)p.n * p.xs_n * 2);
  const int grid = g.tiles < 512 ? g.tiles : 512;   // two persistent workgroups per CU
  const bool aligned = (p.sw * p.cin) % 2 == 0;
  if (dtype == kF16) {
    if (aligned)
      hipLaunchKernelGGL((conv_rows_kernel<_Float16, true>), dim3(grid), dim3(256), 0, s, p, g,
                         (const _Float16*)x, (const _Float16*)w, (_Float16*)y, xb);
    else
      hipLaunchKernelGGL((conv_rows_kernel<_Float16, false>), dim3(grid), dim3(256), 0, s, p, g,
                         (const _Float16*)x, (const _Float16*)w, (_Float16*)y, xb);
  } else {
    if (aligned)
      hipLaunchKernelGGL((conv_rows_kernel<__bf16, true>), dim3(grid), dim3(256), 0, s, p, g,
                         (const __bf16*)x, (const __bf16*)w, (__bf16*)y, xb);
    else
      hipLaunchKernelGGL((conv_rows_kernel<__bf16, false>), dim3(grid), dim3(256), 0, s, p, g,
                         (const __bf16*)x, (const __bf16*)w, (__bf16*)y, xb);
  }
  return hipGetLastError();
}

}  // namespace convfwd
