// conv_params.h -- problem parameters shared by the host API and the gfx950 kernels.
//
// The host derives everything here once per call from the public descriptor
// (output extents, GEMM sizes, element strides of the channels-last input) and
// passes the struct to a kernel by value, so kernels read it from the kernel
// argument segment through scalar loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

struct ConvParams {
  int n, d, h, w;          // input extents
  int cin, cout;           // channels
  int kd, kh, kw;          // filter extents
  int sd, sh, sw;          // strides
  int pd, ph, pw;          // zero padding on the low side (the high side only sets od, oh, ow)
  int ed, eh, ew;          // filter dilation: tap t sits t*e positions past the window origin
  int groups;              // channel groups: output channel co reads the cin_g input
  int cin_g, cout_g;       //   channels of group co / cout_g (cin = groups * cin_g)
  int od, oh, ow;          // output extents
  int M;                   // GEMM rows: n * od * oh * ow
  int ntaps;               // kd * kh * kw
  int K;                   // GEMM depth of one group: ntaps * cin_g (the filter's row length)
  int xs_w, xs_h, xs_d, xs_n;  // element strides of x along w, h, d, n (xs_w == cin)
  // Where output row m = ((n*od + z)*oh + y)*ow + x lives in y.  remap == 0: at
  // m * cout (y dense, the forward pass).  remap == 1: at y_off + n*ys_n +
  // z*ys_d + y*ys_h + x*ys_w elements (one stride phase of backward-data, whose
  // rows are every s-th position of dx).  Only the main, runs and direct
  // kernels honour remap == 1.
  int remap;
  int ys_w, ys_h, ys_d, ys_n, y_off;
};

// The plain convolution: one group, undilated filter.
inline bool plain(const ConvParams& p) { return p.groups == 1 && p.ed == 1 && p.eh == 1 && p.ew == 1; }

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Kernel launchers, one per path.  Each returns hipSuccess or the launch error.
hipError_t launch_direct(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                         hipStream_t s);
hipError_t launch_main(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s);
hipError_t launch_flatk(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s);
hipError_t launch_rows(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s);
hipError_t launch_brick(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s);
hipError_t launch_strip(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s);
hipError_t launch_runs(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s);
hipError_t launch_grouped(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                          hipStream_t s);
hipError_t launch_slab(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s);
hipError_t launch_phase(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                        hipStream_t s);
hipError_t launch_staged(const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                         hipStream_t s);

// Backward-data filter rearrangement (see k_bwd.hip): per dimension the stride
// s, dilation e, low pad p, filter extent K and, per stride phase r < s, the
// first tap k0, the tap count T and the taps of all earlier phases pre.
constexpr int kMaxBwdStride = 16;
struct BwdGeom {
  int cout, cin, groups;   // forward C_out, C_in, G
  int k[3], s[3], e[3], p[3];
  int k0[3][kMaxBwdStride], t[3][kMaxBwdStride], pre[3][kMaxBwdStride];
};
hipError_t launch_bwd_filter(const BwdGeom& g, int dtype, const void* w, void* wt, hipStream_t s);

// The main path's tile configurations by number (0: the size-based choice of
// launch_main); the measured selection in conv_tune times them.
const int* main_tile_configs(int* count);
bool main_config_accepts(const ConvParams& p, int dtype, int config);
hipError_t launch_main_config(const ConvParams& p, int dtype, int config, const void* x, const void* w,
                              void* y, hipStream_t s);

// Main-path problems that share x and y and all take the main path (the
// stride phases of backward-data), launched together: problem i reads its
// filter w_off[i] bytes into w.
hipError_t launch_main_phased(const ConvParams* ps, const uint32_t* w_off, int count, int dtype,
                              const void* x, const void* w, void* y, hipStream_t s);

// Whether a path accepts a problem (host-side rules mirrored in convfwd.h).
bool main_accepts(const ConvParams& p, int dtype);
bool flatk_accepts(const ConvParams& p, int dtype);
bool rows_accepts(const ConvParams& p, int dtype);
bool brick_accepts(const ConvParams& p, int dtype);
bool strip_accepts(const ConvParams& p, int dtype);
bool runs_accepts(const ConvParams& p, int dtype);
bool grouped_accepts(const ConvParams& p, int dtype);
bool slab_accepts(const ConvParams& p, int dtype);
bool phase_accepts(const ConvParams& p, int dtype);
bool staged_accepts(const ConvParams& p, int dtype);

// Compute units of the current device (looked up once per device).
int device_cus();

}  // namespace convfwd
