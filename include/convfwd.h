/*
 * convfwd.h -- C ABI of the channels-last implicit-GEMM convolution library
 * for AMD Instinct MI355X (gfx950): the forward pass, and backward-data (the
 * transposed convolution) built on it.
 *
 * The operation (the "Convolutions" tutorial page, sections 1 and 4, and the
 * MLX pull request "Add implicit matmul pathway for mx.conv3d", benchmark
 * table header for the layouts): for every output position and output
 * channel,
 *
 *   y[n,od,oh,ow,co] = sum_{kd,kh,kw,c} X(n, od*s_d - p_d + kd,
 *                                          oh*s_h - p_h + kh,
 *                                          ow*s_w - p_w + kw, c) * w[co,kd,kh,kw,c]
 *
 * with X the input extended by zeros outside its extent.  The filter is not
 * flipped (the tutorial's worked example fixes the orientation).  Output
 * extents are floor((in + 2p - k)/s) + 1.
 *
 * The variants the tutorial lists among "Convolution variants worth knowing"
 * take the same sum and are reached through convfwd_desc_ex: grouped
 * (channels split into G groups; output channel co reads only the C_in/G input
 * channels of its group g = co / (C_out/G), X's channel g*C_in/G + c), dilated
 * (tap t sits t*e positions past the window origin, "gaps in the kernel"), and
 * padded differently on the low (p) and high (q) side of a dimension; then
 * extents are floor((in + p + q - e*(k-1) - 1)/s) + 1.  The result is computed as an
 * implicit GEMM (tutorial section 5, "Alternatives"): M = N*D_out*H_out*W_out
 * rows, N_gemm = C_out columns, K = C_in*K_d*K_h*K_w, with the im2col operand
 * addressed on the fly inside the kernel and never stored.
 *
 * Layouts (all dense, innermost dimension last, no padding between rows):
 *   x  (N, D, H, W, C_in)                   channels-last input
 *   w  (C_out, K_d, K_h, K_w, C_in/G)       filter, C_in/G fastest (G = 1 unless grouped)
 *   y  (N, D_out, H_out, W_out, C_out)      channels-last output, same dtype as x
 * A 2D problem is the 3D one with d = k_d = s_d = 1 and p_d = 0.
 *
 * Arithmetic: fp16 and bf16 inputs are multiplied exactly and accumulated in
 * fp32; the result is rounded once to the output dtype, round-to-nearest-even.
 * fp32 inputs are accumulated in fp32.  The summation order is unspecified.
 *
 * Ownership: the caller owns x, w, y and the stream.  The library allocates
 * no device memory (no workspace, no im2col buffer), never frees and never
 * synchronises (except conv_tune, which times launches); its one piece of
 * mutable state is the table of measured choices that conv_tune fills, guarded
 * by a mutex, so calls are reentrant and may be made from several host
 * threads.
 *
 * Errors: every entry point validates its arguments before touching the GPU
 * and returns 0 or one of the negative codes below.  Faults inside a kernel
 * are asynchronous: they surface at the caller's next synchronisation on the
 * stream, not in a return code.
 */
#ifndef CONVFWD_H
#define CONVFWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CONVFWD_F32 = 0,
  CONVFWD_F16 = 1,
  CONVFWD_BF16 = 2
} convfwd_dtype;

/* Return codes. */
enum {
  CONVFWD_OK = 0,
  CONVFWD_ERR_NULL = -1,        /* a required pointer is NULL */
  CONVFWD_ERR_BAD_DESC = -2,    /* a non-positive extent, stride or dilation < 1, pad < 0, groups < 1
                                   or not dividing C_in and C_out, or an empty output */
  CONVFWD_ERR_UNSUPPORTED = -3, /* unknown dtype, or a path that cannot take this problem */
  CONVFWD_ERR_TOO_LARGE = -4,   /* a tensor of 2^31 bytes or more, or M >= 2^31 */
  CONVFWD_ERR_ALIAS = -5,       /* y's byte range overlaps x or w */
  CONVFWD_ERR_LAUNCH = -6,      /* the HIP runtime refused the launch */
  CONVFWD_ERR_MISALIGNED = -7   /* a tensor pointer not aligned to its element size */
};

/* Kernel paths.  AUTO lets the library choose; the others force one (for
 * testing every path on every shape it accepts). */
typedef enum {
  CONVFWD_PATH_AUTO = 0,
  CONVFWD_PATH_MAIN = 1,   /* fp16/bf16, C_in/G % 32 == 0, C_out/G % 4 == 0, filter <= 16 per dim:
                              16-byte channels-last loads straight into LDS, MFMA */
  CONVFWD_PATH_FLATK = 2,  /* any C_in, filter <= 16 per dim, G = 1, undilated: element-granular
                              gathers over the flattened (tap, channel) axis, MFMA */
  CONVFWD_PATH_ROWS = 3,   /* fp16/bf16 tiny C_in (C_in * K_w <= 32, 2D or 3D), G = 1, undilated:
                              whole input rows staged in LDS, MFMA */
  CONVFWD_PATH_DIRECT = 4, /* any problem: one thread per output, fp32 FMA (slow, simple) */
  CONVFWD_PATH_BRICK = 5,  /* fp16/bf16, G = 1, undilated, C_in % 16 == 0, C_out % 4 == 0, >= 4 taps, filter <= 16
                              per dim and a brick that fits: the input brick of a box of up to
                              512 outputs staged in LDS per 16-channel chunk, every tap read
                              from it, MFMA */
  CONVFWD_PATH_STRIP = 6,  /* fp16/bf16, G = 1, C_in % 32 == 0, C_out % 4 == 0, stride and dilation 1 along w,
                              W_out % 32 == 0, K_w <= 5, K_d, K_h <= 16: per (channel chunk,
                              kd, kh) one input strip per 32-output w-segment staged in LDS,
                              all K_w taps read from it, 512 x 128 tiles, MFMA */
  CONVFWD_PATH_RUNS = 7,   /* any dtype and C_in, filter <= 16 per dim, x and w of at least 16
                              bytes (the unaligned-channel tail path and fp32): the K_w * C_in
                              columns of each (kd, kh) read as one contiguous run, 16-byte
                              unaligned pieces, MFMA; with few tiles, 16-row tiles whose four
                              waves split the K walk */
  CONVFWD_PATH_GROUPED = 8, /* any dtype, G > 1 with C_in/G in {1, 2, 4, 8, 16}, C_out/G <= 16 and
                              C_out * K_d*K_h*K_w * C_in/G <= 16384 (depthwise and small groups):
                              one thread per (output position, group), fp32 FMA, filter in LDS */
  CONVFWD_PATH_SLAB = 9,   /* fp16/bf16, C_in/G % 32 == 0, C_out % 4 == 0, G = 1 or C_out/G % 64 == 0,
                              stride 1 along h and w, K_h in {2, 3}, K_w <= 3, K_d <= 16,
                              dilation 1 along h and w or 2 along both with K_h = K_w = 3:
                              tiles of 16 output rows x 32 outputs (ragged at the ends) x 128
                              or 64 channels (64 within one group, for C_out <= 64, and when
                              128-channel tiles would be fewer than the device's compute
                              units); per (channel chunk, kd) the input rows those windows
                              cover (18, dilated 20) are staged in LDS once and all K_h * K_w
                              taps read from them, MFMA */
  CONVFWD_PATH_PHASE = 10, /* fp16/bf16, C_in/G % 64 == 0, C_out % 4 == 0, G = 1 or C_out/G % 64 == 0,
                              stride 2 along h and w, K_h and K_w in {2, 3}, dilation 1 along h and
                              w, K_d <= 16: tiles of 8 output rows x 16 outputs (ragged at the
                              ends) x 64 channels; per (64-channel chunk, kd) the input rows the
                              windows cover are staged in LDS split by stride phase (even rows and
                              odd rows, each row's even positions before its odd ones), so every
                              tap reads consecutive slots, MFMA */
  CONVFWD_PATH_STAGED = 11 /* fp16/bf16, G = 1, C_in >= 8 with (C_in % 8) * K_d*K_h*K_w <= 32 (and K_d <= 3
                              when C_in % 8 != 0), stride 1 and dilation 1 along h and w, K_h and
                              K_w in {2, 3}, K_d <= 16,
                              element-aligned tensors suffice: the slab scheme with the input
                              staged through registers (unaligned 16-byte loads, so positions of
                              any channel count), tiles of 16 output rows x 32 outputs x 32, 64
                              or 80 channels; channels below C_in - C_in % 8 walk the slab in
                              32-channel chunks, the C_in % 8 left over are packed across all taps
                              into one extra K block of 32, MFMA */
} convfwd_path;

/* Problem descriptor.  All extents in elements. */
typedef struct {
  int32_t n, d, h, w;        /* input batch and spatial extents (d = 1 for 2D) */
  int32_t c_in, c_out;       /* channels */
  int32_t k_d, k_h, k_w;     /* filter extents (k_d = 1 for 2D) */
  int32_t s_d, s_h, s_w;     /* strides, >= 1 */
  int32_t p_d, p_h, p_w;     /* zero padding added on both sides, >= 0 */
  int32_t groups;            /* channel groups G >= 1 dividing c_in and c_out (1: plain) */
  int32_t dtype;             /* convfwd_dtype; x, w and y share it */
} convfwd_desc;

/* Extended descriptor: as convfwd_desc, plus the padding of the high side of
 * each dimension and the filter dilation.  A convfwd_desc is the extended one
 * with q_* = p_* and e_* = 1. */
typedef struct {
  int32_t n, d, h, w;        /* input batch and spatial extents (d = 1 for 2D) */
  int32_t c_in, c_out;       /* channels */
  int32_t k_d, k_h, k_w;     /* filter extents (taps per dimension) */
  int32_t s_d, s_h, s_w;     /* strides, >= 1 */
  int32_t p_d, p_h, p_w;     /* zero padding before the first element (low side), >= 0 */
  int32_t q_d, q_h, q_w;     /* zero padding after the last element (high side), >= 0 */
  int32_t e_d, e_h, e_w;     /* filter dilation, >= 1: tap t sits t*e positions past the origin */
  int32_t groups;            /* channel groups G >= 1 dividing c_in and c_out */
  int32_t dtype;             /* convfwd_dtype; x, w and y share it */
} convfwd_desc_ex;

/* Output shape (N, D_out, H_out, W_out, C_out) into out[5].  Host only; never
 * touches the GPU.  Returns CONVFWD_OK or a validation error. */
int conv_out_shape(const convfwd_desc* desc, int64_t out[5]);

/* The path CONVFWD_PATH_AUTO would take for this descriptor with 16-byte
 * aligned tensors (a positive convfwd_path), or a negative validation error.
 * Host only. */
int conv_select_path(const convfwd_desc* desc);

/* y = conv(x, w) on `stream` (a hipStream_t; NULL means the null stream of the
 * current device).  x, w, y are device pointers on the current device, laid
 * out as above, each aligned to its element size (2 bytes for fp16/bf16, 4 for
 * fp32; else CONVFWD_ERR_MISALIGNED).  The fast paths (slab, phase, strip,
 * main, brick, rows, flatk) move 16-byte pieces counted from the base pointers and
 * need x, w and y all 16-byte aligned: with a tensor that is not, AUTO keeps to
 * the paths that need element alignment only (staged, else runs, else direct;
 * grouped checks its own 16-byte kernel), and a forced 16-byte path returns
 * CONVFWD_ERR_UNSUPPORTED
 * (the MLX pull request's dispatch falls back rather than failing).  Tensors
 * from an allocator are 256-byte aligned; a view at an element offset may not
 * be.  Asynchronous: returns after the launch.  With N = 0 it launches nothing
 * and returns CONVFWD_OK without reading the pointers (a forced path must
 * still accept the problem). */
int conv_fwd(const convfwd_desc* desc, const void* x, const void* w, void* y, void* stream);

/* As conv_fwd, but on the given path; CONVFWD_ERR_UNSUPPORTED if that path
 * cannot take the problem. */
int conv_fwd_path(const convfwd_desc* desc, int path, const void* x, const void* w, void* y,
                  void* stream);

/* The four calls above for an extended descriptor (same arguments, same
 * rules; every path takes groups, dilation and asymmetric padding except as
 * its comment in convfwd_path restricts). */
int conv_out_shape_ex(const convfwd_desc_ex* desc, int64_t out[5]);
int conv_select_path_ex(const convfwd_desc_ex* desc);
int conv_fwd_ex(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream);
int conv_fwd_path_ex(const convfwd_desc_ex* desc, int path, const void* x, const void* w, void* y,
                     void* stream);

/* ---- Measured selection (a table of timed choices) ----
 *
 * The practice the tutorial describes for cuDNN ("Convolutions", section 6,
 * "Under the hood"): try the algorithms on a shape, keep the fastest, and for
 * varying shapes bucket the sizes.  conv_tune times, on `stream`, every path
 * that accepts the problem and every tile configuration of the main path (the
 * direct path only when nothing else accepts the problem or it is small): one
 * warm-up launch and `reps` (1..1000) timed launches each, between two HIP
 * events, so it synchronises the stream.  It records the fastest choice in a
 * process-wide table twice, under the exact descriptor and under its bucket
 * (N, D, H, W rounded up to powers of two, the other fields exact), leaves y
 * holding that choice's result and returns its path (> 0); *best_us (if not
 * NULL) receives its mean launch time.  x, w, y as for conv_fwd; y is written
 * many times.  With N = 0 nothing is timed and the size-based path is
 * returned.
 *
 * From then on CONVFWD_PATH_AUTO (conv_fwd, conv_select_path) takes the
 * recorded choice for the exact descriptor, else for its bucket, when that
 * choice accepts the problem, and the size-based choice otherwise.
 * conv_tuned_path returns the recorded path for a descriptor (exact, then
 * bucket) or 0; conv_tune_clear empties the table.  The table is the
 * library's only mutable state; a mutex guards it, so every call stays safe
 * from several host threads (a lookup on an empty table takes no lock). */
int conv_tune(const convfwd_desc* desc, const void* x, const void* w, void* y, void* stream, int reps,
              float* best_us);
int conv_tune_ex(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream, int reps,
                 float* best_us);
int conv_tuned_path_ex(const convfwd_desc_ex* desc);
int conv_tune_clear(void);

/* ---- Backward-data (the transposed convolution) ----
 *
 * The gradient with respect to x of the forward convolution `desc` (the
 * "Transposed" entry, upsampling convolution, of the tutorial's "Convolution
 * variants worth knowing"; the MLX pull request's general path builds it from
 * input dilation and a flipped filter):
 *
 *   dx[n,id,ih,iw,c] = sum over co of c's group and taps (kd,kh,kw) with
 *       od = (id + p_d - kd*e_d) / s_d a whole number in [0, D_out)  (likewise h, w)
 *     of dy[n,od,oh,ow,co] * w[co,kd,kh,kw,c - g*C_in/G]
 *
 * dx has x's shape, dy has y's shape, w is the forward filter; positions no
 * output window covers get 0.  A transposed convolution layer that upsamples
 * u by stride s is this call with dy = u and desc describing the downsampling
 * convolution whose input has the upsampled shape.  Strides up to 16 per
 * dimension (CONVFWD_ERR_UNSUPPORTED beyond).
 *
 * Two calls.  conv_bwd_data_filter rearranges w into wt, a caller-owned
 * device buffer of w's size and dtype, which must not overlap w: per stride
 * phase (the dx positions with the same index mod s), the taps that reach it,
 * reversed, with input and output channels exchanged.  It depends only on w
 * and the descriptor, so it can be prepared once per filter.  conv_bwd_data
 * then computes dx from dy and wt as s_d*s_h*s_w forward convolutions over dy
 * (one per phase, each writing every s-th position of dx), launched in order
 * on `stream`; dx must overlap neither dy nor wt.  Same pointer, alignment,
 * asynchrony and error rules as conv_fwd; nothing is allocated.
 * conv_bwd_data_path forces the kernel of the phases: CONVFWD_PATH_MAIN,
 * CONVFWD_PATH_RUNS or CONVFWD_PATH_DIRECT (CONVFWD_ERR_UNSUPPORTED if it
 * cannot take a phase; phases that no tap reaches are always zero-filled by
 * the direct kernel); AUTO picks per phase. */
int conv_bwd_data_filter(const convfwd_desc* desc, const void* w, void* wt, void* stream);
int conv_bwd_data(const convfwd_desc* desc, const void* dy, const void* wt, void* dx, void* stream);
int conv_bwd_data_filter_ex(const convfwd_desc_ex* desc, const void* w, void* wt, void* stream);
int conv_bwd_data_ex(const convfwd_desc_ex* desc, const void* dy, const void* wt, void* dx, void* stream);
int conv_bwd_data_path_ex(const convfwd_desc_ex* desc, int path, const void* dy, const void* wt, void* dx,
                          void* stream);

/* Static message for a return code; never NULL. */
const char* conv_strerror(int code);

/* Static name of a path ("auto", "main", "flatk", "rows", "direct", "brick", "strip", "runs",
 * "grouped", "slab", "phase", "staged"); never NULL. */
const char* conv_path_name(int path);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_H */
