// convfwd_api.cpp -- the C ABI declared in include/convfwd.h: descriptor
// validation, output extents, path selection and the launch on the caller's
// stream.  No device memory is allocated here and nothing is synchronised.
#include "../../include/convfwd.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "conv_params.h"

using convfwd::ConvParams;

namespace {

// floor((in + p + q - e*(k-1) - 1) / s) + 1: low / high padding p / q, k taps
// e apart; 0 when the padded input is shorter than the filter's span.
int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t q, int64_t e) {
  const int64_t span = in + p + q - (e * (k - 1) + 1);
  if (span < 0) return 0;
  return span / s + 1;
}

int elem_bytes(int dtype) { return dtype == CONVFWD_F32 ? 4 : 2; }

// Both descriptors as one: the plain one has the same padding on both sides
// of a dimension and an undilated filter.
convfwd_desc_ex widen(const convfwd_desc& d) {
  convfwd_desc_ex e;
  e.n = d.n; e.d = d.d; e.h = d.h; e.w = d.w;
  e.c_in = d.c_in; e.c_out = d.c_out;
  e.k_d = d.k_d; e.k_h = d.k_h; e.k_w = d.k_w;
  e.s_d = d.s_d; e.s_h = d.s_h; e.s_w = d.s_w;
  e.p_d = d.p_d; e.p_h = d.p_h; e.p_w = d.p_w;
  e.q_d = d.p_d; e.q_h = d.p_h; e.q_w = d.p_w;
  e.e_d = 1; e.e_h = 1; e.e_w = 1;
  e.groups = d.groups;
  e.dtype = d.dtype;
  return e;
}

// Validates the descriptor and fills the kernel parameters.  Returns an error
// code; on success every extent is positive except possibly n (n == 0 is a
// valid empty problem).
int make_params(const convfwd_desc_ex* d, ConvParams* p, int64_t* x_bytes, int64_t* w_bytes,
                int64_t* y_bytes) {
  if (!d) return CONVFWD_ERR_NULL;
  if (d->n < 0 || d->d < 1 || d->h < 1 || d->w < 1 || d->c_in < 1 || d->c_out < 1)
    return CONVFWD_ERR_BAD_DESC;
  if (d->k_d < 1 || d->k_h < 1 || d->k_w < 1) return CONVFWD_ERR_BAD_DESC;
  if (d->s_d < 1 || d->s_h < 1 || d->s_w < 1) return CONVFWD_ERR_BAD_DESC;
  if (d->p_d < 0 || d->p_h < 0 || d->p_w < 0) return CONVFWD_ERR_BAD_DESC;
  if (d->q_d < 0 || d->q_h < 0 || d->q_w < 0) return CONVFWD_ERR_BAD_DESC;
  if (d->e_d < 1 || d->e_h < 1 || d->e_w < 1) return CONVFWD_ERR_BAD_DESC;
  if (d->groups < 1) return CONVFWD_ERR_BAD_DESC;
  if (d->c_in % d->groups != 0 || d->c_out % d->groups != 0) return CONVFWD_ERR_BAD_DESC;
  if (d->dtype != CONVFWD_F32 && d->dtype != CONVFWD_F16 && d->dtype != CONVFWD_BF16)
    return CONVFWD_ERR_UNSUPPORTED;
  const int64_t od = out_extent(d->d, d->k_d, d->s_d, d->p_d, d->q_d, d->e_d);
  const int64_t oh = out_extent(d->h, d->k_h, d->s_h, d->p_h, d->q_h, d->e_h);
  const int64_t ow = out_extent(d->w, d->k_w, d->s_w, d->p_w, d->q_w, d->e_w);
  if (od < 1 || oh < 1 || ow < 1) return CONVFWD_ERR_BAD_DESC;

  const int64_t eb = elem_bytes(d->dtype);
  const int64_t spatial = (int64_t)d->d * d->h * d->w;
  const int64_t xe = (int64_t)d->n * spatial * d->c_in;
  const int64_t ntaps = (int64_t)d->k_d * d->k_h * d->k_w;
  const int64_t cin_g = d->c_in / d->groups;
  const int64_t ke = ntaps * cin_g;
  const int64_t we = (int64_t)d->c_out * ke;
  const int64_t M = (int64_t)d->n * od * oh * ow;
  const int64_t ye = M * d->c_out;
  const int64_t lim = (int64_t)1 << 31;
  // 32-bit signed byte offsets inside every tensor; also covers element offsets.
  if (spatial * d->c_in * eb >= lim || xe * eb >= lim || we * eb >= lim || ye * eb >= lim ||
      M >= lim || ke >= lim)
    return CONVFWD_ERR_TOO_LARGE;

  p->n = d->n; p->d = d->d; p->h = d->h; p->w = d->w;
  p->cin = d->c_in; p->cout = d->c_out;
  p->kd = d->k_d; p->kh = d->k_h; p->kw = d->k_w;
  p->sd = d->s_d; p->sh = d->s_h; p->sw = d->s_w;
  p->pd = d->p_d; p->ph = d->p_h; p->pw = d->p_w;
  p->ed = d->e_d; p->eh = d->e_h; p->ew = d->e_w;
  p->groups = d->groups;
  p->cin_g = (int)cin_g;
  p->cout_g = d->c_out / d->groups;
  p->od = (int)od; p->oh = (int)oh; p->ow = (int)ow;
  p->M = (int)M;
  p->ntaps = (int)ntaps;
  p->K = (int)ke;
  p->xs_w = d->c_in;
  p->xs_h = d->w * d->c_in;
  p->xs_d = d->h * d->w * d->c_in;
  p->xs_n = (int)(spatial * d->c_in);
  *x_bytes = xe * eb;
  *w_bytes = we * eb;
  *y_bytes = ye * eb;
  return CONVFWD_OK;
}

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// The brick path is available on request; on the measured shapes the
// per-tap-gather main path is faster, so AUTO does not pick it.
int auto_path(const ConvParams& p, int dtype) {
  // Few channels per group (down to depthwise): the memory-bound vector-ALU form.
  if (convfwd::grouped_accepts(p, dtype)) return CONVFWD_PATH_GROUPED;
  // The strip path wins once the w-taps share a strip (K_w >= 2); with K_w = 1
  // it is the main path with a larger tile and the main path is faster.
  if (p.kw >= 2 && convfwd::strip_accepts(p, dtype)) return CONVFWD_PATH_STRIP;
  if (convfwd::main_accepts(p, dtype)) return CONVFWD_PATH_MAIN;
  if (convfwd::rows_accepts(p, dtype)) return CONVFWD_PATH_ROWS;
  if (convfwd::runs_accepts(p, dtype)) return CONVFWD_PATH_RUNS;
  return CONVFWD_PATH_DIRECT;
}

bool path_accepts(int path, const ConvParams& p, int dtype) {
  switch (path) {
    case CONVFWD_PATH_MAIN: return convfwd::main_accepts(p, dtype);
    case CONVFWD_PATH_FLATK: return convfwd::flatk_accepts(p, dtype);
    case CONVFWD_PATH_ROWS: return convfwd::rows_accepts(p, dtype);
    case CONVFWD_PATH_DIRECT: return true;
    case CONVFWD_PATH_BRICK: return convfwd::brick_accepts(p, dtype);
    case CONVFWD_PATH_STRIP: return convfwd::strip_accepts(p, dtype);
    case CONVFWD_PATH_RUNS: return convfwd::runs_accepts(p, dtype);
    case CONVFWD_PATH_GROUPED: return convfwd::grouped_accepts(p, dtype);
    default: return false;
  }
}

int run(const convfwd_desc_ex* desc, int path, const void* x, const void* w, void* y, void* stream) {
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  if (path == CONVFWD_PATH_AUTO) path = auto_path(p, desc->dtype);
  if (!path_accepts(path, p, desc->dtype)) return CONVFWD_ERR_UNSUPPORTED;
  if (p.n == 0) return CONVFWD_OK;  // empty batch: nothing to read or write
  if (!x || !w || !y) return CONVFWD_ERR_NULL;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb)) return CONVFWD_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  switch (path) {
    case CONVFWD_PATH_MAIN: e = convfwd::launch_main(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_FLATK: e = convfwd::launch_flatk(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_ROWS: e = convfwd::launch_rows(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_BRICK: e = convfwd::launch_brick(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_STRIP: e = convfwd::launch_strip(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_RUNS: e = convfwd::launch_runs(p, desc->dtype, x, w, y, s); break;
    case CONVFWD_PATH_GROUPED: e = convfwd::launch_grouped(p, desc->dtype, x, w, y, s); break;
    default: e = convfwd::launch_direct(p, desc->dtype, x, w, y, s); break;
  }
  if (e != hipSuccess) return CONVFWD_ERR_LAUNCH;
  return CONVFWD_OK;
}

}  // namespace

extern "C" {

int conv_out_shape_ex(const convfwd_desc_ex* desc, int64_t out[5]) {
  if (!out) return CONVFWD_ERR_NULL;
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  out[0] = p.n; out[1] = p.od; out[2] = p.oh; out[3] = p.ow; out[4] = p.cout;
  return CONVFWD_OK;
}

int conv_select_path_ex(const convfwd_desc_ex* desc) {
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  return auto_path(p, desc->dtype);
}

int conv_fwd_ex(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream) {
  return run(desc, CONVFWD_PATH_AUTO, x, w, y, stream);
}

int conv_fwd_path_ex(const convfwd_desc_ex* desc, int path, const void* x, const void* w, void* y,
                     void* stream) {
  if (path < CONVFWD_PATH_AUTO || path > CONVFWD_PATH_GROUPED) return CONVFWD_ERR_UNSUPPORTED;
  return run(desc, path, x, w, y, stream);
}

int conv_out_shape(const convfwd_desc* desc, int64_t out[5]) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return conv_out_shape_ex(&e, out);
}

int conv_select_path(const convfwd_desc* desc) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return conv_select_path_ex(&e);
}

int conv_fwd(const convfwd_desc* desc, const void* x, const void* w, void* y, void* stream) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return conv_fwd_ex(&e, x, w, y, stream);
}

int conv_fwd_path(const convfwd_desc* desc, int path, const void* x, const void* w, void* y,
                  void* stream) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return conv_fwd_path_ex(&e, path, x, w, y, stream);
}

const char* conv_strerror(int code) {
  switch (code) {
    case CONVFWD_OK: return "success";
    case CONVFWD_ERR_NULL: return "a required pointer is NULL";
    case CONVFWD_ERR_BAD_DESC: return "bad descriptor: non-positive extent, stride or dilation < 1, pad < 0, groups not dividing the channels, or empty output";
    case CONVFWD_ERR_UNSUPPORTED: return "unsupported: unknown dtype, or the path cannot take this problem";
    case CONVFWD_ERR_TOO_LARGE: return "too large: a tensor reaches 2^31 bytes or M reaches 2^31";
    case CONVFWD_ERR_ALIAS: return "the output overlaps an input";
    case CONVFWD_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

const char* conv_path_name(int path) {
  switch (path) {
    case CONVFWD_PATH_AUTO: return "auto";
    case CONVFWD_PATH_MAIN: return "main";
    case CONVFWD_PATH_FLATK: return "flatk";
    case CONVFWD_PATH_ROWS: return "rows";
    case CONVFWD_PATH_DIRECT: return "direct";
    case CONVFWD_PATH_BRICK: return "brick";
    case CONVFWD_PATH_STRIP: return "strip";
    case CONVFWD_PATH_RUNS: return "runs";
    case CONVFWD_PATH_GROUPED: return "grouped";
    default: return "unknown";
  }
}

}  // extern "C"
