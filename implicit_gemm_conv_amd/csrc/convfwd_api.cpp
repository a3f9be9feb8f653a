// convfwd_api.cpp -- the C ABI declared in include/convfwd.h: descriptor
// validation, output extents, path selection and the launch on the caller's
// stream.  No device memory is allocated here and nothing is synchronised.
#include "../../include/convfwd.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "conv_params.h"

namespace convfwd {

// Compute units of the current device, looked up once per device (relaxed
// atomics: threads that race on the first lookup store the same value).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    v = cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace convfwd

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
  p->remap = 0;
  p->ys_w = d->c_out;
  p->ys_h = (int)(ow * d->c_out);
  p->ys_d = (int)(oh * ow * d->c_out);
  p->ys_n = (int)(od * oh * ow * d->c_out);
  p->y_off = 0;
  *x_bytes = xe * eb;
  *w_bytes = we * eb;
  *y_bytes = ye * eb;
  return CONVFWD_OK;
}

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// Paths whose kernels move x, w and y in 16-byte pieces at offsets counted
// from the base pointers (direct-to-LDS buffer loads, 16-byte stores): they
// need all three tensors 16-byte aligned.  The runs, direct and grouped paths
// need element alignment only (the grouped path checks for its 16-byte
// kernel itself).
bool needs_16(int path) {
  switch (path) {
    case CONVFWD_PATH_SLAB:
    case CONVFWD_PATH_STRIP:
    case CONVFWD_PATH_MAIN:
    case CONVFWD_PATH_BRICK:
    case CONVFWD_PATH_ROWS:
    case CONVFWD_PATH_FLATK:
    case CONVFWD_PATH_PHASE: return true;
    default: return false;
  }
}

bool aligned_to(const void* a, const void* b, const void* c, uintptr_t bytes) {
  return (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & (bytes - 1)) == 0;
}

// The brick path is available on request; on the measured shapes the
// per-tap-gather main path is faster, so AUTO does not pick it.  With tensors
// that are not all 16-byte aligned AUTO keeps to the paths that need element
// alignment only (staged, runs, else direct), the fall-back-rather-than-fail
// rule of the MLX pull request's dispatch.
int auto_path(const ConvParams& p, int dtype, bool al16 = true) {
  // Few channels per group (down to depthwise): the memory-bound vector-ALU form.
  if (convfwd::grouped_accepts(p, dtype)) return CONVFWD_PATH_GROUPED;
  // The slab and staged paths compute whole blocks of 16 rows x 32 outputs;
  // they are taken when at least 70% of that area lies inside the output (on
  // (32,56^2,256) with 77% the slab path runs 1.17x faster than the main path).
  const int64_t wpad = (p.ow + 31) / 32 * 32, hpad = (p.oh + 15) / 16 * 16;
  const bool blocks_fit = 10 * (int64_t)p.ow * p.oh >= 7 * wpad * hpad;
  const bool staged = blocks_fit && convfwd::staged_accepts(p, dtype);
  if (!al16) {
    if (staged) return CONVFWD_PATH_STAGED;
    return convfwd::runs_accepts(p, dtype) ? CONVFWD_PATH_RUNS : CONVFWD_PATH_DIRECT;
  }
  // Once the w-taps share a strip (K_w >= 2): the slab path where the h-taps
  // share its staged rows too, else the strip path.  With K_w = 1 the strip
  // path is the main path with a larger tile and the main path is faster.
  if (p.kw >= 2 && blocks_fit && convfwd::slab_accepts(p, dtype)) return CONVFWD_PATH_SLAB;
  if (p.kw >= 2 && convfwd::strip_accepts(p, dtype)) return CONVFWD_PATH_STRIP;
  // Stride 2 along h and w with 64-channel chunks: the stride-phase staging.
  if (convfwd::phase_accepts(p, dtype)) return CONVFWD_PATH_PHASE;
  if (convfwd::main_accepts(p, dtype)) return CONVFWD_PATH_MAIN;
  if (convfwd::rows_accepts(p, dtype)) return CONVFWD_PATH_ROWS;
  // Channel counts the 16-byte paths cannot take (C_in = 65): the slab scheme
  // staged through registers, else whole-window runs.
  if (staged) return CONVFWD_PATH_STAGED;
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
    case CONVFWD_PATH_SLAB: return convfwd::slab_accepts(p, dtype);
    case CONVFWD_PATH_PHASE: return convfwd::phase_accepts(p, dtype);
    case CONVFWD_PATH_STAGED: return convfwd::staged_accepts(p, dtype);
    default: return false;
  }
}

hipError_t launch_path(int path, const ConvParams& p, int dtype, const void* x, const void* w, void* y,
                       hipStream_t s) {
  switch (path) {
    case CONVFWD_PATH_MAIN: return convfwd::launch_main(p, dtype, x, w, y, s);
    case CONVFWD_PATH_FLATK: return convfwd::launch_flatk(p, dtype, x, w, y, s);
    case CONVFWD_PATH_ROWS: return convfwd::launch_rows(p, dtype, x, w, y, s);
    case CONVFWD_PATH_BRICK: return convfwd::launch_brick(p, dtype, x, w, y, s);
    case CONVFWD_PATH_STRIP: return convfwd::launch_strip(p, dtype, x, w, y, s);
    case CONVFWD_PATH_RUNS: return convfwd::launch_runs(p, dtype, x, w, y, s);
    case CONVFWD_PATH_GROUPED: return convfwd::launch_grouped(p, dtype, x, w, y, s);
    case CONVFWD_PATH_SLAB: return convfwd::launch_slab(p, dtype, x, w, y, s);
    case CONVFWD_PATH_PHASE: return convfwd::launch_phase(p, dtype, x, w, y, s);
    case CONVFWD_PATH_STAGED: return convfwd::launch_staged(p, dtype, x, w, y, s);
    default: return convfwd::launch_direct(p, dtype, x, w, y, s);
  }
}

// ---- measured selection: a table of timed choices keyed by the descriptor ----
//
// The tutorial page ("Convolutions", section 6, *Under the hood*) describes
// the cuDNN practice: try the algorithms on a shape, cache the fastest, and
// for varying shapes bucket the sizes.  conv_tune times every path (and every
// main-path tile configuration) that accepts a problem and records the
// fastest twice: under the exact descriptor and under its bucket (batch and
// spatial extents rounded up to powers of two).  AUTO looks up the exact key,
// then the bucket, then falls back to the size-based choice; a recorded
// choice is used only if it accepts the problem at hand.

struct TuneKey {
  int32_t f[24];
  bool operator==(const TuneKey& o) const { return std::memcmp(f, o.f, sizeof(f)) == 0; }
};
struct TuneKeyHash {
  size_t operator()(const TuneKey& k) const {
    uint64_t h = 1469598103934665603ull;   // FNV-1a over the key's bytes
    const unsigned char* b = (const unsigned char*)k.f;
    for (size_t i = 0; i < sizeof(k.f); ++i) h = (h ^ b[i]) * 1099511628211ull;
    return (size_t)h;
  }
};
struct Choice {
  int path, config;
  float us;
};

std::mutex& tune_mutex() {
  static std::mutex m;
  return m;
}
std::unordered_map<TuneKey, Choice, TuneKeyHash>& tune_table() {
  static std::unordered_map<TuneKey, Choice, TuneKeyHash> t;
  return t;
}
std::atomic<int>& tune_count() {
  static std::atomic<int> c{0};
  return c;
}

int32_t pow2_ceil(int32_t v) {
  int32_t r = 1;
  while (r < v && r < (1 << 30)) r <<= 1;
  return r;
}

TuneKey tune_key(const convfwd_desc_ex& d, bool bucket) {
  TuneKey k;
  std::memset(&k, 0, sizeof(k));
  const int32_t v[23] = {d.n, d.d, d.h, d.w, d.c_in, d.c_out, d.k_d, d.k_h, d.k_w, d.s_d, d.s_h, d.s_w,
                         d.p_d, d.p_h, d.p_w, d.q_d, d.q_h, d.q_w, d.e_d, d.e_h, d.e_w, d.groups, d.dtype};
  std::memcpy(k.f, v, sizeof(v));
  if (bucket)
    for (int i = 0; i < 4; ++i) k.f[i] = pow2_ceil(k.f[i]);
  k.f[23] = bucket ? 1 : 0;
  return k;
}

bool choice_accepts(const Choice& c, const ConvParams& p, int dtype) {
  if (c.path == CONVFWD_PATH_MAIN) return convfwd::main_config_accepts(p, dtype, c.config);
  return path_accepts(c.path, p, dtype);
}

// The recorded choice for the descriptor (exact key, then bucket) if it
// accepts the problem; false when there is none.
bool tuned_choice(const convfwd_desc_ex& d, const ConvParams& p, Choice* out) {
  if (tune_count().load(std::memory_order_acquire) == 0) return false;
  std::lock_guard<std::mutex> lock(tune_mutex());
  for (int b = 0; b < 2; ++b) {
    auto it = tune_table().find(tune_key(d, b == 1));
    if (it != tune_table().end() && choice_accepts(it->second, p, d.dtype)) {
      *out = it->second;
      return true;
    }
  }
  return false;
}

hipError_t launch_choice(const Choice& c, const ConvParams& p, int dtype, const void* x, const void* w,
                         void* y, hipStream_t s) {
  if (c.path == CONVFWD_PATH_MAIN) return convfwd::launch_main_config(p, dtype, c.config, x, w, y, s);
  return launch_path(c.path, p, dtype, x, w, y, s);
}

int run(const convfwd_desc_ex* desc, int path, const void* x, const void* w, void* y, void* stream) {
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  const bool al16 = aligned_to(x, w, y, 16);
  Choice tuned;
  bool use_tuned = path == CONVFWD_PATH_AUTO && tuned_choice(*desc, p, &tuned);
  if (use_tuned && !al16 && needs_16(tuned.path)) use_tuned = false;
  if (path == CONVFWD_PATH_AUTO) path = use_tuned ? tuned.path : auto_path(p, desc->dtype, al16);
  if (!path_accepts(path, p, desc->dtype)) return CONVFWD_ERR_UNSUPPORTED;
  if (!al16 && needs_16(path)) return CONVFWD_ERR_UNSUPPORTED;   // a forced 16-byte path
  if (p.n == 0) return CONVFWD_OK;  // empty batch: nothing to read or write
  if (!x || !w || !y) return CONVFWD_ERR_NULL;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb)) return CONVFWD_ERR_ALIAS;
  if (!aligned_to(x, w, y, (uintptr_t)elem_bytes(desc->dtype))) return CONVFWD_ERR_MISALIGNED;
  const hipError_t e = use_tuned ? launch_choice(tuned, p, desc->dtype, x, w, y, (hipStream_t)stream)
                                 : launch_path(path, p, desc->dtype, x, w, y, (hipStream_t)stream);
  if (e != hipSuccess) return CONVFWD_ERR_LAUNCH;
  return CONVFWD_OK;
}

int run_tune(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream, int reps,
             float* best_us) {
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  if (reps < 1 || reps > 1000) return CONVFWD_ERR_BAD_DESC;
  if (p.n == 0) return auto_path(p, desc->dtype);   // nothing to time
  if (!x || !w || !y) return CONVFWD_ERR_NULL;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb)) return CONVFWD_ERR_ALIAS;
  if (!aligned_to(x, w, y, (uintptr_t)elem_bytes(desc->dtype))) return CONVFWD_ERR_MISALIGNED;
  // candidates: every accepting path (the 16-byte ones only for 16-byte aligned
  // tensors), the main path once per tile configuration; the direct path only
  // when nothing else takes the problem or it is small
  const bool al16 = aligned_to(x, w, y, 16);
  Choice cand[64];
  int nc = 0;
  const int paths[] = {CONVFWD_PATH_SLAB, CONVFWD_PATH_STRIP, CONVFWD_PATH_PHASE, CONVFWD_PATH_STAGED,
                       CONVFWD_PATH_GROUPED, CONVFWD_PATH_ROWS, CONVFWD_PATH_RUNS, CONVFWD_PATH_FLATK,
                       CONVFWD_PATH_BRICK};
  for (int q : paths)
    if (path_accepts(q, p, desc->dtype) && (al16 || !needs_16(q))) cand[nc++] = Choice{q, 0, 0.f};
  int ncfg = 0;
  const int* cfgs = convfwd::main_tile_configs(&ncfg);
  for (int i = 0; i < ncfg && al16; ++i)
    if (convfwd::main_config_accepts(p, desc->dtype, cfgs[i])) cand[nc++] = Choice{CONVFWD_PATH_MAIN, cfgs[i], 0.f};
  const double macs = (double)p.M * p.cout_g * p.K;
  if (nc == 0 || macs < 1e8) cand[nc++] = Choice{CONVFWD_PATH_DIRECT, 0, 0.f};

  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return CONVFWD_ERR_LAUNCH;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return CONVFWD_ERR_LAUNCH;
  }
  int best = -1;
  int err = CONVFWD_OK;
  for (int i = 0; i < nc && err == CONVFWD_OK; ++i) {
    if (launch_choice(cand[i], p, desc->dtype, x, w, y, s) != hipSuccess) { err = CONVFWD_ERR_LAUNCH; break; }
    if (hipEventRecord(e0, s) != hipSuccess) { err = CONVFWD_ERR_LAUNCH; break; }
    for (int r = 0; r < reps; ++r)
      if (launch_choice(cand[i], p, desc->dtype, x, w, y, s) != hipSuccess) { err = CONVFWD_ERR_LAUNCH; break; }
    if (err != CONVFWD_OK) break;
    float ms = 0.f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      err = CONVFWD_ERR_LAUNCH;
      break;
    }
    cand[i].us = ms * 1000.f / reps;
    if (best < 0 || cand[i].us < cand[best].us) best = i;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != CONVFWD_OK) return err;
  // leave y holding the chosen path's result
  if (launch_choice(cand[best], p, desc->dtype, x, w, y, s) != hipSuccess) return CONVFWD_ERR_LAUNCH;
  {
    std::lock_guard<std::mutex> lock(tune_mutex());
    tune_table()[tune_key(*desc, false)] = cand[best];
    tune_table()[tune_key(*desc, true)] = cand[best];
    tune_count().store((int)tune_table().size(), std::memory_order_release);
  }
  if (best_us) *best_us = cand[best].us;
  return cand[best].path;
}

// ---- backward-data: stride phases (see k_bwd.hip for the derivation) ----

// One dimension's share of one stride phase r: J dx positions j*s + r, the T
// taps k0, k0 + s', ... that reach them, and the phase convolution over dy at
// unit stride with dilation ep and low pad P (negative when the window starts
// past the output position).
struct PhaseDim {
  int J, k0, T, P, ep;
};

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

void phase_dims(int I, int K, int s, int p, int e, PhaseDim* out) {
  const int g = gcd_int(e, s), sp = s / g, ep = e / g;
  for (int r = 0; r < s; ++r) {
    PhaseDim& d = out[r];
    d.J = r < I ? (I - r + s - 1) / s : 0;
    d.ep = ep;
    d.k0 = -1;
    for (int k = 0; k < sp; ++k)
      if ((((k * e - r - p) % s) + s) % s == 0) {
        d.k0 = k;
        break;
      }
    if (d.k0 < 0 || d.k0 >= K) {
      d.k0 = 0; d.T = 0; d.P = 0;
      continue;
    }
    d.T = (K - d.k0 + sp - 1) / sp;
    const int q0 = (r + p - d.k0 * e) / s;   // exact: k0*e = r + p (mod s)
    d.P = (d.T - 1) * ep - q0;
  }
}

struct BwdPlan {
  ConvParams fwd;
  int64_t x_bytes, w_bytes, y_bytes;
  convfwd::BwdGeom geom;
  PhaseDim ph[3][convfwd::kMaxBwdStride];
};

int make_bwd_plan(const convfwd_desc_ex* d, BwdPlan* b) {
  const int rc = make_params(d, &b->fwd, &b->x_bytes, &b->w_bytes, &b->y_bytes);
  if (rc != CONVFWD_OK) return rc;
  const ConvParams& f = b->fwd;
  const int st[3] = {f.sd, f.sh, f.sw}, ks[3] = {f.kd, f.kh, f.kw}, pads[3] = {f.pd, f.ph, f.pw};
  const int dil[3] = {f.ed, f.eh, f.ew}, in[3] = {f.d, f.h, f.w};
  for (int i = 0; i < 3; ++i)
    if (st[i] > convfwd::kMaxBwdStride) return CONVFWD_ERR_UNSUPPORTED;
  convfwd::BwdGeom& g = b->geom;
  g.cout = f.cout; g.cin = f.cin; g.groups = f.groups;
  for (int i = 0; i < 3; ++i) {
    g.k[i] = ks[i]; g.s[i] = st[i]; g.e[i] = dil[i]; g.p[i] = pads[i];
    phase_dims(in[i], ks[i], st[i], pads[i], dil[i], b->ph[i]);
    int acc = 0;
    for (int r = 0; r < convfwd::kMaxBwdStride; ++r) {
      const bool live = r < st[i];
      g.k0[i][r] = live ? b->ph[i][r].k0 : 0;
      g.t[i][r] = live ? b->ph[i][r].T : 0;
      g.pre[i][r] = acc;
      if (live) acc += b->ph[i][r].T;
    }
  }
  return CONVFWD_OK;
}

// The forward problem one stride phase computes: x = dy, y = the phase's dx
// rows, filter = the phase's block of the rearranged filter.
ConvParams phase_params(const BwdPlan& b, int rd, int rh, int rw) {
  const ConvParams& f = b.fwd;
  const PhaseDim& a = b.ph[0][rd];
  const PhaseDim& c = b.ph[1][rh];
  const PhaseDim& e = b.ph[2][rw];
  ConvParams q;
  q.n = f.n; q.d = f.od; q.h = f.oh; q.w = f.ow;
  q.cin = f.cout; q.cout = f.cin;
  q.groups = f.groups; q.cin_g = f.cout_g; q.cout_g = f.cin_g;
  q.kd = a.T; q.kh = c.T; q.kw = e.T;
  q.sd = q.sh = q.sw = 1;
  q.pd = a.P; q.ph = c.P; q.pw = e.P;
  q.ed = a.ep; q.eh = c.ep; q.ew = e.ep;
  q.od = a.J; q.oh = c.J; q.ow = e.J;
  q.M = f.n * a.J * c.J * e.J;
  q.ntaps = a.T * c.T * e.T;
  q.K = q.ntaps * q.cin_g;
  q.xs_w = q.cin; q.xs_h = q.w * q.cin; q.xs_d = q.h * q.w * q.cin; q.xs_n = q.d * q.h * q.w * q.cin;
  const bool unit = f.sd == 1 && f.sh == 1 && f.sw == 1;
  q.remap = unit ? 0 : 1;
  q.ys_w = f.sw * f.cin;
  q.ys_h = f.sh * f.w * f.cin;
  q.ys_d = f.sd * f.h * f.w * f.cin;
  q.ys_n = f.d * f.h * f.w * f.cin;
  q.y_off = (rd * f.h * f.w + rh * f.w + rw) * f.cin;
  return q;
}

// Element offset of a phase's block in the rearranged filter.
int64_t phase_filter_offset(const BwdPlan& b, int rd, int rh, int rw) {
  const convfwd::BwdGeom& g = b.geom;
  const int64_t og = b.fwd.cout_g;
  return og * g.cin *
         ((int64_t)g.pre[0][rd] * g.k[1] * g.k[2] + (int64_t)g.t[0][rd] * g.pre[1][rh] * g.k[2] +
          (int64_t)g.t[0][rd] * g.t[1][rh] * g.pre[2][rw]);
}

// Path for one phase: AUTO takes the forward choice when the phase writes a
// dense dx with non-negative pads (unit stride), else main, runs or direct,
// the kernels that write remapped rows.  A phase without taps writes zeros
// through the direct kernel.  al16: dy, the phase's filter block and dx are
// all 16-byte aligned (else only the element-aligned paths run).
int phase_path(const ConvParams& q, int path, int dtype, bool al16) {
  if (q.ntaps == 0) return CONVFWD_PATH_DIRECT;
  if (path != CONVFWD_PATH_AUTO) return path_accepts(path, q, dtype) && (al16 || !needs_16(path)) ? path : -1;
  if (!q.remap && q.pd >= 0 && q.ph >= 0 && q.pw >= 0) return auto_path(q, dtype, al16);
  if (al16 && convfwd::main_accepts(q, dtype)) return CONVFWD_PATH_MAIN;
  if (convfwd::runs_accepts(q, dtype)) return CONVFWD_PATH_RUNS;
  return CONVFWD_PATH_DIRECT;
}

int run_bwd_data(const convfwd_desc_ex* desc, int path, const void* dy, const void* wt, void* dx,
                 void* stream) {
  if (path != CONVFWD_PATH_AUTO && path != CONVFWD_PATH_MAIN && path != CONVFWD_PATH_RUNS &&
      path != CONVFWD_PATH_DIRECT)
    return CONVFWD_ERR_UNSUPPORTED;
  BwdPlan b;
  const int rc = make_bwd_plan(desc, &b);
  if (rc != CONVFWD_OK) return rc;
  const ConvParams& f = b.fwd;
  const int eb = elem_bytes(desc->dtype);
  // whether phase (rd, rh, rw)'s tensors (dy, its filter block, dx) are 16-byte aligned
  // (integer arithmetic: wt may be NULL for an empty batch)
  auto phase_al16 = [&](int rd, int rh, int rw) {
    const uintptr_t wq = (uintptr_t)wt + (uintptr_t)(phase_filter_offset(b, rd, rh, rw) * eb);
    return aligned_to(dy, (const void*)wq, dx, 16);
  };
  // every phase must be runnable before the first launch
  for (int rd = 0; rd < f.sd; ++rd)
    for (int rh = 0; rh < f.sh; ++rh)
      for (int rw = 0; rw < f.sw; ++rw) {
        const ConvParams q = phase_params(b, rd, rh, rw);
        if (q.od == 0 || q.oh == 0 || q.ow == 0) continue;
        if (phase_path(q, path, desc->dtype, phase_al16(rd, rh, rw)) < 0) return CONVFWD_ERR_UNSUPPORTED;
      }
  if (f.n == 0) return CONVFWD_OK;
  if (!dy || !wt || !dx) return CONVFWD_ERR_NULL;
  if (overlaps(dx, b.x_bytes, dy, b.y_bytes) || overlaps(dx, b.x_bytes, wt, b.w_bytes))
    return CONVFWD_ERR_ALIAS;
  if (!aligned_to(dy, wt, dx, (uintptr_t)eb)) return CONVFWD_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  // Phases on the main path share one launch (their start-up and tails
  // overlap); the others run one launch each.
  ConvParams batch[convfwd::kMaxBwdStride * convfwd::kMaxBwdStride];
  uint32_t batch_off[convfwd::kMaxBwdStride * convfwd::kMaxBwdStride];
  int nbatch = 0;
  for (int rd = 0; rd < f.sd; ++rd)
    for (int rh = 0; rh < f.sh; ++rh)
      for (int rw = 0; rw < f.sw; ++rw) {
        const ConvParams q = phase_params(b, rd, rh, rw);
        if (q.od == 0 || q.oh == 0 || q.ow == 0) continue;
        const int64_t off = phase_filter_offset(b, rd, rh, rw) * eb;
        const int qp = phase_path(q, path, desc->dtype, phase_al16(rd, rh, rw));
        if (qp == CONVFWD_PATH_MAIN && q.remap && nbatch < (int)(sizeof(batch) / sizeof(batch[0]))) {
          batch[nbatch] = q;
          batch_off[nbatch++] = (uint32_t)off;
          continue;
        }
        if (launch_path(qp, q, desc->dtype, dy, (const char*)wt + off, dx, s) != hipSuccess)
          return CONVFWD_ERR_LAUNCH;
      }
  // Phases with more taps take longer: put them first so that the short ones
  // fill the tail (insertion sort, at most s_d*s_h*s_w entries).
  for (int i = 1; i < nbatch; ++i)
    for (int j = i; j > 0 && batch[j].ntaps > batch[j - 1].ntaps; --j) {
      const ConvParams tq = batch[j];
      batch[j] = batch[j - 1];
      batch[j - 1] = tq;
      const uint32_t to = batch_off[j];
      batch_off[j] = batch_off[j - 1];
      batch_off[j - 1] = to;
    }
  if (convfwd::launch_main_phased(batch, batch_off, nbatch, desc->dtype, dy, wt, dx, s) != hipSuccess)
    return CONVFWD_ERR_LAUNCH;
  return CONVFWD_OK;
}

int run_bwd_filter(const convfwd_desc_ex* desc, const void* w, void* wt, void* stream) {
  BwdPlan b;
  const int rc = make_bwd_plan(desc, &b);
  if (rc != CONVFWD_OK) return rc;
  if (!w || !wt) return CONVFWD_ERR_NULL;
  if (overlaps(wt, b.w_bytes, w, b.w_bytes)) return CONVFWD_ERR_ALIAS;
  if (!aligned_to(w, wt, wt, (uintptr_t)elem_bytes(desc->dtype))) return CONVFWD_ERR_MISALIGNED;
  if (convfwd::launch_bwd_filter(b.geom, desc->dtype, w, wt, (hipStream_t)stream) != hipSuccess)
    return CONVFWD_ERR_LAUNCH;
  return CONVFWD_OK;
}

}  // namespace

extern "C" {

int conv_bwd_data_filter_ex(const convfwd_desc_ex* desc, const void* w, void* wt, void* stream) {
  return run_bwd_filter(desc, w, wt, stream);
}

int conv_bwd_data_ex(const convfwd_desc_ex* desc, const void* dy, const void* wt, void* dx, void* stream) {
  return run_bwd_data(desc, CONVFWD_PATH_AUTO, dy, wt, dx, stream);
}

int conv_bwd_data_path_ex(const convfwd_desc_ex* desc, int path, const void* dy, const void* wt, void* dx,
                          void* stream) {
  return run_bwd_data(desc, path, dy, wt, dx, stream);
}

int conv_bwd_data_filter(const convfwd_desc* desc, const void* w, void* wt, void* stream) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return run_bwd_filter(&e, w, wt, stream);
}

int conv_bwd_data(const convfwd_desc* desc, const void* dy, const void* wt, void* dx, void* stream) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return run_bwd_data(&e, CONVFWD_PATH_AUTO, dy, wt, dx, stream);
}


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
  Choice c;
  if (tuned_choice(*desc, p, &c)) return c.path;
  return auto_path(p, desc->dtype);
}

int conv_tune_ex(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream, int reps,
                 float* best_us) {
  return run_tune(desc, x, w, y, stream, reps, best_us);
}

int conv_tune(const convfwd_desc* desc, const void* x, const void* w, void* y, void* stream, int reps,
              float* best_us) {
  if (!desc) return CONVFWD_ERR_NULL;
  const convfwd_desc_ex e = widen(*desc);
  return run_tune(&e, x, w, y, stream, reps, best_us);
}

int conv_tuned_path_ex(const convfwd_desc_ex* desc) {
  ConvParams p;
  int64_t xb, wb, yb;
  const int rc = make_params(desc, &p, &xb, &wb, &yb);
  if (rc != CONVFWD_OK) return rc;
  Choice c;
  return tuned_choice(*desc, p, &c) ? c.path : 0;
}

int conv_tune_clear(void) {
  std::lock_guard<std::mutex> lock(tune_mutex());
  tune_table().clear();
  tune_count().store(0, std::memory_order_release);
  return CONVFWD_OK;
}

int conv_fwd_ex(const convfwd_desc_ex* desc, const void* x, const void* w, void* y, void* stream) {
  return run(desc, CONVFWD_PATH_AUTO, x, w, y, stream);
}

int conv_fwd_path_ex(const convfwd_desc_ex* desc, int path, const void* x, const void* w, void* y,
                     void* stream) {
  if (path < CONVFWD_PATH_AUTO || path > CONVFWD_PATH_STAGED) return CONVFWD_ERR_UNSUPPORTED;
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
    case CONVFWD_ERR_MISALIGNED: return "a tensor pointer is not aligned to its element size";
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
    case CONVFWD_PATH_SLAB: return "slab";
    case CONVFWD_PATH_PHASE: return "phase";
    case CONVFWD_PATH_STAGED: return "staged";
    default: return "unknown";
  }
}

}  // extern "C"
