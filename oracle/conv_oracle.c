/*
 * conv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow CPU oracle for the forward pass of a dense 2D/3D convolution
 * in channels-last layout.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU product path never calls,
 * links or includes it, and it shares no code with that path.
 *
 * What it computes (sources: the "Convolutions" tutorial page, sections
 * "1. What is it?" and "4. Tiny example"; the MLX pull request "Add implicit
 * matmul pathway for mx.conv3d", benchmark tables, for the channels-last
 * layouts and the per-dimension stride and pads):
 *
 *   y[n,od,oh,ow,co] = sum over kd<KD, kh<KH, kw<KW, c<C_in/G of
 *        X(n, od*sd - pd + kd*ed, oh*sh - ph + kh*eh, ow*sw - pw + kw*ew, g*C_in/G + c)
 *          * w[co,kd,kh,kw,c],          g = co / (C_out/G)
 *
 *   X(n,d,h,w,c) = x[n,d,h,w,c] inside the input, 0 outside (zero padding).
 *
 * The plain convolution has G = 1, dilation e = 1 and the same padding on
 * both sides of a dimension.  The variants the tutorial lists ("Convolution
 * variants worth knowing") take the same sum: grouped convolution splits the
 * channels into G groups, an output channel reading only the input channels
 * of its own group (the filter then holds C_in/G channels per tap); a dilated
 * filter puts its taps e positions apart ("gaps in the kernel"); and padding
 * may differ between the low side (p) and the high side (q) of a dimension.
 *
 * The filter is slid over the input and NOT flipped: the tutorial's worked
 * example indexes the input at (i+di, j+dj) against kernel entry (di, dj)
 * (a cross-correlation), and its printed result [[-4,-4],[-4,-4]] tells the
 * two orientations apart.  Output extents use floor division:
 * out = floor((in + 2p - k) / s) + 1, which gives the tutorial's 224 -> 112
 * for a 7x7 stride-2 layer with padding 3 (ResNet-50 first layer, section 4),
 * 3 -> 2 and 5 -> 3 for its unpadded examples.  In general a filter of K taps
 * e apart spans e*(K-1)+1 positions, so out = floor((in + p + q - e*(K-1) - 1)
 * / s) + 1.
 *
 * Layouts: x is (N, D, H, W, C_in), w is (C_out, KD, KH, KW, C_in/G), y is
 * (N, D_out, H_out, W_out, C_out), all dense, C fastest.  A 2D problem is the
 * 3D one with D = KD = sd = 1 and pd = 0.
 *
 * Backward-data (the gradient with respect to x, "dgrad") is the transposed
 * convolution of the tutorial's variant list ("Convolution variants worth
 * knowing": transposed, upsampling convolution): the adjoint of the forward
 * map.  Every forward product x(n, i, c) * w[co, k, c] that feeds y[n, o, co]
 * sends dy[n, o, co] * w[co, k, c] back to dx[n, i, c]:
 *
 *   dx[n,id,ih,iw,c] = sum over co of c's group, kd, kh, kw such that
 *        od = (id + pd - kd*ed) / sd is a whole number with 0 <= od < D_out
 *        (likewise oh, ow) of dy[n,od,oh,ow,co] * w[co,kd,kh,kw,c - g*C_in/G]
 *
 * Written out this way it is also what the MLX pull request's general path
 * ("input dilation", "flip") computes: a forward convolution of dy with s-1
 * zeros inserted between neighbours, against the spatially flipped filter with
 * input and output channels exchanged.  dx has x's shape; positions that no
 * output window covers get 0.
 *
 * Arithmetic: every value is a double; every product of two fp16, bf16 or
 * fp32 inputs is exact in double, and the sum is accumulated in double in
 * the loop order below.  The loop runs over every tap, padding included,
 * exactly as the definition reads, so the count of multiply-adds it performs
 * is N*D_out*H_out*W_out * C_out * (C_in/G)*KD*KH*KW, the quantity the tutorial's
 * FLOP formula doubles.  The only parallelism is an OpenMP split over output
 * positions, which does not change any output value.
 */
#include <stdint.h>
#include <stddef.h>

typedef struct {
  int64_t n, d, h, w, c_in, c_out; /* input batch, depth, height, width, channels; output channels */
  int64_t k_d, k_h, k_w;           /* filter extents */
  int64_t s_d, s_h, s_w;           /* strides, >= 1 */
  int64_t p_d, p_h, p_w;           /* zero padding on the low side, >= 0 */
  int64_t q_d, q_h, q_w;           /* zero padding on the high side, >= 0 */
  int64_t e_d, e_h, e_w;           /* filter dilation: tap t sits t*e positions past the origin */
  int64_t groups;                  /* channel groups G, dividing C_in and C_out */
} oracle_conv_shape;

/* Output positions along one dimension for low / high padding p / q and a
 * filter of k taps e apart: floor((in + p + q - e*(k-1) - 1) / s) + 1, or 0
 * when the padded input is shorter than the filter's span. */
int64_t oracle_out_extent_ex(int64_t in, int64_t k, int64_t s, int64_t p, int64_t q, int64_t e) {
  int64_t span = in + p + q - (e * (k - 1) + 1);
  if (s < 1 || e < 1 || span < 0) return 0;
  return span / s + 1;
}

/* The plain case: the same padding on both sides, undilated filter. */
int64_t oracle_out_extent(int64_t in, int64_t k, int64_t s, int64_t p) {
  return oracle_out_extent_ex(in, k, s, p, p, 1);
}

/* The input with zero padding: X(n,d,h,w,c). */
static double x_at(const oracle_conv_shape* s, const double* x,
                   int64_t n, int64_t d, int64_t h, int64_t w, int64_t c) {
  if (d < 0 || d >= s->d) return 0.0;
  if (h < 0 || h >= s->h) return 0.0;
  if (w < 0 || w >= s->w) return 0.0;
  return x[(((n * s->d + d) * s->h + h) * s->w + w) * s->c_in + c];
}

static double w_at(const oracle_conv_shape* s, const double* wt,
                   int64_t co, int64_t kd, int64_t kh, int64_t kw, int64_t c) {
  return wt[(((co * s->k_d + kd) * s->k_h + kh) * s->k_w + kw) * (s->c_in / s->groups) + c];
}

/*
 * Computes the output rows listed in `rows` (flat output-position indices
 * m = ((n*D_out + od)*H_out + oh)*W_out + ow), or every row when rows is NULL
 * (then nrows is ignored and y receives the whole output).  Row r of y holds
 * the C_out outputs of rows[r].  Returns the number of multiply-adds done, or
 * -1 for a malformed shape or an out-of-range row index.
 */
int64_t oracle_conv_fwd(const oracle_conv_shape* s, const double* x, const double* wt,
                        const int64_t* rows, int64_t nrows, double* y) {
  if (s->n < 0 || s->d < 1 || s->h < 1 || s->w < 1 || s->c_in < 1 || s->c_out < 1) return -1;
  if (s->k_d < 1 || s->k_h < 1 || s->k_w < 1) return -1;
  if (s->s_d < 1 || s->s_h < 1 || s->s_w < 1) return -1;
  if (s->p_d < 0 || s->p_h < 0 || s->p_w < 0) return -1;
  if (s->q_d < 0 || s->q_h < 0 || s->q_w < 0) return -1;
  if (s->e_d < 1 || s->e_h < 1 || s->e_w < 1) return -1;
  if (s->groups < 1 || s->c_in % s->groups != 0 || s->c_out % s->groups != 0) return -1;
  const int64_t od_n = oracle_out_extent_ex(s->d, s->k_d, s->s_d, s->p_d, s->q_d, s->e_d);
  const int64_t oh_n = oracle_out_extent_ex(s->h, s->k_h, s->s_h, s->p_h, s->q_h, s->e_h);
  const int64_t ow_n = oracle_out_extent_ex(s->w, s->k_w, s->s_w, s->p_w, s->q_w, s->e_w);
  const int64_t cg = s->c_in / s->groups;    /* input channels per group */
  const int64_t og = s->c_out / s->groups;   /* output channels per group */
  const int64_t m_total = s->n * od_n * oh_n * ow_n;
  const int64_t count = rows ? nrows : m_total;
  if (count < 0) return -1;
  if (rows) {
    for (int64_t r = 0; r < count; ++r)
      if (rows[r] < 0 || rows[r] >= m_total) return -1;
  }
  int64_t macs = 0;

#pragma omp parallel for schedule(dynamic, 16) reduction(+ : macs)
  for (int64_t r = 0; r < count; ++r) {
    const int64_t m = rows ? rows[r] : r;
    const int64_t ow = m % ow_n;
    const int64_t oh = (m / ow_n) % oh_n;
    const int64_t od = (m / (ow_n * oh_n)) % od_n;
    const int64_t n = m / (ow_n * oh_n * od_n);
    for (int64_t co = 0; co < s->c_out; ++co) {
      const int64_t g = co / og;
      double acc = 0.0;
      for (int64_t kd = 0; kd < s->k_d; ++kd)
        for (int64_t kh = 0; kh < s->k_h; ++kh)
          for (int64_t kw = 0; kw < s->k_w; ++kw)
            for (int64_t c = 0; c < cg; ++c) {
              acc += x_at(s, x, n, od * s->s_d - s->p_d + kd * s->e_d, oh * s->s_h - s->p_h + kh * s->e_h,
                          ow * s->s_w - s->p_w + kw * s->e_w, g * cg + c) *
                     w_at(s, wt, co, kd, kh, kw, c);
              macs += 1;
            }
      y[r * s->c_out + co] = acc;
    }
  }
  return macs;
}

/*
 * Backward-data: dx (x's shape) from dy (y's shape) and the forward filter w,
 * for the forward problem *s.  Computes the input positions listed in `rows`
 * (flat indices ((n*D + d)*H + h)*W + w), or all of them when rows is NULL;
 * row r of dx receives the C_in values of rows[r].  Returns the number of
 * multiply-adds done, or -1 for a malformed shape or an out-of-range row.
 */
int64_t oracle_conv_bwd_data(const oracle_conv_shape* s, const double* dy, const double* wt,
                             const int64_t* rows, int64_t nrows, double* dx) {
  if (s->n < 0 || s->d < 1 || s->h < 1 || s->w < 1 || s->c_in < 1 || s->c_out < 1) return -1;
  if (s->k_d < 1 || s->k_h < 1 || s->k_w < 1) return -1;
  if (s->s_d < 1 || s->s_h < 1 || s->s_w < 1) return -1;
  if (s->p_d < 0 || s->p_h < 0 || s->p_w < 0) return -1;
  if (s->q_d < 0 || s->q_h < 0 || s->q_w < 0) return -1;
  if (s->e_d < 1 || s->e_h < 1 || s->e_w < 1) return -1;
  if (s->groups < 1 || s->c_in % s->groups != 0 || s->c_out % s->groups != 0) return -1;
  const int64_t od_n = oracle_out_extent_ex(s->d, s->k_d, s->s_d, s->p_d, s->q_d, s->e_d);
  const int64_t oh_n = oracle_out_extent_ex(s->h, s->k_h, s->s_h, s->p_h, s->q_h, s->e_h);
  const int64_t ow_n = oracle_out_extent_ex(s->w, s->k_w, s->s_w, s->p_w, s->q_w, s->e_w);
  if (od_n < 1 || oh_n < 1 || ow_n < 1) return -1;
  const int64_t cg = s->c_in / s->groups;
  const int64_t og = s->c_out / s->groups;
  const int64_t positions = s->n * s->d * s->h * s->w;
  const int64_t count = rows ? nrows : positions;
  if (count < 0) return -1;
  if (rows) {
    for (int64_t r = 0; r < count; ++r)
      if (rows[r] < 0 || rows[r] >= positions) return -1;
  }
  int64_t macs = 0;

#pragma omp parallel for schedule(dynamic, 16) reduction(+ : macs)
  for (int64_t r = 0; r < count; ++r) {
    const int64_t pos = rows ? rows[r] : r;
    const int64_t iw = pos % s->w;
    const int64_t ih = (pos / s->w) % s->h;
    const int64_t id = (pos / (s->w * s->h)) % s->d;
    const int64_t n = pos / (s->w * s->h * s->d);
    for (int64_t c = 0; c < s->c_in; ++c) {
      const int64_t g = c / cg;
      double sum = 0.0;
      for (int64_t co = g * og; co < (g + 1) * og; ++co)
        for (int64_t kd = 0; kd < s->k_d; ++kd) {
          const int64_t td = id + s->p_d - kd * s->e_d;
          if (td < 0 || td % s->s_d != 0 || td / s->s_d >= od_n) continue;
          for (int64_t kh = 0; kh < s->k_h; ++kh) {
            const int64_t th = ih + s->p_h - kh * s->e_h;
            if (th < 0 || th % s->s_h != 0 || th / s->s_h >= oh_n) continue;
            for (int64_t kw = 0; kw < s->k_w; ++kw) {
              const int64_t tw = iw + s->p_w - kw * s->e_w;
              if (tw < 0 || tw % s->s_w != 0 || tw / s->s_w >= ow_n) continue;
              const int64_t o = ((n * od_n + td / s->s_d) * oh_n + th / s->s_h) * ow_n + tw / s->s_w;
              sum += dy[o * s->c_out + co] * w_at(s, wt, co, kd, kh, kw, c - g * cg);
              macs += 1;
            }
          }
        }
      dx[r * s->c_in + c] = sum;
    }
  }
  return macs;
}
