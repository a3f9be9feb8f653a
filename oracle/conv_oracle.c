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
 *   y[n,od,oh,ow,co] = sum over kd<KD, kh<KH, kw<KW, c<C_in of
 *        X(n, od*sd - pd + kd, oh*sh - ph + kh, ow*sw - pw + kw, c)
 *          * w[co,kd,kh,kw,c]
 *
 *   X(n,d,h,w,c) = x[n,d,h,w,c] inside the input, 0 outside (zero padding).
 *
 * The filter is slid over the input and NOT flipped: the tutorial's worked
 * example indexes the input at (i+di, j+dj) against kernel entry (di, dj)
 * (a cross-correlation), and its printed result [[-4,-4],[-4,-4]] tells the
 * two orientations apart.  Output extents use floor division:
 * out = floor((in + 2p - k) / s) + 1, which gives the tutorial's 224 -> 112
 * for a 7x7 stride-2 layer with padding 3 (ResNet-50 first layer, section 4),
 * 3 -> 2 and 5 -> 3 for its unpadded examples.
 *
 * Layouts: x is (N, D, H, W, C_in), w is (C_out, KD, KH, KW, C_in), y is
 * (N, D_out, H_out, W_out, C_out), all dense, C fastest.  A 2D problem is the
 * 3D one with D = KD = sd = 1 and pd = 0.
 *
 * Arithmetic: every value is a double; every product of two fp16, bf16 or
 * fp32 inputs is exact in double, and the sum is accumulated in double in
 * the loop order below.  The loop runs over every tap, padding included,
 * exactly as the definition reads, so the count of multiply-adds it performs
 * is N*D_out*H_out*W_out * C_out * C_in*KD*KH*KW, the quantity the tutorial's
 * FLOP formula doubles.  The only parallelism is an OpenMP split over output
 * positions, which does not change any output value.
 */
#include <stdint.h>
#include <stddef.h>

typedef struct {
  int64_t n, d, h, w, c_in, c_out; /* input batch, depth, height, width, channels; output channels */
  int64_t k_d, k_h, k_w;           /* filter extents */
  int64_t s_d, s_h, s_w;           /* strides, >= 1 */
  int64_t p_d, p_h, p_w;           /* zero padding on both sides, >= 0 */
} oracle_conv_shape;

/* Number of output positions along one dimension: floor((in + 2p - k) / s) + 1,
 * or 0 when the padded input is shorter than the filter. */
int64_t oracle_out_extent(int64_t in, int64_t k, int64_t s, int64_t p) {
  int64_t span = in + 2 * p - k;
  if (s < 1 || span < 0) return 0;
  return span / s + 1;
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
  return wt[(((co * s->k_d + kd) * s->k_h + kh) * s->k_w + kw) * s->c_in + c];
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
  const int64_t od_n = oracle_out_extent(s->d, s->k_d, s->s_d, s->p_d);
  const int64_t oh_n = oracle_out_extent(s->h, s->k_h, s->s_h, s->p_h);
  const int64_t ow_n = oracle_out_extent(s->w, s->k_w, s->s_w, s->p_w);
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
      double acc = 0.0;
      for (int64_t kd = 0; kd < s->k_d; ++kd)
        for (int64_t kh = 0; kh < s->k_h; ++kh)
          for (int64_t kw = 0; kw < s->k_w; ++kw)
            for (int64_t c = 0; c < s->c_in; ++c) {
              acc += x_at(s, x, n, od * s->s_d - s->p_d + kd, oh * s->s_h - s->p_h + kh,
                          ow * s->s_w - s->p_w + kw, c) *
                     w_at(s, wt, co, kd, kh, kw, c);
              macs += 1;
            }
      y[r * s->c_out + co] = acc;
    }
  }
  return macs;
}
