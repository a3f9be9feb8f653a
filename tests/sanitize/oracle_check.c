/*
 * oracle_check.c -- runs the CPU oracle (oracle/conv_oracle.c, compiled into
 * this program) on random small problems for sanitizer builds (AddressSanitizer
 * + UndefinedBehaviorSanitizer).  Test infrastructure.
 *
 * Every buffer is allocated at exactly the size the problem needs, so a read
 * or write past an end is reported by the sanitizer.  Two consistency checks
 * keep the run honest: the rows-subset form of the forward pass returns the
 * same rows as the whole-output form, and the backward-data pass is the
 * adjoint of the forward one, <conv(x, w), dy> = <x, dgrad(dy, w)>.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/conv_oracle.c"

static uint64_t state = 88172645463325252ull;
static uint32_t next_u32(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)(state >> 11);
}
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u32() % (uint32_t)(hi - lo + 1)); }
static double uniform(void) { return (double)next_u32() / 2097152.0 - 1.0; }   /* 2^21 buckets of [-1, 1) */

static double* filled(int64_t count) {
  double* p = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
  for (int64_t i = 0; i < count; ++i) p[i] = uniform();
  return p;
}

int main(int argc, char** argv) {
  const int problems = argc > 1 ? atoi(argv[1]) : 300;
  int bad = 0, ran = 0;
  for (int it = 0; it < problems; ++it) {
    oracle_conv_shape s;
    s.groups = range(1, 3);
    s.n = range(1, 2);
    s.d = range(1, 5);
    s.h = range(1, 7);
    s.w = range(1, 8);
    s.c_in = s.groups * range(1, 4);
    s.c_out = s.groups * range(1, 4);
    s.k_d = range(1, 3);
    s.k_h = range(1, 4);
    s.k_w = range(1, 4);
    s.s_d = range(1, 3);
    s.s_h = range(1, 3);
    s.s_w = range(1, 4);
    s.p_d = range(0, 2);
    s.p_h = range(0, 3);
    s.p_w = range(0, 3);
    s.q_d = range(0, 2);
    s.q_h = range(0, 3);
    s.q_w = range(0, 3);
    s.e_d = range(1, 2);
    s.e_h = range(1, 3);
    s.e_w = range(1, 2);
    const int64_t od = oracle_out_extent_ex(s.d, s.k_d, s.s_d, s.p_d, s.q_d, s.e_d);
    const int64_t oh = oracle_out_extent_ex(s.h, s.k_h, s.s_h, s.p_h, s.q_h, s.e_h);
    const int64_t ow = oracle_out_extent_ex(s.w, s.k_w, s.s_w, s.p_w, s.q_w, s.e_w);
    if (od < 1 || oh < 1 || ow < 1) continue;
    ++ran;
    const int64_t xe = s.n * s.d * s.h * s.w * s.c_in;
    const int64_t we = s.c_out * s.k_d * s.k_h * s.k_w * (s.c_in / s.groups);
    const int64_t m = s.n * od * oh * ow;
    double* x = filled(xe);
    double* w = filled(we);
    double* y = filled(m * s.c_out);
    double* dy = filled(m * s.c_out);
    double* dx = filled(xe);
    if (oracle_conv_fwd(&s, x, w, NULL, 0, y) < 0 || oracle_conv_bwd_data(&s, dy, w, NULL, 0, dx) < 0) {
      fprintf(stderr, "problem %d rejected\n", it);
      ++bad;
    }
    /* every third row through the subset form */
    const int64_t nr = (m + 2) / 3;
    int64_t* rows = (int64_t*)malloc((size_t)nr * sizeof(int64_t));
    for (int64_t r = 0; r < nr; ++r) rows[r] = m - 1 - 3 * r;
    double* ys = filled(nr * s.c_out);
    oracle_conv_fwd(&s, x, w, rows, nr, ys);
    for (int64_t r = 0; r < nr; ++r)
      for (int64_t c = 0; c < s.c_out; ++c)
        if (ys[r * s.c_out + c] != y[rows[r] * s.c_out + c]) {
          ++bad;
          r = nr;
          break;
        }
    double lhs = 0.0, rhs = 0.0, scale = 0.0;
    for (int64_t i = 0; i < m * s.c_out; ++i) {
      lhs += y[i] * dy[i];
      scale += fabs(y[i] * dy[i]);
    }
    for (int64_t i = 0; i < xe; ++i) rhs += x[i] * dx[i];
    if (fabs(lhs - rhs) > 1e-9 * (scale + 1.0)) {
      fprintf(stderr, "problem %d: adjoint identity %.17g vs %.17g\n", it, lhs, rhs);
      ++bad;
    }
    free(rows);
    free(ys);
    free(x);
    free(w);
    free(y);
    free(dy);
    free(dx);
  }
  /* malformed shapes are refused without touching the buffers */
  oracle_conv_shape z = {0};
  if (oracle_conv_fwd(&z, NULL, NULL, NULL, 0, NULL) != -1) ++bad;
  printf("oracle_check: %d problems, %d failures\n", ran, bad);
  return bad == 0 ? 0 : 1;
}
