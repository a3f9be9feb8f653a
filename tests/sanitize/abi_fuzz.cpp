// abi_fuzz.cpp -- host-side stress of the C ABI's validation, path choice and
// backward-data planning, for sanitizer builds (AddressSanitizer +
// UndefinedBehaviorSanitizer, ThreadSanitizer).  Test infrastructure.
//
// Every call made here returns before any kernel launch: descriptors are
// random (valid and invalid), the batch is empty or the pointers are rejected
// (NULL, overlapping, not aligned to the element size), so the program runs
// on a machine without a GPU.  It checks only that the library's own answers
// are consistent (a valid shape gives positive extents; a path the library
// picks accepts the problem) and leaves memory errors, undefined behaviour
// and data races to the sanitizer the library was built with.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <thread>
#include <vector>

#include "../../include/convfwd.h"

namespace {

struct Lcg {
  uint64_t s;
  explicit Lcg(uint64_t seed) : s(seed * 6364136223846793005ull + 1442695040888963407ull) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  }
  int range(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }
};

convfwd_desc_ex random_desc(Lcg& r) {
  convfwd_desc_ex d;
  const bool bad = r.range(0, 9) == 0;   // one in ten may carry an invalid field
  d.n = r.range(bad ? -1 : 0, 3);
  d.d = r.range(bad ? 0 : 1, 12);
  d.h = r.range(bad ? 0 : 1, 40);
  d.w = r.range(bad ? 0 : 1, 70);
  d.groups = r.range(bad ? 0 : 1, 4);
  d.c_in = d.groups * r.range(1, 70) + (bad ? r.range(0, 1) : 0);
  d.c_out = d.groups * r.range(1, 70);
  d.k_d = r.range(bad ? 0 : 1, d.d > 3 ? 3 : d.d);
  d.k_h = r.range(bad ? 0 : 1, 8);
  d.k_w = r.range(bad ? 0 : 1, r.range(0, 20) == 0 ? 18 : 7);
  d.s_d = r.range(bad ? 0 : 1, 3);
  d.s_h = r.range(bad ? 0 : 1, r.range(0, 10) == 0 ? 17 : 3);
  d.s_w = r.range(bad ? 0 : 1, 3);
  d.p_d = r.range(bad ? -1 : 0, 2);
  d.p_h = r.range(bad ? -1 : 0, 4);
  d.p_w = r.range(0, 4);
  d.q_d = r.range(0, 2);
  d.q_h = r.range(0, 4);
  d.q_w = r.range(bad ? -1 : 0, 4);
  d.e_d = r.range(1, 2);
  d.e_h = r.range(bad ? 0 : 1, 3);
  d.e_w = r.range(1, 3);
  d.dtype = r.range(bad ? -1 : 0, bad ? 3 : 2);
  return d;
}

int check(bool ok, const char* what, int i) {
  if (ok) return 0;
  fprintf(stderr, "inconsistent answer: %s (descriptor %d)\n", what, i);
  return 1;
}

// One worker: `count` random descriptors through every host-side entry point.
int run_worker(uint64_t seed, int count) {
  Lcg r(seed);
  int bad = 0;
  char* const base = (char*)(uintptr_t)(1u << 24);   // never dereferenced
  for (int i = 0; i < count; ++i) {
    convfwd_desc_ex d = random_desc(r);
    int64_t out[5] = {0, 0, 0, 0, 0};
    const int rc = conv_out_shape_ex(&d, out);
    if (rc == CONVFWD_OK)
      bad += check(out[0] == d.n && out[1] > 0 && out[2] > 0 && out[3] > 0 && out[4] == d.c_out, "extents", i);
    const int path = conv_select_path_ex(&d);
    bad += check((rc == CONVFWD_OK) == (path > 0), "select_path agrees with validation", i);
    (void)conv_tuned_path_ex(&d);
    // empty batch: every path's rules run, nothing is read or launched
    convfwd_desc_ex e = d;
    e.n = 0;
    for (int p = CONVFWD_PATH_AUTO; p <= CONVFWD_PATH_SLAB + 1; ++p) {
      const int f = conv_fwd_path_ex(&e, p, nullptr, nullptr, nullptr, nullptr);
      if (rc == CONVFWD_OK && p == CONVFWD_PATH_AUTO) bad += check(f == CONVFWD_OK, "AUTO takes any valid problem", i);
      if (rc == CONVFWD_OK && p == path) bad += check(f == CONVFWD_OK, "the chosen path accepts", i);
    }
    (void)conv_bwd_data_path_ex(&e, CONVFWD_PATH_AUTO, nullptr, nullptr, nullptr, nullptr);
    (void)conv_bwd_data_path_ex(&e, CONVFWD_PATH_MAIN, nullptr, nullptr, nullptr, nullptr);
    (void)conv_tune_ex(&e, nullptr, nullptr, nullptr, nullptr, 3, nullptr);
    // pointers the host rejects before a launch
    if (d.n > 0 && rc == CONVFWD_OK) {
      bad += check(conv_fwd_ex(&d, nullptr, base, base, nullptr) == CONVFWD_ERR_NULL, "NULL x", i);
      bad += check(conv_fwd_ex(&d, base, base + (1 << 22), base + 2, nullptr) == CONVFWD_ERR_ALIAS, "alias", i);
      bad += check(conv_fwd_ex(&d, base + 1, base + (1 << 26), base + (1 << 27), nullptr) == CONVFWD_ERR_MISALIGNED,
                   "odd x", i);
      bad += check(conv_bwd_data_filter_ex(&d, base, nullptr, nullptr) == CONVFWD_ERR_NULL ||
                       conv_bwd_data_filter_ex(&d, base, nullptr, nullptr) == CONVFWD_ERR_UNSUPPORTED,
                   "NULL wt", i);
      const int b = conv_bwd_data_ex(&d, base + 1, base + (1 << 26), base + (1 << 27), nullptr);
      bad += check(b == CONVFWD_ERR_MISALIGNED || b == CONVFWD_ERR_UNSUPPORTED, "odd dy", i);
    }
    (void)conv_strerror(rc);
    (void)conv_path_name(path);
  }
  return bad;
}

}  // namespace

int main(int argc, char** argv) {
  const int threads = argc > 1 ? atoi(argv[1]) : 1;
  const int count = argc > 2 ? atoi(argv[2]) : 20000;
  std::vector<std::thread> pool;
  std::vector<int> bad(threads, 0);
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([t, count, &bad] {
      bad[t] = run_worker(1000 + t, count);
      if (t % 2 == 1) conv_tune_clear();   // the table's lock against concurrent lookups
    });
  for (auto& th : pool) th.join();
  int total = 0;
  for (int b : bad) total += b;
  printf("abi_fuzz: %d threads x %d descriptors, %d inconsistent answers\n", threads, count, total);
  return total == 0 ? 0 : 1;
}
