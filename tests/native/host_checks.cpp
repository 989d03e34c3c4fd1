// Host-only driver of the library's pure C++ parts (the argument checks of
// args.cpp and the job tables of plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py. Every check
// here states a property of the C ABI (include/zyfa.h); any failed check,
// memory error or undefined behaviour (signed overflow included) ends the
// run with a non-zero status.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "args.h"
#include "plan.h"
#include "zyfa.h"

using namespace zyfa;

static int g_failed = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++g_failed;                                                        \
    }                                                                    \
  } while (0)

static void shapes() {
  CHECK(check_shape(1, 256, 4, 4, 128, 128, ZYFA_LAYOUT_BSHD, ZYFA_DTYPE_BF16) == ZYFA_OK);
  CHECK(check_shape(2, 32000, 32, 8, 128, 128, ZYFA_LAYOUT_BSHD, ZYFA_DTYPE_FP8_E4M3FN) == ZYFA_OK);
  CHECK(check_shape(1, 16384, 16, 16, 192, 128, ZYFA_LAYOUT_BHSD, ZYFA_DTYPE_BF16) == ZYFA_OK);
  CHECK(check_shape(0, 1, 1, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, 0, 1, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, -5, 1, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, 1, 0, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, 1, 1, 0, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, kMaxSeqlen, 1, 1, 128, 128, 0, 0) == ZYFA_OK);
  CHECK(check_shape(1, kMaxSeqlen + 1, 1, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(1, INT_MAX, 1, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);
  CHECK(check_shape(INT_MAX, 1, INT_MAX, 1, 128, 128, 0, 0) == ZYFA_ERR_SHAPE);   // batch * nheads >= 2^31
  CHECK(check_shape(65536, 1, 32767, 1, 128, 128, 0, 0) == ZYFA_OK);
  CHECK(check_shape(1, 1, 1, 1, 64, 64, 0, 0) == ZYFA_ERR_HEADDIM);
  CHECK(check_shape(1, 1, 1, 1, 192, 192, 0, 0) == ZYFA_ERR_HEADDIM);
  CHECK(check_shape(1, 1, 6, 4, 128, 128, 0, 0) == ZYFA_ERR_GQA);
  CHECK(check_shape(1, 1, 4, 4, 128, 128, 0, 7) == ZYFA_ERR_DTYPE);
  CHECK(check_shape(1, 1, 4, 4, 128, 128, 0, ZYFA_DTYPE_FP32) == ZYFA_ERR_DTYPE);
  CHECK(check_shape(1, 1, 4, 4, 128, 128, 2, 0) == ZYFA_ERR_LAYOUT);
}

static void strides_and_ranges() {
  long long sb, sh, ss;
  layout_strides(ZYFA_LAYOUT_BSHD, 1000, 8, 128, &sb, &sh, &ss);
  CHECK(sb == 1000LL * 8 * 128 && sh == 128 && ss == 8 * 128);
  layout_strides(ZYFA_LAYOUT_BHSD, 1000, 8, 192, &sb, &sh, &ss);
  CHECK(sb == 8LL * 1000 * 192 && sh == 1000LL * 192 && ss == 192);
  layout_strides(ZYFA_LAYOUT_BSHD, kMaxSeqlen, 65536, 192, &sb, &sh, &ss);   // no overflow in 64 bits
  CHECK(sb == (long long)kMaxSeqlen * 65536 * 192);
  CHECK(rows_in_31_bits(32 * 128, 128, 2));
  CHECK(rows_in_31_bits(65536LL * 128, 128, 2));          // 16 MiB rows: 64 of them are 1 GiB
  CHECK(!rows_in_31_bits(262144LL * 128, 128, 2));        // 64 rows of 64 MiB exceed 2^31
  CHECK(!rows_in_31_bits(LLONG_MAX, 128, 2));
  CHECK(!rows_in_31_bits(-1, 128, 1));
  CHECK(clamp_delta(0, 0, 100, 100) == 0);
  CHECK(clamp_delta(700, 0, 300, 1000) == 700);
  CHECK(clamp_delta(5000, 0, 300, 1000) == 1000);
  CHECK(clamp_delta(0, 5000, 300, 1000) == -812);
  CHECK(clamp_delta(LLONG_MAX, LLONG_MIN, 300, 1000) == 1000);   // the difference overflows 64 bits
  CHECK(clamp_delta(LLONG_MIN, LLONG_MAX, 300, 1000) == -812);
  CHECK(clamp_delta(0, 0, kMaxSeqlen, kMaxSeqlen) == 0);
  CHECK(clamp_delta(LLONG_MIN, 0, kMaxSeqlen, kMaxSeqlen) == -kMaxSeqlen - 512);
}

static void signs() {
  unsigned m[4];
  std::vector<signed char> s(128, 1);
  CHECK(sign_mask(nullptr, 128, m) == ZYFA_OK && m[0] == 0 && m[3] == 0);
  s[0] = -1;
  s[37] = -1;
  s[127] = -1;
  CHECK(sign_mask(s.data(), 128, m) == ZYFA_OK);
  CHECK(m[0] == 1u && m[1] == (1u << 5) && m[2] == 0 && m[3] == (1u << 31));
  s[100] = 0;
  CHECK(sign_mask(s.data(), 128, m) == ZYFA_ERR_SIGNS);
  CHECK(sign_mask(s.data(), 64, m) == ZYFA_ERR_HEADDIM);
  CHECK(sign_mask(s.data(), 192, m) == ZYFA_ERR_HEADDIM);
  int x = 0;
  CHECK(aligned(&x, 4) && aligned(reinterpret_cast<char*>(256), 16) && !aligned(reinterpret_cast<char*>(24), 16));
}

// Every query tile of every (batch, head) appears in exactly one job, each
// once, rows past the last job are {-1, -1}, and the table has the shape
// the plan reports.
static void job_tables() {
  const int seqs[] = {1, 2, 127, 128, 129, 255, 256, 257, 1000, 4097, 16384, 32000, 131072};
  const int heads[][2] = {{1, 1}, {4, 1}, {4, 4}, {32, 8}, {64, 8}, {16, 16}};
  const int cus[] = {1, 3, 80, 256, 304};
  for (int b = 1; b <= 3; ++b)
    for (int s : seqs)
      for (auto& hh : heads)
        for (int tq : {128, 256})
          for (int c : cus) {
            const JobTable t = build_job_table(b, s, hh[0], hh[1], tq, c);
            const int n = (s + tq - 1) / tq;
            CHECK(t.tile_q == tq && t.n_qtiles == n);
            CHECK(t.entries.size() == 2ull * t.num_wgs * t.jobs_per_wg);
            CHECK(t.num_wgs >= 1 && t.num_wgs <= c);
            std::vector<int> seen((size_t)b * hh[0] * n, 0);
            long long jobs = 0;
            for (size_t i = 0; i + 1 < t.entries.size(); i += 2) {
              const int bh = t.entries[i], tile = t.entries[i + 1];
              if (bh < 0) {
                CHECK(tile == -1);
                continue;
              }
              ++jobs;
              CHECK(bh < b * hh[0] && tile >= 0 && tile <= n - 1 - tile);
              seen[(size_t)bh * n + tile] += 1;
              if (n - 1 - tile != tile) seen[(size_t)bh * n + n - 1 - tile] += 1;
            }
            CHECK(jobs == (long long)b * hh[0] * ((n + 1) / 2));
            for (int v : seen) CHECK(v == 1);
            const int choice = tile_q_rows(b, s, hh[0], 128, ZYFA_DTYPE_BF16, c);
            CHECK(choice == 128 || choice == 256);
          }
  // the largest sequences the checks admit do not overflow the plan's sizes
  const JobTable big = build_job_table(1, kMaxSeqlen, 1, 1, 128, 256);
  CHECK(big.n_qtiles == kMaxSeqlen / 128);
  CHECK(tile_q_rows(1, kMaxSeqlen, 1, 128, ZYFA_DTYPE_BF16, 256) == 256);
  CHECK(tile_q_rows(1, 16384, 4, 128, ZYFA_DTYPE_FP8_E4M3FN, 256) == 128);
}

int main() {
  shapes();
  strides_and_ranges();
  signs();
  job_tables();
  if (g_failed) {
    std::fprintf(stderr, "%d checks failed\n", g_failed);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
