// Work distribution for the persistent causal kernels ("ZYFA" README,
// Kernel design: work distribution). See plan.h.
#include "plan.h"

#include <algorithm>

namespace zyfa {

static constexpr int kNumXcd = 8;

// Throughput of a compute unit running 128-row tiles (16 query rows per
// wave) relative to 256-row tiles (32 per wave): each K and V fragment read
// from LDS then feeds half as many matrix instructions. Measured on MI355X
// at 16K tokens with every compute unit busy: 0.81 (bf16, d 128) to 0.88
// (fp8, d 192).
static constexpr double kRate128 = 0.82;

// Estimated time of a launch with tile_q-row tiles: rounds of jobs over the
// compute units times the work of the longest job. A pair job (i, n-1-i)
// spans n + 1 key tiles of tile_q x tile_q; a single tile (n = 1) one.
static double est_time(int batch, int seqlen, int nheads, int tile_q, int num_cus, double rate) {
  const long long n = (seqlen + tile_q - 1) / tile_q;
  const long long jobs = (long long)batch * nheads * ((n + 1) / 2);
  const long long rounds = (jobs + num_cus - 1) / num_cus;
  const double work = (n >= 2 ? (double)(n + 1) : 1.0) * tile_q * tile_q;
  return (double)rounds * work / rate;
}

int tile_q_rows(int batch, int seqlen, int nheads, int d_qk, int dtype, int num_cus) {
  (void)d_qk;
  (void)dtype;
  // 256-row tiles (8 waves x 32 rows) unless 128-row tiles finish sooner:
  // when a shape has too few 256-row jobs to occupy every compute unit, the
  // shorter tiles make twice as many jobs of half the work.
  const int c = num_cus > 0 ? num_cus : 1;
  return est_time(batch, seqlen, nheads, 128, c, kRate128) < est_time(batch, seqlen, nheads, 256, c, 1.0) ? 128
                                                                                                           : 256;
}

JobTable build_job_table(int batch, int seqlen, int nheads, int nheads_k, int tile_q, int num_cus) {
  JobTable t;
  t.tile_q = tile_q;
  t.n_qtiles = (seqlen + tile_q - 1) / tile_q;
  const int pairs = (t.n_qtiles + 1) / 2;  // the middle tile of an odd count runs alone
  // Job order: batch, then KV head, then the query heads of its group, then
  // pairs. Query heads of one group are adjacent, so nearby jobs read the
  // same K/V.
  const int group = nheads / nheads_k;
  std::vector<int32_t> jobs;
  jobs.reserve(size_t(batch) * nheads * pairs * 2);
  for (int b = 0; b < batch; ++b)
    for (int hk = 0; hk < nheads_k; ++hk)
      for (int h = hk * group; h < (hk + 1) * group; ++h)
        for (int i = 0; i < pairs; ++i) {
          jobs.push_back(b * nheads + h);
          jobs.push_back(i);
        }
  const long long njobs = (long long)jobs.size() / 2;
  t.num_wgs = (int)std::max<long long>(1, std::min<long long>(njobs, num_cus));
  t.jobs_per_wg = (int)((njobs + t.num_wgs - 1) / t.num_wgs);
  t.entries.assign(size_t(2) * t.num_wgs * t.jobs_per_wg, -1);
  // Workgroups of XCD x are {x, x + 8, ...}; list them per XCD.
  std::vector<std::vector<int>> xcd_wgs(kNumXcd);
  for (int w = 0; w < t.num_wgs; ++w) xcd_wgs[w % kNumXcd].push_back(w);
  long long next = 0;
  for (int r = 0; r < t.jobs_per_wg && next < njobs; ++r) {
    // This row hands out jobs [next, next + num_wgs): XCD x takes a
    // contiguous run of them, one per workgroup it owns.
    for (int x = 0; x < kNumXcd && next < njobs; ++x)
      for (int w : xcd_wgs[x]) {
        if (next >= njobs) break;
        const size_t e = 2 * (size_t(r) * t.num_wgs + w);
        t.entries[e] = jobs[2 * next];
        t.entries[e + 1] = jobs[2 * next + 1];
        ++next;
      }
  }
  return t;
}

}  // namespace zyfa
