// Work distribution for the persistent causal kernels ("ZYFA" README,
// Kernel design: work distribution). See plan.h.
#include "plan.h"

#include <algorithm>

namespace zyfa {

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
  const long long n = ((long long)seqlen + tile_q - 1) / tile_q;
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
  t.n_qtiles = (int)(((long long)seqlen + tile_q - 1) / tile_q);
  const int pairs = (t.n_qtiles + 1) / 2;  // the middle tile of an odd count runs alone
  const long long njobs = (long long)batch * nheads * pairs;
  t.num_wgs = (int)std::max<long long>(1, std::min<long long>(njobs, num_cus));
  t.jobs_per_wg = (int)((njobs + t.num_wgs - 1) / t.num_wgs);
  t.entries.assign(size_t(2) * t.num_wgs * t.jobs_per_wg, -1);
  for (int r = 0; r < t.jobs_per_wg; ++r)
    for (int w = 0; w < t.num_wgs; ++w) {
      const JobEntry e = job_entry(r, w, njobs, t.num_wgs, pairs, nheads / nheads_k);
      const size_t i = 2 * (size_t(r) * t.num_wgs + w);
      t.entries[i] = e.bh;
      t.entries[i + 1] = e.tile;
    }
  return t;
}

}  // namespace zyfa
