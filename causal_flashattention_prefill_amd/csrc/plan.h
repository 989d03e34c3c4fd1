// Host-side work distribution for the persistent causal attention kernels.
// Pure C++ (no HIP): unit-testable on any machine.
#pragma once
#include <cstdint>
#include <vector>

namespace zyfa {

// Query-tile height (rows per workgroup job tile): 256, or 128 when that
// shape has too few 256-row jobs to keep num_cus compute units busy.
int tile_q_rows(int batch, int seqlen, int nheads, int d_qk, int dtype, int num_cus);

struct JobTable {
  int tile_q = 0;        // query rows per tile
  int n_qtiles = 0;      // tiles per (batch, head)
  int num_wgs = 0;       // persistent grid size
  int jobs_per_wg = 0;   // rows of the table
  std::vector<int32_t> entries;  // 2 * num_wgs * jobs_per_wg: {bh, tile} or {-1, -1}
};

// Build the job table: query tiles of each (batch, head) paired first with
// last, persistent grid of min(#jobs, num_cus) workgroups, and jobs of one
// time step handed out so that workgroups on the same XCD (blockIdx % 8) get
// consecutive jobs (the same KV head, hence the same K/V in that XCD's L2).
JobTable build_job_table(int batch, int seqlen, int nheads, int nheads_k, int tile_q, int num_cus);

constexpr int kNumXcd = 8;

// Entry (row r, workgroup w) of the job table as {bh, tile} (bh = batch *
// nheads + head; the job covers query tiles tile and n - 1 - tile), or
// {-1, -1} past the last job. Jobs are numbered by batch, then KV head,
// then pair, then the `group` query heads of the KV head (consecutive query
// heads share a KV head): j = ((b * nheads_k + hk) * pairs + tile) * group
// + (h - hk * group). Row r hands out jobs r * num_wgs .. in XCD order: the
// workgroups of XCD 0 (w % 8 == 0, by increasing w), then those of XCD 1,
// and so on, so the workgroups of one XCD take the same pairs of every
// query head of one KV head, which read the same K and V at the same time.
// A constexpr function, so the host plan and the device-side table builder
// share this one definition.
struct JobEntry {
  int bh, tile;
};
constexpr JobEntry job_entry(int r, int w, long long njobs, int num_wgs, int pairs, int group) {
  const int x = w % kNumXcd;
  long long before = 0;   // workgroups of the XCDs before x
  for (int y = 0; y < x; ++y) before += (num_wgs - y + kNumXcd - 1) / kNumXcd;
  const long long j = (long long)r * num_wgs + before + w / kNumXcd;
  if (j >= njobs) return JobEntry{-1, -1};
  const long long per_kv = (long long)pairs * group;   // jobs of one (batch, KV head)
  const long long kv = j / per_kv, idx = j - kv * per_kv;
  return JobEntry{(int)(kv * group + idx % group), (int)(idx / group)};
}

}  // namespace zyfa
