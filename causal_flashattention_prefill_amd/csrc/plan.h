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
// consecutive jobs (same head, hence the same K/V in that XCD's L2).
JobTable build_job_table(int batch, int seqlen, int nheads, int nheads_k, int tile_q, int num_cus);

}  // namespace zyfa
