// Internal declarations shared by the host API and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace zyfa {

// One (batch, head) slice of a tensor: base offset strides in elements.
struct TensorDesc {
  const void* ptr;
  long long stride_b;   // elements between batches
  long long stride_h;   // elements between heads
  long long stride_s;   // elements between positions (rows)
};

struct AttnArgs {
  TensorDesc q, k, v;
  void* out;
  long long o_stride_b, o_stride_h, o_stride_s;
  float* lse;                 // may be null
  int batch, nheads, nheads_k;
  int seqlen_q, seqlen_k;     // query rows and keys per (batch, head)
  int delta;                  // key c is visible to query row r when c <= r + delta
  int n_qtiles;               // query tiles per (batch, head)
  int jobs_per_wg;
  int num_wgs;                // workgroups of the launch (the job table's row length)
  const int2* jobs;           // [jobs_per_wg][gridDim.x]
  float scale_log2;           // softmax_scale * log2(e)
  const float* q_descale;     // fp8 only
  const float* k_descale;
  const float* v_descale;
};

// tile_q: query rows per tile, 256 (32 per wave) or 128 (16 per wave)
hipError_t launch_attn_bf16(const AttnArgs& a, int d_qk, bool with_lse, int tile_q, int grid, hipStream_t s);
// How the FP8 kernel rounds probabilities (and, precise, computes scores);
// zyfa_p_mode resolved for the call's head dim.
enum class FP8Mode { kExact, kLean, kPrecise };
hipError_t launch_attn_fp8(const AttnArgs& a, int d_qk, bool with_lse, FP8Mode mode, int tile_q, int grid,
                           hipStream_t s);
// x8 doubles as the scratch of the amax partials (overwritten by the codes)
hipError_t launch_fp8_quantize(const void* x, int x_dtype, long long numel, void* x8, float* descale,
                               hipStream_t s);
// d: 128; sign_mask: four words, bit i set when channel i's sign is -1
// shift: null, or a device vector per (batch, head) slot subtracted from
// each row before the rotation (rows in the tensor's memory order, seqlen
// positions and nheads heads per batch, bshd or bhsd)
hipError_t launch_fp8_quantize_rotated(const void* x, int x_dtype, long long rows, int d, const unsigned* sign_mask,
                                       const float* shift, int seqlen, int nheads, bool bshd, void* x8,
                                       float* descale, hipStream_t s);
hipError_t launch_key_mean(const void* x, int x_dtype, int batch, int seqlen, int nheads, int d, bool bshd,
                           float* mean, hipStream_t s);
// zyfa_fwd_noalloc: the static job-table buffer (its capacity in entries and
// its device address on device dev, looked up on first use) and the kernel
// that writes a job table into it.
int noalloc_scratch_entries();
hipError_t noalloc_scratch(int dev, int2** out);
hipError_t launch_build_jobs(int2* table, int rows, int num_wgs, long long njobs, int pairs, int group,
                             hipStream_t s);
hipError_t launch_lse_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b, void* out,
                            float* lse, int batch, int seqlen, int nheads, int d_v, bool bshd, hipStream_t s);

}  // namespace zyfa
