// Host side of the C ABI (include/zyfa.h): argument checks, the per-shape
// plan cache, and kernel launches. Nothing here computes attention; every
// step of the path runs in the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "zyfa.h"
#include "args.h"
#include "plan.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

struct PlanKey {
  int device, batch, seqlen, nheads, nheads_k, d_qk, dtype;
  int tile_q;  // 0 in a shape's key, the query-tile height in a plan's key
  bool operator<(const PlanKey& o) const {
    return std::tie(device, batch, seqlen, nheads, nheads_k, d_qk, dtype, tile_q) <
           std::tie(o.device, o.batch, o.seqlen, o.nheads, o.nheads_k, o.d_qk, o.dtype, o.tile_q);
  }
};

struct Plan {
  int2* jobs = nullptr;  // device copy of the job table
  int num_wgs = 0;
  int jobs_per_wg = 0;
  int n_qtiles = 0;
  int tile_q = 0;
};

std::mutex g_mu;
std::map<PlanKey, Plan> g_plans;
std::map<PlanKey, int> g_tile_choice;   // query-tile heights set by zyfa_set_tile_q
// compute units per device, looked up once (a fixed array: zyfa_fwd_noalloc
// allocates nothing, host memory included)
constexpr int kMaxDevices = 64;
int g_num_cus[kMaxDevices] = {};

int current_device(int* dev) {
  return hipGetDevice(dev) == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

int num_cus(int dev) {
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && g_num_cus[dev] > 0) return g_num_cus[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (cached) g_num_cus[dev] = n;
  return n;
}

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// Finds or builds the plan of a shape (shape.tile_q == 0): with tile_q
// rows when given, else with the height set for the shape, else the
// automatic one; caller holds g_mu.
int get_plan(const PlanKey& shape, hipStream_t stream, const Plan** out, int tile_q = 0) {
  const int cus = num_cus(shape.device);
  const auto ch = g_tile_choice.find(shape);
  PlanKey key = shape;
  key.tile_q = tile_q                    ? tile_q
               : ch != g_tile_choice.end() ? ch->second
                                           : tile_q_rows(shape.batch, shape.seqlen, shape.nheads, shape.d_qk,
                                                         shape.dtype, cus);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *out = &it->second;
    return ZYFA_OK;
  }
  if (stream_capturing(stream)) return ZYFA_ERR_CAPTURE;
  JobTable t = build_job_table(key.batch, key.seqlen, key.nheads, key.nheads_k, key.tile_q, cus);
  Plan p;
  p.num_wgs = t.num_wgs;
  p.jobs_per_wg = t.jobs_per_wg;
  p.n_qtiles = t.n_qtiles;
  p.tile_q = t.tile_q;
  const size_t bytes = t.entries.size() * sizeof(int32_t);
  if (hipMalloc(&p.jobs, bytes) != hipSuccess) return ZYFA_ERR_HIP;
  if (hipMemcpy(p.jobs, t.entries.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p.jobs);
    return ZYFA_ERR_HIP;
  }
  *out = &(g_plans[key] = p);
  return ZYFA_OK;
}

bool aligned16(const void* p) { return aligned(p, 16); }

// Whole-sequence attention is the range call with seqlen_q == seqlen_k and
// q_pos0 == k_pos0.
// noalloc: no plan cache; the job table is written by a kernel into the
// library's static buffer (zyfa_fwd_noalloc).
int fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen,
             int seqlen_k, long long q_pos0, long long k_pos0, int nheads, int nheads_k, int d_qk, int d_v,
             int layout, int dtype, const float* q_descale, const float* k_descale, const float* v_descale,
             float softmax_scale, int p_mode, void* stream_, bool noalloc = false) {
  int rc = check_shape(batch, seqlen, nheads, nheads_k, d_qk, d_v, layout, dtype);
  if (rc) return rc;
  if (seqlen_k <= 0 || seqlen_k > kMaxSeqlen) return ZYFA_ERR_SHAPE;
  if (p_mode != ZYFA_P_DEFAULT && p_mode != ZYFA_P_EXACT && p_mode != ZYFA_P_LEAN && p_mode != ZYFA_P_PRECISE)
    return ZYFA_ERR_PMODE;
  if (!q || !k || !v || !out) return ZYFA_ERR_NULL;
  if (dtype == ZYFA_DTYPE_FP8_E4M3FN && (!q_descale || !k_descale || !v_descale)) return ZYFA_ERR_DESCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ZYFA_ERR_ALIGN;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int esz = dtype == ZYFA_DTYPE_BF16 ? 2 : 1;

  int dev;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  const Plan* plan = nullptr;
  Plan na_plan;   // noalloc: the plan's sizes, its table in the static buffer
  PlanKey key{dev, batch, seqlen, nheads, nheads_k, d_qk, dtype, 0};
  // the precise FP8 mode runs on 128-row query tiles only
  const bool precise = dtype == ZYFA_DTYPE_FP8_E4M3FN && p_mode == ZYFA_P_PRECISE;
  if (noalloc) {
    const auto ch = g_tile_choice.find(key);
    const int tq = precise ? 128 : ch != g_tile_choice.end() ? ch->second
                                                            : tile_q_rows(batch, seqlen, nheads, d_qk, dtype,
                                                                          num_cus(dev));
    const int n_qtiles = (seqlen + tq - 1) / tq;
    const int pairs = (n_qtiles + 1) / 2;
    const long long njobs = (long long)batch * nheads * pairs;
    const long long wgs = std::max<long long>(1, std::min<long long>(njobs, num_cus(dev)));
    const long long rows = (njobs + wgs - 1) / wgs;
    if (rows * wgs > noalloc_scratch_entries()) return ZYFA_ERR_SCRATCH;
    int2* table = nullptr;
    if (noalloc_scratch(dev, &table) != hipSuccess) return ZYFA_ERR_HIP;
    na_plan.jobs = table;
    na_plan.num_wgs = (int)wgs;
    na_plan.jobs_per_wg = (int)rows;
    na_plan.n_qtiles = n_qtiles;
    na_plan.tile_q = tq;
    plan = &na_plan;
  } else if ((rc = get_plan(key, stream, &plan, precise ? 128 : 0))) {
    return rc;
  }

  AttnArgs a{};
  a.q.ptr = q;
  a.k.ptr = k;
  a.v.ptr = v;
  layout_strides(layout, seqlen, nheads, d_qk, &a.q.stride_b, &a.q.stride_h, &a.q.stride_s);
  layout_strides(layout, seqlen_k, nheads_k, d_qk, &a.k.stride_b, &a.k.stride_h, &a.k.stride_s);
  layout_strides(layout, seqlen_k, nheads_k, d_v, &a.v.stride_b, &a.v.stride_h, &a.v.stride_s);
  layout_strides(layout, seqlen, nheads, d_v, &a.o_stride_b, &a.o_stride_h, &a.o_stride_s);
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.seqlen_q = seqlen;
  a.seqlen_k = seqlen_k;
  // key c is visible to query row r when c <= r + delta
  a.delta = clamp_delta(q_pos0, k_pos0, seqlen, seqlen_k);
  a.nheads = nheads;
  a.nheads_k = nheads_k;
  a.n_qtiles = plan->n_qtiles;
  a.jobs_per_wg = plan->jobs_per_wg;
  a.num_wgs = plan->num_wgs;
  a.jobs = plan->jobs;
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)d_qk);
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  // The kernels address each wave's query rows and each half key tile (at
  // most 64 rows) through a buffer resource of its own with a 64-bit base,
  // so only 64 rows of a tensor must fit in 31 bits of byte offset; tensors
  // and (batch, head) slices may span more than 4 GiB.
  if (!rows_in_31_bits(a.q.stride_s, d_qk, esz) || !rows_in_31_bits(a.k.stride_s, d_qk, esz) ||
      !rows_in_31_bits(a.v.stride_s, d_v, esz))
    return ZYFA_ERR_RANGE;

  hipError_t e;
  if (noalloc) {
    const int pairs = (plan->n_qtiles + 1) / 2;
    e = launch_build_jobs(const_cast<int2*>(plan->jobs), plan->jobs_per_wg, plan->num_wgs,
                          (long long)batch * nheads * pairs, pairs, nheads / nheads_k, stream);
    if (e != hipSuccess) return ZYFA_ERR_HIP;
  }
  if (dtype == ZYFA_DTYPE_BF16)
    e = launch_attn_bf16(a, d_qk, lse != nullptr, plan->tile_q, plan->num_wgs, stream);
  else
    e = launch_attn_fp8(a, d_qk, lse != nullptr,
                        p_mode == ZYFA_P_PRECISE                                       ? FP8Mode::kPrecise
                        : p_mode == ZYFA_P_LEAN || (p_mode == ZYFA_P_DEFAULT && d_qk == 128) ? FP8Mode::kLean
                                                                                           : FP8Mode::kExact,
                        plan->tile_q, plan->num_wgs, stream);
  return e == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

}  // namespace
}  // namespace zyfa

using namespace zyfa;

namespace {

int quantize_rotated_impl(const void* x, int x_dtype, long long rows, int d, const signed char* signs,
                          const float* shift, int seqlen, int nheads, bool bshd, void* x8, float* descale,
                          void* stream_) {
  if (x_dtype != ZYFA_DTYPE_BF16 && x_dtype != ZYFA_DTYPE_FP32) return ZYFA_ERR_DTYPE;
  if (rows < 0) return ZYFA_ERR_SHAPE;
  unsigned mask[4];
  const int rc = sign_mask(signs, d, mask);
  if (rc) return rc;
  if (!descale || (rows > 0 && (!x || !x8))) return ZYFA_ERR_NULL;
  if (rows > 0 && (!aligned16(x) || !aligned16(x8))) return ZYFA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(descale) & 3u) return ZYFA_ERR_ALIGN;
  if (shift && !aligned16(shift)) return ZYFA_ERR_ALIGN;
  hipError_t e = launch_fp8_quantize_rotated(x, x_dtype == ZYFA_DTYPE_BF16 ? 0 : 2, rows, d, mask, shift, seqlen,
                                             nheads, bshd, x8, descale, reinterpret_cast<hipStream_t>(stream_));
  return e == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

}  // namespace

extern "C" {

int zyfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen, int nheads,
             int nheads_k, int d_qk, int d_v, int layout, int dtype, const float* q_descale, const float* k_descale,
             const float* v_descale, void* stream) {
  return fwd_impl(q, k, v, out, lse, batch, seqlen, seqlen, 0, 0, nheads, nheads_k, d_qk, d_v, layout, dtype,
                  q_descale, k_descale, v_descale, 0.f, ZYFA_P_DEFAULT, stream);
}

int zyfa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen,
                int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype, const float* q_descale,
                const float* k_descale, const float* v_descale, float softmax_scale, int p_mode, void* stream) {
  return fwd_impl(q, k, v, out, lse, batch, seqlen, seqlen, 0, 0, nheads, nheads_k, d_qk, d_v, layout, dtype,
                  q_descale, k_descale, v_descale, softmax_scale, p_mode, stream);
}

int zyfa_fwd_range(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen_q,
                   int seqlen_k, long long q_pos0, long long k_pos0, int nheads, int nheads_k, int d_qk, int d_v,
                   int layout, int dtype, const float* q_descale, const float* k_descale, const float* v_descale,
                   float softmax_scale, int p_mode, void* stream) {
  return fwd_impl(q, k, v, out, lse, batch, seqlen_q, seqlen_k, q_pos0, k_pos0, nheads, nheads_k, d_qk, d_v, layout,
                  dtype, q_descale, k_descale, v_descale, softmax_scale, p_mode, stream);
}

int zyfa_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen,
                     int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype, const float* q_descale,
                     const float* k_descale, const float* v_descale, float softmax_scale, int p_mode, void* stream) {
  return fwd_impl(q, k, v, out, lse, batch, seqlen, seqlen, 0, 0, nheads, nheads_k, d_qk, d_v, layout, dtype,
                  q_descale, k_descale, v_descale, softmax_scale, p_mode, stream, true);
}

int zyfa_lse_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b, void* out,
                   float* lse, int batch, int seqlen, int nheads, int d_v, int layout, void* stream) {
  if (batch <= 0 || seqlen <= 0 || nheads <= 0) return ZYFA_ERR_SHAPE;
  if (d_v != 128) return ZYFA_ERR_HEADDIM;
  if (layout != ZYFA_LAYOUT_BSHD && layout != ZYFA_LAYOUT_BHSD) return ZYFA_ERR_LAYOUT;
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return ZYFA_ERR_NULL;
  if (!aligned16(out_a) || !aligned16(out_b) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse_a) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_b) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ZYFA_ERR_ALIGN;
  const hipError_t e = launch_lse_merge(out_a, lse_a, out_b, lse_b, out, lse, batch, seqlen, nheads, d_v,
                                        layout == ZYFA_LAYOUT_BSHD, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

int zyfa_prepare(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype,
                 int with_lse, void* stream) {
  (void)with_lse;
  int rc = check_shape(batch, seqlen, nheads, nheads_k, d_qk, d_v, layout, dtype);
  if (rc) return rc;
  int dev;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  const Plan* plan = nullptr;
  PlanKey key{dev, batch, seqlen, nheads, nheads_k, d_qk, dtype, 0};
  if ((rc = get_plan(key, reinterpret_cast<hipStream_t>(stream), &plan))) return rc;
  // FP8: also the 128-row plan of the precise mode
  if (dtype == ZYFA_DTYPE_FP8_E4M3FN) rc = get_plan(key, reinterpret_cast<hipStream_t>(stream), &plan, 128);
  return rc;
}

int zyfa_set_tile_q(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int dtype, int tile_q) {
  int rc = check_shape(batch, seqlen, nheads, nheads_k, d_qk, 128, ZYFA_LAYOUT_BSHD, dtype);
  if (rc) return rc;
  if (tile_q != 0 && tile_q != 128 && tile_q != 256) return ZYFA_ERR_SHAPE;
  int dev;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  const PlanKey shape{dev, batch, seqlen, nheads, nheads_k, d_qk, dtype, 0};
  if (tile_q == 0) g_tile_choice.erase(shape);
  else g_tile_choice[shape] = tile_q;
  return ZYFA_OK;
}

int zyfa_fp8_quantize(const void* x, int x_dtype, long long numel, void* x8, float* descale, void* stream_) {
  if (x_dtype != ZYFA_DTYPE_BF16 && x_dtype != ZYFA_DTYPE_FP32) return ZYFA_ERR_DTYPE;
  if (numel < 0) return ZYFA_ERR_SHAPE;
  if (!descale || (numel > 0 && (!x || !x8))) return ZYFA_ERR_NULL;
  if (numel > 0 && (!aligned16(x) || !aligned16(x8))) return ZYFA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(descale) & 3u) return ZYFA_ERR_ALIGN;
  hipError_t e = launch_fp8_quantize(x, x_dtype == ZYFA_DTYPE_BF16 ? 0 : 2, numel, x8, descale,
                                     reinterpret_cast<hipStream_t>(stream_));
  return e == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

int zyfa_fp8_quantize_rotated(const void* x, int x_dtype, long long rows, int d, const signed char* signs, void* x8,
                              float* descale, void* stream) {
  return quantize_rotated_impl(x, x_dtype, rows, d, signs, nullptr, 1, 1, true, x8, descale, stream);
}

int zyfa_fp8_quantize_rotated_shifted(const void* x, int x_dtype, int batch, int seqlen, int nheads, int d,
                                      int layout, const signed char* signs, const float* shift, void* x8,
                                      float* descale, void* stream) {
  if (batch <= 0 || seqlen <= 0 || nheads <= 0) return ZYFA_ERR_SHAPE;
  if (layout != ZYFA_LAYOUT_BSHD && layout != ZYFA_LAYOUT_BHSD) return ZYFA_ERR_LAYOUT;
  if (!shift) return ZYFA_ERR_NULL;
  const long long rows = (long long)batch * seqlen * nheads;
  if (rows > 0x7FFFFFFFll) return ZYFA_ERR_RANGE;   // rows are indexed in 32 bits here
  return quantize_rotated_impl(x, x_dtype, rows, d, signs, shift, seqlen, nheads, layout == ZYFA_LAYOUT_BSHD, x8,
                               descale, stream);
}

int zyfa_key_mean(const void* k, int k_dtype, int batch, int seqlen, int nheads_k, int d, int layout, float* mean,
                  void* stream) {
  if (k_dtype != ZYFA_DTYPE_BF16 && k_dtype != ZYFA_DTYPE_FP32) return ZYFA_ERR_DTYPE;
  if (batch <= 0 || seqlen <= 0 || nheads_k <= 0) return ZYFA_ERR_SHAPE;
  if (d != 128 && d != 192) return ZYFA_ERR_HEADDIM;
  if (layout != ZYFA_LAYOUT_BSHD && layout != ZYFA_LAYOUT_BHSD) return ZYFA_ERR_LAYOUT;
  if (!k || !mean) return ZYFA_ERR_NULL;
  if (!aligned16(k) || (reinterpret_cast<uintptr_t>(mean) & 3u)) return ZYFA_ERR_ALIGN;
  const hipError_t e = launch_key_mean(k, k_dtype == ZYFA_DTYPE_BF16 ? 0 : 2, batch, seqlen, nheads_k, d,
                                       layout == ZYFA_LAYOUT_BSHD, mean, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZYFA_OK : ZYFA_ERR_HIP;
}

const char* zyfa_status_string(int status) {
  switch (status) {
    case ZYFA_OK: return "ok";
    case ZYFA_ERR_NULL: return "a required pointer is NULL";
    case ZYFA_ERR_SHAPE: return "batch, seqlen, nheads and nheads_k must be positive (numel non-negative)";
    case ZYFA_ERR_HEADDIM: return "unsupported head dims: (d_qk, d_v) must be (128, 128) or (192, 128)";
    case ZYFA_ERR_GQA: return "nheads must be a multiple of nheads_k";
    case ZYFA_ERR_DTYPE: return "unknown dtype";
    case ZYFA_ERR_LAYOUT: return "unknown layout (0 = bshd, 1 = bhsd)";
    case ZYFA_ERR_DESCALE: return "FP8 inputs need q, k and v descale pointers";
    case ZYFA_ERR_CAPTURE: return "the plan for this shape must be built (zyfa_prepare) before graph capture";
    case ZYFA_ERR_HIP: return "a HIP runtime call failed";
    case ZYFA_ERR_RANGE: return "the row stride is too large: 64 rows must span at most 2^31 bytes";
    case ZYFA_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case ZYFA_ERR_PMODE: return "unknown FP8 probability mode";
    case ZYFA_ERR_SIGNS: return "rotation signs must each be +1 or -1";
    case ZYFA_ERR_SCRATCH: return "the call's job table exceeds the no-allocation buffer (65536 entries)";
    default: return "unknown status";
  }
}

void zyfa_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  // hipFree waits for work still using the memory; errors are ignored (the
  // cache is emptied either way)
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_plans) {
    (void)hipSetDevice(kv.first.device);
    (void)hipFree(kv.second.jobs);
  }
  g_plans.clear();
  (void)hipSetDevice(cur);
}

int zyfa_plan_jobs(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int dtype, int num_cus_, int* out_tile_q,
                   int* out_num_wgs, int* out_jobs_per_wg, int* table, long long table_capacity) {
  int rc = check_shape(batch, seqlen, nheads, nheads_k, d_qk, 128, ZYFA_LAYOUT_BSHD, dtype);
  if (rc) return rc;
  if (num_cus_ <= 0) return ZYFA_ERR_SHAPE;
  if (!out_tile_q || !out_num_wgs || !out_jobs_per_wg) return ZYFA_ERR_NULL;
  JobTable t = build_job_table(batch, seqlen, nheads, nheads_k,
                               tile_q_rows(batch, seqlen, nheads, d_qk, dtype, num_cus_), num_cus_);
  *out_tile_q = t.tile_q;
  *out_num_wgs = t.num_wgs;
  *out_jobs_per_wg = t.jobs_per_wg;
  if (table) {
    if (table_capacity < (long long)t.entries.size()) return ZYFA_ERR_SHAPE;
    for (size_t i = 0; i < t.entries.size(); ++i) table[i] = t.entries[i];
  }
  return ZYFA_OK;
}

}  // extern "C"
