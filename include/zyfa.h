/*
 * zyfa.h - C ABI of the causal prefill attention library for MI355X (gfx950).
 *
 * What the library computes is defined on the "ZYFA" README (GitHub page of
 * Zyphra/zyfa), sections Usage and Supported configurations: the causal
 * forward attention pass of LLM prefill (seqlen_q == seqlen_k),
 *     out[i] = sum_{j<=i} softmax_j(scale * <q_i, k_j>) * v_j,
 * with an optional natural-log log-sum-exp per row, for BF16 inputs or FP8
 * e4m3fn inputs with one descale per tensor, for MHA, GQA and MQA, and for
 * head dims d_qk = d_v = 128 or d_qk = 192 with d_v = 128. The output is
 * always BF16.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to contiguous tensors owned by the
 *    caller; the library never frees or retains them past the call.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Work is
 *    enqueued asynchronously; no call waits on the host in the steady state.
 *  - Every call returns ZYFA_OK (0) or a negative ZYFA_ERR_* status and
 *    never throws. Argument checks happen before anything is enqueued.
 */
#ifndef ZYFA_H
#define ZYFA_H

#ifdef __cplusplus
extern "C" {
#endif

enum zyfa_status {
  ZYFA_OK = 0,
  ZYFA_ERR_NULL = -1,      /* a required pointer is NULL */
  ZYFA_ERR_SHAPE = -2,     /* batch, seqlen, nheads or nheads_k <= 0, or numel < 0 */
  ZYFA_ERR_HEADDIM = -3,   /* (d_qk, d_v) not (128, 128) or (192, 128) */
  ZYFA_ERR_GQA = -4,       /* nheads is not a multiple of nheads_k */
  ZYFA_ERR_DTYPE = -5,     /* unknown dtype enum */
  ZYFA_ERR_LAYOUT = -6,    /* unknown layout enum */
  ZYFA_ERR_DESCALE = -7,   /* FP8 call without all three descale pointers */
  ZYFA_ERR_CAPTURE = -8,   /* a per-shape plan must be built while the stream is capturing */
  ZYFA_ERR_HIP = -9,       /* a HIP runtime call failed (launch, allocation, copy) */
  ZYFA_ERR_RANGE = -10,    /* 64 rows of one tensor span more than 2^31 bytes (tensors and
                              slices beyond 4 GiB are fine) */
  ZYFA_ERR_ALIGN = -11,    /* a tensor pointer is not 16-byte aligned */
  ZYFA_ERR_PMODE = -12,    /* unknown FP8 probability mode */
  ZYFA_ERR_SIGNS = -13,    /* a rotation sign other than +1 or -1 */
  ZYFA_ERR_SCRATCH = -14   /* zyfa_fwd_noalloc: the job table exceeds the static buffer */
};

enum zyfa_layout {
  ZYFA_LAYOUT_BSHD = 0,    /* (batch, seqlen, heads, head_dim) */
  ZYFA_LAYOUT_BHSD = 1     /* (batch, heads, seqlen, head_dim) */
};

enum zyfa_dtype {
  ZYFA_DTYPE_BF16 = 0,
  ZYFA_DTYPE_FP8_E4M3FN = 1,  /* OCP e4m3fn: 4 exponent bits (bias 7), 3 mantissa bits, max 448 */
  ZYFA_DTYPE_FP32 = 2         /* accepted by zyfa_fp8_quantize as its input only */
};

/*
 * zyfa_fwd - causal forward attention ("ZYFA" README: Usage; Supported
 * configurations).
 *
 *  q    [batch, seqlen, nheads,   d_qk] (bshd) or [batch, nheads,   seqlen, d_qk] (bhsd)
 *  k    [batch, seqlen, nheads_k, d_qk] or [batch, nheads_k, seqlen, d_qk]
 *  v    [batch, seqlen, nheads_k, d_v ] or [batch, nheads_k, seqlen, d_v ]
 *  out  q's layout with head dim d_v, always bf16, written for real rows only.
 *  lse  NULL, or fp32 [batch, nheads, seqlen]: natural-log log-sum-exp of
 *       each row of scaled scores. For FP8 it is taken from the same rounded
 *       probabilities that multiply V (README, Accuracy).
 *  dtype ZYFA_DTYPE_BF16 (q, k, v bf16) or ZYFA_DTYPE_FP8_E4M3FN (q, k, v
 *       e4m3fn codes). For FP8, q_descale/k_descale/v_descale each point to
 *       ONE positive normal fp32 value in device memory; the kernel reads and
 *       applies them itself, and does not check them (README, Usage). They
 *       are ignored (may be NULL) for BF16.
 *  Query head h uses KV head floor(h * nheads_k / nheads) (consecutive
 *  query heads share a KV head). The softmax scale is 1/sqrt(d_qk).
 *  Any seqlen >= 1 works: rows past seqlen read as zeros up to the kernel's
 *  query-tile multiple, which is exact for causal attention (README, Usage).
 *  A shape's plan (its job table) is made on its first call, with a
 *  blocking host-to-device copy; call zyfa_prepare first if the call is to
 *  be captured into a graph.
 */
int zyfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v,
             int layout, int dtype,
             const float* q_descale, const float* k_descale, const float* v_descale,
             void* stream);

/*
 * How the FP8 kernels turn scores into e4m3fn probabilities ("ZYFA" README,
 * Kernel design: lean P, per-block scaling). Every mode rounds the
 * probabilities of each 32-key block relative to a power of two, multiplies
 * V by the rounded values and divides by their sum (README, Accuracy).
 *  ZYFA_P_DEFAULT  ZYFA_P_LEAN at d_qk = 128, ZYFA_P_EXACT at d_qk = 192
 *                  (the README's choice per head dim).
 *  ZYFA_P_EXACT    exact P: e4m3fn RNE of exp2 of the base-2 score.
 *  ZYFA_P_LEAN     lean P for keys below the query's own 256-row block
 *                  (keys j < 256 floor(i / 256) of row i, at either query-
 *                  tile height): the code of 2^y
 *                  is RNE(8 y + 56 + 8 log2(2 ln^2 2)) read as an integer
 *                  (interpolates 2^y linearly between powers of two,
 *                  unbiased on average); keys from that tile on, which
 *                  include every key of the rows with fewest keys, keep
 *                  exact P.
 *  ZYFA_P_PRECISE  for inputs whose channels differ widely in magnitude
 *                  (activations with outlier channels): the scores are
 *                  computed on the bf16 matrix instruction from the e4m3
 *                  codes (exact products, fp32-accurate sums; the FP8
 *                  matrix instructions sum to about 2^-11.5 of
 *                  sum_c |q_c k_c| there), and each probability is split
 *                  into two e4m3 values hi = RNE(p), lo = RNE(p - hi), both
 *                  multiplied into V and summed into the denominator (about
 *                  7 significant bits of p instead of 4). Exact P
 *                  otherwise. Always runs on 128-row query tiles (its
 *                  operands do not fit the register file at 256 rows);
 *                  slower than the other modes.
 * BF16 calls ignore the mode.
 */
enum zyfa_p_mode {
  ZYFA_P_DEFAULT = 0,
  ZYFA_P_EXACT = 1,
  ZYFA_P_LEAN = 2,
  ZYFA_P_PRECISE = 3
};

/* zyfa_fwd with an explicit softmax scale (flash-attn's softmax_scale
 * argument, README: Differences from flash-attn; softmax_scale <= 0 selects
 * 1/sqrt(d_qk)) and an FP8 probability mode (enum zyfa_p_mode; any other
 * value returns ZYFA_ERR_PMODE). */
int zyfa_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v,
                int layout, int dtype,
                const float* q_descale, const float* k_descale, const float* v_descale,
                float softmax_scale, int p_mode, void* stream);

/*
 * zyfa_fwd_noalloc - zyfa_fwd_ex for callers that cannot allocate device
 * memory: code under graph capture that has not called zyfa_prepare, tight
 * serving loops, harnesses that forbid allocation. Same arguments and
 * results (bitwise equal to zyfa_fwd_ex). Instead of the cached per-shape
 * plan it writes the job table with a small kernel, on `stream` just before
 * the attention kernel, into a static device buffer of the library (65536
 * entries of 8 bytes, 512 KiB, held on each GPU the library runs on until
 * the process ends): no hipMalloc, no hipFree, no host-to-device copy. Calls
 * on one GPU share that buffer, so calls that overlap (other streams,
 * parallel graph branches) race: serialize them. The buffer's address is
 * looked up once per device on the first call there.
 * Returns ZYFA_ERR_SCRATCH when the table (nheads * batch * ceil(tiles / 2)
 * jobs, rounded up to a multiple of the grid) exceeds 65536 entries, e.g.
 * beyond about 512K tokens at 32 heads; other errors as zyfa_fwd_ex.
 */
int zyfa_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                     int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v,
                     int layout, int dtype,
                     const float* q_descale, const float* k_descale, const float* v_descale,
                     float softmax_scale, int p_mode, void* stream);

/*
 * zyfa_fwd_range - causal attention of a block of queries over a range of
 * keys, returning the partial output and its LSE so that results over
 * different key ranges can be merged ("ZYFA" README, Accuracy: the FP8 LSE
 * is computed from the same rounded probabilities as the output, which keeps
 * merges over key ranges consistent; the flash-attention RDNA3 page's split
 * of the keys with an LSE merge). Uses: chunked prefill
 * (a chunk of new queries over the cached prefix and itself) and a sequence
 * split over devices.
 *  Query row r sits at absolute position q_pos0 + r, key c at k_pos0 + c;
 *  key c is visible to row r when k_pos0 + c <= q_pos0 + r.
 *  q       [batch, seqlen_q, nheads, d_qk] (bshd) or [batch, nheads, seqlen_q,
 *          d_qk] (bhsd); k and v the same with seqlen_k and nheads_k.
 *  out     q's layout with head dim d_v, bf16. lse: fp32 [batch, nheads,
 *          seqlen_q], natural log, or NULL.
 *  A row that sees no key gets out = 0 and lse = -inf (the merge's
 *  identity). q_pos0 == k_pos0 with seqlen_q == seqlen_k is zyfa_fwd_ex.
 *  Every other argument, the errors and the plan (keyed by seqlen_q: pass
 *  seqlen = seqlen_q to zyfa_prepare) are those of zyfa_fwd_ex;
 *  seqlen_k <= 0 returns ZYFA_ERR_SHAPE.
 */
int zyfa_fwd_range(const void* q, const void* k, const void* v, void* out, float* lse,
                   int batch, int seqlen_q, int seqlen_k, long long q_pos0, long long k_pos0,
                   int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype,
                   const float* q_descale, const float* k_descale, const float* v_descale,
                   float softmax_scale, int p_mode, void* stream);

/*
 * zyfa_lse_merge - merge two partial results of the same query rows over
 * disjoint key sets (as zyfa_fwd_range returns them) into the result over
 * both. Per row, with L_a, L_b the partial LSEs:
 *   L = ln(e^L_a + e^L_b),  out = e^(L_a - L) out_a + e^(L_b - L) out_b
 * and L = -inf, out = 0 when both are -inf. Arithmetic in fp32, out rounded
 * to bf16 (RNE).
 *  out_a, out_b, out  bf16, [batch, seqlen, nheads, d_v] (bshd) or
 *                     [batch, nheads, seqlen, d_v] (bhsd), 16-byte aligned;
 *  lse_a, lse_b, lse  fp32 [batch, nheads, seqlen].
 *  out may be out_a or out_b and lse may be lse_a or lse_b (merging in
 *  place); other overlaps are undefined. d_v must be 128
 *  (ZYFA_ERR_HEADDIM otherwise). Asynchronous on `stream`; allocates
 *  nothing.
 */
int zyfa_lse_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                   void* out, float* lse, int batch, int seqlen, int nheads, int d_v, int layout,
                   void* stream);

/*
 * zyfa_prepare - build (or find) the per-shape plan ahead of time so that a
 * later zyfa_fwd with the same shape allocates nothing and copies nothing
 * from the host (README, Usage: run each new shape once before capturing).
 * For FP8 it also builds the 128-row plan of ZYFA_P_PRECISE. with_lse is
 * accepted for symmetry and ignored (plans do not depend on it).
 * Returns ZYFA_ERR_CAPTURE if the plan is missing and `stream` is capturing.
 */
int zyfa_prepare(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v,
                 int layout, int dtype, int with_lse, void* stream);

/*
 * zyfa_set_tile_q - set the query-tile height that calls of one shape use
 * on the current device from now on. The README's work distribution pairs
 * query tiles of one (batch, head) first with last and hands the pairs to
 * a persistent grid; a shape with too few 256-row pairs to occupy every
 * compute unit finishes sooner with 128-row tiles (16 query rows per wave,
 * twice the pairs at half the work each), which the library picks by
 * itself from a cost estimate. This call overrides that choice.
 *  shape     as for zyfa_prepare (seqlen: query rows of the call; d_v 128)
 *  tile_q    128 or 256, or 0 to return to the automatic choice
 * Reads the current device and allocates nothing; the plan of the chosen
 * height is built on the next zyfa_prepare or attention call of the shape
 * on that device, and plans already built stay valid (a plan is kept per
 * height). The setting outlives zyfa_release. zyfa_plan_jobs shows the
 * automatic choice only.
 * Returns ZYFA_ERR_SHAPE for another tile_q, and the shape errors of
 * zyfa_prepare.
 */
int zyfa_set_tile_q(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int dtype, int tile_q);

/*
 * zyfa_fp8_quantize - per-tensor power-of-two FP8 quantization (README,
 * Usage: fp8_quantize returns the e4m3 tensor and its descale as a device
 * fp32 scalar).
 *   amax    = max |x| over all numel elements (x finite)
 *   descale = 2^ceil(log2(amax / 448)), or 1 when amax == 0, and never
 *             below 2^-126 (a descale must be a normal float32)
 *   x8[i]   = e4m3fn code of x[i] / descale, round to nearest even
 *  x       device pointer, numel elements of x_dtype (ZYFA_DTYPE_BF16 or
 *          ZYFA_DTYPE_FP32)
 *  x8      device pointer, numel bytes (caller-owned)
 *  descale device pointer to one fp32 (caller-owned); written on device, the
 *          host never reads it.
 *  numel == 0 writes descale = 1. Deterministic: the result does not depend
 *  on timing. x8 also holds the partial maxima between the passes (they are
 *  overwritten by the codes), so a call reads and writes nothing but its own
 *  arguments and calls on different streams do not interfere; x8 must not
 *  overlap x. Allocates nothing.
 */
int zyfa_fp8_quantize(const void* x, int x_dtype, long long numel, void* x8, float* descale,
                      void* stream);

/*
 * zyfa_fp8_quantize_rotated - rotate each row of d = 128 channels by an
 * orthogonal matrix R, then quantize the rotated tensor as zyfa_fp8_quantize does
 * ("ZYFA" README, "Using FP8 attention in a model": a Hadamard rotation of
 * q and k before quantization; (q R)(k R)^T = q k^T, so attention on the
 * rotated q and k equals attention on the originals up to rounding, and the
 * rotation mixes the few large channels into all of them, so one
 * power-of-two scale fits the tensor better and its codes lose less).
 * Rotate q and k with the same signs; leave v unrotated.
 *   R = diag(s) H_128 / sqrt(128), H Sylvester's Hadamard matrix
 *   y = x R (computed in fp32 with a fast Walsh-Hadamard transform), then
 *   descale = 2^ceil(log2(max|y| / 448)) (1 when y == 0, >= 2^-126) and
 *   x8 = e4m3fn RNE of y / descale.
 *  x       device pointer, rows * d values of x_dtype (ZYFA_DTYPE_BF16 or
 *          ZYFA_DTYPE_FP32), rows contiguous; 16-byte aligned.
 *  d       128 (ZYFA_ERR_HEADDIM otherwise).
 *  signs   host pointer to d values, each +1 or -1 (ZYFA_ERR_SIGNS
 *          otherwise), or NULL for all +1. Read during the call only.
 *  x8      device pointer, rows * d bytes; descale: device pointer to one
 *          fp32. Both caller-owned, written on the device.
 *  Asynchronous on `stream`; deterministic; allocates nothing. As in
 *  zyfa_fp8_quantize, x8 also holds the partial maxima between the passes
 *  and must not overlap x.
 */
int zyfa_fp8_quantize_rotated(const void* x, int x_dtype, long long rows, int d, const signed char* signs,
                              void* x8, float* descale, void* stream);

/*
 * zyfa_key_mean - mean key of each (batch, head) over the sequence, for K
 * smoothing ("ZYFA" README, "Using FP8 attention in a model": subtracting
 * the mean key of each head before the rotation lowers the quantization
 * error further; the mean cancels in the softmax because every key of a
 * row loses the same vector, so the output is unchanged and the LSE moves
 * by softmax_scale * q . mean).
 *   mean[b][h][c] = (1 / seqlen) sum_s k[b][s][h][c]   (fp32, fixed order)
 *  k       device pointer, bf16 or fp32 (k_dtype), [batch, seqlen, nheads_k,
 *          d] (bshd) or [batch, nheads_k, seqlen, d] (bhsd), 16-byte aligned.
 *  mean    device pointer, batch * nheads_k * d fp32 (caller-owned).
 *  d is 128 or 192. Deterministic; asynchronous on `stream`. When the keys
 *  of a sequence are quantized in several calls (chunks, a cached prefix),
 *  every key of a row must lose the same vector: compute the mean once and
 *  pass that same vector to every call.
 */
int zyfa_key_mean(const void* k, int k_dtype, int batch, int seqlen, int nheads_k, int d, int layout,
                  float* mean, void* stream);

/*
 * zyfa_fp8_quantize_rotated_shifted - zyfa_fp8_quantize_rotated of
 * (x - shift[b][h]): the vector of each (batch, head) is subtracted from
 * every position of that head before the rotation (K smoothing with the
 * vector from zyfa_key_mean, or one fixed in advance).
 *  x       [batch, seqlen, nheads, d] (bshd) or [batch, nheads, seqlen, d]
 *          (bhsd), bf16 or fp32, 16-byte aligned; batch * seqlen * nheads
 *          below 2^31 (ZYFA_ERR_RANGE otherwise).
 *  shift   device pointer, batch * nheads * d fp32, 16-byte aligned.
 *  Everything else as zyfa_fp8_quantize_rotated.
 */
int zyfa_fp8_quantize_rotated_shifted(const void* x, int x_dtype, int batch, int seqlen, int nheads, int d,
                                      int layout, const signed char* signs, const float* shift, void* x8,
                                      float* descale, void* stream);

/* zyfa_status_string - static, human-readable text of a status code. */
const char* zyfa_status_string(int status);

/* zyfa_release - free every cached plan on every device (device memory of
 * the job tables). Must not race with calls in flight. Plans are kept until
 * this call: one per shape and query-tile height, 8 bytes per job-table
 * entry (8 KiB for 16K tokens at 32 heads), so a server that sees many
 * distinct shapes can release them between phases. */
void zyfa_release(void);

/*
 * zyfa_plan_jobs - host-only view of the job table a shape would use (no HIP
 * call, no device memory), for inspection and tests. The work distribution
 * follows the README's Kernel design list (work distribution): query tiles
 * of one (batch, head) are paired first with last so every job has the same
 * work, a persistent grid of num_wgs workgroups loops over jobs, and
 * consecutive jobs go to workgroups on the same XCD (blockIdx % 8).
 *  num_cus      compute units to fill (256 on MI355X)
 *  out_tile_q   receives the query-tile height in rows
 *  out_num_wgs  receives the persistent grid size
 *  out_jobs_per_wg receives the number of table rows
 *  table        NULL, or int[2 * num_wgs * jobs_per_wg] receiving, for row r
 *               and workgroup w at index 2*(r*num_wgs + w), the pair
 *               {batch*nheads + head, first tile i} (the job covers query
 *               tiles i and n-1-i, or only i when they coincide); {-1, -1}
 *               marks the end of a workgroup's list.
 *  table_capacity number of ints available in table (ignored when NULL).
 */
int zyfa_plan_jobs(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int dtype,
                   int num_cus, int* out_tile_q, int* out_num_wgs, int* out_jobs_per_wg,
                   int* table, long long table_capacity);

#ifdef __cplusplus
}
#endif
#endif /* ZYFA_H */
