// Causal forward attention, FP8 e4m3fn inputs with one descale per tensor,
// BF16 output, for gfx950 (CDNA4).
//
// What is computed: "ZYFA" README, Usage (descales read from device memory
// and applied by the kernel), Supported configurations, Accuracy (the row
// sum that normalises the output, and the LSE, are taken over exactly the
// rounded probabilities that weight V, which keeps partial results over
// separate key ranges mergeable). Query row r sits at position
// r + delta relative to the keys (key c is visible to row r when
// c <= r + delta): delta = 0 with seqlen_q == seqlen_k is whole-sequence
// causal attention, other values give partial results over a key range.
// Rows that see no key get O = 0 and LSE = -inf.
//
// Structure (shared with the BF16 kernel: persistent 8-wave workgroups, jobs
// = pairs of query tiles, QG 16-row groups of query rows per wave (256-row
// tiles with two, 128-row tiles with one), transposed scores):
//  - Keys stream in 128-key tiles through four-slot K and V rings in LDS,
//    filled by direct global-to-LDS loads two tiles (K) and one tile (V)
//    ahead of use; the lag wave group issues the K loads and the lead
//    group the V loads.
//  - Ping-pong (README, Kernel design: ping-pong schedule): the two waves
//    that share a SIMD run half a tile apart, so while one issues the
//    matrix instructions of a tile the other runs the vector work of its
//    own; one barrier per interval keeps the groups in step.
//  - S^T = K Q^T with v_mfma_scale_f32_16x16x128_f8f6f4 (neutral scales);
//    the three descales and the softmax scale are folded into one base-2
//    factor read from device memory at kernel start.
//  - Per-block power-of-two scaling (README, Kernel design: per-block
//    scaling): each 32-key block of a query row (the scale block of the
//    scaled MFMA) gets e_b = floor(block max - m_ref) in base-2 units, so its
//    largest probability divided by 2^e_b lies in [1, 2) and stays normal;
//    the PV MFMA multiplies 2^e_b back in through its B-scale operand.
//  - Exact P: y = s - m_ref - e_b, p = exp2(y) rounded to e4m3fn (RNE,
//    v_cvt_pk_fp8_f32); e_b is folded into the exponent's bias, so no
//    scaling conversion is needed.
//  - Lean P (README, Kernel design: lean P): the e4m3fn code of a positive
//    value grows by 8 per doubling, so the code of 2^y is written directly as
//    RNE(8 y + C), clamped to 0..255 (one FMA per score and one packing
//    conversion per two scores instead of an exponential and an FP8
//    conversion).
//    C = 56 + 8 log2(2 ln^2 2) makes the piecewise-linear value unbiased.
//    Lean P is used on key tiles that lie wholly before the 256-row block
//    of query rows that holds the workgroup's query tile; the key tiles that
//    overlap the block keep exact P, so the rows with the fewest keys (rows
//    0..255) are exact throughout, at either tile height.
//    The choice is uniform over the workgroup.
//  - The row sum is one extra MFMA of the rounded, scaled P against a block
//    of ones (README, Kernel design: row sum on the matrix unit), so the
//    denominator is the sum of exactly the values that multiply V.
//  - V^T is read from LDS with ds_read_b64_tr_b8 (transposes bytes during
//    the read), so V is stored as it arrives.
//  - Lazy rescale (README, Kernel design: lazy rescaling): a row's reference
//    moves to the tile maximum only when that exceeds it by more than kTau;
//    one wave ballot decides whether any row of the wave moves.
//  - K rows are written to LDS with key bits [5:4] and [3:2] swapped, so the
//    score layout of the MFMA puts key 16g + 4c + i (and 64 + ...) in lane
//    group g: the MFMA k index of P equals the key's offset in the tile and
//    each E8M0 scale block is 32 consecutive keys.
//  - d_qk = 192: with two query groups per wave, d 128..191 of all 32
//    query columns and 128 keys take four v_mfma_scale_f32_32x32x64_f8f6f4,
//    the FP8 rate of the 16x16x128 instruction; their results reach the
//    16x16 score layout through v_permlane16_swap (one per pair of values)
//    and start the accumulators of the 16x16x128 products over d 0..127.
//    With one query group (16 columns, too few for the 32-column product)
//    each score block adds two v_mfma_f32_16x16x32_fp8_fp8, which run at
//    half that rate.
//  - Precise mode (for inputs whose channels differ widely in magnitude,
//    such as activations with outlier channels): gfx950's FP8 matrix
//    instructions sum their products with an error of up to 2^-11.5 of
//    sum |q_c k_c| on such rows, enough to move the softmax weights of keys
//    whose scores are close. Here the e4m3 codes of q and k are converted to
//    bf16 (exactly: every e4m3 value is a bf16 value) and S^T = K Q^T runs on
//    v_mfma_f32_16x16x32_bf16, whose sums hold to ~2^-22; and each
//    probability of a block is split into two e4m3 values, hi = RNE(p) and
//    lo = RNE(p - hi), multiplied into V (and into the row sum) by two PV
//    matrix instructions with the block's scale, which carries p to about
//    7 significant bits instead of 4. Exact P only.
//
// Fragment layout of the 16x16x128 FP8 MFMA (lane = 16*g + r, g = lane/16):
// A (16 x 128): lane holds row r, bytes 0..15 = k 16g..16g+15 and bytes
// 16..31 = k 64+16g..; B (128 x 16) likewise for column r; D: lane holds
// rows 4g..4g+3 of column r. The scale of A row r (B column r) for k-block
// b (32 wide) comes from lane r + 16b.
#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

constexpr int kThreads = 512;
constexpr int kTileK = 128;
constexpr int kSlots = 4;             // K and V ring depth
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRefFloor = -1e30f;      // initial reference maximum, base-2 units
constexpr int kE8M0One = 127;           // E8M0 scale 2^0
// Lean-P constant 56 + 8 log2(2 ln(2)^2).
constexpr float kLeanC = 55.539734f;
constexpr float kInv65535 = 1.0f / 65535.0f;

// 16-byte chunk swizzle of V row r: bits 1..2 and 4 of r.
__device__ __forceinline__ int vsw(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }

// Key held by LDS row r of a K tile: bits [5:4] and [3:2] of r swapped.
__device__ __forceinline__ int kswap(int r) { return (r & ~0x3C) | ((r & 0x30) >> 2) | ((r & 0x0C) << 2); }

// Chunk swizzle of the 64-byte d 128..191 K rows. Each 16-lane group of a
// read should touch 16 distinct 16-byte bank groups of the 256 bytes the
// LDS serves per cycle; a row's 256-byte offset is its bits 0, 1. The 8-byte
// reads of the one-group kernels cover rows 16 kb + n (n < 16): swizzle by
// bits 2, 3. The 16-byte reads of the 32x32x64 operand cover rows 16 j +
// 8 h + i (j < 2): swizzle by bits 3, 4.
template <bool WIDE>
__device__ __forceinline__ int kbsw_of(int r) { return WIDE ? ((r >> 3) & 3) : ((r >> 2) & 3); }

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Probability modes of the kernel template (zyfa_p_mode resolved per call).
constexpr int kPmExact = 0;
constexpr int kPmLean = 1;
constexpr int kPmPrecise = 2;

// Eight e4m3fn codes (two words, byte j = element j) -> eight bf16 values,
// exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1, two codes per
// instruction). Words are passed by value.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned w0, unsigned w1) {
  const unsigned r0 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  const unsigned r1 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  const unsigned r2 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  const unsigned r3 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8, u32x4{r0, r1, r2, r3});
}

// e4m3fn codes 0, 1 (HI false) or 2, 3 (HI true) of word w as floats.
template <bool HI>
__device__ __forceinline__ f32x2 fp8_pair_to_f32(unsigned w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// a * b rounded to fp32 on its own: never fused with a following add.
__device__ __forceinline__ float mul_nofma(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Largest power of two <= x for x > 0 (exponent field only), at least 2^-126.
__device__ __forceinline__ float pow2_floor(float x) {
  const unsigned e = __builtin_bit_cast(unsigned, x) & 0x7F800000u;
  return __builtin_bit_cast(float, e < 0x00800000u ? 0x00800000u : e);
}

// Four floats -> four e4m3fn codes (RNE) in one word. The first conversion
// keeps the upper half of its destination, which the second one then writes,
// so the word may start from any value; written as assembly so that no
// instruction zeroes it first (the builtin form always does).
__device__ __forceinline__ unsigned cvt4_fp8(float a, float b, float c, float d) {
  unsigned w;
  asm("v_cvt_pk_fp8_f32 %0, %1, %2\n\tv_cvt_pk_fp8_f32 %0, %3, %4 op_sel:[0,0,1]"
      : "=&v"(w)
      : "v"(a), "v"(b), "v"(c), "v"(d));
  return w;
}

template <int DQK, bool WITH_LSE, int PM, int QG>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(const AttnArgs a) {
  constexpr int DV = 128;
  constexpr bool LEAN = PM == kPmLean;
  constexpr bool PRECISE = PM == kPmPrecise;
  constexpr int NCB = DQK / 32;                     // bf16 MFMA k-steps over d_qk (precise mode)
  constexpr int RW = 16 * QG;                       // query rows per wave (QG 16-row groups)
  constexpr int kTileQ = 8 * RW;                    // query rows per tile
  constexpr bool D192 = DQK == 192;
  // d_qk = 192 with two query groups: the scores over d 128..191 come from
  // the 32x32x64 scaled instruction at the full FP8 rate and are brought
  // into the 16x16 layout by lane swaps; with one group (16 query columns
  // per wave, too few for a 32-column product) they come from two 16x16x32
  // FP8 instructions per block, which run at half the rate
  constexpr bool kWide = D192 && QG == 2 && !PRECISE;
  auto kbsw = [](int r) { return kbsw_of<kWide>(r); };
  constexpr int KA_BYTES = kTileK * 128;            // K region for d 0..127
  constexpr int KB_BYTES = D192 ? kTileK * 64 : 0;  // K region for d 128..191
  constexpr int K_SLOT = KA_BYTES + KB_BYTES;
  // LDS fragment prefetch distance of the matrix cluster (16-key or
  // 16-column blocks); d 192 has fewer registers to spare
  constexpr int kPfV = D192 ? 1 : 2;
  constexpr int kPfK = D192 ? 1 : 2;
  constexpr int V_SLOT = kTileK * DV;
  static_assert(KA_BYTES == 16 * 1024 && V_SLOT == 16 * 1024 && (!D192 || KB_BYTES == 8 * 1024), "tile split");

  __shared__ __attribute__((aligned(16))) char smem[kSlots * (K_SLOT + V_SLOT)];
  char* const kring = smem;
  char* const vring = smem + kSlots * K_SLOT;
  // the rings' LDS byte addresses, for the direct-to-LDS loads
  const unsigned kring_lds = lds_addr(smem);
  const unsigned vring_lds = kring_lds + kSlots * K_SLOT;

  // work-item and group ids from the hardware registers directly (the
  // device-library accessors are not inlined into a kernel compiled with
  // IEEE mode off, and a call would spill every live register)
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int lane = tid & 63;
  // wave-uniform values live in scalar registers
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  // Waves w and w + 4 share a SIMD. Waves 4..7 (the lead group, which also
  // holds the query rows with more keys) run half a key tile ahead of waves
  // 0..3 (the lag group).
  const bool lead = wave >= 4;
  // The wave's index within its group, as a scalar, so the load
  // addresses built from it stay in scalar registers.
  const int wsc = __builtin_amdgcn_readfirstlane(wave & 3);
  const int ws = __builtin_amdgcn_readfirstlane(wave);
  const int Sq = a.seqlen_q;
  const int Sk = a.seqlen_k;
  const int dl = a.delta;
  // Scores in base-2 units: S_codes * (softmax_scale * log2 e * dq * dk).
  const float sl2 = a.scale_log2 * a.q_descale[0] * a.k_descale[0];
  const float c8s = 8.0f * sl2 * kInv65535;
  // ds_bpermute source of the lane's E8M0 scale: lane groups 1 and 2 swap
  const int psc_addr = 4 * (((g == 1) || (g == 2)) ? (lane ^ 48) : lane);
  // LDS bases of this lane's d 128..191 K reads on the 32x32x64
  // instruction: instruction row x = lane % 32 = 8 j + 4 h + i on LDS row
  // 16 j + 8 h + i (+ 64 p + 4 o), chunks 2 (lane / 32) (lo) and
  // 2 (lane / 32) + 1 (hi), swizzled as kbsw below
  const int x32 = lane & 31;
  const int krow0 = 16 * (x32 >> 3) + 8 * ((x32 >> 2) & 1) + (x32 & 3);
  const int khb_lo = kTileK * 128 + krow0 * 64 + (((2 * (lane >> 5)) ^ ((krow0 >> 3) & 3)) << 4);
  const int khb_hi = kTileK * 128 + krow0 * 64 + (((2 * (lane >> 5) + 1) ^ ((krow0 >> 3) & 3)) << 4);
  const float dvs = a.v_descale[0];
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3fn 1.0

  for (int it = 0; it < a.jobs_per_wg; ++it) {
    const int2 jv = a.jobs[it * a.num_wgs + wg];
    const int2 job = {__builtin_amdgcn_readfirstlane(jv.x), __builtin_amdgcn_readfirstlane(jv.y)};
    if (job.x < 0) break;
    const int b = job.x / a.nheads;
    const int h = job.x - b * a.nheads;
    const int hk = (int)(((long long)h * a.nheads_k) / a.nheads);
    const char* qbase = (const char*)a.q.ptr + (b * a.q.stride_b + h * a.q.stride_h);
    const char* kbase = (const char*)a.k.ptr + (b * a.k.stride_b + hk * a.k.stride_h);
    const char* vbase = (const char*)a.v.ptr + (b * a.v.stride_b + hk * a.v.stride_h);
    const int qrs = (int)a.q.stride_s;
    const int krs = (int)a.k.stride_s;
    const int vrs = (int)a.v.stride_s;

    const int tA = job.y;
    const int tB = a.n_qtiles - 1 - job.y;
    const int ntiles = (tA == tB) ? 1 : 2;
    for (int tt = 0; tt < ntiles; ++tt) {
      // the longer tile first: the workgroups of one chiplet then stream the
      // same keys at the same time for longer, so K and V stay in its L2
      const int qt = tt == 0 ? tB : tA;
      const int q0 = qt * kTileQ;
      const int qw0 = q0 + wave * RW;
      const int qend = min(q0 + kTileQ, Sq);
      // key tiles that some row of the query tile sees (when any: the
      // tile's last row sees qend + delta keys, capped at seqlen_k)
      const bool any_key = qend + dl > 0;
      const int n_kt = (min(Sk, qend + dl) - 1) / kTileK + 1;
      // this wave's last key tile (the one holding its diagonal), -1 if the
      // wave has no rows or its rows see no key
      const int lk_w = min(Sk - 1, qw0 + RW - 1 + dl);
      const int kt_w = (qw0 < Sq && lk_w >= 0) ? min(lk_w / kTileK, n_kt - 1) : -1;
      // key tiles from K0 on reach the diagonal band of the 256-row block
      // that holds this query tile: exact P and (on the diagonal) the causal
      // mask; tiles before K0, whose keys every row of the block sees, take
      // lean P (with LEAN). The block is 256 rows whatever the tile height,
      // so rows 0..255, which have the fewest keys, are exact throughout and
      // the rounding does not depend on the tiling; in a call over a range
      // of keys, a block whose first row sees fewer than 256 keys is exact
      // throughout as well.
      const int qb = q0 & ~255;
      const int K0 = min(qb + dl + 1, Sk) >= 256 ? (qb + dl + 1) / kTileK : 0;

      // Q fragments (B operand): lane (g, n) holds q[row n][16g..16g+15] and
      // q[row n][64+16g..]; for d 192 with one query group also
      // q[row n][128+8g..+7] and q[row n][160+8g..+7], the B operands of two
      // 16x16x32 FP8 MFMAs over d 128..191. They are read through a resource
      // based at the wave's first row.
      const int qr0 = q0 + RW * ws;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase + (unsigned long long)qr0 * (unsigned)qrs,
                                                  rows_extent(min(Sq - qr0, RW), qrs, DQK));
      i32x8 qf[QG];
      long qx[QG][2];
      // kWide: the B operand of the 32x32x64 instruction over d 128..191,
      // lane l holding q[row l % 32][128 + 32 (l / 32) .. +31]
      i32x8 qh = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const int off = (16 * qg + n) * qrs;
        const u32x4 lo = buf_load16(rq, off + 16 * g);
        const u32x4 hi = buf_load16(rq, off + 64 + 16 * g);
        qf[qg] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (D192 && !kWide) {
          qx[qg][0] = __builtin_bit_cast(long, buf_load8(rq, off + 128 + 8 * g));
          qx[qg][1] = __builtin_bit_cast(long, buf_load8(rq, off + 160 + 8 * g));
        }
      }
      if (kWide) {
        const int off = (lane & 31) * qrs + 128 + 32 * (lane >> 5);
        const u32x4 lo = buf_load16(rq, off), hi = buf_load16(rq, off + 16);
        qh = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      // Precise mode: the B operands of the bf16 score MFMAs, k-step c of
      // lane group g holding the same d values as the K operand: c = 0..3
      // are bytes 8 (c % 2) .. of the 16-byte chunks g (c < 2) and 4 + g
      // (c >= 2), c = 4, 5 the d 128..191 words.
      bf16x8 qbf[PRECISE ? QG : 1][PRECISE ? NCB : 1];
      if (PRECISE) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const unsigned w0 = (unsigned)qf[qg][2 * c], w1 = (unsigned)qf[qg][2 * c + 1];
            qbf[qg][c] = fp8x8_to_bf16(w0, w1);
          }
          if (D192) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const unsigned long long x = (unsigned long long)qx[qg][c];
              qbf[qg][4 + c] = fp8x8_to_bf16((unsigned)x, (unsigned)(x >> 32));
            }
          }
        }
      }

      f32x4 o[QG][8];
      f32x4 lacc[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        lacc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // Reference maxima start at a finite floor, so rows that have seen no
      // key yet give exp2(-inf - m) = 0 and rescale factors of 1, never NaN.
      float mref[QG];
      // lazy-rescale threshold in raw score units, (m + tau) / sl2, and the
      // lean-P offset (C - 8 m) / 65535 of each query group
      float thr[QG];
      float lcs[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        mref[qg] = kRefFloor;
        thr[qg] = neg_inf();
        lcs[qg] = 0.f;
      }
      // scores of the tile in flight (made by a matrix cluster, turned into P
      // codes by the next vector cluster), the P codes and the E8M0 exponent
      // this lane supplies to the PV MFMA
      f32x4 s[QG][8];
      i32x8 pf[QG];
      i32x8 pl[PRECISE ? QG : 1];   // precise mode: the lo parts of P
      int psc[QG];

      // Direct global-to-LDS tile loads; K row r of a slot holds key
      // kswap(r), V row r holds key r; 16-byte chunks XOR-swizzled by row:
      //  K d 0..127:   row * 128 + ((c ^ ((row >> 1) & 7)) << 4)
      //  K d 128..191: row * 64  + ((c ^ kbsw(row)) << 4)
      //  V:            row * 128 + ((c ^ vsw(row)) << 4)
      // The V swizzle puts the sixteen rows that a half-wave of each
      // transposing read touches (8 consecutive keys in each of two lane
      // groups) on distinct banks.
      // Per-lane byte offsets of the tile loads (fixed for the job); the
      // offset of the tile, or of its upper 64-row half, goes into the
      // buffer resource, whose extent still ends at the slice end, so rows
      // past seqlen read as zeros. One wave group loads each whole tile (the
      // lag group K, the lead group V), wave wsc of it instructions 2 wsc,
      // 2 wsc + 1 (and wsc for d 128..191) of each half; the same offsets serve both halves (64 rows apart is a
      // multiple of every swizzle period and kswap keeps bit 6).
      int kvo[3], vvo[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = (wsc * 2 + u) * 1024 + lane * 16;
        const int row = p >> 7, slot = (p & 127) >> 4;
        kvo[u] = kswap(row) * krs + (slot ^ ((row >> 1) & 7)) * 16;
        vvo[u] = row * vrs + (slot ^ vsw(row)) * 16;
      }
      if (D192) {
        const int p = wsc * 1024 + lane * 16;
        const int row = p >> 6, x = ((p & 63) >> 4) ^ kbsw(row);
        kvo[2] = kswap(row) * krs + 128 + x * 16;
      }
      // resource at rows 64 hs .. of key tile kt
      auto tile_rsrc = [&](const char* base, int stride, int row_bytes, int kt, int hs) {
        const int r0 = kt * kTileK + 64 * hs;
        return make_rsrc_words(base + (unsigned long long)r0 * (unsigned)stride,
                               rows_extent(min(Sk - r0, 64), stride, row_bytes));
      };
      auto issue_k = [&](int kt) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const unsigned base = kring_lds + (kt % kSlots) * K_SLOT;
          const i32x4 r = tile_rsrc(kbase, krs, DQK, kt, hs);
#pragma unroll
          for (int u = 0; u < 2; ++u) dma16(r, kvo[u], base + hs * (KA_BYTES / 2) + (wsc * 2 + u) * 1024);
          if (D192) dma16(r, kvo[2], base + KA_BYTES + hs * (KB_BYTES / 2) + wsc * 1024);
        }
      };
      auto issue_v = [&](int kt) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const unsigned base = vring_lds + (kt % kSlots) * V_SLOT;
          const i32x4 r = tile_rsrc(vbase, vrs, DV, kt, hs);
#pragma unroll
          for (int u = 0; u < 2; ++u) dma16(r, vvo[u], base + hs * (V_SLOT / 2) + (wsc * 2 + u) * 1024);
        }
      };

      // V^T fragment of 16-column block db: byte 8t + r of lane group g is
      // key 64 (t / 2) + 16 g + 8 (t % 2) + r; lane 2r + hh supplies that
      // row, columns 16 db + 8 hh .. +7.
      auto v_frag = [&](const char* vs, int db) {
        i32x8 vf;
        const int r = n >> 1, hh = n & 1;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = 64 * (t >> 1) + 16 * g + 8 * (t & 1) + r;
          const i32x2 w = lds_read_tr8(vs + row * 128 + ((db ^ vsw(row)) << 4) + hh * 8);
          vf[2 * t] = w[0];
          vf[2 * t + 1] = w[1];
        }
        return vf;
      };

      // K fragments of 16-key block kb (A operand): lane (g, n) holds key
      // row 16 kb + n, d 16g..16g+15 and 64+16g.. (and, for d 192, d
      // 128+8g..+7 and 160+8g..+7).
      struct KFrag {
        i32x8 a;
        long b0, b1;
      };
      auto k_frag = [&](const char* ka, int kb) {
        KFrag f;
        const int row = 16 * kb + n;
        const int sw = (row >> 1) & 7;
        const u32x4 lo = lds_load<u32x4>(ka + row * 128 + ((g ^ sw) << 4));
        const u32x4 hi = lds_load<u32x4>(ka + row * 128 + (((4 + g) ^ sw) << 4));
        f.a = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (D192 && !kWide) {
          // 64-byte rows, 16-byte chunks swizzled by (row >> 2) & 3: d
          // 128+8g.. is half g & 1 of chunk g >> 1, d 160+8g.. of chunk
          // 2 + (g >> 1)
          const char* kr = ka + KA_BYTES + row * 64 + (g & 1) * 8;
          const int sw2 = kbsw(row);
          f.b0 = __builtin_bit_cast(long, lds_load<u32x2>(kr + (((g >> 1) ^ sw2) << 4)));
          f.b1 = __builtin_bit_cast(long, lds_load<u32x2>(kr + (((2 + (g >> 1)) ^ sw2) << 4)));
        }
        return f;
      };

      // kWide: K operand of 32x32x64 instruction w = 2 p + o over d
      // 128..191. Lane l supplies row x = l % 32 = 8 j + 4 h + i of the
      // instruction, bytes 32 (l / 32) .. +31 of the key's d 128..191. Row x
      // of instruction w is key 64 p + 16 (2 h + o) + 4 j + i, so that after
      // the lane swaps lane group g holds the keys of the 16x16 layout
      // (16 g .., 64 + 16 g ..). kswap puts that key on LDS row 64 p + 16 j +
      // 8 h + 4 o + i, whose chunk swizzle (rows bits 3, 4: h + 2 (j % 2))
      // does not depend on p and o: every read is one of the lane's two base
      // addresses plus 4096 p + 256 o.
      auto khi_frag = [&](const char* ka, int w) {
        const int off = 4096 * (w >> 1) + 256 * (w & 1);
        const u32x4 lo = lds_load<u32x4>(ka + khb_lo + off);
        const u32x4 hi = lds_load<u32x4>(ka + khb_hi + off);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };

      // Matrix cluster of tile t: O^T += V^T P^T and the row sum for tile
      // t - 1 (P codes from the previous vector cluster), then the scores
      // S^T = K Q^T of tile t.
      auto matrix_cluster = [&](int t) {
        __builtin_amdgcn_s_setprio(1);
        const bool pv = t >= 1 && t - 1 <= kt_w;
        if (pv && !PRECISE) {
          const char* vs = vring + ((t - 1) % kSlots) * V_SLOT;
          i32x8 vfb[kPfV];
#pragma unroll
          for (int u = 0; u < kPfV; ++u) vfb[u] = v_frag(vs, u);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) lacc[qg] = mfma_fp8(ones, pf[qg], lacc[qg], kE8M0One, psc[qg]);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4 * kPfV, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const i32x8 cur = vfb[db % kPfV];
            if (db + kPfV < 8) vfb[db % kPfV] = v_frag(vs, db + kPfV);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) o[qg][db] = mfma_fp8(cur, pf[qg], o[qg][db], kE8M0One, psc[qg]);
            if (db + kPfV < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
          }
        }
        if (pv && PRECISE) {
          // hi parts of column block db at step db, lo parts at step db + 1,
          // so two products into one accumulator are never adjacent
          const char* vs = vring + ((t - 1) % kSlots) * V_SLOT;
          i32x8 vfb[kPfV];
#pragma unroll
          for (int u = 0; u < kPfV; ++u) vfb[u] = v_frag(vs, u);
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) lacc[qg] = mfma_fp8(ones, pf[qg], lacc[qg], kE8M0One, psc[qg]);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4 * kPfV, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
          i32x8 prev = vfb[0];
#pragma unroll
          for (int st = 0; st <= 8; ++st) {
            i32x8 cur = prev;
            if (st < 8) {
              cur = vfb[st % kPfV];
              if (st + kPfV < 8) vfb[st % kPfV] = v_frag(vs, st + kPfV);
#pragma unroll
              for (int qg = 0; qg < QG; ++qg) o[qg][st] = mfma_fp8(cur, pf[qg], o[qg][st], kE8M0One, psc[qg]);
            }
            if (st >= 1) {
#pragma unroll
              for (int qg = 0; qg < QG; ++qg)
                o[qg][st - 1] = mfma_fp8(prev, pl[qg], o[qg][st - 1], kE8M0One, psc[qg]);
            }
            prev = cur;
            if (st + kPfV < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
            if (st == 0 || st == 8) __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
            else __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * QG, 0);
          }
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) lacc[qg] = mfma_fp8(ones, pl[qg], lacc[qg], kE8M0One, psc[qg]);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
        }
        if (t <= kt_w && PRECISE) {
          // scores on the bf16 instruction: each K fragment's codes become
          // NCB bf16 operands, k-steps in the order of the Q operands. Two
          // key blocks are interleaved, so the k-steps accumulating into one
          // score block are never adjacent; the next pair's fragments are
          // read while this pair's instructions run.
          const char* ka = kring + (t % kSlots) * K_SLOT;
          KFrag kfb[2][2];
          kfb[0][0] = k_frag(ka, 0);
          kfb[0][1] = k_frag(ka, 1);
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const KFrag c0 = kfb[pr & 1][0], c1 = kfb[pr & 1][1];
            if (pr < 3) {
              kfb[(pr + 1) & 1][0] = k_frag(ka, 2 * pr + 2);
              kfb[(pr + 1) & 1][1] = k_frag(ka, 2 * pr + 3);
            }
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const KFrag& cur = j ? c1 : c0;
                bf16x8 kc;
                if (c < 4) {
                  const unsigned w0 = (unsigned)cur.a[2 * c], w1 = (unsigned)cur.a[2 * c + 1];
                  kc = fp8x8_to_bf16(w0, w1);
                } else {
                  const unsigned long long x = (unsigned long long)(c == 4 ? cur.b0 : cur.b1);
                  kc = fp8x8_to_bf16((unsigned)x, (unsigned)(x >> 32));
                }
                const int kb = 2 * pr + j;
#pragma unroll
                for (int qg = 0; qg < QG; ++qg)
                  s[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, qbf[qg][c],
                                                                      c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[qg][kb],
                                                                      0, 0, 0);
              }
            }
          }
        }
        if (t <= kt_w && !PRECISE) {
          const char* ka = kring + (t % kSlots) * K_SLOT;
          // kWide: the d 128..191 scores first, four 32x32x64 instructions
          // (keys 0..63, then 64..127; in each half the keys of lane groups
          // 0, 2, then of lane groups 1, 3); they start where the PV
          // instructions end, so the matrix pipe stays busy
          f32x16 hw[kWide ? 4 : 1];
          if (kWide) {
            i32x8 kh = khi_frag(ka, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const i32x8 cur = kh;
              if (w < 3) kh = khi_frag(ka, w + 1);
              hw[w] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur, qh, f32x16{}, 0, 0, 0, kE8M0One, 0, kE8M0One);
              if (w < 3) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
              __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            }
            // all four issued before the first swap, which then finds the
            // results of instructions 0 and 1 ready while 3 still runs
            __builtin_amdgcn_sched_barrier(0);
          }
          // K fragments are read kPfK 16-key blocks ahead of their MFMAs
          KFrag kfb[kPfK];
#pragma unroll
          for (int u = 0; u < kPfK; ++u) kfb[u] = k_frag(ka, u);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, (D192 && !kWide ? 4 : 2) * kPfK, 0);
          // d_qk = 192 with one query group: the pair of 16x16x32 FP8
          // instructions over d 128..191 accumulates onto the result of the
          // scaled instruction. Issued straight after that result, such a
          // pair was given no wait states and read a stale accumulator on the
          // GPU, so the scaled instruction of block kb + 1 always sits between
          // them (the pair of block kb - 1 is issued after the scaled
          // instruction of block kb), held there by a scheduling barrier; a
          // CPU test checks the order in the built code.
          constexpr bool kDefer = D192 && !kWide;
          static_assert(!kDefer || QG == 1 || PRECISE, "two-group d 192 kernels take the 32x32x64 path");
          long pb0 = 0, pb1 = 0;   // d 128..191 K fragments of the deferred block
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const KFrag cur = kfb[kb % kPfK];
            if (kb + kPfK < 8) kfb[kb % kPfK] = k_frag(ka, kb + kPfK);
            if (kWide) {
              // Lane swaps. Value 4 j + i of instruction w = 2 p + o holds, in
              // lane group g, the score of query column 16 (g % 2) + n and
              // key 64 p + 16 (2 (g / 2) + o) + 4 j + i: lane groups 0, 2 of
              // w = 2 p and 1, 3 of w = 2 p + 1 already hold their own keys;
              // v_permlane16_swap trades the odd lane groups of its first
              // operand for the even lane groups of its second, after which
              // the first holds query group 0 and the second query group 1,
              // in the 16x16 layout of key block 4 p + j.
              const int pw = 2 * (kb >> 2), j = kb & 3;
              // (elements are copied to scalars before the bit casts: a bit
              // cast of a vector element in place has been compiled as a
              // cast of element 0)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float e0 = hw[pw][4 * j + i], e1 = hw[pw + 1][4 * j + i];
                const auto pr = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, e0),
                                                                 __builtin_bit_cast(unsigned, e1), false, false);
                const unsigned r0 = pr[0], r1 = pr[1];
                s[0][kb][i] = __builtin_bit_cast(float, r0);
                s[1][kb][i] = __builtin_bit_cast(float, r1);
              }
              __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
            }
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              s[qg][kb] = mfma_fp8(cur.a, qf[qg], kWide ? s[qg][kb] : f32x4{0.f, 0.f, 0.f, 0.f}, kE8M0One, kE8M0One);
            if (kDefer) {
              if (kb >= 1) {
                // keeps the pair after this block's scaled instruction
                __builtin_amdgcn_sched_barrier(0);
                s[0][kb - 1] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pb0, qx[0][0], s[0][kb - 1], 0, 0, 0);
                s[0][kb - 1] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pb1, qx[0][1], s[0][kb - 1], 0, 0, 0);
              }
              pb0 = cur.b0;
              pb1 = cur.b1;
            }
            if (kb + kPfK < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, D192 && !kWide ? 4 : 2, 0);
            if (kDefer && kb == 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(kSchedMfma, (D192 && !kWide ? 3 : 1) * QG, 0);
          }
          if (kDefer) {
            // the pair of the last block follows the pair of block 6
            __builtin_amdgcn_sched_barrier(0);
            s[0][7] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pb0, qx[0][0], s[0][7], 0, 0, 0);
            s[0][7] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pb1, qx[0][1], s[0][7], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };

      // Vector cluster of tile t: causal mask (diagonal tile), maxima, lazy
      // rescale, block exponents and P codes. Cross-lane exchanges go
      // through the LDS unit (ds_swizzle, ds_bpermute), which is idle here,
      // so they take no vector-ALU issue slots.
      auto vector_cluster = [&](int t) {
        if (t > kt_w) return;
        const int kt0 = t * kTileK;
        // ---- causal mask, on the diagonal tile only; score (kb, i) of lane
        // group g is key 64 (kb / 4) + 16 g + 4 (kb % 4) + i of the tile. Row r
        // sees keys up to min(r + delta, seqlen_k - 1): the cap masks the zero
        // rows past the last key when every key is visible.
        if (__builtin_expect(kt0 + kTileK - 1 > min(qw0 + dl, Sk - 1), 0)) {
          const float ninf = neg_inf();
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            const int q = min(qw0 + 16 * qg + n + dl, Sk - 1) - kt0 - 16 * g;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) s[qg][kb][i] = mask_above(s[qg][kb][i], 64 * (kb >> 2) + 4 * (kb & 3) + i, q, ninf);
          }
        }
        // ---- lane maxima of the raw scores per scale half (kb 0..3: keys
        // 16g..16g+15, kb 4..7: keys 64+16g..), then the maxima of the
        // 32-key scale blocks (held by lane groups g and g ^ 1)
        float x0[QG], x1[QG], b0[QG], b1[QG];
        bool need = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float y0 = fmaxf(fmaxf(s[qg][0][0], s[qg][0][1]), s[qg][0][2]);
          float y1 = fmaxf(fmaxf(s[qg][4][0], s[qg][4][1]), s[qg][4][2]);
#pragma unroll
          for (int j = 3; j < 15; j += 2) {
            y0 = fmaxf(fmaxf(y0, s[qg][j >> 2][j & 3]), s[qg][(j + 1) >> 2][(j + 1) & 3]);
            y1 = fmaxf(fmaxf(y1, s[qg][4 + (j >> 2)][j & 3]), s[qg][4 + ((j + 1) >> 2)][(j + 1) & 3]);
          }
          x0[qg] = fmaxf(y0, s[qg][3][3]);
          x1[qg] = fmaxf(y1, s[qg][7][3]);
          b0[qg] = fmaxf(x0[qg], swap16(x0[qg]));
          b1[qg] = fmaxf(x1[qg], swap16(x1[qg]));
        }
        // ---- lazy test in raw score units, one ballot per tile
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) need = need || (fmaxf(x0[qg], x1[qg]) > thr[qg]);
        if (__builtin_expect(wave_any(need), 0)) {
          // keep the rescale a real branch (with f == 1 it is harmless, so
          // the compiler would otherwise run it on every tile)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            const float rm = max_xor32(fmaxf(b0[qg], b1[qg])) * sl2;
            const float mn = rm > mref[qg] + kTau ? rm : mref[qg];
            const float f = fast_exp2(mref[qg] - mn);
            lacc[qg] *= f;
#pragma unroll
            for (int db = 0; db < 8; ++db) o[qg][db] *= f;
            mref[qg] = mn;
            thr[qg] = (mn + kTau) / sl2;
            lcs[qg] = (kLeanC - 8.0f * mn) * kInv65535;
          }
        }
        // ---- block exponents e_b = floor(block max - m) (base 2, >= -126)
        // and P codes
        const bool lean = LEAN && t < K0;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          // the block maximum is rounded to fp32 before m is subtracted,
          // exactly as m itself was (a fused multiply-subtract would give
          // e_b = -1 instead of 0 for the block that holds the maximum
          // whenever the product rounds up)
          const float e0 = fmaxf(floorf(mul_nofma(b0[qg], sl2) - mref[qg]), -126.0f);
          const float e1 = fmaxf(floorf(mul_nofma(b1[qg], sl2) - mref[qg]), -126.0f);
          // lane 16 b + n supplies the scale of block b; group g holds
          // blocks g / 2 (half 0) and 2 + g / 2 (half 1), so groups 1 and 2
          // fetch theirs from each other
          const float es = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                         psc_addr, __builtin_bit_cast(int, (g & 1) ? e1 : e0)));
          if (lean) {
            // code = RNE(8 y + C) with y = s sl2 - m - e_b, clamped at 0:
            // v_cvt_pknorm_u16_f32 rounds (8 y + C) / 65535 * 65535 and
            // clamps, two scores per instruction
            const float o0 = __builtin_fmaf(e0, -8.0f * kInv65535, lcs[qg]);
            const float o1 = __builtin_fmaf(e1, -8.0f * kInv65535, lcs[qg]);
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
              const float off = kb < 4 ? o0 : o1;
              const u16x2 lo = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(s[qg][kb][0], c8s, off),
                                                               __builtin_fmaf(s[qg][kb][1], c8s, off));
              const u16x2 hi = __builtin_amdgcn_cvt_pknorm_u16(__builtin_fmaf(s[qg][kb][2], c8s, off),
                                                               __builtin_fmaf(s[qg][kb][3], c8s, off));
              pf[qg][kb] = (int)__builtin_amdgcn_perm(__builtin_bit_cast(unsigned, hi), __builtin_bit_cast(unsigned, lo),
                                                      0x06040200u);
            }
          } else {
            const float nm0 = -(mref[qg] + e0);
            const float nm1 = -(mref[qg] + e1);
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
              f32x4 p;
#pragma unroll
              for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], sl2, kb < 4 ? nm0 : nm1));
              const unsigned hi = cvt4_fp8(p[0], p[1], p[2], p[3]);
              pf[qg][kb] = (int)hi;
              if (PRECISE) {
                // lo = RNE(p - hi); p - hi is exact in fp32
                const f32x2 h01 = fp8_pair_to_f32<false>(hi), h23 = fp8_pair_to_f32<true>(hi);
                const float h0 = h01[0], h1 = h01[1], h2 = h23[0], h3 = h23[1];
                pl[qg][kb] = (int)cvt4_fp8(p[0] - h0, p[1] - h1, p[2] - h2, p[3] - h3);
              }
            }
          }
          psc[qg] = (int)es + 127;
        }
      };

      // Ping-pong over intervals closed by one barrier each. In interval i
      // the lead group runs the vector cluster of tile i - 1 and then the
      // matrix cluster of tile i; the lag group runs the matrix cluster of
      // tile i - 1 and then its vector cluster. On every SIMD one wave is in
      // a matrix cluster while the other computes a softmax. Interval i
      // reads K(i - 1), K(i), V(i - 2) and V(i - 1). The lag group issues
      // K(i + 2) between its two clusters and the lead group issues V(i + 1)
      // at the start of the interval, into the slots last read in interval
      // i - 1 (four-slot rings); before the barrier each wave waits for the
      // loads it issued one interval earlier (read from interval i + 1 on).
      // A wave that issues direct-to-LDS loads is held until the address
      // unit accepts them; issued by one group alone they lengthen its chain
      // past the other's, and issued in a burst by all waves at the start of
      // an interval they queue in the address unit and stall every wave.
      // The lag group's last tile (its PV) ends in interval kt_w + 2, the
      // lead's in kt_w + 1.
      const int lag_last = q0 + 4 * RW - 1 + dl >= 0 ? min((q0 + 4 * RW - 1 + dl) / kTileK, n_kt - 1) : -1;
      const int n_int = max(n_kt + 1, lag_last + 3);
      __syncthreads();   // the previous query tile's last reads of the rings are done
      if (any_key) {     // a query tile whose rows see no key skips the loop
        if (lead) {
          issue_v(0);
        } else {
          issue_k(0);
          if (n_kt > 1) issue_k(1);
        }
        wait_vm<0>();
        __syncthreads();
        for (int i = 0; i < n_int; ++i) {
          if (lead) {
            if (i + 1 < n_kt) issue_v(i + 1);
            if (i >= 1) vector_cluster(i - 1);
            matrix_cluster(i);
            if (i + 1 < n_kt) wait_vm<4>();
            else wait_vm<0>();
          } else {
            if (i >= 1) matrix_cluster(i - 1);
            if (i + 2 < n_kt) issue_k(i + 2);
            if (i >= 1) vector_cluster(i - 1);
            if (i + 2 < n_kt) wait_vm<D192 ? 6 : 4>();
            else wait_vm<0>();
          }
          __syncthreads();
        }
      }

      // ---- epilogue: O * dv / l (RNE to bf16), LSE = ln2 * (m + log2 l)
      if (qw0 < Sq) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          const float lt = lacc[qg][0];
          const float f = lt > 0.f ? dvs / lt : 0.f;   // l = 0: the row saw no key
          const int q = qw0 + 16 * qg + n;
          if (q < Sq) {
            __bf16* orow = (__bf16*)a.out + (b * a.o_stride_b + h * a.o_stride_h + (long long)q * a.o_stride_s);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const u32x2 w = {pack_bf16x2(o[qg][db][0] * f, o[qg][db][1] * f),
                               pack_bf16x2(o[qg][db][2] * f, o[qg][db][3] * f)};
              *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g) = w;
            }
            if (WITH_LSE && g == 0)
              a.lse[((long long)b * a.nheads + h) * Sq + q] = (mref[qg] + fast_log2(lt)) * kLn2;
          }
        }
      }
    }
  }
}

}  // namespace

template <int DQK, int PM, int QG>
static void launch_fp8(const AttnArgs& a, bool with_lse, dim3 gd, dim3 bd, hipStream_t s) {
  if (with_lse) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, true, PM, QG>), gd, bd, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, false, PM, QG>), gd, bd, 0, s, a);
}

// The precise mode runs on 128-row tiles only (one 16-row group per wave):
// with two groups its bf16 Q operands and lo parts do not fit the register
// file beside the scores and accumulators.
template <int DQK, int QG>
static hipError_t launch_fp8_p(const AttnArgs& a, bool with_lse, int pm, dim3 gd, dim3 bd, hipStream_t s) {
  if (pm == kPmLean) launch_fp8<DQK, kPmLean, QG>(a, with_lse, gd, bd, s);
  else if (pm == kPmExact) launch_fp8<DQK, kPmExact, QG>(a, with_lse, gd, bd, s);
  else if constexpr (QG == 1) launch_fp8<DQK, kPmPrecise, QG>(a, with_lse, gd, bd, s);
  else return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_attn_fp8(const AttnArgs& a, int d_qk, bool with_lse, FP8Mode mode, int tile_q, int grid,
                           hipStream_t s) {
  const dim3 gd(grid), bd(kThreads);
  if (tile_q != 128 && tile_q != 256) return hipErrorInvalidValue;
  const int pm = mode == FP8Mode::kLean ? kPmLean : mode == FP8Mode::kPrecise ? kPmPrecise : kPmExact;
  const bool tall = tile_q == 256;
  hipError_t e;
  if (d_qk == 128) e = tall ? launch_fp8_p<128, 2>(a, with_lse, pm, gd, bd, s) : launch_fp8_p<128, 1>(a, with_lse, pm, gd, bd, s);
  else e = tall ? launch_fp8_p<192, 2>(a, with_lse, pm, gd, bd, s) : launch_fp8_p<192, 1>(a, with_lse, pm, gd, bd, s);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace zyfa
