// Causal forward attention, FP8 e4m3fn inputs with one descale per tensor,
// BF16 output, for gfx950 (CDNA4).
//
// What is computed: "ZYFA" README, Usage (descales read from device memory
// and applied by the kernel), Supported configurations, Accuracy (the output
// is divided by the sum of the same rounded probabilities that multiply V,
// and the LSE comes from those rounded probabilities).
//
// Structure (shared with the BF16 kernel: persistent 8-wave workgroups, jobs
// = pairs of 256-row query tiles, 32 query rows per wave, transposed scores):
//  - Keys stream in 128-key tiles through a two-stage LDS ring filled by
//    direct global-to-LDS loads issued one tile ahead.
//  - S^T = K Q^T with v_mfma_scale_f32_16x16x128_f8f6f4 (neutral scales);
//    the three descales and the softmax scale are folded into one base-2
//    factor read from device memory at kernel start.
//  - Per-block power-of-two scaling (README, Kernel design: per-block
//    scaling): each 32-key block of a query row (the scale block of the
//    scaled MFMA) gets e_b = floor(block max - m_ref) in base-2 units, so its
//    largest probability divided by 2^e_b lies in [1, 2) and stays normal;
//    the PV MFMA multiplies 2^e_b back in through its B-scale operand.
//  - Exact P: p = exp2(s - m_ref) rounded to e4m3fn as p / 2^e_b
//    (v_cvt_scalef32_pk_fp8_f32, RNE).
//  - Lean P (README, Kernel design: lean P): the e4m3fn code of a positive
//    value grows by 8 per doubling, so the code of 2^y is written directly as
//    RNE(8 y + C), clamped to 0..255 by v_cvt_pk_u8_f32 (one FMA and one
//    conversion per score instead of an exponential and an FP8 conversion).
//    C = 56 + 8 log2(2 ln^2 2) makes the piecewise-linear value unbiased.
//    Lean P is used on key tiles that lie wholly before the workgroup's
//    256-row query tile; the key tiles that overlap the query tile keep exact
//    P, so the rows with the fewest keys (query tile 0) are exact throughout.
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
//  - d_qk = 192 adds one MFMA per score block over d 128..191 with the
//    remaining half of the K dimension zero.
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
constexpr int kTileQ = 256;
constexpr int kTileK = 128;
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kE8M0One = 127;           // E8M0 scale 2^0
// sched_group_barrier instruction classes.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// Lean-P constant 56 + 8 log2(2 ln(2)^2).
constexpr float kLeanC = 55.539734f;

// 16-byte chunk swizzle of V row r: bits 1..2 and 4 of r.
__device__ __forceinline__ int vsw(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }

// Key held by LDS row r of a K tile: bits [5:4] and [3:2] of r swapped.
__device__ __forceinline__ int kswap(int r) { return (r & ~0x3C) | ((r & 0x30) >> 2) | ((r & 0x0C) << 2); }

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Largest power of two <= x for x > 0 (exponent field only), at least 2^-126.
__device__ __forceinline__ float pow2_floor(float x) {
  const unsigned e = __builtin_bit_cast(unsigned, x) & 0x7F800000u;
  return __builtin_bit_cast(float, e < 0x00800000u ? 0x00800000u : e);
}

// Four floats / scale -> four e4m3fn codes (RNE) in one word.
__device__ __forceinline__ unsigned cvt4_fp8(float a, float b, float c, float d, float scale) {
  i16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
  return __builtin_bit_cast(unsigned, w);
}

template <int DQK, bool WITH_LSE, bool LEAN>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(const AttnArgs a) {
  constexpr int DV = 128;
  constexpr bool D192 = DQK == 192;
  constexpr int KA_BYTES = kTileK * 128;       // K region for d 0..127
  constexpr int KB_BYTES = D192 ? kTileK * 64 : 0;  // K region for d 128..191
  constexpr int V_BYTES = kTileK * DV;
  constexpr int STAGE = KA_BYTES + KB_BYTES + V_BYTES;
  static_assert(KA_BYTES == 16 * 1024 && V_BYTES == 16 * 1024 && (!D192 || KB_BYTES == 8 * 1024), "tile split");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int S = a.seqlen;
  // Scores in base-2 units: S_codes * (softmax_scale * log2 e * dq * dk).
  const float sl2 = a.scale_log2 * a.q_descale[0] * a.k_descale[0];
  const float dvs = a.v_descale[0];
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3fn 1.0

  for (int it = 0; it < a.jobs_per_wg; ++it) {
    const int2 job = a.jobs[it * (int)gridDim.x + (int)blockIdx.x];
    if (job.x < 0) break;
    const int b = job.x / a.nheads;
    const int h = job.x - b * a.nheads;
    const int hk = (int)(((long long)h * a.nheads_k) / a.nheads);
    const char* qbase = (const char*)a.q.ptr + (b * a.q.stride_b + h * a.q.stride_h);
    const char* kbase = (const char*)a.k.ptr + (b * a.k.stride_b + hk * a.k.stride_h);
    const char* vbase = (const char*)a.v.ptr + (b * a.v.stride_b + hk * a.v.stride_h);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, a.q_bytes);
    const i32x4 rk = make_rsrc_words(kbase, a.k_bytes);
    const i32x4 rv = make_rsrc_words(vbase, a.v_bytes);
    const int qrs = (int)a.q.stride_s;
    const int krs = (int)a.k.stride_s;
    const int vrs = (int)a.v.stride_s;

    const int tA = job.y;
    const int tB = a.n_qtiles - 1 - job.y;
    const int ntiles = (tA == tB) ? 1 : 2;
    for (int tt = 0; tt < ntiles; ++tt) {
      const int qt = tt == 0 ? tA : tB;
      const int q0 = qt * kTileQ;
      const int qw0 = q0 + wave * 32;
      const int qend = min(q0 + kTileQ, S);
      const int n_kt = (qend - 1) / kTileK + 1;
      const int kt_w = (qw0 < S) ? min((qw0 + 31) / kTileK, n_kt - 1) : -1;

      // Q fragments (B operand): lane (g, n) holds q[row n][16g..16g+15] and
      // q[row n][64+16g..]; for d 192 also q[row n][128+16g..] (upper half 0).
      i32x8 qf[2], qf2[2];
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const int off = (qw0 + 16 * qg + n) * qrs;
        const u32x4 lo = buf_load16(rq, off + 16 * g);
        const u32x4 hi = buf_load16(rq, off + 64 + 16 * g);
        qf[qg] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (D192) {
          const u32x4 x = buf_load16(rq, off + 128 + 16 * g);
          qf2[qg] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
        }
      }

      f32x4 o[2][8];
      f32x4 lacc[2];
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        lacc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float mref[2] = {neg_inf(), neg_inf()};

      // Direct global-to-LDS tile loads (see the BF16 kernel); K row r of the
      // LDS tile holds key kswap(r), V row r holds key r; 16-byte chunks
      // XOR-swizzled by row:
      //  K d 0..127:   row * 128 + ((c ^ ((row >> 1) & 7)) << 4)
      //  K d 128..191: row * 64  + ((c ^ ((row >> 2) & 3)) << 4)
      //  V:            row * 128 + ((c ^ vsw(row)) << 4)
      // The V swizzle puts the sixteen rows that a half-wave of each
      // transposing read touches (8 consecutive keys in each of two lane
      // groups) on distinct banks, and does not depend on the read index t.
      auto issue_kv = [&](int kt, char* base) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int I = wave * 2 + u;
          const int p = I * 1024 + lane * 16;
          const int row = p >> 7, slot = (p & 127) >> 4;
          dma16(rk, (kt * kTileK + kswap(row)) * krs + (slot ^ ((row >> 1) & 7)) * 16, base + I * 1024);
          dma16(rv, (kt * kTileK + row) * vrs + (slot ^ vsw(row)) * 16,
                base + KA_BYTES + KB_BYTES + I * 1024);
        }
        if (D192) {
          const int p = wave * 1024 + lane * 16;
          const int row = p >> 6, x = ((p & 63) >> 4) ^ ((row >> 2) & 3);
          dma16(rk, (kt * kTileK + kswap(row)) * krs + 128 + x * 16, base + KA_BYTES + wave * 1024);
        }
      };

      // One key tile read from ring stage `cur` while the next streams into `nxt`.
      auto step = [&](char* const cur, char* const nxt, int kt) {
        const bool more = kt + 1 < n_kt;
        if (more) issue_kv(kt + 1, nxt);
        if (kt <= kt_w) {
          const char* ka = cur;
          const char* kb2 = cur + KA_BYTES;
          const char* vs = cur + KA_BYTES + KB_BYTES;
          // ---- S^T = K Q^T (8 blocks of 16 keys)
          f32x4 s[2][8];
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const int row = 16 * kb + n;
            const int sw = (row >> 1) & 7;
            const u32x4 lo = lds_load<u32x4>(ka + row * 128 + ((g ^ sw) << 4));
            const u32x4 hi = lds_load<u32x4>(ka + row * 128 + (((4 + g) ^ sw) << 4));
            const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
            for (int qg = 0; qg < 2; ++qg)
              s[qg][kb] = mfma_fp8(kf, qf[qg], f32x4{0.f, 0.f, 0.f, 0.f}, kE8M0One, kE8M0One);
            if (D192) {
              const u32x4 x = lds_load<u32x4>(kb2 + row * 64 + ((g ^ ((row >> 2) & 3)) << 4));
              const i32x8 kf2 = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
#pragma unroll
              for (int qg = 0; qg < 2; ++qg) s[qg][kb] = mfma_fp8(kf2, qf2[qg], s[qg][kb], kE8M0One, kE8M0One);
            }
          }
          // ---- causal mask, on the diagonal tile only; score (kb, i) of lane
          // group g is key 64 (kb / 4) + 16 g + 4 (kb % 4) + i of the tile
          const int kbase = kt * kTileK;
          const bool diag = kbase + kTileK - 1 > qw0;
          if (__builtin_expect(diag, 0)) {
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
              const int q = qw0 + 16 * qg + n - kbase - 16 * g;
#pragma unroll
              for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (64 * (kb >> 2) + 4 * (kb & 3) + i > q) s[qg][kb][i] = neg_inf();
            }
          }
          // ---- lane maxima of the raw scores per scale half (kb 0..3: keys
          // 16g..16g+15, kb 4..7: keys 64+16g..), lazy test and one ballot
          // per tile
          float m0[2], m1[2];
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) {
            float a0 = fmaxf(fmaxf(s[qg][0][0], s[qg][0][1]), s[qg][0][2]);
            float a1 = fmaxf(fmaxf(s[qg][4][0], s[qg][4][1]), s[qg][4][2]);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
              for (int i = (kb == 0 ? 3 : 0); i < 4; i += 2) {
                if (i == 3) {
                  a0 = fmaxf(a0, s[qg][kb][3]);
                  a1 = fmaxf(a1, s[qg][kb + 4][3]);
                } else {
                  a0 = fmaxf(fmaxf(a0, s[qg][kb][i]), s[qg][kb][i + 1]);
                  a1 = fmaxf(fmaxf(a1, s[qg][kb + 4][i]), s[qg][kb + 4][i + 1]);
                }
              }
            }
            m0[qg] = a0 * sl2;
            m1[qg] = a1 * sl2;
          }
          const bool need = (fmaxf(m0[0], m1[0]) > mref[0] + kTau) || (fmaxf(m0[1], m1[1]) > mref[1] + kTau);
          if (__builtin_expect(wave_any(need), 0)) {
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
              float rm = fmaxf(fmaxf(m0[qg], m1[qg]), __shfl_xor(fmaxf(m0[qg], m1[qg]), 16));
              rm = fmaxf(rm, __shfl_xor(rm, 32));
              const float mn = rm > mref[qg] + kTau ? rm : mref[qg];
              const float f = fast_exp2(mref[qg] - mn);
              lacc[qg] *= f;
#pragma unroll
              for (int db = 0; db < 8; ++db) o[qg][db] *= f;
              mref[qg] = mn;
            }
          }
          // ---- P codes and per-block exponents
          i32x8 pf[2];
          int psc[2];
          const bool lean = LEAN && kbase + kTileK <= q0;
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) {
            // block maxima: the 32-key block of half 0 (1) is held by lane
            // groups g and g ^ 1
            const float b0 = fmaxf(m0[qg], __shfl_xor(m0[qg], 16));
            const float b1 = fmaxf(m1[qg], __shfl_xor(m1[qg], 16));
            const float e0 = fmaxf(floorf(b0 - mref[qg]), -126.0f);
            const float e1 = fmaxf(floorf(b1 - mref[qg]), -126.0f);
            // lane 16 b + n supplies the scale of block b: groups 1 and 2
            // swap the exponents they do not hold themselves
            const float other = __shfl_xor((g & 1) ? e1 : e0, 48);
            const float mine = g == 0 ? e0 : (g == 3 ? e1 : other);
            psc[qg] = (int)mine + 127;
            if (lean) {
              const float c8 = 8.0f * sl2;
              const float o0 = kLeanC - 8.0f * (mref[qg] + e0);
              const float o1 = kLeanC - 8.0f * (mref[qg] + e1);
#pragma unroll
              for (int kb = 0; kb < 8; ++kb) {
                const float o = kb < 4 ? o0 : o1;
                unsigned w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[qg][kb][0], c8, o), 0, 0u);
                w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[qg][kb][1], c8, o), 1, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[qg][kb][2], c8, o), 2, w);
                w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[qg][kb][3], c8, o), 3, w);
                pf[qg][kb] = (int)w;
              }
            } else {
              const float nm = -mref[qg];
              const float sc0 = __builtin_bit_cast(float, (unsigned)((int)e0 + 127) << 23);
              const float sc1 = __builtin_bit_cast(float, (unsigned)((int)e1 + 127) << 23);
#pragma unroll
              for (int kb = 0; kb < 8; ++kb) {
                f32x4 p;
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], sl2, nm));
                pf[qg][kb] = (int)cvt4_fp8(p[0], p[1], p[2], p[3], kb < 4 ? sc0 : sc1);
              }
            }
          }
          // ---- row sum of the rounded P on the matrix unit
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) lacc[qg] = mfma_fp8(ones, pf[qg], lacc[qg], kE8M0One, psc[qg]);
          // ---- O^T += V^T P^T; V fragments are read two 16-column blocks
          // ahead of their MFMAs, so the LDS latency hides behind the
          // matrix work
          auto v_frag = [&](int db) {
            i32x8 vf;
            const int r = n >> 1, hh = n & 1;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              // byte 8t + r of lane group g is key 64 (t / 2) + 16 g +
              // 8 (t % 2) + r; lane 2r + hh supplies that row, columns
              // 16db + 8hh .. +7
              const int row = 64 * (t >> 1) + 16 * g + 8 * (t & 1) + r;
              const i32x2 w = lds_read_tr8(vs + row * 128 + ((db ^ vsw(row)) << 4) + hh * 8);
              vf[2 * t] = w[0];
              vf[2 * t + 1] = w[1];
            }
            return vf;
          };
          i32x8 vfb[2] = {v_frag(0), v_frag(1)};
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const i32x8 cur = vfb[db & 1];
            if (db + 2 < 8) vfb[db & 1] = v_frag(db + 2);
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) o[qg][db] = mfma_fp8(cur, pf[qg], o[qg][db], kE8M0One, psc[qg]);
            if (db + 2 < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
          }
        }
        if (more) wait_vm<0>();
        __syncthreads();
      };

      __syncthreads();   // the previous tile's last reads of the ring are done
      issue_kv(0, smem);
      wait_vm<0>();
      __syncthreads();
      for (int kt = 0; kt < n_kt; ++kt) {
        const int st = kt & 1;
        step(smem + st * STAGE, smem + (st ^ 1) * STAGE, kt);
      }

      // ---- epilogue: O * dv / l (RNE to bf16), LSE = ln2 * (m + log2 l)
      if (kt_w >= 0) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
          const float lt = lacc[qg][0];
          const float f = dvs / lt;
          const int q = qw0 + 16 * qg + n;
          if (q < S) {
            __bf16* orow = (__bf16*)a.out + (b * a.o_stride_b + h * a.o_stride_h + (long long)q * a.o_stride_s);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const u32x2 w = {pack_bf16x2(o[qg][db][0] * f, o[qg][db][1] * f),
                               pack_bf16x2(o[qg][db][2] * f, o[qg][db][3] * f)};
              *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g) = w;
            }
            if (WITH_LSE && g == 0)
              a.lse[((long long)b * a.nheads + h) * S + q] = (mref[qg] + fast_log2(lt)) * kLn2;
          }
        }
      }
    }
  }
}

}  // namespace

template <int DQK, bool LEAN>
static void launch_fp8(const AttnArgs& a, bool with_lse, dim3 gd, dim3 bd, hipStream_t s) {
  if (with_lse) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, true, LEAN>), gd, bd, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, false, LEAN>), gd, bd, 0, s, a);
}

hipError_t launch_attn_fp8(const AttnArgs& a, int d_qk, bool with_lse, bool lean, int grid, hipStream_t s) {
  const dim3 gd(grid), bd(kThreads);
  if (d_qk == 128) {
    if (lean) launch_fp8<128, true>(a, with_lse, gd, bd, s);
    else launch_fp8<128, false>(a, with_lse, gd, bd, s);
  } else {
    if (lean) launch_fp8<192, true>(a, with_lse, gd, bd, s);
    else launch_fp8<192, false>(a, with_lse, gd, bd, s);
  }
  return hipGetLastError();
}

}  // namespace zyfa
