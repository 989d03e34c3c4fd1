// Causal forward attention, BF16 inputs, for gfx950 (CDNA4).
//
// What is computed: "ZYFA" README, Usage and Supported configurations
// (causal, seqlen_q == seqlen_k, GQA head sharing, natural-log LSE, BF16
// output, zero padding to the query-tile multiple).
//
// Structure (one workgroup = 8 waves = 512 threads, persistent):
//  - A job is a pair of 256-row query tiles (i, n-1-i) of one (batch, head)
//    (README, Kernel design: work distribution). Each wave owns 32 query
//    rows (two 16-row groups) for the whole key loop.
//  - Keys stream in 64-key tiles through a two-stage LDS ring filled by
//    direct global-to-LDS loads (buffer_load ... lds): the loads of tile t+1
//    are issued before the MFMA work on tile t and waited for after it.
//  - Scores are computed transposed, S^T = K Q^T, with K as the MFMA A
//    operand (README, Kernel design: transposed scores), using
//    v_mfma_f32_16x16x32_bf16. Lane (g, n) (g = lane/16, n = lane%16) then
//    holds, for query column n, the keys 16*kb + 4*g + i of each 16-key
//    block kb: a lane owns part of one query row, and P goes from registers
//    straight into the PV product as the B operand.
//  - O^T += V^T P^T with V^T read from LDS by ds_read_b64_tr_b16, which
//    transposes 16-bit values during the read, so V is stored in LDS as it
//    arrives from memory.
//  - One barrier per key tile; at d_qk = 128 the key loop is unrolled by the
//    two ring stages so every LDS offset is an immediate.
//  - Online softmax in base 2 (log2(e) folded into the scale, one FMA per
//    score before the exponential) with a lazy reference maximum: it moves
//    only when some score passes it by kTau; one wave-wide ballot decides,
//    and the rescale runs out of line (README, Kernel design: lazy
//    rescaling). The causal mask is applied on diagonal tiles only.
//  - Row sums: with LSE requested, an fp32 sum of the unrounded
//    probabilities (so the LSE holds to ~1e-7 relative); otherwise one MFMA
//    of the bf16 P against ones per 32 keys, so the output is divided by the
//    sum of exactly the rounded weights that multiply V.
//  - Every conversion rounds to nearest even (README, Kernel design).
#include <type_traits>

#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

constexpr int kThreads = 512;
constexpr int kTileQ = 256;
constexpr int kTileK = 64;
constexpr int kStages = 2;
constexpr float kTau = 8.0f;           // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;

template <int DQK, bool WITH_LSE>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(const AttnArgs a) {
  constexpr int DV = 128;
  constexpr int KCH = DQK / 8;                 // 16-byte chunks per K row
  constexpr int KPITCH = DQK * 2;              // bytes per K row in LDS
  constexpr int VPITCH = DV * 2;
  constexpr int KSWZ = (KCH % 16 == 0) ? 15 : 7;
  constexpr int KBYTES = kTileK * KPITCH;
  constexpr int VBYTES = kTileK * VPITCH;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int NC = DQK / 32;                 // MFMA k-steps over d_qk
  constexpr int KLD = KBYTES / 1024 / 8;       // 1 KiB direct-to-LDS loads per wave per tile
  constexpr int VLD = VBYTES / 1024 / 8;
  static_assert(KLD * 8 * 1024 == KBYTES && VLD * 8 * 1024 == VBYTES, "tile split");

  __shared__ __attribute__((aligned(16))) char smem[kStages * STAGE];

  // work-item and group ids from the hardware registers directly (the
  // device-library accessors are not inlined into a kernel compiled with
  // IEEE mode off, and a call would spill every live register)
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int lane = tid & 63;
  // wave-uniform values live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int S = a.seqlen;
  const float sl2 = a.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  for (int it = 0; it < a.jobs_per_wg; ++it) {
    const int2 jv = a.jobs[it * a.num_wgs + wg];
    const int2 job = {__builtin_amdgcn_readfirstlane(jv.x), __builtin_amdgcn_readfirstlane(jv.y)};
    if (job.x < 0) break;
    const int b = job.x / a.nheads;
    const int h = job.x - b * a.nheads;
    const int hk = (int)(((long long)h * a.nheads_k) / a.nheads);

    const char* qbase = (const char*)a.q.ptr + 2 * (b * a.q.stride_b + h * a.q.stride_h);
    const char* kbase = (const char*)a.k.ptr + 2 * (b * a.k.stride_b + hk * a.k.stride_h);
    const char* vbase = (const char*)a.v.ptr + 2 * (b * a.v.stride_b + hk * a.v.stride_h);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, a.q_bytes);
    const i32x4 rk = make_rsrc_words(kbase, a.k_bytes);
    const i32x4 rv = make_rsrc_words(vbase, a.v_bytes);
    const int qrs = (int)(2 * a.q.stride_s);
    const int krs = (int)(2 * a.k.stride_s);
    const int vrs = (int)(2 * a.v.stride_s);

    const int tA = job.y;
    const int tB = a.n_qtiles - 1 - job.y;
    const int ntiles = (tA == tB) ? 1 : 2;
    for (int tt = 0; tt < ntiles; ++tt) {
      // the longer tile first: the workgroups of one chiplet then stream the
      // same keys at the same time for longer, so K and V stay in its L2
      const int qt = tt == 0 ? tB : tA;
      const int q0 = qt * kTileQ;
      const int qw0 = q0 + wave * 32;
      const int qend = min(q0 + kTileQ, S);
      const int n_kt = (qend - 1) / kTileK + 1;
      const int kt_w = (qw0 < S) ? min((qw0 + 31) / kTileK, n_kt - 1) : -1;

      // Q fragments, MFMA B operand: lane (g, n) holds q[row n][32c + 8g .. +7].
      bf16x8 qf[2][NC];
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          qf[qg][c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (qw0 + 16 * qg + n) * qrs + (32 * c + 8 * g) * 2));

      f32x4 o[2][8];
      f32x4 lacc[2];
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        lacc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float mref[2] = {neg_inf(), neg_inf()};
      float lsum[2] = {0.f, 0.f};

      // K/V tiles go straight from memory into LDS. Wave-instruction I fills
      // bytes [1024 I, 1024 I + 1024) of a region; lane L's 16 bytes land at
      // p = 1024 I + 16 L, which is row p / pitch, chunk slot (p % pitch) / 16,
      // so the lane fetches the global chunk that belongs in that slot. K
      // chunks are XOR-swizzled by row so the 16 lanes that read one chunk
      // column of 16 rows hit distinct banks; V chunks are swizzled by even
      // values, keeping the 8-byte halves the transposing read needs intact.
      auto issue_kv = [&](int kt, char* stage) {
#pragma unroll
        for (int u = 0; u < KLD; ++u) {
          const int I = wave * KLD + u;
          const int p = I * 1024 + lane * 16;
          const int row = p / KPITCH, x = ((p % KPITCH) >> 4) ^ (row & KSWZ);
          dma16(rk, (kt * kTileK + row) * krs + x * 16, stage + I * 1024);
        }
#pragma unroll
        for (int u = 0; u < VLD; ++u) {
          const int I = wave * VLD + u;
          const int p = I * 1024 + lane * 16;
          const int row = p / VPITCH, x = ((p % VPITCH) >> 4) ^ ((row & 7) << 1);
          dma16(rv, (kt * kTileK + row) * vrs + x * 16, stage + KBYTES + I * 1024);
        }
      };

      // Key tiles are visited in ascending order for the first (longer)
      // query tile of the pair and in descending order for the second. A
      // pair's tiles together span the same number of key tiles for every
      // pair, so the workgroups of a chiplet that have moved on to their
      // second tiles all read the same key tile at the same time and share
      // it in L2.
      const bool rev = tt == 1;
      auto tile_of = [&](int j) { return rev ? n_kt - 1 - j : j; };
      // Step j: key tile tile_of(j) is read from ring stage `cur` while the
      // next streams into `nxt`: S^T = K Q^T, softmax, O^T += V^T P^T.
      auto step = [&](char* const cur, char* const nxt, int j) {
        const int kt = tile_of(j);
        const bool more = j + 1 < n_kt;
        if (more) issue_kv(tile_of(j + 1), nxt);
        if (kt <= kt_w) {
          // ---- S^T = K Q^T
          f32x4 s[2][4];
#pragma unroll
          for (int qg = 0; qg < 2; ++qg)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[qg][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const int row = 16 * kb + n;
              const int x = 4 * c + g;
              const bf16x8 kf = lds_load<bf16x8>(cur + row * KPITCH + ((x ^ (row & KSWZ)) << 4));
#pragma unroll
              for (int qg = 0; qg < 2; ++qg)
                s[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qg][c], s[qg][kb], 0, 0, 0);
            }
          // ---- causal mask, on diagonal tiles only (kept a real branch)
          const int kbase = kt * kTileK;
          if (__builtin_expect(kbase + kTileK - 1 > qw0, 0)) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
              const int q = qw0 + 16 * qg + n - kbase - 4 * g;
#pragma unroll
              for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (16 * kb + i > q) s[qg][kb][i] = neg_inf();
            }
          }
          // ---- lazy max: a lane-local test and one ballot per tile
          float mx[2];
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) {
            float m = fmaxf(fmaxf(s[qg][0][0], s[qg][0][1]), s[qg][0][2]);
            m = fmaxf(fmaxf(m, s[qg][0][3]), s[qg][1][0]);
            m = fmaxf(fmaxf(m, s[qg][1][1]), s[qg][1][2]);
            m = fmaxf(fmaxf(m, s[qg][1][3]), s[qg][2][0]);
            m = fmaxf(fmaxf(m, s[qg][2][1]), s[qg][2][2]);
            m = fmaxf(fmaxf(m, s[qg][2][3]), s[qg][3][0]);
            m = fmaxf(fmaxf(m, s[qg][3][1]), s[qg][3][2]);
            mx[qg] = fmaxf(m, s[qg][3][3]) * sl2;
          }
          if (__builtin_expect(wave_any((mx[0] > mref[0] + kTau) || (mx[1] > mref[1] + kTau)), 0)) {
            // Keep this branch real: with f == 1 the multiplies are harmless,
            // so the compiler would otherwise run them on every tile.
            asm volatile("" ::: "memory");
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
              const float rm = max_xor32(max_xor16(mx[qg]));
              const float mn = fmaxf(mref[qg], rm);
              const float f = fast_exp2(mref[qg] - mn);
              lsum[qg] *= f;
              lacc[qg] *= f;
#pragma unroll
              for (int db = 0; db < 8; ++db) o[qg][db] *= f;
              mref[qg] = mn;
            }
          }
          // ---- P = exp2(s * scale - m), RNE to bf16. Operands are assembled
          // as whole 32-bit words: building them element by element from
          // 16-bit values has been compiled incorrectly (every slot took
          // element 0).
          bf16x8 pb[2][2];
#pragma unroll
          for (int qg = 0; qg < 2; ++qg) {
            const float nm = -mref[qg];
            float ls = 0.f;
            u32x4 w[2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              f32x4 p;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], sl2, nm));
                if (WITH_LSE) ls += p[i];
              }
              w[kb >> 1][2 * (kb & 1) + 0] = pack_bf16x2(p[0], p[1]);
              w[kb >> 1][2 * (kb & 1) + 1] = pack_bf16x2(p[2], p[3]);
            }
            pb[qg][0] = __builtin_bit_cast(bf16x8, w[0]);
            pb[qg][1] = __builtin_bit_cast(bf16x8, w[1]);
            if (WITH_LSE) lsum[qg] += ls;
          }
          // ---- O^T += V^T P^T (and the row sum of the rounded P when no LSE)
#pragma unroll
          for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              u32x2 t[2];
#pragma unroll
              for (int hf = 0; hf < 2; ++hf) {
                const int row = 32 * kc + 16 * hf + 4 * g + (n >> 2);
                const int x = 2 * db + ((n & 3) >> 1);
                const char* p = cur + KBYTES + row * VPITCH + ((x ^ ((row & 7) << 1)) << 4) + (n & 1) * 8;
                t[hf] = __builtin_bit_cast(u32x2, lds_read_tr16(p));
              }
              const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{t[0][0], t[0][1], t[1][0], t[1][1]});
#pragma unroll
              for (int qg = 0; qg < 2; ++qg)
                o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[qg][kc], o[qg][db], 0, 0, 0);
            }
          if (!WITH_LSE) {
#pragma unroll
            for (int qg = 0; qg < 2; ++qg)
#pragma unroll
              for (int kc = 0; kc < 2; ++kc)
                lacc[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg][kc], lacc[qg], 0, 0, 0);
          }
        }
        if (more) wait_vm<0>();
        __syncthreads();
      };

      __syncthreads();   // the previous tile's last reads of the ring are done
      issue_kv(tile_of(0), smem);
      wait_vm<0>();
      __syncthreads();
      if (DQK == 128) {
        // unrolled by the two stages: every LDS offset is an immediate
        for (int j = 0; j < n_kt; j += 2) {
          step(smem, smem + STAGE, j);
          if (j + 1 < n_kt) step(smem + STAGE, smem, j + 1);
        }
      } else {
        // d_qk = 192 keeps 48 registers of Q; a rolled loop leaves room
        for (int j = 0; j < n_kt; ++j) {
          const int st = j & 1;
          step(smem + st * STAGE, smem + (st ^ 1) * STAGE, j);
        }
      }

      // ---- epilogue: O / l (RNE to bf16), LSE = ln2 * (m + log2 l)
      if (kt_w >= 0) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
          float lt;
          if (WITH_LSE) {
            lt = lsum[qg] + swap16(lsum[qg]);
            lt += __shfl_xor(lt, 32);
          } else {
            lt = lacc[qg][0];
          }
          const float inv = 1.0f / lt;
          const int q = qw0 + 16 * qg + n;
          if (q < S) {
            __bf16* orow = (__bf16*)a.out + (b * a.o_stride_b + h * a.o_stride_h + (long long)q * a.o_stride_s);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const u32x2 w = {pack_bf16x2(o[qg][db][0] * inv, o[qg][db][1] * inv),
                               pack_bf16x2(o[qg][db][2] * inv, o[qg][db][3] * inv)};
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

hipError_t launch_attn_bf16(const AttnArgs& a, int d_qk, bool with_lse, int grid, hipStream_t s) {
  const dim3 gd(grid), bd(kThreads);
  if (d_qk == 128) {
    if (with_lse) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), gd, bd, 0, s, a);
  } else {
    if (with_lse) hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, false>), gd, bd, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zyfa
