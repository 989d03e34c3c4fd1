// LSE merge of two partial attention results over disjoint key sets, for
// gfx950 (CDNA4).
//
// What is computed: the README's Accuracy note (the LSE is returned so that
// results over different key ranges merge consistently) and the RDNA3
// page's split-and-merge (partial outputs with their LSE, combined by an
// LSE reduction). For one query row with partial results (O_a, L_a) and
// (O_b, L_b):
//     L = ln(e^L_a + e^L_b),  O = e^(L_a - L) O_a + e^(L_b - L) O_b
// and L = -inf, O = 0 when both are empty (L_a = L_b = -inf).
//
// Memory-bound: each row reads two bf16 outputs of d_v = 128 values and
// two LSE values and writes one of each. Sixteen lanes handle one row, 16
// bytes each; a row never spans two waves, and every lane reads its inputs
// before any lane of the wave writes, so the output may alias either input.
#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const u32x4* oa, const float* lse_a,
                                                                  const u32x4* ob, const float* lse_b,
                                                                  u32x4* out, float* lse, long long rows, int seqlen,
                                                                  int nheads, bool bshd) {
  const long long t = (long long)blockIdx.x * kMergeThreads + threadIdx.x;
  const long long r = t >> 4;          // output row in memory order
  const int c = (int)(t & 15);         // 16-byte chunk of the row
  if (r >= rows) return;
  // LSE index (b, h, s) of the row
  long long li = r;
  if (bshd) {
    const long long bs = r / nheads;
    const int h = (int)(r - bs * nheads);
    const long long b = bs / seqlen;
    const int s = (int)(bs - b * seqlen);
    li = (b * nheads + h) * seqlen + s;
  }
  const float la = lse_a[li], lb = lse_b[li];
  const u32x4 xa = oa[r * 16 + c], xb = ob[r * 16 + c];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, L = neg_inf();
  if (m > neg_inf()) {
    const float ea = __builtin_amdgcn_exp2f((la - m) * kLog2e);
    const float eb = __builtin_amdgcn_exp2f((lb - m) * kLog2e);
    const float tot = ea + eb;
    wa = ea / tot;
    wb = eb / tot;
    L = m + __builtin_amdgcn_logf(tot) * kLn2;
  }
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // two bf16 per word: the value is the high half of an fp32
    const float a0 = __builtin_bit_cast(float, xa[i] << 16), a1 = __builtin_bit_cast(float, xa[i] & 0xFFFF0000u);
    const float b0 = __builtin_bit_cast(float, xb[i] << 16), b1 = __builtin_bit_cast(float, xb[i] & 0xFFFF0000u);
    y[i] = pack_bf16x2(wa * a0 + wb * b0, wa * a1 + wb * b1);
  }
  out[r * 16 + c] = y;
  if (c == 0) lse[li] = L;
}

}  // namespace

hipError_t launch_lse_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b, void* out,
                            float* lse, int batch, int seqlen, int nheads, int d_v, bool bshd, hipStream_t s) {
  (void)d_v;   // 128: 16 chunks of 16 bytes per row
  const long long rows = (long long)batch * seqlen * nheads;
  const long long threads = rows * 16;
  const long long blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, (const u32x4*)out_a,
                     lse_a, (const u32x4*)out_b, lse_b, (u32x4*)out, lse, rows, seqlen, nheads, bshd);
  return hipGetLastError();
}

}  // namespace zyfa
