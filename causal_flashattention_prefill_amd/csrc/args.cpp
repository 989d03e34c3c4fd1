// Argument checks of the C ABI; see args.h.
#include "args.h"

#include <algorithm>
#include <cstdint>

#include "zyfa.h"

namespace zyfa {

int check_shape(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype) {
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || nheads_k <= 0) return ZYFA_ERR_SHAPE;
  if (seqlen > kMaxSeqlen || (long long)batch * nheads > 0x7FFFFFFFll) return ZYFA_ERR_SHAPE;
  if (!((d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128))) return ZYFA_ERR_HEADDIM;
  if (nheads % nheads_k != 0) return ZYFA_ERR_GQA;
  if (dtype != ZYFA_DTYPE_BF16 && dtype != ZYFA_DTYPE_FP8_E4M3FN) return ZYFA_ERR_DTYPE;
  if (layout != ZYFA_LAYOUT_BSHD && layout != ZYFA_LAYOUT_BHSD) return ZYFA_ERR_LAYOUT;
  return ZYFA_OK;
}

void layout_strides(int layout, int seqlen, int heads, int dim, long long* sb, long long* sh, long long* ss) {
  if (layout == ZYFA_LAYOUT_BSHD) {
    *sb = (long long)seqlen * heads * dim;
    *sh = dim;
    *ss = (long long)heads * dim;
  } else {
    *sb = (long long)heads * seqlen * dim;
    *sh = (long long)seqlen * dim;
    *ss = dim;
  }
}

int clamp_delta(long long q_pos0, long long k_pos0, int seqlen_q, int seqlen_k) {
  const __int128 dl = (__int128)q_pos0 - (__int128)k_pos0;   // exact for any two positions
  const __int128 lo = -(__int128)seqlen_q - 512, hi = seqlen_k;
  return (int)std::max(lo, std::min(dl, hi));
}

bool rows_in_31_bits(long long row_stride, int dim, int esz) {
  if (row_stride < 0 || row_stride > (1ll << 40)) return false;
  return (64 * row_stride + dim) * esz <= 0x7FFFFFFFll;
}

int sign_mask(const signed char* signs, int d, unsigned mask[4]) {
  if (d != 128) return ZYFA_ERR_HEADDIM;
  for (int i = 0; i < 4; ++i) mask[i] = 0;
  if (!signs) return ZYFA_OK;
  for (int i = 0; i < d; ++i) {
    if (signs[i] != 1 && signs[i] != -1) return ZYFA_ERR_SIGNS;
    if (signs[i] < 0) mask[i >> 5] |= 1u << (i & 31);
  }
  return ZYFA_OK;
}

bool aligned(const void* p, unsigned bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

}  // namespace zyfa
