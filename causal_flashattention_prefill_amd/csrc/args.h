// Argument checks and derived launch quantities of the C ABI (include/zyfa.h).
// Pure C++ (no HIP): a host build with sanitizers exercises them, with the
// job-table code of plan.h, in the CPU test suite.
#pragma once

namespace zyfa {

// Longest sequence (query rows, or keys of a range call) a call accepts:
// the kernels index rows, and row + offset sums, in 32-bit integers.
constexpr int kMaxSeqlen = 1 << 30;

// ZYFA_OK, or the status of the first failed check: sizes positive,
// seqlen <= kMaxSeqlen and batch * nheads < 2^31 (ZYFA_ERR_SHAPE), head
// dims (HEADDIM), nheads a multiple of nheads_k (GQA), dtype, layout.
int check_shape(int batch, int seqlen, int nheads, int nheads_k, int d_qk, int d_v, int layout, int dtype);

// Strides (elements) of a (batch, heads, seqlen, dim) view of a contiguous
// bshd or bhsd tensor.
void layout_strides(int layout, int seqlen, int heads, int dim, long long* sb, long long* sh, long long* ss);

// delta = q_pos0 - k_pos0 (key c visible to query row r when c <= r +
// delta), clamped to [-(seqlen_q + 512), seqlen_k]: offsets beyond act
// alike (every key, or no key, visible), and the kernels' row + delta sums
// stay inside int.
int clamp_delta(long long q_pos0, long long k_pos0, int seqlen_q, int seqlen_k);

// Whether 64 rows of `row_stride` elements (the last holding `dim` of them)
// of esz-byte elements span at most 2^31 - 1 bytes: the kernels address a
// wave's rows through a buffer resource with a 32-bit offset.
bool rows_in_31_bits(long long row_stride, int dim, int esz);

// Rotation signs (d = 128 values, each +1 or -1; NULL: all +1) as four
// words of sign bits, bit i set when sign i is -1. ZYFA_ERR_SIGNS for
// another value, ZYFA_ERR_HEADDIM for d other than 128 (the rotation is the
// 128-point Hadamard transform).
int sign_mask(const signed char* signs, int d, unsigned mask[4]);

bool aligned(const void* p, unsigned bytes);

}  // namespace zyfa
