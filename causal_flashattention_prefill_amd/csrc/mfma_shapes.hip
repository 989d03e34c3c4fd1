// Equal-FLOP streams of matrix instructions of two tile shapes, for choosing
// the attention kernels' MFMA shape on gfx950 (the "Attention at the Power
// Cap" post compares 16x16x32 and 32x32x16 bf16 streams at the board's power
// cap, section 3.2), and the rate of the older 16x16x32 FP8 instruction
// that takes the last 64 channels of a d_qk = 192 score product. Not part
// of the attention library: built into its own shared library and driven by
// bench_mfma_shapes.py.
//
// Every wave of a persistent 512-thread workgroup (8 waves per CU, as in the
// attention kernels) issues, per iteration, independent matrix instructions
// worth 2^17 (bf16) or 2^19 (fp8) FLOP, alternating between two operand
// sets loaded from memory (random values, so the multipliers toggle as on
// real data), and writes the sum of its accumulators at the end. All loads
// and stores stay inside the two buffers: in[] holds 16 words per thread of
// the grid, out[] one float per thread.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

enum Kind { kBf16_16x16x32 = 0, kBf16_32x32x16 = 1, kFp8_16x16x128 = 2, kFp8_32x32x64 = 3, kFp8_16x16x32 = 4 };

template <int KIND>
__global__ __launch_bounds__(512, 1) void mfma_stream(const u32x4* in, float* out, int iters) {
  const int gid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const u32x4 w0 = in[4 * gid], w1 = in[4 * gid + 1], w2 = in[4 * gid + 2], w3 = in[4 * gid + 3];
  float sum = 0.f;
  if (KIND == kBf16_16x16x32 || KIND == kBf16_32x32x16) {
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, w0), b0 = __builtin_bit_cast(bf16x8, w1);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, w2), b1 = __builtin_bit_cast(bf16x8, w3);
    if (KIND == kBf16_16x16x32) {
      f32x4 acc[8] = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((j & 1) ? a1 : a0, (j & 1) ? b1 : b0, acc[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
      f32x16 acc[4] = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((j & 1) ? a1 : a0, (j & 1) ? b1 : b0, acc[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[j][e];
    }
  } else if (KIND == kFp8_16x16x32) {
    const long a0 = __builtin_bit_cast(long, u32x2{w0[0], w0[1]}), b0 = __builtin_bit_cast(long, u32x2{w0[2], w0[3]});
    const long a1 = __builtin_bit_cast(long, u32x2{w1[0], w1[1]}), b1 = __builtin_bit_cast(long, u32x2{w1[2], w1[3]});
    f32x4 acc[8] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 32; ++j)
        acc[j & 7] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((j & 1) ? a1 : a0, (j & 1) ? b1 : b0, acc[j & 7], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    const i32x8 a0 = {(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
    const i32x8 a1 = {(int)w2[0], (int)w2[1], (int)w2[2], (int)w2[3], (int)w3[0], (int)w3[1], (int)w3[2], (int)w3[3]};
    if (KIND == kFp8_16x16x128) {
      f32x4 acc[8] = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4((j & 1) ? a1 : a0, (j & 1) ? a0 : a1, acc[j], 0, 0,
                                                                     0, 127, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
      f32x16 acc[4] = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((j & 1) ? a1 : a0, (j & 1) ? a0 : a1, acc[j], 0, 0,
                                                                    0, 127, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[j][e];
    }
  }
  out[gid] = sum;
}

}  // namespace

extern "C" {

// FLOP of one iteration of one wave.
long long mfma_shapes_flop_per_wave_iter(int kind) { return kind < 2 ? (1ll << 17) : (1ll << 19); }

// Words of `in` (uint32) and floats of `out` a launch of `grid` workgroups needs.
long long mfma_shapes_in_words(int grid) { return 16ll * 512 * grid; }
long long mfma_shapes_out_floats(int grid) { return 512ll * grid; }

int mfma_shapes_launch(int kind, const void* in, float* out, int iters, int grid, void* stream) {
  if (kind < 0 || kind > 4 || iters < 1 || grid < 1 || !in || !out) return -1;
  const dim3 g(grid), b(512);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const u32x4* x = static_cast<const u32x4*>(in);
  switch (kind) {
    case kBf16_16x16x32: hipLaunchKernelGGL(mfma_stream<kBf16_16x16x32>, g, b, 0, s, x, out, iters); break;
    case kBf16_32x32x16: hipLaunchKernelGGL(mfma_stream<kBf16_32x32x16>, g, b, 0, s, x, out, iters); break;
    case kFp8_16x16x128: hipLaunchKernelGGL(mfma_stream<kFp8_16x16x128>, g, b, 0, s, x, out, iters); break;
    case kFp8_32x32x64: hipLaunchKernelGGL(mfma_stream<kFp8_32x32x64>, g, b, 0, s, x, out, iters); break;
    default: hipLaunchKernelGGL(mfma_stream<kFp8_16x16x32>, g, b, 0, s, x, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
