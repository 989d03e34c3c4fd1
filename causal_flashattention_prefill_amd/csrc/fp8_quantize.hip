// Per-tensor power-of-two FP8 (e4m3fn) quantization for gfx950.
//
// "ZYFA" README, Usage: fp8_quantize gives one power-of-two scale per tensor
// and returns the descale as a device scalar; every conversion rounds to
// nearest even (Kernel design). Rule: amax = max|x|; descale = the smallest
// power of two d with amax / d <= 448 (1 when amax == 0, and at least 2^-126
// so that it is a normal float); code = RNE_e4m3fn(x / d).
//
// Three kernels on one stream, no atomics, so the result never depends on
// timing:
//  1. amax_partial: each block reduces a strided share of |x| to one value
//     (non-negative floats compare like their bit patterns).
//  2. amax_final: one block reduces the partials and writes the descale.
//  3. convert: x * (1/d) is exact (d is a power of two), then
//     v_cvt_pk_fp8_f32 rounds to nearest even.
#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

constexpr int kQThreads = 256;
constexpr int kMaxPartials = 1024;

// Scalars are passed by value: __builtin_bit_cast applied directly to an
// element of an ext_vector (w[1]) has been compiled as a cast of element 0.
__device__ __forceinline__ float as_float(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ unsigned block_max_u32(unsigned v, unsigned* red) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  unsigned r = 0;
  if (threadIdx.x == 0)
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, red[i]);
  return r;  // valid in thread 0
}

// x_dtype 0: bf16 (8 values per 16 bytes), 2: fp32 (4 values per 16 bytes).
template <int XDT>
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(const void* x, long long numel, unsigned* partial) {
  __shared__ unsigned red[kQThreads / 64];
  constexpr int PER = XDT == 0 ? 8 : 4;
  const long long nvec = numel / PER;
  unsigned m = 0;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 w = reinterpret_cast<const u32x4*>(x)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (XDT == 0) {
        m = max(m, __builtin_bit_cast(unsigned, fabsf(bf16_lo(w[j]))));
        m = max(m, __builtin_bit_cast(unsigned, fabsf(bf16_hi(w[j]))));
      } else {
        m = max(m, w[j] & 0x7FFFFFFFu);
      }
    }
  }
  // tail (numel not a multiple of the vector width): block 0 only
  if (blockIdx.x == 0) {
    for (long long i = nvec * PER + threadIdx.x; i < numel; i += blockDim.x) {
      float v = XDT == 0 ? __builtin_bit_cast(float, ((unsigned)reinterpret_cast<const unsigned short*>(x)[i]) << 16)
                         : reinterpret_cast<const float*>(x)[i];
      m = max(m, __builtin_bit_cast(unsigned, fabsf(v)));
    }
  }
  const unsigned r = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

// descale = smallest power of two d >= 2^-126 with amax <= 448 * d.
// With amax = m * 2^E (1 <= m < 2): 448 = 1.75 * 2^8, so
// amax <= 448 * 2^e  <=>  e >= E - 8 when m <= 1.75, else e >= E - 7.
__device__ __forceinline__ float pow2_descale_from_bits(unsigned amax_bits) {
  if (amax_bits == 0) return 1.0f;
  int E;
  unsigned mant;
  const unsigned ef = amax_bits >> 23;
  if (ef == 0) {  // subnormal amax: normalise
    const int lz = __clz(amax_bits) - 8;     // leading zeros within the 23-bit field + 1
    E = -126 - lz;
    mant = (amax_bits << lz) & 0x7FFFFFu;
  } else {
    E = (int)ef - 127;
    mant = amax_bits & 0x7FFFFFu;
  }
  int e = E - 8 + (mant > 0x600000u ? 1 : 0);  // 0x600000: mantissa field of 1.75
  if (e < -126) e = -126;
  return __builtin_bit_cast(float, (unsigned)(e + 127) << 23);
}

__global__ __launch_bounds__(kQThreads) void amax_final_kernel(const unsigned* partial, int np, float* descale) {
  __shared__ unsigned red[kQThreads / 64];
  unsigned m = 0;
  for (int i = threadIdx.x; i < np; i += blockDim.x) m = max(m, partial[i]);
  const unsigned r = block_max_u32(m, red);
  if (threadIdx.x == 0) *descale = pow2_descale_from_bits(r);
}

template <int XDT>
__global__ __launch_bounds__(kQThreads) void convert_kernel(const void* x, long long numel, const float* descale,
                                                            unsigned char* x8) {
  const float inv = 1.0f / *descale;  // exact: descale is a power of two
  constexpr int PER = XDT == 0 ? 8 : 4;
  const long long nvec = numel / PER;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 w = reinterpret_cast<const u32x4*>(x)[i];
    if (XDT == 0) {
      u32x2 outw;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * j]) * inv, bf16_hi(w[2 * j]) * inv, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * j + 1]) * inv, bf16_hi(w[2 * j + 1]) * inv, p, true);
        outw[j] = (unsigned)p;
      }
      reinterpret_cast<u32x2*>(x8)[i] = outw;
    } else {
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(as_float(w[0]) * inv,
                                              as_float(w[1]) * inv, 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(as_float(w[2]) * inv,
                                          as_float(w[3]) * inv, p, true);
      reinterpret_cast<unsigned*>(x8)[i] = (unsigned)p;
    }
  }
  if (blockIdx.x == 0) {
    for (long long i = nvec * PER + threadIdx.x; i < numel; i += blockDim.x) {
      float v = XDT == 0 ? __builtin_bit_cast(float, ((unsigned)reinterpret_cast<const unsigned short*>(x)[i]) << 16)
                         : reinterpret_cast<const float*>(x)[i];
      const int p = __builtin_amdgcn_cvt_pk_fp8_f32(v * inv, 0.0f, 0, false);
      x8[i] = (unsigned char)(p & 0xFF);
    }
  }
}

}  // namespace

int quantize_scratch_slots() { return kMaxPartials; }

hipError_t launch_fp8_quantize(const void* x, int x_dtype, long long numel, void* x8, float* descale,
                               unsigned* scratch_amax, int scratch_slots, hipStream_t s) {
  const int per = x_dtype == 0 ? 8 : 4;
  const long long nvec = numel / per;
  long long want = (nvec + kQThreads * 4 - 1) / (kQThreads * 4);
  int blocks = (int)(want < 1 ? 1 : (want > scratch_slots ? scratch_slots : want));
  if (x_dtype == 0)
    hipLaunchKernelGGL(amax_partial_kernel<0>, dim3(blocks), dim3(kQThreads), 0, s, x, numel, scratch_amax);
  else
    hipLaunchKernelGGL(amax_partial_kernel<2>, dim3(blocks), dim3(kQThreads), 0, s, x, numel, scratch_amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(kQThreads), 0, s, scratch_amax, blocks, descale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  long long cw = (nvec + kQThreads - 1) / kQThreads;
  int cblocks = (int)(cw < 1 ? 1 : (cw > 8192 ? 8192 : cw));
  if (x_dtype == 0)
    hipLaunchKernelGGL(convert_kernel<0>, dim3(cblocks), dim3(kQThreads), 0, s, x, numel, descale, (unsigned char*)x8);
  else
    hipLaunchKernelGGL(convert_kernel<2>, dim3(cblocks), dim3(kQThreads), 0, s, x, numel, descale, (unsigned char*)x8);
  return hipGetLastError();
}

}  // namespace zyfa
