// Per-tensor power-of-two FP8 (e4m3fn) quantization for gfx950.
//
// "ZYFA" README, Usage: fp8_quantize gives one power-of-two scale per tensor
// and returns the descale as a device scalar; every conversion rounds to
// nearest even (Kernel design). Rule: amax = max|x|; descale = the smallest
// power of two d with amax / d <= 448 (1 when amax == 0, and at least 2^-126
// so that it is a normal float); code = RNE_e4m3fn(x / d).
//
// Three kernels on one stream, no atomics, so the result never depends on
// timing (the rotated variant at the end of the file has the same shape):
//  1. amax_partial: each block reduces a strided share of |x| to one value
//     (non-negative floats compare like their bit patterns).
//  2. amax_final: one block reduces the partials and writes the descale.
//  3. convert: x * (1/d) is exact (d is a power of two), then
//     v_cvt_pk_fp8_f32 rounds to nearest even.
// The partial maxima are kept in the first bytes of the call's own output
// x8 (at most one 4-byte partial per 4 output bytes), which step 3 then
// overwrites: a call touches no memory but its own arguments, so calls on
// different streams, or in parallel branches of a graph, cannot interfere.
// A grid of one block (small tensors) writes the descale in step 1.
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

// x_dtype 0: bf16 (8 values per 16 bytes), 2: fp32 (4 values per 16 bytes).
// FINAL: a grid of one block, which writes the descale itself.
template <int XDT, bool FINAL>
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(const void* x, long long numel, unsigned* partial,
                                                                 float* descale) {
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
  if (threadIdx.x == 0) {
    if (FINAL) *descale = pow2_descale_from_bits(r);
    else partial[blockIdx.x] = r;
  }
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

// ---- Rotation before quantization ("ZYFA" README, "Using FP8 attention in
// a model"): each row x of d = 128 channels becomes y = x R with
//   R = diag(s) H_128 / sqrt(128)  (Sylvester Hadamard, signs s)
// and the rotated tensor is quantized as above. Half a wave (32 lanes)
// holds one row, lane l channels 4 l .. 4 l + 3. The fast Walsh-Hadamard
// transform does the butterflies on channel bits held in a lane in
// registers and those held across lanes with xor shuffles inside the half
// wave; butterfly (u, w) -> (u + w, u - w) keeps natural order, so the
// result is x H. The two passes (maximum, then conversion) both rotate, so
// the rotated tensor is never stored.

// bit i set when s_i = -1
struct SignMask {
  unsigned w[4];
};

constexpr float kInvSqrt128 = 0.0883883476483184405f;

template <int D>
struct Rot {
  static_assert(D == 128, "the rotation is the 128-point Hadamard transform");
  static constexpr int V = 4;  // values per lane
};

// Sign bits of this lane's channels, as float sign-bit masks.
template <int D>
__device__ __forceinline__ void lane_signs(const SignMask& sm, int hl, unsigned (&sg)[Rot<D>::V]) {
  const unsigned w = hl < 8 ? sm.w[0] : hl < 16 ? sm.w[1] : hl < 24 ? sm.w[2] : sm.w[3];
#pragma unroll
  for (int t = 0; t < 4; ++t) sg[t] = ((w >> ((4 * hl + t) & 31)) & 1u) << 31;
}

// butterfly across lanes: the partner at lane ^ M (within the 32-lane half
// wave; ds_swizzle in bit mode, xor mask M) holds the channel with that bit
// flipped
template <int M>
__device__ __forceinline__ float bfly_x(float v, bool upper) {
  const float p = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (M << 10)));
  return upper ? p - v : v + p;
}

// raw channel values of one row held by this lane (zeros past the last row)
template <int D, int XDT>
__device__ __forceinline__ void load_row(const void* x, long long row, bool live, int hl, float (&y)[Rot<D>::V]) {
  const char* base = reinterpret_cast<const char*>(x);
  if (XDT == 0) {
    u32x2 w = {0u, 0u};
    if (live) w = *reinterpret_cast<const u32x2*>(base + row * 256 + hl * 8);
    const unsigned w0 = w[0], w1 = w[1];
    y[0] = bf16_lo(w0); y[1] = bf16_hi(w0); y[2] = bf16_lo(w1); y[3] = bf16_hi(w1);
  } else {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4*>(base + row * 512 + hl * 16);
    const unsigned w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    y[0] = as_float(w0); y[1] = as_float(w1); y[2] = as_float(w2); y[3] = as_float(w3);
  }
}

template <int D, int M>
__device__ __forceinline__ void bfly_stage(float (&y)[Rot<D>::V], int hl) {
  const bool up = (hl & M) != 0;
#pragma unroll
  for (int t = 0; t < Rot<D>::V; ++t) y[t] = bfly_x<M>(y[t], up);
}

// y <- (y * s) R for one row (signs as float sign-bit masks)
template <int D>
__device__ __forceinline__ void transform(float (&y)[Rot<D>::V], int hl, const unsigned (&sg)[Rot<D>::V]) {
#pragma unroll
  for (int t = 0; t < Rot<D>::V; ++t) y[t] = as_float(__builtin_bit_cast(unsigned, y[t]) ^ sg[t]);
  // channel bits 0, 1 in the lane
  const float a0 = y[0] + y[1], a1 = y[0] - y[1], a2 = y[2] + y[3], a3 = y[2] - y[3];
  y[0] = a0 + a2; y[2] = a0 - a2; y[1] = a1 + a3; y[3] = a1 - a3;
  // the remaining channel bits across the lanes (lane bits 0..4)
  bfly_stage<D, 1>(y, hl);
  bfly_stage<D, 2>(y, hl);
  bfly_stage<D, 4>(y, hl);
  bfly_stage<D, 8>(y, hl);
  bfly_stage<D, 16>(y, hl);
#pragma unroll
  for (int t = 0; t < 4; ++t) y[t] *= kInvSqrt128;
}

// Each half wave takes kRotRows rows per step: their loads go out together,
// so enough bytes are in flight to keep HBM busy.
constexpr int kRotRows = 4;

// Optional vector subtracted from every row of a (batch, head) before the
// rotation (K smoothing: the mean key of the head). Row r of the rotated
// tensor belongs to head slot bh = b * nheads + h, whose vector is
// shift[bh * d ..]; rows are counted in the tensor's memory order.
struct ShiftDesc {
  const float* shift;  // null: nothing subtracted
  unsigned seqlen, nheads;
  bool bshd;
};

__device__ __forceinline__ unsigned shift_slot(unsigned r, const ShiftDesc& sd) {
  if (!sd.bshd) return r / sd.seqlen;                 // bhsd: rows of one head are contiguous
  const unsigned bs = r / sd.nheads;                  // bshd: (batch, position) then head
  return (bs / sd.seqlen) * sd.nheads + (r - bs * sd.nheads);
}

// this lane's channels of the row's shift vector
template <int D>
__device__ __forceinline__ void load_shift(const float* v, int hl, float (&sv)[Rot<D>::V]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(v + 4 * hl);
  const unsigned w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
  sv[0] = as_float(w0); sv[1] = as_float(w1); sv[2] = as_float(w2); sv[3] = as_float(w3);
}

template <int D, bool SHIFT>
__device__ __forceinline__ void subtract_shift(float (&y)[Rot<D>::V], long long r, bool live, int hl,
                                               const ShiftDesc& sd) {
  if (!SHIFT || !live) return;
  float sv[Rot<D>::V];
  load_shift<D>(sd.shift + (size_t)shift_slot((unsigned)r, sd) * D, hl, sv);
#pragma unroll
  for (int t = 0; t < Rot<D>::V; ++t) y[t] -= sv[t];
}

template <int D, int XDT, bool SHIFT, bool FINAL>
__global__ __launch_bounds__(kQThreads) void rot_amax_kernel(const void* x, long long rows, SignMask sm, ShiftDesc sd,
                                                             unsigned* partial, float* descale) {
  __shared__ unsigned red[kQThreads / 64];
  const int hl = threadIdx.x & 31;
  unsigned sg[Rot<D>::V];
  lane_signs<D>(sm, hl, sg);
  const long long nh = ((long long)gridDim.x * kQThreads) >> 5;
  unsigned m = 0;
  for (long long r0 = (((long long)blockIdx.x * kQThreads + threadIdx.x) >> 5) * kRotRows; r0 < rows;
       r0 += nh * kRotRows) {
    float y[kRotRows][Rot<D>::V];
#pragma unroll
    for (int u = 0; u < kRotRows; ++u) {
      load_row<D, XDT>(x, r0 + u, r0 + u < rows, hl, y[u]);
      subtract_shift<D, SHIFT>(y[u], r0 + u, r0 + u < rows, hl, sd);
    }
#pragma unroll
    for (int u = 0; u < kRotRows; ++u) {
      transform<D>(y[u], hl, sg);   // rows past the end are zero and stay zero
#pragma unroll
      for (int t = 0; t < Rot<D>::V; ++t) m = max(m, __builtin_bit_cast(unsigned, fabsf(y[u][t])));
    }
  }
  const unsigned r = block_max_u32(m, red);
  if (threadIdx.x == 0) {
    if (FINAL) *descale = pow2_descale_from_bits(r);
    else partial[blockIdx.x] = r;
  }
}

template <int D, int XDT, bool SHIFT>
__global__ __launch_bounds__(kQThreads) void rot_convert_kernel(const void* x, long long rows, SignMask sm,
                                                                ShiftDesc sd, const float* descale,
                                                                unsigned char* x8) {
  const float inv = 1.0f / *descale;  // exact: descale is a power of two
  const int hl = threadIdx.x & 31;
  unsigned sg[Rot<D>::V];
  lane_signs<D>(sm, hl, sg);
  const long long nh = ((long long)gridDim.x * kQThreads) >> 5;
  for (long long r0 = (((long long)blockIdx.x * kQThreads + threadIdx.x) >> 5) * kRotRows; r0 < rows;
       r0 += nh * kRotRows) {
    float y[kRotRows][Rot<D>::V];
#pragma unroll
    for (int u = 0; u < kRotRows; ++u) {
      load_row<D, XDT>(x, r0 + u, r0 + u < rows, hl, y[u]);
      subtract_shift<D, SHIFT>(y[u], r0 + u, r0 + u < rows, hl, sd);
    }
#pragma unroll
    for (int u = 0; u < kRotRows; ++u) {
      transform<D>(y[u], hl, sg);
      const long long r = r0 + u;
      if (r >= rows) continue;
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(y[u][0] * inv, y[u][1] * inv, 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(y[u][2] * inv, y[u][3] * inv, p, true);
      *reinterpret_cast<unsigned*>(x8 + r * 128 + 4 * hl) = (unsigned)p;
    }
  }
}

// Number of amax partials: one per block, capped so that they fit in the
// first bytes of the output (4 bytes each) and at kMaxPartials.
long long partial_blocks(long long want, long long out_bytes) {
  long long b = want < 1 ? 1 : want;
  if (b > out_bytes / 4) b = out_bytes / 4;
  if (b > kMaxPartials) b = kMaxPartials;
  return b < 1 ? 1 : b;
}

template <int D, int XDT, bool SHIFT>
hipError_t launch_rot(const void* x, long long rows, const SignMask& sm, const ShiftDesc& sd, void* x8,
                      float* descale, hipStream_t s) {
  constexpr int kRowsPerBlock = kQThreads / 32 * kRotRows;
  const int blocks = (int)partial_blocks((rows + kRowsPerBlock * 2 - 1) / (kRowsPerBlock * 2), rows * D);
  unsigned* partial = reinterpret_cast<unsigned*>(x8);
  if (blocks == 1) {
    hipLaunchKernelGGL((rot_amax_kernel<D, XDT, SHIFT, true>), dim3(1), dim3(kQThreads), 0, s, x, rows, sm, sd,
                       partial, descale);
  } else {
    hipLaunchKernelGGL((rot_amax_kernel<D, XDT, SHIFT, false>), dim3(blocks), dim3(kQThreads), 0, s, x, rows, sm,
                       sd, partial, descale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(kQThreads), 0, s, partial, blocks, descale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long long cw = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int cblocks = (int)(cw < 1 ? 1 : (cw > 8192 ? 8192 : cw));
  hipLaunchKernelGGL((rot_convert_kernel<D, XDT, SHIFT>), dim3(cblocks), dim3(kQThreads), 0, s, x, rows, sm, sd,
                     descale, (unsigned char*)x8);
  return hipGetLastError();
}

template <int D, bool SHIFT>
hipError_t launch_rot_dt(const void* x, int x_dtype, long long rows, const SignMask& sm, const ShiftDesc& sd,
                         void* x8, float* descale, hipStream_t s) {
  return x_dtype == 0 ? launch_rot<D, 0, SHIFT>(x, rows, sm, sd, x8, descale, s)
                      : launch_rot<D, 2, SHIFT>(x, rows, sm, sd, x8, descale, s);
}

// ---- Mean over positions of each (batch, head), for K smoothing: one
// workgroup of 1024 threads per (batch, head); d / 8 threads cover a row (8
// channels each), 1024 / (d / 8) rows at a time; each thread sums its rows
// in order, then one thread per channel adds the partial sums in order, so
// the result does not depend on timing.
constexpr int kMeanThreads = 1024;

template <int D, int XDT>
__global__ __launch_bounds__(kMeanThreads) void key_mean_kernel(const void* x, int seqlen, int nheads, bool bshd,
                                                               float* mean) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RP = kMeanThreads / TPR;     // rows in parallel
  __shared__ float part[RP][D];
  const int bh = blockIdx.x;
  const int b = bh / nheads, h = bh - (bh / nheads) * nheads;
  const int t = threadIdx.x;
  const int rp = t / TPR, c0 = (t - rp * TPR) * 8;
  const long long row_stride = bshd ? (long long)nheads * D : D;
  const long long base = bshd ? ((long long)b * seqlen * nheads + h) * D : (long long)bh * seqlen * D;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (rp < RP) {
    for (int sp = rp; sp < seqlen; sp += RP) {
      const long long e = base + sp * row_stride + c0;
      if (XDT == 0) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned short*>(x) + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned wj = w[j];
          acc[2 * j] += bf16_lo(wj);
          acc[2 * j + 1] += bf16_hi(wj);
        }
      } else {
        const float* f = reinterpret_cast<const float*>(x) + e;
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(f), w1 = *reinterpret_cast<const u32x4*>(f + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned a0 = w0[j], a1 = w1[j];
          acc[j] += as_float(a0);
          acc[4 + j] += as_float(a1);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part[rp][c0 + j] = acc[j];
  }
  __syncthreads();
  if (t < D) {
    float sum = 0.f;
    for (int i = 0; i < RP; ++i) sum += part[i][t];
    mean[(long long)bh * D + t] = sum / (float)seqlen;
  }
}

}  // namespace

hipError_t launch_fp8_quantize_rotated(const void* x, int x_dtype, long long rows, int d, const unsigned* sign_mask,
                                       const float* shift, int seqlen, int nheads, bool bshd, void* x8,
                                       float* descale, hipStream_t s) {
  if (d != 128) return hipErrorInvalidValue;
  SignMask sm;
  for (int i = 0; i < 4; ++i) sm.w[i] = sign_mask[i];
  const ShiftDesc sd{shift, (unsigned)seqlen, (unsigned)nheads, bshd};
  return shift ? launch_rot_dt<128, true>(x, x_dtype, rows, sm, sd, x8, descale, s)
               : launch_rot_dt<128, false>(x, x_dtype, rows, sm, sd, x8, descale, s);
}

hipError_t launch_key_mean(const void* x, int x_dtype, int batch, int seqlen, int nheads, int d, bool bshd,
                           float* mean, hipStream_t s) {
  const dim3 g((unsigned)(batch * nheads)), b(kMeanThreads);
  if (d == 128) {
    if (x_dtype == 0) hipLaunchKernelGGL((key_mean_kernel<128, 0>), g, b, 0, s, x, seqlen, nheads, bshd, mean);
    else hipLaunchKernelGGL((key_mean_kernel<128, 2>), g, b, 0, s, x, seqlen, nheads, bshd, mean);
  } else {
    if (x_dtype == 0) hipLaunchKernelGGL((key_mean_kernel<192, 0>), g, b, 0, s, x, seqlen, nheads, bshd, mean);
    else hipLaunchKernelGGL((key_mean_kernel<192, 2>), g, b, 0, s, x, seqlen, nheads, bshd, mean);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* x, int x_dtype, long long numel, void* x8, float* descale,
                               hipStream_t s) {
  const int per = x_dtype == 0 ? 8 : 4;
  const long long nvec = numel / per;
  const int blocks = (int)partial_blocks((nvec + kQThreads * 4 - 1) / (kQThreads * 4), numel);
  unsigned* partial = reinterpret_cast<unsigned*>(x8);
  if (blocks == 1) {
    if (x_dtype == 0)
      hipLaunchKernelGGL((amax_partial_kernel<0, true>), dim3(1), dim3(kQThreads), 0, s, x, numel, partial, descale);
    else
      hipLaunchKernelGGL((amax_partial_kernel<2, true>), dim3(1), dim3(kQThreads), 0, s, x, numel, partial, descale);
  } else {
    if (x_dtype == 0)
      hipLaunchKernelGGL((amax_partial_kernel<0, false>), dim3(blocks), dim3(kQThreads), 0, s, x, numel, partial,
                         descale);
    else
      hipLaunchKernelGGL((amax_partial_kernel<2, false>), dim3(blocks), dim3(kQThreads), 0, s, x, numel, partial,
                         descale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(kQThreads), 0, s, partial, blocks, descale);
  }
  hipError_t e = hipGetLastError();
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
