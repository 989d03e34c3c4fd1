// Device-side helpers shared by the gfx950 kernels: vector types, buffer
// resources (range-checked loads that return zero past the end), LDS access
// and the few CDNA4 builtins the kernels use.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace zyfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

// Word 3 of a gfx9-family buffer resource: 32-bit data format, raw access.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, kBufferWord3);
}

// Extent of a resource based at some row of a slice: `rows` rows of
// `stride` bytes are readable from it (rows <= 0: none), the last one
// holding `row_bytes`. Reads of later rows fall outside and return zero,
// which is how rows past seqlen read as zero padding. The kernels place a
// resource at every wave's query rows and at every half key tile (a 64-bit
// base), so rows * stride stays below 2^31 even when a tensor or a slice
// spans more than 4 GiB.
__device__ __forceinline__ unsigned rows_extent(int rows, int stride, int row_bytes) {
  return rows > 0 ? (unsigned)((rows - 1) * stride + row_bytes) : 0u;
}

// 16-byte load at a byte offset; returns zeros when the offset is past the
// resource's extent (this is how rows past seqlen read as zero padding).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 8-byte load at a byte offset; zeros past the resource's extent.
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// Raw buffer resource as four scalar words (for inline assembly operands).
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, unsigned nbytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a & 0xFFFFFFFFull));
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = kBufferWord3;
  return r;
}

// Direct global-to-LDS load issued as inline assembly, so the compiler does
// not track it: otherwise it waits for every such load before any later LDS
// read (it cannot tell which ring slot a read touches), which would expose
// the full memory latency once per key tile. The caller orders these loads
// with wait_vm() and barriers itself. Lane L's 16 bytes go to
// lds_wave_base + 16 L (M0 holds the wave-uniform base); past the resource's
// extent they are zero.
// lds_wave_base is an LDS byte address (see lds_addr), kept in 32 bits: a
// generic pointer would be converted, null check included, at every load.
__device__ __forceinline__ void dma16(const i32x4& rsrc, int voff, unsigned lds_wave_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array (taken once per
// kernel from the array itself, whose address the compiler knows).
__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// s_waitcnt vmcnt(N) leaving the LDS and export counters alone (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <class T>
__device__ __forceinline__ T lds_load(const char* p) {
  return *reinterpret_cast<const T*>(p);
}

// ds_read_b64_tr_b16: within each 16-lane group, the lanes' 8-byte reads
// form a 4 x 16 block of 16-bit values (row r from lanes 4r..4r+3); lane i
// receives column i, rows 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const_cast<char*>(p)));
}

// ds_read_b64_tr_b8: within each 16-lane group, the lanes' 8-byte reads
// form an 8 x 16 block of bytes (row r from lanes 2r, 2r+1); lane i receives
// column i, rows 0..7.
__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(const_cast<char*>(p)));
}

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, low
// half first (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Bit casts of scalars passed by value (a bit cast applied directly to an
// element of an ext_vector has been compiled as a cast of element 0).
__device__ __forceinline__ float as_f32(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned as_u32(float f) { return __builtin_bit_cast(unsigned, f); }

// x of lane l ^ 16 (ds_swizzle in bit-mask mode, xor mask 16): runs on the
// LDS unit without touching memory, so it takes no vector-ALU issue slot.
__device__ __forceinline__ float swap16(float x) {
  return as_f32((unsigned)__builtin_amdgcn_ds_swizzle((int)as_u32(x), 0x401F));
}

// v_permlane16_swap_b32 with both operands x: the first result holds rows
// (16-lane groups) 0, 0, 2, 2 of x and the second rows 1, 1, 3, 3, so their
// maximum is max(x[l], x[l ^ 16]) in every lane l.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(as_f32(a), as_f32(b));
}

// v_permlane32_swap_b32 with both operands x: max(x[l], x[l ^ 32]).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(as_f32(a), as_f32(b));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// x = -inf where key offset ko > q (the causal mask). One compare into VCC
// and one select per score; written as assembly so that the compiler does
// not compute all compares first into scalar register pairs (which it then
// spills).
__device__ __forceinline__ float mask_above(float x, int ko, int q, float ninf) {
  asm volatile("v_cmp_gt_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
               : "+v"(x)
               : "s"(ko), "v"(q), "v"(ninf)
               : "vcc");
  return x;
}

// sched_group_barrier instruction classes.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedValu = 0x002;

}  // namespace zyfa
