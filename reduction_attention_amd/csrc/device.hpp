// device.hpp -- gfx950 building blocks shared by the attention kernels:
// element types, 128-bit vectors, MFMA wrappers, cross-lane reductions.
//
// MFMA operand convention used throughout.  For v_mfma_f32_32x32x16_{bf16,f16}
// lane l supplies row (l % 32) of A and column (l % 32) of B, and eight
// consecutive reduction "slots" selected by its half (l / 32) and register
// position.  A and B use the same slot numbering, so any assignment of the
// reduction index to (half, position) gives the right contraction provided
// both operands follow it; the kernels pick assignments that make their
// memory reads contiguous.  The 32x32 accumulator gives lane l column
// (l % 32) and rows 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
// For v_mfma_f32_16x16x32_* lane l supplies row/column (l % 16), slots by
// (l / 16) and position; the 16x16 accumulator gives lane l column (l % 16)
// and rows 4*(l/16) + r, r = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element traits: the storage type, its 8-wide MFMA operand vector,
// the MFMA builtins and the fp32 -> 16-bit conversion (round to nearest even).
struct BF16 {
  typedef __bf16 elem;
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec8 cvt8(f32x8 x) { return __builtin_convertvector(x, vec8); }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return __uint_as_float(uint32_t(bits) << 16);
  }
};

struct F16 {
  typedef _Float16 elem;
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec8 cvt8(f32x8 x) { return __builtin_convertvector(x, vec8); }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, bits);
    return float(h);
  }
};

template <class V>
__device__ __forceinline__ V as(u32x4 x) { return __builtin_bit_cast(V, x); }

// 128-bit global load / store through the vector memory path.
__device__ __forceinline__ u32x4 ldg128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void stg128(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }
// Non-temporal (streaming) loads for data read exactly once, such as the K/V
// of a decode step: on MI355X a stream of these sustains about 7 TB/s where
// plain loads level off near 6.
__device__ __forceinline__ u32x4 ldg128_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ldg64_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Buffer resource over [base, base + bytes): a 16-byte buffer load at byte
// offset voff (a VGPR) returns zeros, and touches no memory, when voff lies
// at or beyond bytes.  Word 3 holds the gfx9 raw-buffer format bits (32-bit
// data, no swizzle, stride 0).  Only the VGPR offset enters the range check,
// so callers put every row-dependent offset there and pass no scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7fffffff;
  const int n = int(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load128(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Pick 16-bit halves: lo16(a) | lo16(b) << 16, and hi16(a) | hi16(b) << 16.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// x from lane (lane ^ 32): one LDS permute with a lane address computed once
// by the caller (addr = (lane ^ 32) * 4), instead of __shfl_xor's per-call
// index arithmetic.
__device__ __forceinline__ float swap_halves(float x, int addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x)));
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// x combined with its partner lane l ^ 32, in every lane, through the
// cross-half lane swap (a VALU op, no LDS round trip): swapping the upper
// half of one copy of x with the lower half of another leaves, in each
// lane, x of both partners.
__device__ __forceinline__ float max_halves(float x) {
  const int b = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const int b = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

}  // namespace rattn
