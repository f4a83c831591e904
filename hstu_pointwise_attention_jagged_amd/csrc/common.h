// Internal helpers shared by the gfx950 kernels of libhstu (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32], fp32 accumulate.
// Operand lane layout (64 lanes): lane l holds A row (l % 32), k = 8*(l/32) .. +8, and
// B column (l % 32), k = 8*(l/32) .. +8.  D: lane l holds column (l % 32) and rows
// 8*(i/4) + 4*(l/32) + (i%4) for its 16 values i.
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same operand layout with fp16 inputs (v_mfma_f32_32x32x16_f16, same rate as bf16).
__device__ __forceinline__ f32x16 mfma32_f16(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f16x8 as_f16x8(const u32x4 &v) {
  return __builtin_bit_cast(f16x8, v);
}

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
// ds_read_b64_tr_b16, gfx950's transposing 8-byte LDS read: in each group of 16 lanes,
// lane 4 j + q gives the address of 4 consecutive 16-bit values (columns 4 q .. 4 q + 3
// of row j of a 4 x 16 block) and lane i receives column i, rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char *p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Two fp32 -> packed fp16 (round to nearest even; v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// As pack_f16, saturating to the finite fp16 range first (no infinities).
__device__ __forceinline__ uint32_t pack_f16_sat(float lo, float hi) {
  return pack_f16(__builtin_amdgcn_fmed3f(lo, -65504.0f, 65504.0f),
                  __builtin_amdgcn_fmed3f(hi, -65504.0f, 65504.0f));
}

__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(f16x2, v)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(f16x2, v)[1];
}

// SiLU(x) = x / (1 + 2^(-x log2 e)).  For x << 0 the power overflows to +inf and the
// reciprocal gives 0, so the result is a signed zero, never NaN.
__device__ __forceinline__ float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// floor(log2(1 + dt)) for the non-negative time gap dt = ts_q - ts_k taken over the full
// int32 range (0 when ts_q <= ts_k).  Integer only: the bit length of (1 + dt) minus 1.
__device__ __forceinline__ int time_log2_bucket(int32_t ts_q, int32_t ts_k) {
  const uint32_t dt = ts_q > ts_k ? (uint32_t)ts_q - (uint32_t)ts_k : 0u;
  const uint32_t x = dt + 1u;  // wraps to 0 only for dt = 2^32 - 1, whose log2 is 32
  return x == 0u ? 32 : 31 - (int)__builtin_clz(x);
}

}  // namespace hstu
