// Matrix-core helpers shared by the decode and prefill kernels (gfx950
// v_mfma_f32_16x16x32 / 16x16x16 in f16 and bf16).
#pragma once

#include "pa_device.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 half4_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8v_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

constexpr float kMfmaNegInf = -__builtin_huge_valf();

// 16-bit operand type of the matrix products
template <typename QT>
struct Mma;

template <>
struct Mma<F16> {
  static __device__ __forceinline__ float4_t qk(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float4_t pv(u32x2_t a, u32x2_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
  }
  // two floats -> packed 16-bit pair (round to nearest even)
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return (uint32_t)to_f16_bits(lo) | ((uint32_t)to_f16_bits(hi) << 16);
  }
  // the same as one v_cvt_pk_f16_f32
  static __device__ __forceinline__ uint32_t pack_pk(float lo, float hi) {
    const half2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static constexpr uint32_t kOne2 = 0x3C003C00u;   // packed pair of 1.0
  // acc + the two 16-bit values of w (exact products, one fp32 sum)
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(as_half2(w), one, acc, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
  // e4m3fn bytes 0,1 (HI: 2,3) of w -> packed f16 pair (exact; scale 1)
  template <bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
};

template <>
struct Mma<BF16> {
  static __device__ __forceinline__ float4_t qk(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v_t, a),
                                                   __builtin_bit_cast(bf16x8v_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float4_t pv(u32x2_t a, u32x2_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf162_t r;
    r[0] = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ uint32_t pack_pk(float lo, float hi) { return pack(lo, hi); }
  static constexpr uint32_t kOne2 = 0x3F803F80u;   // packed pair of 1.0
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    const bf162_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf162(w), one, acc, false);
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
};

// Head dim of element e (0..7) of k-chunk c for lane group g in the QK
// product; 16-bit caches read 16 contiguous bytes per chunk, fp8 caches read
// 16 bytes (16 dims) that serve two consecutive chunks.
template <int ESZ>
__device__ __forceinline__ int qk_dim(int c, int g) {
  if constexpr (ESZ == 2) return 32 * c + 8 * g;
  else return 64 * (c >> 1) + 16 * g + 8 * (c & 1);
}

}  // namespace pa
