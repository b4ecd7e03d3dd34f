// Device-side helpers shared by the gfx950 kernels of libpa: element types,
// raw buffer loads, DPP cross-lane reductions and the base-2 exponential.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(2))) float float2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type tags.  kBytes is the storage size; a 16-byte lane load holds
// 16 / kBytes elements.
struct F16 { static constexpr int kBytes = 2; };
struct BF16 { static constexpr int kBytes = 2; };
struct FP8 { static constexpr int kBytes = 1; };

// ---------------------------------------------------------------------------
// Raw buffer loads.  The descriptor base is the (uniform) tile address; a
// descriptor with num_records = 0 turns every lane's load into a zero fill
// with no memory access, which keeps prefetch loads unconditional at the end
// of a range.  Word 3 = 0x00020000 is the raw-buffer format for gfx9-family
// parts (32-bit data format, no swizzle).

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy of loads of data that a launch reads once (the K/V tiles of
// the decode kernels): non-temporal, the `nt` bit (bit 1 of the policy
// operand on this target).  With the default policy the Llama-7B-shaped
// decode streams ~10% slower.
constexpr int kStreamOnce = 2;

__device__ __forceinline__ u32x4_t stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kStreamOnce));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}

// ---------------------------------------------------------------------------
// DPP lane permutes (within 16-lane rows).

constexpr int dpp_quad(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kDppRowRor = 0x120;       // + n, n in 1..15
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {1, 2, 4, 8, 16}); every lane of
// the group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N == 16) {
    x += dpp<kDppRowRor + 8>(x);
    x += dpp<kDppRowRor + 4>(x);
    x += dpp<kDppRowRor + 2>(x);
    x += dpp<kDppRowRor + 1>(x);
  } else if constexpr (N == 8) {
    x += dpp<kDppRowHalfMirror>(x);
    x += dpp<dpp_quad(3, 2, 1, 0)>(x);
    x += dpp<dpp_quad(1, 0, 3, 2)>(x);
  } else if constexpr (N == 4) {
    x += dpp<dpp_quad(2, 3, 0, 1)>(x);
    x += dpp<dpp_quad(1, 0, 3, 2)>(x);
  } else if constexpr (N == 2) {
    x += dpp<dpp_quad(1, 0, 3, 2)>(x);
  }
  return x;
}

// ---------------------------------------------------------------------------
// Reductions across lanes further apart than a quad.  Default build: the
// exchanges go through ds_bpermute (__shfl_xor), an LDS-unit instruction.
// PA_XLANE_DPP=1 builds them from DPP row operations and gfx950's
// v_permlane16_swap / v_permlane32_swap (no LDS instruction); bench.py can
// load that build to compare the two.

#ifndef PA_XLANE_DPP
#define PA_XLANE_DPP 0
#endif

#if PA_XLANE_DPP
// The values of lanes l and l ^ O (O = 16 or 32), in both lanes of the pair:
// v_permlane{16,32}_swap exchanges the odd 16- (32-) lane rows of its first
// register with the even rows of its second, so with x in both, the first
// ends up holding the even rows' values and the second the odd rows'.  Both
// registers are written; written as inline assembly because this compiler's
// builtin returns the first register twice (a lane-layout probe on the GPU
// showed it).  The compiler does not insert the wait states around inline
// assembly that it inserts around its own permlane instructions, so the
// s_nops provide them on both sides.
template <int O>
__device__ __forceinline__ float2_t pair_values(float x) {
  static_assert(O == 16 || O == 32, "distance");
  int a = __builtin_bit_cast(int, x), b = a;
  if constexpr (O == 32)
    asm("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
  else
    asm("s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
  return float2_t{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}
#endif

// x + (x of lane l ^ O), O in {4, 8, 16, 32}, the same in both lanes of the
// pair.  (For O = 4 the DPP build adds lane (l + 4) mod 16 instead, which
// gives the same totals once O = 8 follows.)
template <int O>
__device__ __forceinline__ float xor_add(float x) {
#if PA_XLANE_DPP
  if constexpr (O == 4 || O == 8) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), 0x120 + O, 0xF, 0xF,
                                             false));
  } else {
    const float2_t v = pair_values<O>(x);
    return v[0] + v[1];
  }
#else
  return x + __shfl_xor(x, O, kWave);
#endif
}

// max(x, x of lane l ^ O), O in {16, 32}.
template <int O>
__device__ __forceinline__ float xor_max(float x) {
#if PA_XLANE_DPP
  const float2_t v = pair_values<O>(x);
  return fmaxf(v[0], v[1]);
#else
  return fmaxf(x, __shfl_xor(x, O, kWave));
#endif
}

// Maximum over the whole wavefront, in every lane.
__device__ __forceinline__ float wave_max(float x) {
#if PA_XLANE_DPP
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
  return xor_max<32>(xor_max<16>(x));
#else
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
#endif
}

// Sum over the lanes that share lane % O (O in {4, 8, 16, 32, 64}; 64: x).
template <int O>
__device__ __forceinline__ float sum_lanes_mod(float x) {
  static_assert(O >= 4, "distance");
  if constexpr (O >= kWave) return x;
  else return sum_lanes_mod<2 * O>(xor_add<O>(x));
}

// Value of lane (lane ^ M) for M in {1, 2} (quad permutes).
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  static_assert(M == 1 || M == 2, "xor distance");
  if constexpr (M == 1) return dpp<dpp_quad(1, 0, 3, 2)>(x);
  else return dpp<dpp_quad(2, 3, 0, 1)>(x);
}

// ---------------------------------------------------------------------------
// Arithmetic helpers.

// Reinterpret one 32-bit word as a pair of 16-bit floats.  The word is taken
// as a scalar parameter: bit-casting an ext-vector element expression
// (v[i]) in place does not select element i with this compiler.
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ bf162_t as_bf162(uint32_t w) { return __builtin_bit_cast(bf162_t, w); }

// 2^x with the hardware transcendental (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w)[1];
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// Two e4m3fn codes (bytes 0,1 or 2,3 of w) -> two floats, with the gfx950
// conversion instruction (OCP e4m3fn on this target).
template <bool HI>
__device__ __forceinline__ float2_t fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// Round-to-nearest-even float -> 16-bit storage.
__device__ __forceinline__ uint16_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);   // v_cvt_pk_bf16_f32 on gfx950
}

// fp32 -> OCP e4m3fn code: clamp to +-448 (saturating, also +-inf), round to
// nearest even, NaN stays NaN; integer operations from the format definition
// (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9,
// S.1111.111 = NaN, largest finite 1.75 * 2^8).
__device__ __forceinline__ uint32_t e4m3fn_encode(float y) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, y) >> 24) & 0x80u;
  const float a = __builtin_fminf(__builtin_fabsf(y), 448.0f);   // saturate (also +-inf)
  const uint32_t ua = __builtin_bit_cast(uint32_t, a);
  // normal range: keep 3 mantissa bits, round half to even (the carry may
  // bump the exponent); exponent field = unbiased exponent + 7
  const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
  const uint32_t normal = ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u)) & 0x7Fu;
  // below 2^-6: quantum 2^-9, rint rounds half to even (8 = 2^-6)
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t code = ua < 0x3C800000u ? sub : normal;       // 0x3C800000 = 2^-6
  return y != y ? (sign | 0x7Fu) : (sign | code);
}

template <typename T>
__device__ __forceinline__ uint16_t to_bits16(float x);
template <>
__device__ __forceinline__ uint16_t to_bits16<F16>(float x) { return to_f16_bits(x); }
template <>
__device__ __forceinline__ uint16_t to_bits16<BF16>(float x) { return to_bf16_bits(x); }

}  // namespace pa
