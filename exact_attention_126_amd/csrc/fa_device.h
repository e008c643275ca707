// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware transcendental unit (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32), x > 0 normal.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t b = __float_as_uint(x);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> packed bf16 pair (low half = a), round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// x rounded to bf16 (the same conversion as pack_bf16x2, round to nearest even) and widened back.
__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

// max(a, b, c): lowers to one v_maximum3_f32.  Unlike fmaxf (which first quiets each input the
// compiler cannot prove canonical, such as MFMA results, with an extra instruction) it needs no
// canonicalisation; it propagates NaN, and scores are never NaN here.  Being visible to the
// compiler, it also gets the wait states a VALU read of a fresh MFMA result requires.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Max of a value across the two 32-lane halves of a wave (lane l and lane l ^ 32).
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte LDS accesses.
__device__ __forceinline__ u32x4_t lds_load16(const FA_LDS char* p) { return *(const FA_LDS u32x4_t*)p; }
__device__ __forceinline__ void lds_store16(FA_LDS char* p, u32x4_t v) { *(FA_LDS u32x4_t*)p = v; }

// Debug aid, off by default: built with FA_DEBUG_POISON_LDS=1, the waves that refill a slot of an
// LDS tile ring first overwrite their share of it with NaN, after the barrier that retires the
// slot and before their tile loads are issued.  With the barriers right no wave ever reads the
// NaN (the loads overwrite it first), so such a build gives bit for bit the outputs of the normal
// one; a missing or misplaced barrier would let a wave read the poison and turn its rows of O
// into NaN.
#ifndef FA_DEBUG_POISON_LDS
#define FA_DEBUG_POISON_LDS 0
#endif
constexpr uint32_t kPoisonBf16 = 0x7FC07FC0u;  // two bf16 NaNs
constexpr uint32_t kPoisonF32 = 0x7FC00000u;   // fp32 NaN
constexpr uint32_t kPoisonE4M3 = 0x7F7F7F7Fu;  // four OCP E4M3 NaNs
__device__ __forceinline__ void poison16(FA_LDS char* p, uint32_t w) { lds_store16(p, u32x4_t{w, w, w, w}); }
// waits for this wave's poison stores, so that they land before the tile loads that follow
__device__ __forceinline__ void poison_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte rows addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ i16x4_t lds_load8_tr16(const FA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p);
}

__device__ __forceinline__ u32x4_t gload16(const void* p) { return *(const u32x4_t*)p; }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef __attribute__((address_space(3))) void* lptr_t;

// Raw buffer resource over the bytes [base, base + bytes).  Word 3 selects the 32-bit data format:
// untyped buffer accesses need a non-zero format on this architecture.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time loop).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace fa
