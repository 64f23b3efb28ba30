// pa_mfma.h -- matrix-core helpers shared by the decode and prefill kernels:
// 16x16 MFMA contractions in bf16 or f16, fp32 -> 16-bit packing and e4m3
// widening, all for gfx950 (wave64).
//
// Lane layout of a 16x16 MFMA (lane l, lo = l % 16, grp = l / 16):
//   A (16 x K): row lo, a run of K/4 values picked by (grp, element);
//   B (K x 16): column lo, the same (grp, element) -> k pairing as A;
//   D (16 x 16, four fp32 per lane): D[4*grp + r][lo] in element r.
// Only the pairing of A and B slots matters for a contraction, so a kernel
// may assign head-dim positions (or tokens) to (grp, element) slots freely as
// long as both operands use the same assignment.
#pragma once

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// MFMA operand type (the query dtype): contractions, packing of fp32 weights
// and widening of e4m3 codes.
template <int MT>
struct Mfma;

template <>
struct Mfma<PA_BF16> {
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16
  __device__ static f32x4 qk(const uint32_t* a, const uint32_t* b, f32x4 c) {
    const u32x4 av = {a[0], a[1], a[2], a[3]};
    const u32x4 bv = {b[0], b[1], b[2], b[3]};
    return mma32(av, bv, c);
  }
  // D += A B with K = 32: eight bf16 per lane and operand
  __device__ static f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
    const u32x2 av = {a0, a1};
    const u32x2 bv = {b0, b1};
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av),
                                                     __builtin_bit_cast(s16x4, bv), c, 0, 0, 0);
  }
  // two fp32 -> bf16 pair, round to nearest even
  __device__ static uint32_t pack2(float x, float y) {
    const bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
    return __builtin_bit_cast(uint32_t, v);
  }
  // sum of the two values of a packed bf16 pair (exact widening)
  __device__ static float pair_sum(uint32_t u) { return u2f(u << 16) + u2f(u & 0xffff0000u); }
  // four e4m3 codes -> two dwords of bf16 pairs (exact)
  __device__ static void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  // four e5m2 codes -> two dwords of bf16 pairs (exact)
  __device__ static void widen4_e5m2(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true));
  }
};

template <>
struct Mfma<PA_F16> {
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // (1.0, 1.0) in f16
  __device__ static f32x4 qk(const uint32_t* a, const uint32_t* b, f32x4 c) {
    const u32x4 av = {a[0], a[1], a[2], a[3]};
    const u32x4 bv = {b[0], b[1], b[2], b[3]};
    return mma32(av, bv, c);
  }
  // D += A B with K = 32: eight f16 per lane and operand
  __device__ static f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
    const u32x2 av = {a0, a1};
    const u32x2 bv = {b0, b1};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, av),
                                                 __builtin_bit_cast(f16x4, bv), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y) {
    const f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
    return __builtin_bit_cast(uint32_t, v);
  }
  // sum of the two values of a packed f16 pair (exact widening)
  __device__ static float pair_sum(uint32_t u) {
    const f16x2 h = __builtin_bit_cast(f16x2, u);
    return static_cast<float>(h[0]) + static_cast<float>(h[1]);
  }
  __device__ static void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  __device__ static void widen4_e5m2(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true));
  }
};

// Four 8-bit codes of cache format KV (e4m3 or e5m2) -> two dwords of pairs of
// the operand type Q (bf16 and f16 hold every value of both formats exactly).
template <int Q, int KV>
__device__ __forceinline__ void widen_fp8(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (KV == PA_FP8_E5M2) Mfma<Q>::widen4_e5m2(w, lo, hi);
  else Mfma<Q>::widen4(w, lo, hi);
}

// Half `sel` (0 = low, 1 = high) of dwords a and b, packed as (a_half, b_half).
__device__ __forceinline__ uint32_t pick_halves(uint32_t a, uint32_t b, int sel) {
  // one v_perm_b32: bytes 0-3 index the second operand (a), 4-7 the first (b)
  return __builtin_amdgcn_perm(b, a, sel ? 0x07060302u : 0x05040100u);
}

}  // namespace pa
