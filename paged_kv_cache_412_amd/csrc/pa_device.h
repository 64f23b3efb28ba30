// pa_device.h -- device-side helpers for the gfx950 kernels of libpa:
// element types, 16-byte chunk loads and conversions, wave64 DPP reductions
// and the OCP e4m3 codec.
//
// Written for CDNA4 (gfx950, wave64).  No code here is shared with the CPU
// oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// One 16-byte chunk of a K or V row: the unit every lane loads.
struct alignas(16) Chunk {
  uint32_t w[4];
};

__device__ __forceinline__ Chunk load_chunk(const void* p) {
  // global_load_dwordx4; the pools are read once per decode step, so the
  // loads are marked non-temporal to keep L2/MALL for the block tables and q.
  const uint32_t __attribute__((ext_vector_type(4)))* vp =
      reinterpret_cast<const uint32_t __attribute__((ext_vector_type(4)))*>(p);
  auto v = __builtin_nontemporal_load(vp);
  Chunk c;
  c.w[0] = v[0];
  c.w[1] = v[1];
  c.w[2] = v[2];
  c.w[3] = v[3];
  return c;
}

// ---------------------------------------------------------------- buffer loads

// Buffer resource (V#) over `bytes` bytes at `base`: raw buffer loads through
// it return zeros, without touching memory, for offsets at or past `bytes`.
// A resource with bytes = 0 therefore turns every load of a block that must
// not be read into a no-op, so the loop can issue the same loads on every path.
// Dword 3 (0x00020000: 32-bit data format) is the raw-buffer setting for gfx9
// parts, gfx950 included.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// A pointer that is the same in every lane, made provably so (v_readfirstlane
// of both halves; free when it already sits in scalar registers).  Buffer
// resources need one: built from a value the compiler takes as per-lane,
// every buffer access becomes a loop over the distinct resources.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Cache-policy bits of a buffer load: non-temporal (the pools are read once
// per decode step; L2 and the MALL are left to the block tables and queries).
constexpr int kLoadNT = 2;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// N dwords (1, 2 or 4) at byte voff + soff + IMM of the resource.
template <int N, int IMM = 0>
__device__ __forceinline__ void buffer_load(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                            uint32_t* out) {
  if constexpr (N == 4) {
    const u32x4_t v = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff + IMM, soff, kLoadNT));
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
    out[3] = v[3];
  } else if constexpr (N == 2) {
    const u32x2_t v = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff + IMM, soff, kLoadNT));
    out[0] = v[0];
    out[1] = v[1];
  } else {
    out[0] = __builtin_bit_cast(uint32_t,
                                __builtin_amdgcn_raw_buffer_load_b32(r, voff + IMM, soff, kLoadNT));
  }
}

// N dwords (1, 2 or 4) at byte IMM of a per-lane address (non-temporal, as
// the buffer loads).  For reads whose rows lie in different blocks per lane.
template <int N, int IMM = 0>
__device__ __forceinline__ void global_load(const char* p, uint32_t* out) {
  if constexpr (N == 4) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + IMM));
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
    out[3] = v[3];
  } else if constexpr (N == 2) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p + IMM));
    out[0] = v[0];
    out[1] = v[1];
  } else {
    out[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + IMM));
  }
}

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------- dtype traits

template <int DT>
struct Elem;
template <>
struct Elem<PA_F32> {
  static constexpr int bytes = 4;
};
template <>
struct Elem<PA_F16> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<PA_BF16> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<PA_FP8_E4M3> {
  static constexpr int bytes = 1;
};
template <>
struct Elem<PA_FP8_E5M2> {
  static constexpr int bytes = 1;
};

// Whether a cache dtype is one of the 8-bit formats.
constexpr bool is_fp8(int dt) { return dt == PA_FP8_E4M3 || dt == PA_FP8_E5M2; }

// Scalar element of a 16-bit or 32-bit type -> fp32 (exact).
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t i);
template <>
__device__ __forceinline__ float load_elem<PA_F32>(const void* base, size_t i) {
  return static_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float load_elem<PA_F16>(const void* base, size_t i) {
  return static_cast<float>(static_cast<const _Float16*>(base)[i]);
}
template <>
__device__ __forceinline__ float load_elem<PA_BF16>(const void* base, size_t i) {
  return u2f(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Store one output element; out_dtype is F32, F16 or BF16.
__device__ __forceinline__ void store_out(void* base, size_t i, float v, int out_dtype) {
  if (out_dtype == PA_F32) {
    static_cast<float*>(base)[i] = v;
  } else if (out_dtype == PA_F16) {
    static_cast<_Float16*>(base)[i] = static_cast<_Float16>(v);  // v_cvt_f16_f32, RNE
  } else {
    static_cast<uint16_t*>(base)[i] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------- e4m3 codec

// Decode four e4m3 codes packed in a 32-bit word to fp32 with the gfx950
// conversion instruction (OCP e4m3: bias 7, S.1111.111 = NaN, max 448).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* out) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Encode fp32 -> e4m3 code: round to nearest even, magnitudes that round
// beyond 448 (and +-inf) saturate to +-448, NaN -> 0x7F with the NaN's sign.
// Integer arithmetic on the fp32 fields, written from the format definition:
//   |y| <  2^-6 : subnormal binade, code = rint(|y| * 2^9)   (0..8; 8 is 2^-6)
//   |y| >= 2^-6 : y = (1.f) * 2^e, keep 3 fraction bits, round the 20
//                 dropped bits half to even; a carry moves into the exponent.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float y) {
  const uint32_t u = f2u(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return sign | 0x7fu;                 // NaN
  if (ua >= 0x43e80000u) return sign | 0x7eu;               // |y| >= 464 (incl. inf)
  if (ua < 0x3c800000u) {                                    // |y| < 2^-6
    const float m = __builtin_rintf(u2f(ua) * 512.0f);       // exact scale, RNE
    return sign | static_cast<uint32_t>(m);
  }
  const uint32_t e = (ua >> 23) - 127u + 7u;                 // biased e4m3 exponent, 1..8+7
  const uint32_t frac = ua & 0x7fffffu;
  const uint32_t keep = frac >> 20;
  const uint32_t rest = frac & 0xfffffu;
  const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  uint32_t code = ((e << 3) | keep) + up;
  if (code > 0x7eu) code = 0x7eu;                            // [448, 464) rounds into 0x7E
  return sign | code;
}

// ---------------------------------------------------------------- e5m2 codec

// Decode four e5m2 codes to fp32 (gfx950 bf8 conversion; OCP e5m2: bias 15,
// IEEE-style inf/NaN, max 57344).
__device__ __forceinline__ void e5m2x4_to_f32(uint32_t w, float* out) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Encode fp32 -> e5m2 code: round to nearest even, magnitudes that round
// beyond 57344 (and +-inf) saturate to +-57344, NaN -> 0x7F with the NaN's
// sign.  Integer arithmetic on the fp32 fields, from the format definition:
//   |y| <  2^-14 : subnormal binade, code = rint(|y| * 2^16)  (0..4; 4 is 2^-14)
//   |y| >= 2^-14 : keep 2 fraction bits, round the 21 dropped bits half to
//                  even; a carry moves into the exponent.
__device__ __forceinline__ uint32_t f32_to_e5m2_rne_sat(float y) {
  const uint32_t u = f2u(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return sign | 0x7fu;                 // NaN
  if (ua >= 0x47600000u) return sign | 0x7bu;               // |y| >= 57344 (incl. inf)
  if (ua < 0x38800000u) {                                    // |y| < 2^-14
    const float m = __builtin_rintf(u2f(ua) * 65536.0f);     // exact scale, RNE
    return sign | static_cast<uint32_t>(m);
  }
  const uint32_t e = (ua >> 23) - 127u + 15u;                // biased e5m2 exponent, 1..30
  const uint32_t frac = ua & 0x7fffffu;
  const uint32_t keep = frac >> 21;
  const uint32_t rest = frac & 0x1fffffu;
  const uint32_t up = (rest > 0x100000u) || (rest == 0x100000u && (keep & 1u));
  uint32_t code = ((e << 2) | keep) + up;
  if (code > 0x7bu) code = 0x7bu;
  return sign | code;
}

// 8-bit code of fp32 y in the cache format FMT (PA_FP8_E4M3 or PA_FP8_E5M2).
template <int FMT>
__device__ __forceinline__ uint32_t f32_to_fp8(float y) {
  if constexpr (FMT == PA_FP8_E5M2) return f32_to_e5m2_rne_sat(y);
  else return f32_to_e4m3_rne_sat(y);
}

// Four 8-bit codes of format FMT to fp32 (exact).
template <int FMT>
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  if constexpr (FMT == PA_FP8_E5M2) e5m2x4_to_f32(w, out);
  else e4m3x4_to_f32(w, out);
}

// ---------------------------------------------------------------- DPP reductions

// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm, row mirror, row half mirror.
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return u2f(static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(f2u(v)), CTRL, 0xF, 0xF, true)));
}

// Sum over aligned groups of N consecutive lanes (N = 1..64, a power of two);
// every lane of a group receives the group's sum.  Within rows of 16 lanes the
// exchange uses DPP; across rows it uses ds_swizzle-free bpermute shuffles.
// Additions pair lanes symmetrically, so all lanes of a group hold bitwise
// identical sums.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
  if constexpr (N >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
  if constexpr (N >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
