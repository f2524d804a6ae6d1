// Internal helpers shared by the gfx950 kernels of liblca.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lca.h"

namespace lca {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even: gfx950 converts a pair in one instruction
// (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// Element types: 16-byte vectors hold 8 bf16 or 4 f32.
struct BF16 {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]); v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]); v.w = pack_bf16x2(f[6], f[7]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ float round(float f) { return round_bf16(f); }
};

struct F32 {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    uint4 v;
    v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
    v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ float round(float f) { return f; }
};

__device__ __forceinline__ uint4 ldg16(const void* base, int64_t byte_off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ void stg16(void* base, int64_t byte_off, uint4 v) {
  *reinterpret_cast<uint4*>(reinterpret_cast<char*>(base) + byte_off) = v;
}

// ---------------------------------------------------------------- reductions
// Butterfly over `width` lanes (a power of two <= 64) of one wavefront.
__device__ __forceinline__ float wave_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f32(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Sum over aligned groups of N consecutive lanes (N = 4 .. 64); every lane of
// a group gets the same total.  Quad permutes, the half-row and row mirrors
// (DPP, no LDS traffic), then lane reads across 16-lane rows.  Every lane of
// the wave must be active.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group of 4 to 64 lanes");
  v += dpp_f32<0xB1>(v);                          // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);                          // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if constexpr (N >= 16) v += dpp_f32<0x140>(v);  // row_mirror
  if constexpr (N == 32) {
    const float lo = readlane_f32(v, 0) + readlane_f32(v, 16);
    const float hi = readlane_f32(v, 32) + readlane_f32(v, 48);
    v = (threadIdx.x & 32) ? hi : lo;
  } else if constexpr (N == 64) {
    v = (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps with
// DPP row shifts inside each 16-lane row, then the row broadcasts of lanes 15
// and 31 into the rows above them.  Every lane of the wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111, 0xF>(x);  // row_shr:1
  x += dpp_u32<0x112, 0xF>(x);  // row_shr:2
  x += dpp_u32<0x114, 0xF>(x);  // row_shr:4
  x += dpp_u32<0x118, 0xF>(x);  // row_shr:8
  x += dpp_u32<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_u32<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// ---------------------------------------------------------------- windows
// Complete windows of length w at stride m among the first L tokens.
__device__ __host__ __forceinline__ int64_t n_windows(int64_t L, int m, int w) {
  return L < w ? 0 : (L - w) / m + 1;
}

// ---------------------------------------------------------------- ordering
// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 is folded into +0 so that the two zeros tie, as they compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- launch status
// Implemented in lca_abi.cpp: records a message for lca_last_error().
void set_error(const char* fmt, ...);

}  // namespace lca
