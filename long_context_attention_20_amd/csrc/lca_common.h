// Internal helpers shared by the gfx950 kernels of liblca.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "lca.h"

namespace lca {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
// Every 64-byte line of the kernel's argument block (its first BYTES bytes)
// requested at once at the kernel's start: the argument reads that follow
// then hit the scalar cache, where the compiler would otherwise request the
// lines one dependent wait at a time, each a memory round trip.
template <int BYTES>
__device__ __forceinline__ void warm_kernargs() {
  const __attribute__((address_space(4))) uint32_t* kp =
      (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t x = 0;
#pragma unroll
  for (int o = 0; o < BYTES; o += 64) x ^= kp[o / 4];
  asm volatile("" : : "s"(x));
}

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

// ---------------------------------------------------------------- rotary embedding
// "DeepSeek-V4" spec sheet, Core block and Provenance 16: partial RoPE on the
// last dims of a head.  The last `dims` channels of a C-channel vector turn
// pair by pair, pair p (channels C - dims + 2p and the next) as a complex
// number times exp(i pos theta_p), theta_p = base^(-2p / dims).
//
// theta_p is the product of t2k[k] = base^(-2 * 2^k / dims) over the set bits
// k of p (at most 8 double products, so a few ulp of a double), the angle
// pos * theta_p is formed and reduced to revolutions in double (positions
// reach 2^20, where a float product would lose most of the angle), and the
// sine and cosine of the reduced angle come from Taylor polynomials on a
// quarter turn (degree 9 and 8: truncation below 3e-8 on |r| <= pi/4), moved
// to the right quadrant by the usual identities.
struct RopeTab {
  int dims;        // rotated channels (0: none)
  double t2k[8];   // base^(-2 * 2^k / dims)
};

inline RopeTab make_rope_tab(int dims, float base) {
  RopeTab t{};
  t.dims = dims;
  for (int k = 0; k < 8; ++k) t.t2k[k] = dims > 0 ? std::pow((double)base, -2.0 * (double)(1 << k) / dims) : 0.0;
  return t;
}

// theta_p of a table (a product of its powers, double precision).
__device__ __forceinline__ double rope_theta(int p, const RopeTab& t) {
  double theta = 1.0;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if ((p >> k) & 1) theta *= t.t2k[k];
  return theta;
}

// Sine and cosine of an angle given in quarter turns f, |f| <= 2.
__device__ __forceinline__ void sincos_quarters(float f, float* sn, float* cs) {
  const float q = rintf(f);
  const float r = (f - q) * 1.57079632679489661923f;  // [-pi/4, pi/4]
  const float r2 = r * r;
  const float s = r * (1.f + r2 * (-1.f / 6 + r2 * (1.f / 120 + r2 * (-1.f / 5040 + r2 * (1.f / 362880)))));
  const float c = 1.f + r2 * (-0.5f + r2 * (1.f / 24 + r2 * (-1.f / 720 + r2 * (1.f / 40320))));
  const int qi = (int)q & 3;                          // angle = qi quarter turns + r
  *sn = qi == 0 ? s : qi == 1 ? c : qi == 2 ? -s : -c;
  *cs = qi == 0 ? c : qi == 1 ? -s : qi == 2 ? -c : s;
}

constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

__device__ __forceinline__ void rope_sincos(double pos, int p, const RopeTab& t, float* sn, float* cs) {
  double rev = pos * rope_theta(p, t) * kInvTwoPi;
  rev -= rint(rev);                                   // [-1/2, 1/2] of a turn
  sincos_quarters((float)(rev * 4.0), sn, cs);        // quarter turns, [-2, 2]
}

// Channels [ch0, ch0 + N) of a C-channel vector turned by the angles of
// position base + off, where base's angles are given (rot[p]: cosine and
// sine of base * theta_p) and off is small (a few thousand at most): the
// offset's angle off * theta_p is formed in float (turns[p] = theta_p / 2 pi)
// and the two rotations are composed.
template <int N>
__device__ __forceinline__ void rope_turn_near(float (&v)[N], int ch0, int C, int dims, const float2* rot,
                                               const float* turns, float off) {
  static_assert(N % 2 == 0, "pairs");
  const int lo = C - dims;
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const int c = ch0 + k;
    if (dims > 0 && c >= lo) {
      const int p = (c - lo) >> 1;
      float rev = off * turns[p];
      rev -= rintf(rev);
      float s1, c1;
      sincos_quarters(rev * 4.f, &s1, &c1);
      const float2 b = rot[p];
      const float cs = b.x * c1 - b.y * s1, sn = b.y * c1 + b.x * s1;
      const float x0 = v[k], x1 = v[k + 1];
      v[k] = x0 * cs - x1 * sn;
      v[k + 1] = x0 * sn + x1 * cs;
    }
  }
}

// Channels [ch0, ch0 + N) of a C-channel vector (ch0 and N even), turned by
// the angles of position pos.
template <int N>
__device__ __forceinline__ void rope_turn(float (&v)[N], int ch0, int C, const RopeTab& t, double pos) {
  static_assert(N % 2 == 0, "pairs");
  const int lo = C - t.dims;
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const int c = ch0 + k;
    if (t.dims > 0 && c >= lo) {
      float sn, cs;
      rope_sincos(pos, (c - lo) >> 1, t, &sn, &cs);
      const float x0 = v[k], x1 = v[k + 1];
      v[k] = x0 * cs - x1 * sn;
      v[k + 1] = x0 * sn + x1 * cs;
    }
  }
}

// Channels [ch0, ch0 + N) of a C-channel vector (ch0 and N even) turned by
// the angles of a table (tab[p]: cosine and sine of the angle of pair p, as
// rope_sincos gives them), or by minus those angles (back: the sine negated,
// which is rope_sincos of the negated position exactly, its reduction being
// odd in the position).
template <int N>
__device__ __forceinline__ void rope_turn_tab(float (&v)[N], int ch0, int C, int dims, const float2* tab, bool back) {
  static_assert(N % 2 == 0, "pairs");
  const int lo = C - dims;
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const int c = ch0 + k;
    if (dims > 0 && c >= lo) {
      const float2 t = tab[(c - lo) >> 1];
      const float cs = t.x, sn = back ? -t.y : t.y;
      const float x0 = v[k], x1 = v[k + 1];
      v[k] = x0 * cs - x1 * sn;
      v[k + 1] = x0 * sn + x1 * cs;
    }
  }
}

// ---------------------------------------------------------------- ordering
// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 is folded into +0 so that the two zeros tie, as they compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- LDS ordering
// The lanes of one wave exchange data through LDS (each lane writes words that
// other lanes then update or read): the hardware keeps a wave's LDS
// operations in order, and the fence keeps the compiler from moving a lane's
// LDS access across this point or forwarding its own earlier store to a later
// load (which would miss the other lanes' writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A block barrier that orders LDS only: global loads in flight (a prefetch,
// loads straight into LDS) stay in flight, where __syncthreads would wait for
// every one of them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- launch status
// Implemented in lca_abi.hip: records a message for lca_last_error().
void set_error(const char* fmt, ...);

}  // namespace lca
