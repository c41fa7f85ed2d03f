// m3_device.h -- device-side helpers shared by the libm3ssm kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "m3_launch.h"

namespace m3 {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bh8 __attribute__((ext_vector_type(8)));
typedef __bf16 bh2 __attribute__((ext_vector_type(2)));

// bf16 travels as raw 16-bit patterns; fp32 as float.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}

// round-to-nearest-even fp32 -> bf16 (NaN stays NaN)
__device__ __forceinline__ bf16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t{static_cast<uint16_t>((u >> 16) | 0x40u)};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t{static_cast<uint16_t>(u >> 16)};
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return to_bf16(v); }

template <typename T>
__device__ __forceinline__ float ld1(const T* __restrict__ p, int64_t i) {
  return to_f32(p[i]);
}

// p[i] when p is set, else v; f4 likewise (i a multiple of 4).  Every lane
// reads a valid address (a sink when p is null) and the value is selected
// afterwards: no branch surrounds the read, so it need not wait there.  The
// sink is only read; it is not const so that it lives in global memory like
// p (a pointer that may be either stays a global one, not a generic one).
static __device__ __align__(16) float kReadSink[4];
typedef __attribute__((address_space(1))) const float gfloat;   // global memory
typedef __attribute__((address_space(1))) const f4 gf4;
__device__ __forceinline__ float ld_or(const float* p, int64_t i, float v) {
  const float r = *(const gfloat*)(p ? p + i : kReadSink);
  return p ? r : v;
}
__device__ __forceinline__ f4 ld4_or(const float* p, int64_t i, f4 v) {
  const f4 r = *(const gf4*)(p ? p + i : kReadSink);
  return p ? r : v;
}

// one element as loaded (a bf16 keeps its bit pattern), for a read issued
// early and turned into a float only where it is used: the conversion does
// not make the read wait at the place it is issued
template <typename T>
struct Raw1;
template <>
struct Raw1<float> {
  float v;
  __device__ __forceinline__ void load(const float* __restrict__ p, int64_t i) { v = p[i]; }
  __device__ __forceinline__ float f() const { return v; }
};
template <>
struct Raw1<bf16_t> {
  uint32_t u;
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p, int64_t i) { u = p[i].bits; }
  __device__ __forceinline__ float f() const { return __uint_as_float(u << 16); }
};

// K consecutive elements as loaded (bf16 keeps its bit patterns; the first
// element aligned to the whole vector), likewise converted only where used
template <typename T, int K>
struct RawVec;
template <int K>
struct RawVec<float, K> {
  float v[K];
  __device__ __forceinline__ void load(const float* __restrict__ p) {
    if constexpr (K % 4 == 0) {
#pragma unroll
      for (int i = 0; i < K / 4; ++i) {
        const f4 q = reinterpret_cast<const f4*>(p)[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else if constexpr (K == 2) {
      const f2 q = *reinterpret_cast<const f2*>(p);
      v[0] = q.x; v[1] = q.y;
    } else {
#pragma unroll
      for (int i = 0; i < K; ++i) v[i] = p[i];
    }
  }
  __device__ __forceinline__ void get(float* o) const {
#pragma unroll
    for (int i = 0; i < K; ++i) o[i] = v[i];
  }
};
template <int K>
struct RawVec<bf16_t, K> {
  static constexpr int W = (K + 1) / 2;   // 32-bit words
  uint32_t u[W];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p) {
    if constexpr (K == 1) {
      u[0] = p->bits;
    } else if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        u[4 * i] = q.x; u[4 * i + 1] = q.y; u[4 * i + 2] = q.z; u[4 * i + 3] = q.w;
      }
    } else if constexpr (W == 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      u[0] = q.x; u[1] = q.y;
    } else {
      u[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __device__ __forceinline__ void get(float* o) const {
    if constexpr (K == 1) {
      o[0] = __uint_as_float(u[0] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        o[2 * i] = __uint_as_float(u[i] << 16);
        o[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  }
};

// Raw 16-byte vectors of eight input elements, held in registers between
// the load that is issued early and the store into LDS.
template <typename TI>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { u = uint4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
  }
  // the values, or zeros when keep is false
  __device__ __forceinline__ void get(float* v, bool keep) const {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    const uint4 k = uint4{u.x & m, u.y & m, u.z & m, u.w & m};
    v[0] = __uint_as_float(k.x << 16); v[1] = __uint_as_float(k.x & 0xffff0000u);
    v[2] = __uint_as_float(k.y << 16); v[3] = __uint_as_float(k.y & 0xffff0000u);
    v[4] = __uint_as_float(k.z << 16); v[5] = __uint_as_float(k.z & 0xffff0000u);
    v[6] = __uint_as_float(k.w << 16); v[7] = __uint_as_float(k.w & 0xffff0000u);
  }
};
template <>
struct Vec8<float> {
  f4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f4*>(p);
    b = *reinterpret_cast<const f4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f4{0, 0, 0, 0}; }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void get(float* v, bool keep) const {
    get(v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = keep ? v[j] : 0.0f;
  }
};

// four consecutive elements starting at a multiple of 4 (8-byte / 16-byte loads)
__device__ __forceinline__ f4 ld4(const float* __restrict__ p, int64_t i) {
  return *reinterpret_cast<const f4*>(p + i);
}
__device__ __forceinline__ f4 ld4(const bf16_t* __restrict__ p, int64_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  f4 r;
  r.x = __uint_as_float(u.x << 16);
  r.y = __uint_as_float(u.x & 0xffff0000u);
  r.z = __uint_as_float(u.y << 16);
  r.w = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

// two consecutive elements starting at an even index
__device__ __forceinline__ f2 ld2(const float* __restrict__ p, int64_t i) {
  return *reinterpret_cast<const f2*>(p + i);
}
__device__ __forceinline__ f2 ld2(const bf16_t* __restrict__ p, int64_t i) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p + i);
  f2 r;
  r.x = __uint_as_float(u << 16);
  r.y = __uint_as_float(u & 0xffff0000u);
  return r;
}

// eight consecutive elements starting at a multiple of 8 (16-byte loads)
__device__ __forceinline__ void ld8(const float* __restrict__ p, int64_t i, float* v) {
  const f4 a = *reinterpret_cast<const f4*>(p + i);
  const f4 b = *reinterpret_cast<const f4*>(p + i + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16_t* __restrict__ p, int64_t i, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p + i);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

template <typename T>
__device__ __forceinline__ void st1(T* __restrict__ p, int64_t i, float v) {
  p[i] = from_f32<T>(v);
}

// 16-byte state access, both non-temporal.  A decode step streams a state
// larger than the 256 MB last-level cache, and in a model with several
// layers every step's state was pushed out by the other layers' steps.
// Measured on B=128 H=64 P=64 N=128 single-input steps: 88.0 us when one
// state is updated every step and 88.6 us when two alternate, against 82.3
// and 101.2 us with cached loads (which win only while the last step's
// state is still partly cached, and lose more once it is not).
__device__ __forceinline__ f4 ld4_state(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void st4_stream(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}

// rotate the complex pairs (v.x, v.y) and (v.z, v.w) by the angles whose
// (cos, sin) are c0 and c1
__device__ __forceinline__ f4 rot2pairs(f4 v, f2 c0, f2 c1) {
  f4 r;
  r.x = c0.x * v.x - c0.y * v.y;
  r.y = c0.y * v.x + c0.x * v.y;
  r.z = c1.x * v.z - c1.y * v.w;
  r.w = c1.y * v.z + c1.x * v.w;
  return r;
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of a group receives the group's sum.  Cross-lane steps within
// 16 lanes use DPP (quad permutes, half-row and row mirrors), wider ones a
// single lane permute each.
template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp_get<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (W >= 4) v += dpp_get<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (W >= 8) v += dpp_get<0x141>(v);   // row_half_mirror: 7 - i within 8
  if constexpr (W >= 16) v += dpp_get<0x140>(v);  // row_mirror: 15 - i within 16
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// (cos, sin) of an angle of any size: the angle in turns with its integer
// part removed (exactly), then the hardware sine and cosine, which take
// turns.  The one rounding of phi / 2pi costs |phi| * 6e-8 of phase; the
// hardware functions add at most 3e-7 on the reduced turn.
__device__ __forceinline__ f2 cos_sin_turns(float phi) {
  float t = phi * 0.15915494309189535f;
  t -= rintf(t);
  return f2{__builtin_amdgcn_cosf(t), __builtin_amdgcn_sinf(t)};
}

// Inverse RMS of one rank column of B or C from its sum of squares over the
// N channels (1 when the normalisation is off), with the hardware reciprocal
// square root (about 1 ulp; the correctly rounded sqrt-and-divide sequence
// costs the decode step a few percent).
__device__ __forceinline__ float bc_inv_rms(const BCPrep& p, float sumsq, int N) {
  return p.rms ? __builtin_amdgcn_rsqf(sumsq * (1.0f / (float)N) + p.eps) : 1.0f;
}

}  // namespace m3
