// mfma_pol.h -- MFMA operand policies and LDS row staging shared by the
// chunked prefill kernels and their gradients (gfx950).  Not part of the
// public ABI.
//
// A policy fixes how fp32 operands reach the matrix cores: PolF32 keeps
// them in fp32 (v_mfma_f32_16x16x4_f32, the fp32-input path); PolB16 (the
// bf16-input path, PolHalf) splits each into bf16 hi + lo parts and forms a
// product as hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 (about fp32
// accuracy, fp32's exponent range), with x (a bf16 input, exact) used
// unsplit; PolF16 does the same with fp16 parts (more bits, fp16's range)
// and is kept for comparison.  Fragments follow the 16x16 MFMA lane layout: lane l holds
// row (or column) l % 16 and k group l / 16; a D tile holds column l % 16
// and rows 4 (l / 16) .. 4 (l / 16) + 3, so D tiles turn into A operands
// of the transposed product without a trip through LDS (frag_from_d), and
// fragp / fragx_d read B operands in the same k order.
#pragma once

#include "chunk_common.h"

namespace m3 {

// --------------------------------------------------------------------------
// MFMA operand policies
struct PolF32 {
  static constexpr int KS = 16;  // k per fragment: lane group g holds k = 4g..4g+3
  static constexpr int DT = 1;   // 16x16 D tiles per A fragment built from D
  struct Frag {
    f4 v;
  };
  typedef Frag XFrag;
  template <int ROWS, int K>
  struct Store {
    float v[ROWS][K + 4];
  };
  template <int ROWS, int K>
  struct XStore {
    float v[ROWS][K + 4];
  };
  template <int ROWS, int K>
  static __device__ __forceinline__ void put(Store<ROWS, K>& s, int r, int k, float x) {
    s.v[r][k] = x;
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void putx(XStore<ROWS, K>& s, int r, int k, float x) {
    s.v[r][k] = x;
  }
  // eight consecutive k (k0 a multiple of 8) of one row
  template <int ROWS, int K>
  static __device__ __forceinline__ void put8(Store<ROWS, K>& s, int r, int k0, const float* v) {
    *reinterpret_cast<f4*>(&s.v[r][k0]) = f4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f4*>(&s.v[r][k0 + 4]) = f4{v[4], v[5], v[6], v[7]};
  }
  // M (1, 2 or 4) consecutive k of one row, k0 a multiple of M, one write
  template <int M, class St>
  static __device__ __forceinline__ void putm(St& s, int r, int k0, const float* v) {
    if constexpr (M == 4) {
      *reinterpret_cast<f4*>(&s.v[r][k0]) = f4{v[0], v[1], v[2], v[3]};
    } else if constexpr (M == 2) {
      *reinterpret_cast<f2*>(&s.v[r][k0]) = f2{v[0], v[1]};
    } else {
      static_assert(M == 1, "putm");
      s.v[r][k0] = v[0];
    }
  }
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putn(Store<ROWS, K>& s, int r, int k0, const float* v) {
    putm<M>(s, r, k0, v);
  }
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putxn(XStore<ROWS, K>& s, int r, int k0, const float* v) {
    putm<M>(s, r, k0, v);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag frag(const Store<ROWS, K>& s, int row0, int k0, int lane) {
    return Frag{*reinterpret_cast<const f4*>(&s.v[row0 + (lane & 15)][k0 + 4 * (lane >> 4)])};
  }
  // fragment of KS consecutive values (already rotated) from registers
  static __device__ __forceinline__ Frag make(const float* v) { return Frag{f4{v[0], v[1], v[2], v[3]}}; }
  // B operand from an XStore, k order matching frag_from_d
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_d(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    return Frag{*reinterpret_cast<const f4*>(&s.v[col0 + (lane & 15)][k0 + 4 * (lane >> 4)])};
  }
  // B operand from an XStore, consecutive k order (as frag)
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_c(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    return fragx_d(s, col0, k0, lane);
  }
  static __device__ __forceinline__ Frag frag_from_d(const f4* d) { return Frag{d[0]}; }
  static __device__ __forceinline__ f4 mma(const Frag& a, const Frag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ f4 mma_x(const Frag& a, const XFrag& b, f4 acc) {
    return mma(a, b, acc);
  }
  static __device__ __forceinline__ f4 mma_xa(const XFrag& a, const Frag& b, f4 acc) {
    return mma(a, b, acc);
  }
  // B operand from a Store in the k order of frag_from_d (the natural one here)
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag fragp(const Store<ROWS, K>& s, int col0, int k0, int lane) {
    return frag(s, col0, k0, lane);
  }
};

struct PolF16 {
  static constexpr int KS = 32;  // k per fragment: lane group g holds 8 k values
  static constexpr int DT = 2;
  struct Frag {
    h8 hi, lo;
  };
  typedef h8 XFrag;
  // Rows are padded by 4 halves: a row is then 2 (mod 32) dwords long, so
  // the 16 rows that one 8-byte LDS access phase touches fall on distinct
  // banks.  Rows are only 8-byte aligned, so every access below is made of
  // 8-byte pieces.
  static constexpr int PAD = 4;
  template <int ROWS, int K>
  struct Store {
    _Float16 hi[ROWS][K + PAD];
    _Float16 lo[ROWS][K + PAD];
  };
  template <int ROWS, int K>
  struct XStore {
    _Float16 v[ROWS][K + PAD];
  };
  static __device__ __forceinline__ h8 ld8h(const _Float16* p) {
    const h4 a = *reinterpret_cast<const h4*>(p);
    const h4 b = *reinterpret_cast<const h4*>(p + 4);
    return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  static __device__ __forceinline__ void st8h(_Float16* p, h8 v) {
    *reinterpret_cast<h4*>(p) = h4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<h4*>(p + 4) = h4{v[4], v[5], v[6], v[7]};
  }
  // x = hi + lo to about 2^-22 relative: hi = fp16(x) (round to nearest
  // even), lo = fp16(x - hi) with the difference formed exactly inside
  // v_fma_mix (x * 1 - hi, one rounding).  Written as asm on purpose: x is
  // then one fixed fp32 register value, so FP contraction cannot fold the
  // producer's multiply into lo while hi is rounded from the fp32 product
  // (hi + lo would then miss x by an fp16 ulp).
  static __device__ __forceinline__ void split(float x, _Float16& hi, _Float16& lo) {
    uint32_t h, l = 0;
    asm volatile("v_cvt_f16_f32 %0, %1" : "=v"(h) : "v"(x));
    asm volatile("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "+v"(l) : "v"(x), "v"(h));
    hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xffffu));
    lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(l & 0xffffu));
  }
  // the same for two values, packed (element 0 in the low half)
  static __device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    uint32_t h, l = 0;
    asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(h) : "v"(x0), "v"(x1));
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %3, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "+v"(l)
        : "v"(x0), "v"(h), "v"(x1));
    hi = h;
    lo = l;
  }
  static __device__ __forceinline__ void split8(const float* v, h8& hi, h8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split2(v[2 * q], v[2 * q + 1], h[q], l[q]);
    hi = __builtin_bit_cast(h8, uint4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(h8, uint4{l[0], l[1], l[2], l[3]});
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void put(Store<ROWS, K>& s, int r, int k, float x) {
    split(x, s.hi[r][k], s.lo[r][k]);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void putx(XStore<ROWS, K>& s, int r, int k, float x) {
    s.v[r][k] = static_cast<_Float16>(x);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void put8(Store<ROWS, K>& s, int r, int k0, const float* v) {
    h8 hi, lo;
    split8(v, hi, lo);
    st8h(&s.hi[r][k0], hi);
    st8h(&s.lo[r][k0], lo);
  }
  // M (1, 2 or 4) consecutive k of one row, k0 a multiple of M: one write
  // per part
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putn(Store<ROWS, K>& s, int r, int k0, const float* v) {
    if constexpr (M == 4) {
      uint32_t h0, l0, h1, l1;
      split2(v[0], v[1], h0, l0);
      split2(v[2], v[3], h1, l1);
      *reinterpret_cast<uint2*>(&s.hi[r][k0]) = uint2{h0, h1};
      *reinterpret_cast<uint2*>(&s.lo[r][k0]) = uint2{l0, l1};
    } else if constexpr (M == 2) {
      uint32_t h0, l0;
      split2(v[0], v[1], h0, l0);
      *reinterpret_cast<uint32_t*>(&s.hi[r][k0]) = h0;
      *reinterpret_cast<uint32_t*>(&s.lo[r][k0]) = l0;
    } else {
      static_assert(M == 1, "putn");
      put(s, r, k0, v[0]);
    }
  }
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putxn(XStore<ROWS, K>& s, int r, int k0, const float* v) {
    if constexpr (M == 4) {
      *reinterpret_cast<h4*>(&s.v[r][k0]) = h4{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]),
                                              static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
    } else if constexpr (M == 2) {
      *reinterpret_cast<h2*>(&s.v[r][k0]) = h2{static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1])};
    } else {
      static_assert(M == 1, "putxn");
      s.v[r][k0] = static_cast<_Float16>(v[0]);
    }
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag frag(const Store<ROWS, K>& s, int row0, int k0, int lane) {
    const int r = row0 + (lane & 15), k = k0 + 8 * (lane >> 4);
    return Frag{ld8h(&s.hi[r][k]), ld8h(&s.lo[r][k])};
  }
  static __device__ __forceinline__ Frag make(const float* v) {
    Frag f;
    split8(v, f.hi, f.lo);
    return f;
  }
  // slot 8g+j <-> k0 + 4g + j (j < 4) and k0 + 16 + 4g + (j - 4) (j >= 4)
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_d(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    const int r = col0 + (lane & 15), g = lane >> 4;
    const h4 a = *reinterpret_cast<const h4*>(&s.v[r][k0 + 4 * g]);
    const h4 b = *reinterpret_cast<const h4*>(&s.v[r][k0 + 16 + 4 * g]);
    return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_c(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    return ld8h(&s.v[col0 + (lane & 15)][k0 + 8 * (lane >> 4)]);
  }
  static __device__ __forceinline__ Frag frag_from_d(const f4* d) {
    const float v[8] = {d[0].x, d[0].y, d[0].z, d[0].w, d[1].x, d[1].y, d[1].z, d[1].w};
    return make(v);
  }
  static __device__ __forceinline__ f4 mma(const Frag& a, const Frag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ f4 mma_x(const Frag& a, const XFrag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.hi, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.lo, b, acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ f4 mma_xa(const XFrag& a, const Frag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b.lo, acc, 0, 0, 0);
    return acc;
  }
  // B operand (hi and lo) from a Store in the k order of frag_from_d
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag fragp(const Store<ROWS, K>& s, int col0, int k0, int lane) {
    const int r = col0 + (lane & 15), g = lane >> 4;
    const h4 a = *reinterpret_cast<const h4*>(&s.hi[r][k0 + 4 * g]);
    const h4 b = *reinterpret_cast<const h4*>(&s.hi[r][k0 + 16 + 4 * g]);
    const h4 c = *reinterpret_cast<const h4*>(&s.lo[r][k0 + 4 * g]);
    const h4 d = *reinterpret_cast<const h4*>(&s.lo[r][k0 + 16 + 4 * g]);
    return Frag{h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]},
                h8{c[0], c[1], c[2], c[3], d[0], d[1], d[2], d[3]}};
  }
};


// PolB16: the same three-product split with bf16 parts on
// v_mfma_f32_16x16x32_bf16.  hi = bf16(x) (round to nearest even), lo =
// bf16(x - hi) with x - hi exact in fp32, so hi + lo carries 16-17
// significant bits (relative error <= 2^-17) and, since bf16 has fp32's
// exponent range, every finite fp32 operand splits without overflow or
// precision lost to subnormals (fp16 parts would overflow above 65504 and
// lose bits below about 2^-3 of lo's range).  x, a bf16 input, is exact
// as one bf16 part.
struct PolB16 {
  static constexpr int KS = 32;
  static constexpr int DT = 2;
  struct Frag {
    bh8 hi, lo;
  };
  typedef bh8 XFrag;
  static constexpr int PAD = 4;   // as PolF16: rows 2 (mod 32) dwords long
  template <int ROWS, int K>
  struct Store {
    uint16_t hi[ROWS][K + PAD];
    uint16_t lo[ROWS][K + PAD];
  };
  template <int ROWS, int K>
  struct XStore {
    uint16_t v[ROWS][K + PAD];
  };
  static __device__ __forceinline__ bh8 ld8(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 4);
    return __builtin_bit_cast(bh8, uint4{a.x, a.y, b.x, b.y});
  }
  static __device__ __forceinline__ void st8(uint16_t* p, uint4 v) {
    *reinterpret_cast<uint2*>(p) = uint2{v.x, v.y};
    *reinterpret_cast<uint2*>(p + 4) = uint2{v.z, v.w};
  }
  // two values, packed (element 0 in the low half).  The empty asm makes
  // each input one fixed register value, so FP contraction cannot form lo
  // from an unrounded product that hi was not rounded from.
  static __device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    asm("" : "+v"(x0), "+v"(x1));
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, bh2));
    const float h0 = __uint_as_float(h << 16), h1 = __uint_as_float(h & 0xffff0000u);
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0 - h0, x1 - h1}, bh2));
  }
  static __device__ __forceinline__ void split8(const float* v, uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split2(v[2 * q], v[2 * q + 1], h[q], l[q]);
    hi = uint4{h[0], h[1], h[2], h[3]};
    lo = uint4{l[0], l[1], l[2], l[3]};
  }
  // one bf16 value exactly (x is a bf16 input)
  static __device__ __forceinline__ uint16_t exact(float x) {
    return static_cast<uint16_t>(__float_as_uint(x) >> 16);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void put(Store<ROWS, K>& s, int r, int k, float x) {
    uint32_t h, l;
    split2(x, 0.0f, h, l);
    s.hi[r][k] = static_cast<uint16_t>(h);
    s.lo[r][k] = static_cast<uint16_t>(l);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void putx(XStore<ROWS, K>& s, int r, int k, float x) {
    s.v[r][k] = exact(x);
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ void put8(Store<ROWS, K>& s, int r, int k0, const float* v) {
    uint4 hi, lo;
    split8(v, hi, lo);
    st8(&s.hi[r][k0], hi);
    st8(&s.lo[r][k0], lo);
  }
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putn(Store<ROWS, K>& s, int r, int k0, const float* v) {
    if constexpr (M == 4) {
      uint32_t h0, l0, h1, l1;
      split2(v[0], v[1], h0, l0);
      split2(v[2], v[3], h1, l1);
      *reinterpret_cast<uint2*>(&s.hi[r][k0]) = uint2{h0, h1};
      *reinterpret_cast<uint2*>(&s.lo[r][k0]) = uint2{l0, l1};
    } else if constexpr (M == 2) {
      uint32_t h0, l0;
      split2(v[0], v[1], h0, l0);
      *reinterpret_cast<uint32_t*>(&s.hi[r][k0]) = h0;
      *reinterpret_cast<uint32_t*>(&s.lo[r][k0]) = l0;
    } else {
      static_assert(M == 1, "putn");
      put(s, r, k0, v[0]);
    }
  }
  template <int M, int ROWS, int K>
  static __device__ __forceinline__ void putxn(XStore<ROWS, K>& s, int r, int k0, const float* v) {
    if constexpr (M == 4) {
      *reinterpret_cast<uint2*>(&s.v[r][k0]) =
          uint2{exact(v[0]) | (static_cast<uint32_t>(exact(v[1])) << 16),
                exact(v[2]) | (static_cast<uint32_t>(exact(v[3])) << 16)};
    } else if constexpr (M == 2) {
      *reinterpret_cast<uint32_t*>(&s.v[r][k0]) =
          exact(v[0]) | (static_cast<uint32_t>(exact(v[1])) << 16);
    } else {
      static_assert(M == 1, "putxn");
      s.v[r][k0] = exact(v[0]);
    }
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag frag(const Store<ROWS, K>& s, int row0, int k0, int lane) {
    const int r = row0 + (lane & 15), k = k0 + 8 * (lane >> 4);
    return Frag{ld8(&s.hi[r][k]), ld8(&s.lo[r][k])};
  }
  static __device__ __forceinline__ Frag make(const float* v) {
    uint4 hi, lo;
    split8(v, hi, lo);
    return Frag{__builtin_bit_cast(bh8, hi), __builtin_bit_cast(bh8, lo)};
  }
  // slot 8g+j <-> k0 + 4g + j (j < 4) and k0 + 16 + 4g + (j - 4) (j >= 4)
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_d(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    const int r = col0 + (lane & 15), g = lane >> 4;
    const uint2 a = *reinterpret_cast<const uint2*>(&s.v[r][k0 + 4 * g]);
    const uint2 b = *reinterpret_cast<const uint2*>(&s.v[r][k0 + 16 + 4 * g]);
    return __builtin_bit_cast(bh8, uint4{a.x, a.y, b.x, b.y});
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ XFrag fragx_c(const XStore<ROWS, K>& s, int col0, int k0, int lane) {
    return ld8(&s.v[col0 + (lane & 15)][k0 + 8 * (lane >> 4)]);
  }
  static __device__ __forceinline__ Frag frag_from_d(const f4* d) {
    const float v[8] = {d[0].x, d[0].y, d[0].z, d[0].w, d[1].x, d[1].y, d[1].z, d[1].w};
    return make(v);
  }
  static __device__ __forceinline__ f4 mma(const Frag& a, const Frag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ f4 mma_x(const Frag& a, const XFrag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b, acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ f4 mma_xa(const XFrag& a, const Frag& b, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b.lo, acc, 0, 0, 0);
    return acc;
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag fragp(const Store<ROWS, K>& s, int col0, int k0, int lane) {
    const int r = col0 + (lane & 15), g = lane >> 4;
    const uint2 a = *reinterpret_cast<const uint2*>(&s.hi[r][k0 + 4 * g]);
    const uint2 b = *reinterpret_cast<const uint2*>(&s.hi[r][k0 + 16 + 4 * g]);
    const uint2 c = *reinterpret_cast<const uint2*>(&s.lo[r][k0 + 4 * g]);
    const uint2 d = *reinterpret_cast<const uint2*>(&s.lo[r][k0 + 16 + 4 * g]);
    return Frag{__builtin_bit_cast(bh8, uint4{a.x, a.y, b.x, b.y}),
                __builtin_bit_cast(bh8, uint4{c.x, c.y, d.x, d.y})};
  }
};

// the policy of bf16 inputs
#ifndef M3_HALF_POLICY
#define M3_HALF_POLICY PolB16
#endif
typedef M3_HALF_POLICY PolHalf;

// the B/C preparation of one vector of eight elements (e0 .. e0 + 7 of
// token t's N x R row), in place; NoPrep leaves it as loaded
struct NoPrep {
  __device__ __forceinline__ void operator()(int, int, float*) const {}
};

// B or C rows of a block, rotated by -Phi_t, into st[v - v0][n]
template <class Pol, typename TI, int N, int R, int NT, int ROWS, class Tab, class Prep>
__device__ __forceinline__ void store_rows(const RowBlock<TI, N * R, R, NT, false, ROWS>& rb,
                                           typename Pol::template Store<ROWS, N>& st,
                                           const Tab& tb, int t0, int Lc, const Prep& prep) {
  using RBk = RowBlock<TI, N * R, R, NT, false, ROWS>;
  constexpr int NPAIR = 4 / R;              // complex pairs per vector
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    const int t = t0 + tl;
    const bool ok = t < Lc;
    float v[8], o[8];
    rb.get(i, v);
    if (ok) prep(t, e0, v);
    f2 csr[NPAIR];
    tb.template cs_run<NPAIR>(t, e0 / R / 2, ok, csr);
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
      const f2 cs = csr[pi];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float u0 = v[(2 * pi) * R + r], u1 = v[(2 * pi + 1) * R + r];
        o[(2 * pi) * R + r] = cs.x * u0 + cs.y * u1;        // rotate by -Phi_t
        o[(2 * pi + 1) * R + r] = -cs.y * u0 + cs.x * u1;
      }
    }
    if constexpr (R == 1) {
      Pol::put8(st, tl, e0, o);
    } else {
      // element j is (column e0/R + j/R, rank j%R): row (tl, r) receives
      // 8/R consecutive columns
      constexpr int M = 8 / R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float w[M];
#pragma unroll
        for (int m = 0; m < M; ++m) w[m] = o[m * R + r];
        Pol::template putn<M>(st, tl * R + r, e0 / R, w);
      }
    }
  }
}

// B rows of a block rotated by +(Phi_end - Phi_t) and scaled by W_t,
// transposed: st[n][v - v0]
template <class Pol, typename TI, int N, int R, int NT, bool TF, int ROWS, class Tab, class Prep>
__device__ __forceinline__ void store_rows_T(const RowBlock<TI, N * R, R, NT, TF, ROWS>& rb,
                                             typename Pol::template Store<N, ROWS>& st,
                                             const Tab& tb, const float* w, int t0, int Lc,
                                             const Prep& prep) {
  using RBk = RowBlock<TI, N * R, R, NT, TF, ROWS>;
  constexpr int NPAIR = 4 / R;
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    const int t = t0 + tl;
    const bool ok = t < Lc;
    const float wt = ok ? w[t] : 0.0f;
    float v[8];
    rb.get(i, v);
    if (ok) prep(t, e0, v);
    f2 csr[NPAIR];
    tb.template cs_run<NPAIR>(t, e0 / R / 2, ok, csr);
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
      const int n = e0 / R + 2 * pi;
      const f2 cs = wt * csr[pi];   // the weight folded into the rotation
      float w0[R], w1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float u0 = v[(2 * pi) * R + r], u1 = v[(2 * pi + 1) * R + r];
        w0[r] = cs.x * u0 - cs.y * u1;   // rotate by +angle
        w1[r] = cs.y * u0 + cs.x * u1;
      }
      // the R virtual rows of token tl are consecutive columns of st
      Pol::template putn<R>(st, n, tl * R, w0);
      Pol::template putn<R>(st, n + 1, tl * R, w1);
    }
  }
}

// x rows of a block, transposed: xs[p][v - v0]
template <class Pol, typename TI, int P, int R, int NT, int ROWS, bool TF>
__device__ __forceinline__ void store_x_T(const RowBlock<TI, P * R, R, NT, TF, ROWS>& rb,
                                          typename Pol::template XStore<P, ROWS>& xs) {
  using RBk = RowBlock<TI, P * R, R, NT, TF, ROWS>;
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    float v[8];
    rb.get(i, v);
    if constexpr (R == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) Pol::putx(xs, e0 + j, tl, v[j]);
    } else {
      // element j is (p = e0/R + j/R, rank j%R): the R ranks of one p are
      // consecutive columns
#pragma unroll
      for (int m = 0; m < 8 / R; ++m) Pol::template putxn<R>(xs, e0 / R + m, tl * R, v + m * R);
    }
  }
}

// the P x N entry state of a chunk (fp32) as 16-byte vector pairs
template <int P, int N, int NT>
struct StateBlock {
  static constexpr int NV = P * N / 8;
  static constexpr int IT = (NV + NT - 1) / NT;
  Vec8<float> raw[IT];
  __device__ __forceinline__ void load(const float* __restrict__ src) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = threadIdx.x + NT * i;
      if (vi < NV) raw[i].load(src + (int64_t)vi * 8);
    }
  }
  // rows [p0, p0 + ROWS) only, into st[p - p0][n]
  template <class Pol, int ROWS>
  __device__ __forceinline__ void store_part(typename Pol::template Store<ROWS, N>& st, int p0) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = threadIdx.x + NT * i;
      const int p = (vi * 8) / N;
      if (vi < NV && p >= p0 && p < p0 + ROWS) {
        float v[8];
        raw[i].get(v);
        Pol::put8(st, p - p0, (vi * 8) % N, v);
      }
    }
  }
  template <class Pol>
  __device__ __forceinline__ void store(typename Pol::template Store<P, N>& st) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = threadIdx.x + NT * i;
      if (vi < NV) {
        float v[8];
        raw[i].get(v);
        Pol::put8(st, (vi * 8) / N, (vi * 8) % N, v);
      }
    }
  }
};

}  // namespace m3
