// chunk_common.h -- the pieces of the chunked scan shared by the prefill
// kernels and their gradients (gfx950): chunk geometry, the per-chunk decay
// and phase tables, token indexing and 16-byte row loaders.  Not part of the
// public ABI.
#pragma once

#include <type_traits>

#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

constexpr int kQ = 64;         // default chunk length (the backward's only one)
constexpr int kRB = 64;        // virtual rows per output block / u-block
constexpr double kTwoPi = 6.283185307179586476925286766559;

// (cos, sin) of an angle already reduced to [-pi, pi], from the hardware
// sine/cosine (argument in turns).  Measured on gfx950 over 4M angles in
// [-pi, pi]: max abs error 2.7e-7 (sincosf: 7e-8), far inside every
// tolerance here, at two instructions instead of ~30.
__device__ __forceinline__ f2 cos_sin_reduced(float ang) {
  const float turns = ang * 0.15915494309189535f;
  return f2{__builtin_amdgcn_cosf(turns), __builtin_amdgcn_sinf(turns)};
}

// per-chunk tables in LDS.  ROT: keep (cos, sin) of each angle (computed
// once); otherwise keep the reduced angle and take its sine and cosine where
// a row is staged (half the LDS; each angle is then used once).
//
// The angle table is token-major [t][k] for kernels whose lanes run along
// the pairs of one token, or pair-major [k][t] (rows padded by one entry, so
// both a column and a row of the table fall on distinct banks) for kernels
// whose lanes run along the tokens.  Q is the chunk length.
template <int N, bool ROT, bool KMAJ = false, int Q = kQ>
struct Tables {
  static constexpr int NP = N / 2;
  static constexpr int CQ = Q;
  static constexpr int TS = KMAJ ? Q + 1 : NP;   // row stride
  double cs[Q];       // chunk-local cumulative log-decay sum_{r<=t} dt_r A_r
  float dt[Q];
  float gam[Q];       // lam dt
  float bpr[Q];       // (1 - lam) dt
  float aux[Q];       // e^{cs_t} (outputs) or the chunk-state weights W_t
  double phi_end[NP];
  alignas(16) typename std::conditional<ROT, f2, float>::type tab[(KMAJ ? NP : Q) * TS];
  static __device__ __forceinline__ int at(int t, int k) { return KMAJ ? k * TS + t : t * TS + k; }
  // the phase input of (t, k), held in the angle's own slot until
  // chunk_tables replaces it by the angle (by the same thread)
  __device__ __forceinline__ void put_raw(int t, int k, float v) {
    if constexpr (ROT) {
      tab[at(t, k)] = f2{v, 0.0f};
    } else {
      tab[at(t, k)] = v;
    }
  }
  __device__ __forceinline__ float raw(int t, int k) const {
    if constexpr (ROT) {
      return tab[at(t, k)].x;
    } else {
      return tab[at(t, k)];
    }
  }
  // Phi_t (mode 0) or Phi_end - Phi_t (mode 1), reduced to [-pi, pi]
  __device__ __forceinline__ void set(int t, int k, float ang) {
    if constexpr (ROT) {
      tab[at(t, k)] = cos_sin_reduced(ang);
    } else {
      tab[at(t, k)] = ang;
    }
  }
  __device__ __forceinline__ f2 cs_of(int t, int k) const {
    if constexpr (ROT) {
      return tab[at(t, k)];
    } else {
      return cos_sin_reduced(tab[at(t, k)]);
    }
  }
  // (cos, sin) of pairs k0 .. k0 + M - 1 of token t (identity when !ok); a
  // token-major angle table serves four pairs with one 16-byte read
  template <int M>
  __device__ __forceinline__ void cs_run(int t, int k0, bool ok, f2* out) const {
    if constexpr (M == 4 && !ROT && !KMAJ) {
      const f4 ang = ok ? *reinterpret_cast<const f4*>(&tab[t * TS + k0]) : f4{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < 4; ++m) out[m] = cos_sin_reduced(ang[m]);
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) out[m] = ok ? cs_of(t, k0 + m) : f2{1.0f, 0.0f};
    }
  }
};

__device__ __forceinline__ float reduce_angle(double phi) {
  constexpr double inv = 1.0 / kTwoPi;
  return (float)(phi - kTwoPi * rint(phi * inv));
}

__device__ __forceinline__ int64_t token_index(const PrefillArgs& a, int b, int t, int h) {
  return ((int64_t)b * a.T + t) * a.H + h;
}
// B, C and theta are shared by groups of H / G heads: [Bsz, T, G, ...]
__device__ __forceinline__ int head_group(const PrefillArgs& a, int h) { return h / (a.H / a.G); }
__device__ __forceinline__ int64_t group_index(const PrefillArgs& a, int b, int t, int h) {
  return ((int64_t)b * a.T + t) * a.G + head_group(a, h);
}

// One chunk of the scan: tokens [t0, t0 + Lc) of token row bt, its slot in
// the workspace, and whether its sequence goes on after it.  [Bsz, T]
// inputs: chunk c of batch row b.  Packed sequences: chunk slot c of the
// slot table (row 0 of a [1, T] array), which may be unused.
struct ChunkRef {
  int bt, t0, Lc;
  bool next;
  int64_t id;
};
template <int Q = kQ>
__device__ __forceinline__ bool chunk_ref(const PrefillArgs& a, int c, int h, int b, ChunkRef& r) {
  if (c >= a.nchunk) return false;   // grid padding
  if (a.cmap) {
    const int4 e = a.cmap[c];
    if (e.x < 0) return false;
    r.bt = 0;
    r.t0 = e.y;
    r.Lc = min(Q, e.z - e.y);
    r.next = e.y + Q < e.z;
    r.id = (int64_t)h * a.nchunk + c;
  } else {
    r.bt = b;
    r.t0 = c * Q;
    r.Lc = min(Q, a.T - r.t0);
    r.next = c + 1 < a.nchunk;
    r.id = ((int64_t)b * a.H + h) * a.nchunk + c;
  }
  return true;
}

// One 64-virtual-row block of a per-token array with E elements per token
// (B or C: E = N R; x: E = P R) as 16-byte vectors spread over the block's
// NT threads.  TF: consecutive threads take consecutive tokens (for the
// transposed LDS layouts); otherwise consecutive threads walk one token.
template <typename TI, int E, int R, int NT, bool TF, int ROWS = kRB>
struct RowBlock {
  static constexpr int VPT = E / 8;
  static constexpr int NTOK = ROWS / R;
  static constexpr int NV = NTOK * VPT;
  static constexpr int IT = (NV + NT - 1) / NT;
  Vec8<TI> raw[IT];
  uint32_t okm;   // bit i: raw[i] holds elements of the chunk's rows (else it reads as zeros)
  static __device__ __forceinline__ void where(int vi, int& tl, int& e0) {
    if constexpr (TF) {
      tl = vi % NTOK;
      e0 = (vi / NTOK) * 8;
    } else {
      tl = vi / VPT;
      e0 = (vi % VPT) * 8;
    }
  }
  // rows of x (GRP false: one per head) or of B, C (GRP true: one per group)
  template <bool GRP>
  __device__ __forceinline__ void load(const TI* __restrict__ src, const PrefillArgs& a, int b,
                                       int h, int c0, int Lc, int v0) {
    const int t0 = v0 / R;
    // the chunk's first token is a block-uniform base; per-lane offsets stay
    // in 32 bits (the launcher checks that a chunk spans < 2^31 elements)
    const TI* __restrict__ base = src + (GRP ? group_index(a, b, c0, h) : token_index(a, b, c0, h)) * E;
    const int tstride = (GRP ? a.G : a.H) * E;
    // every lane loads (a lane past the rows re-reads the chunk's first
    // vector and reads as zeros): no branch around a load, so no load waits
    // for the ones before it
    okm = 0u;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = threadIdx.x + NT * i;
      int tl, e0;
      where(vi, tl, e0);
      const bool ok = vi < NV && t0 + tl < Lc;
      raw[i].load(base + (ok ? (t0 + tl) * tstride + e0 : 0));
      okm |= static_cast<uint32_t>(ok) << i;
    }
  }
  __device__ __forceinline__ void get(int i, float* v) const { raw[i].get(v, (okm >> i) & 1u); }
};

// Q x N/2 phase inputs of the chunk plus the token scalars of the first Q
// threads
template <typename TI, int N, int NT, int Q = kQ>
struct ThetaBlock {
  static_assert(NT >= Q, "one thread per token for the token scalars");
  static constexpr int NP = N / 2;
  static constexpr int VPT = NP / 8;
  static constexpr int NV = Q * VPT;
  static constexpr int IT = (NV + NT - 1) / NT;
  Vec8<TI> raw[IT];
  uint32_t okm;      // bit i: raw[i] holds phases of the chunk's tokens
  bool tok;          // this thread's token scalars are a token of the chunk
  float d_, l_, A_;  // as loaded (any value when !tok)
  // every lane loads from a valid address (the chunk's first token when it
  // has none of its own) and the values are masked where they are read: no
  // branch around a load, so no load waits for the ones before it.  With
  // the angle projection the phases are not read (project_theta makes them).
  __device__ __forceinline__ void load(const PrefillArgs& a, int b, int h, int c0, int Lc) {
    okm = 0u;
    if (!a.tp.on) {   // block-uniform
      const TI* __restrict__ th = static_cast<const TI*>(a.theta) + group_index(a, b, c0, h) * NP;
      const int tstride = a.G * NP;
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int vi = threadIdx.x + NT * i;
        const int t = vi / VPT, kv = vi % VPT;
        const bool ok = vi < NV && t < Lc;
        raw[i].load(th + (ok ? t * tstride + 8 * kv : 0));
        okm |= static_cast<uint32_t>(ok) << i;
      }
    }
    const int tid = threadIdx.x;
    tok = tid < Lc;
    const int64_t bth = token_index(a, b, c0, h) + (tok ? tid : 0) * a.H;
    d_ = ld1(static_cast<const TI*>(a.dt), bth);
    l_ = ld1(static_cast<const TI*>(a.lam), bth);
    A_ = (a.flags & kAPerToken) ? a.A[bth] : a.A[h];
  }
  __device__ __forceinline__ void get(int i, float* v) const { raw[i].get(v, (okm >> i) & 1u); }
  // dt, lam and A of token threadIdx.x (zero past the chunk)
  __device__ __forceinline__ float d() const { return tok ? d_ : 0.0f; }
  __device__ __forceinline__ float l() const { return tok ? l_ : 0.0f; }
  __device__ __forceinline__ float A() const { return tok ? A_ : 0.0f; }
};

// The chunk's tables from its loaded inputs: token scalars, the chunk-local
// log-decay prefix (double, one wave shuffle scan) and phase prefix of
// every pair (double; each thread owns one pair and a segment of tokens),
// then the angles reduced to [-pi, pi]: Phi_t (mode 0) or Phi_end - Phi_t
// (mode 1), kept as (cos, sin) or as the angle (see Tables).  scr is LDS
// scratch that is free until the tables are built.
template <int N, int NT, int Q = kQ>
struct TableScratch {
  double seg[NT];        // each thread's total of its segment of one pair's phases
  double wtot[Q / 64];   // each wave's total of the log-decay scan
};

template <typename TI, int N, int NT, bool ROT, bool KMAJ, int Q>
__device__ void chunk_tables(const PrefillArgs& a, const ThetaBlock<TI, N, NT, Q>& tb_in, int Lc,
                             Tables<N, ROT, KMAJ, Q>& tb, TableScratch<N, NT, Q>& scr, int mode) {
  using TB = ThetaBlock<TI, N, NT, Q>;
  static_assert(Q % 64 == 0, "whole waves of tokens");
  constexpr int NP = N / 2;
  const int tid = threadIdx.x;
  double lv = 0.0;
  if (tid < Q) {   // each wave scans its 64 tokens; later waves add the earlier totals below
    const float d = tb_in.d(), l = tb_in.l();
    lv = (double)d * (double)tb_in.A();
    const int lane = tid & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(lv, off, 64);
      if (lane >= off) lv += o;
    }
    if constexpr (Q > 64) {
      if (lane == 63) scr.wtot[tid >> 6] = lv;
    }
    tb.dt[tid] = d;
    tb.gam[tid] = l * d;
    tb.bpr[tid] = (1.0f - l) * d;
  }
  if (!a.tp.on) {   // else project_theta has put the phase inputs (block-uniform)
#pragma unroll
    for (int i = 0; i < TB::IT; ++i) {
      const int vi = tid + NT * i;
      if (vi < TB::NV) {
        float v[8];
        tb_in.get(i, v);
        const int t = vi / TB::VPT, kv = vi % TB::VPT;
#pragma unroll
        for (int j = 0; j < 8; ++j) tb.put_raw(t, 8 * kv + j, v[j]);
      }
    }
  }
  __syncthreads();
  if (tid < Q) {
    if constexpr (Q > 64) {
      for (int w = 0; w < (tid >> 6); ++w) lv += scr.wtot[w];
    }
    tb.cs[tid] = lv;   // read after the barriers below
  }

  constexpr int NSEG = NT / NP;
  constexpr int SEG = Q / NSEG;
  static_assert(NSEG >= 1 && Q % NSEG == 0, "phase segments");
  const int k = tid % NP, sg = tid / NP;
  const bool angle = (a.flags & kThetaIsAngle) != 0;
  double loc[SEG];
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = sg * SEG + i;
    const double tv = (double)tb.raw(t, k);
    run += angle ? tv : tv * (double)tb.dt[t];
    loc[i] = run;
  }
  scr.seg[sg * NP + k] = run;
  __syncthreads();
  double base = 0.0;
  for (int s = 0; s < sg; ++s) base += scr.seg[s * NP + k];
  if (sg == NSEG - 1) tb.phi_end[k] = base + run;
  __syncthreads();
  const double pe = tb.phi_end[k];
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = sg * SEG + i;
    if (t < Lc) {
      const double ph = base + loc[i];
      tb.set(t, k, reduce_angle(mode == 0 ? ph : pe - ph));
    }
  }
  __syncthreads();
}

// The angle projection of a chunk [xxxxx.co.kr Mamba-3 article, section
// 1.2: data-dependent angles]: th[t][k] = sum_j W[g][k][j] u[t][j] for the
// chunk's tokens t < Lc (zero for the rows past them), head group g, into
// the chunk's angle table, where chunk_tables reads them.  A 16 x 16 (token, pair) tile per
// wave at a time on the matrix cores, reading the operands straight from
// global memory in the fragment layout: bf16 inputs on
// v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums), fp32 inputs on
// v_mfma_f32_16x16x4_f32.  Lane l holds token row l % 16 of the A operand and
// pair l % 16 of the B operand; its D values are pair l % 16 of tokens
// 4 (l / 16) .. 4 (l / 16) + 3.
template <typename TI, int N, int NT, int Q, class Tab>
__device__ void project_theta(const PrefillArgs& a, int bt, int h, int c0, int Lc, Tab& tb) {
  constexpr int NP = N / 2;
  constexpr int TT = Q / 16, KT = (NP + 15) / 16;
  const int D = a.tp.dim;
  const TI* __restrict__ U = static_cast<const TI*>(a.tp.u) + ((int64_t)bt * a.T + c0) * D;
  const TI* __restrict__ Wg = static_cast<const TI*>(a.tp.W) + (int64_t)head_group(a, h) * NP * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  for (int tile = wave; tile < TT * KT; tile += NT / 64) {
    const int t0 = 16 * (tile / KT), k0 = 16 * (tile % KT);
    // rows past the chunk or the pairs read a valid row; their results are dropped
    const TI* __restrict__ ur = U + (int64_t)min(t0 + l16, Lc - 1) * D;
    const TI* __restrict__ wr = Wg + (int64_t)min(k0 + l16, NP - 1) * D;
    f4 acc = f4{0, 0, 0, 0};
    if constexpr (std::is_same<TI, bf16_t>::value) {
      for (int j0 = 0; j0 < D; j0 += 32) {
        const uint4 av = *reinterpret_cast<const uint4*>(ur + j0 + 8 * g);
        const uint4 bv = *reinterpret_cast<const uint4*>(wr + j0 + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bh8, av),
                                                      __builtin_bit_cast(bh8, bv), acc, 0, 0, 0);
      }
    } else {
      for (int j0 = 0; j0 < D; j0 += 16) {
        const f4 av = *reinterpret_cast<const f4*>(ur + j0 + 4 * g);
        const f4 bv = *reinterpret_cast<const f4*>(wr + j0 + 4 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc, 0, 0, 0);
      }
    }
    const int k = k0 + l16;
    if (k < NP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i;
        tb.put_raw(t, k, t < Lc ? acc[i] : 0.0f);
      }
    }
  }
}

// element i of an input array of type T
template <typename T>
__device__ __forceinline__ float ldy(const void* p, int64_t i) {
  return ld1(static_cast<const T*>(p), i);
}

// rotate one pair by -angle / +angle given (cos, sin)
__device__ __forceinline__ f2 rot_neg(f2 v, f2 cs) { return f2{cs.x * v.x + cs.y * v.y, -cs.y * v.x + cs.x * v.y}; }
__device__ __forceinline__ f2 rot_pos(f2 v, f2 cs) { return f2{cs.x * v.x - cs.y * v.y, cs.y * v.x + cs.x * v.y}; }

// block-wide sum in a fixed order (all threads receive it); red holds one
// value per wave
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = group_sum<64>(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) s += red[w];
  return s;
}

}  // namespace m3
