// prefill.hip -- chunked prefill scan of the Mamba-3 core recurrence, gfx950.
//
// The recurrence [xxxxx.co.kr Mamba-3 article, sections 1.1-1.3]
//   S_t = R(phi_t) (alpha_t S_{t-1} + beta_t X_{t-1} B_{t-1}^T) + gamma_t X_t B_t^T,
//   y_t = S_t C_t
// is evaluated exactly, chunk by chunk (Q tokens), in the frame that the
// "RoPE trick" of section 1.2 gives: inside a chunk starting at c0, with the
// chunk-local cumulative log-decay cs_t = sum_{r=c0..t} dt_r A_r and phase
// Phi_t = sum_{r=c0..t} dt_r theta_r, rotate B and C by -Phi_t (Bt, Ct); then
//
//   y_t = e^{cs_t} Ct_t . Shat_c                                   (Y_off)
//       + sum_{u=c0..t} e^{cs_t - cs_u} w_{t,u} (Ct_t . Bt_u) x_u  (Y_diag)
//   w_{t,u} = gamma_u + [u < t] (1 - lam_{u+1}) dt_{u+1}
//
// where Shat_c = S_{c0-1} + (1 - lam_{c0}) dt_{c0} x_{c0-1} B_{c0-1}^T is the
// state entering the chunk plus the trapezoid's left-endpoint term of its
// first token (the width-2 convolution reaching back one token).  Chunks are
// linked by
//   S_{end} = e^{cs_end} R(Phi_end) Shat_c + S_c,
//   S_c     = sum_u e^{cs_end - cs_u} w_{end,u} x_u (R(Phi_end - Phi_u) B_u)^T.
// Rank R > 1 turns every token into R "virtual rows" (t, r) of the chunk's
// Gram matrix; the decay mask depends on the tokens only.
//
// Three launches on the caller's stream:
//  k_chunk_state  (batch, head, chunk): decay/phase totals and S_c (MFMA).
//  k_state_pass   (batch, head, 16-row slice): the serial pass over chunks,
//                 turning S_c into Shat_c in place and writing h_T.
//  k_chunk_output (batch, head, chunk, 64-row block): Gram Ct Bt^T, the
//                 decay mask, Y_diag and Y_off (MFMA), y.
// The per-chunk decay and phase prefix sums are recomputed inside the chunk
// kernels (double accumulation, angles reduced mod 2pi before sincos), so no
// precompute pass touches HBM.
//
// MFMA operands: with fp32 inputs, v_mfma_f32_16x16x4_f32 on fp32 operands.
// With bf16 inputs every operand computed in fp32 (rotated B and C, the
// masked Gram, the state) is split into fp16 hi + lo parts and each product
// is hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_f16 (about fp32 accuracy);
// x is exact in fp16 and used unsplit.
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

constexpr int kQ = 64;         // chunk length
constexpr int kRB = 64;        // virtual rows per output block / u-block
constexpr double kTwoPi = 6.283185307179586476925286766559;

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
};

struct PolF16 {
  static constexpr int KS = 32;  // k per fragment: lane group g holds 8 k values
  static constexpr int DT = 2;
  struct Frag {
    h8 hi, lo;
  };
  typedef h8 XFrag;
  template <int ROWS, int K>
  struct Store {
    _Float16 hi[ROWS][K + 8];
    _Float16 lo[ROWS][K + 8];
  };
  template <int ROWS, int K>
  struct XStore {
    _Float16 v[ROWS][K + 8];
  };
  // x = hi + lo to about 2^-22 relative.  The empty asm pins x to one fp32
  // register value: otherwise FP contraction may fold the producer's
  // multiply into the lo subtraction (using the exact product) while hi is
  // rounded from the fp32 product, and hi + lo then misses x by an fp16 ulp.
  static __device__ __forceinline__ void split(float x, _Float16& hi, _Float16& lo) {
    asm volatile("" : "+v"(x));
    hi = static_cast<_Float16>(x);
    lo = static_cast<_Float16>(x - static_cast<float>(hi));
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
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      _Float16 a, b;
      split(v[j], a, b);
      hi[j] = a;
      lo[j] = b;
    }
    *reinterpret_cast<h8*>(&s.hi[r][k0]) = hi;
    *reinterpret_cast<h8*>(&s.lo[r][k0]) = lo;
  }
  template <int ROWS, int K>
  static __device__ __forceinline__ Frag frag(const Store<ROWS, K>& s, int row0, int k0, int lane) {
    const int r = row0 + (lane & 15), k = k0 + 8 * (lane >> 4);
    return Frag{*reinterpret_cast<const h8*>(&s.hi[r][k]), *reinterpret_cast<const h8*>(&s.lo[r][k])};
  }
  static __device__ __forceinline__ Frag make(const float* v) {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      _Float16 h, l;
      split(v[j], h, l);
      f.hi[j] = h;
      f.lo[j] = l;
    }
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
    return *reinterpret_cast<const h8*>(&s.v[col0 + (lane & 15)][k0 + 8 * (lane >> 4)]);
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
};


// --------------------------------------------------------------------------
// launch geometry: one block per chunk; each wave owns TPW 16-row tiles of
// the chunk's Q*R virtual rows (two tiles w and 2NW-1-w when TPW = 2, which
// balances the causal work across waves)
template <int P, int N, int R>
struct Geo {
  static constexpr int ROWS = kQ * R;
  static constexpr int TILES = ROWS / 16;
  static constexpr int NW = TILES >= 8 ? 8 : 4;
  static constexpr int TPW = TILES / NW;
  static constexpr int NT = NW * 64;
  static constexpr int NP = N / 2;
  static constexpr int PT = P / 16;
  static constexpr int NTL = N / 16;
  static constexpr int NUB = ROWS / kRB;
  static_assert(TPW >= 1 && TILES % NW == 0, "tile split");
};

// per-chunk tables in LDS
template <int NT, int N>
struct Tables {
  double cs[kQ];      // chunk-local cumulative log-decay sum_{r<=t} dt_r A_r
  float dt[kQ];
  float gam[kQ];      // lam dt
  float bpr[kQ];      // (1 - lam) dt
  float aux[kQ];      // e^{cs_t} (outputs) or the chunk-state weights W_t
  double seg[NT];
  double phi_end[N / 2];
  f2 rot[kQ][N / 2];  // (cos, sin) of Phi_t (mode 0) or of Phi_end - Phi_t (mode 1)
};

__device__ __forceinline__ float reduce_angle(double phi) {
  constexpr double inv = 1.0 / kTwoPi;
  return (float)(phi - kTwoPi * rint(phi * inv));
}

__device__ __forceinline__ int64_t token_index(const PrefillArgs& a, int b, int t, int h) {
  return ((int64_t)b * a.T + t) * a.H + h;
}

// Token scalars, the chunk-local log-decay prefix (double, one wave) and the
// chunk-local phase prefix of every pair (double; each thread owns one pair
// and a segment of tokens), then (cos, sin) of the reduced angles.  th_raw
// is scratch for the chunk's theta (Q x N/2 floats) and is free on return.
template <typename TI, int N, int NT>
__device__ void chunk_tables(const PrefillArgs& a, int b, int h, int c0, int Lc,
                             Tables<NT, N>& tb, float* th_raw, int mode) {
  constexpr int NP = N / 2;
  constexpr int VPT = NP / 8;                 // 16-byte vectors per token
  constexpr int NV = kQ * VPT;
  constexpr int IT = (NV + NT - 1) / NT;
  const int tid = threadIdx.x;
  const TI* __restrict__ th = static_cast<const TI*>(a.theta);
  float v[IT][8];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    const int t = vi / VPT, kv = vi % VPT;
    if (vi < NV && t < Lc) {
      ld8(th, token_index(a, b, c0 + t, h) * NP + 8 * kv, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
  if (tid < 64) {
    double lv = 0.0;
    float d = 0.0f, gm = 0.0f, bp = 0.0f;
    if (tid < Lc) {
      const int64_t bth = token_index(a, b, c0 + tid, h);
      d = ld1(static_cast<const TI*>(a.dt), bth);
      const float l = ld1(static_cast<const TI*>(a.lam), bth);
      const float A = (a.flags & kAPerToken) ? a.A[bth] : a.A[h];
      lv = (double)d * (double)A;
      gm = l * d;
      bp = (1.0f - l) * d;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(lv, off, 64);
      if (tid >= off) lv += o;
    }
    tb.cs[tid] = lv;
    tb.dt[tid] = d;
    tb.gam[tid] = gm;
    tb.bpr[tid] = bp;
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    if (vi < NV) {
      const int t = vi / VPT, kv = vi % VPT;
#pragma unroll
      for (int j = 0; j < 8; ++j) th_raw[t * NP + 8 * kv + j] = v[i][j];
    }
  }
  __syncthreads();

  constexpr int NSEG = NT / NP;
  constexpr int SEG = kQ / NSEG;
  static_assert(NSEG >= 1 && kQ % NSEG == 0, "phase segments");
  const int k = tid % NP, sg = tid / NP;
  const bool angle = (a.flags & kThetaIsAngle) != 0;
  double loc[SEG];
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = sg * SEG + i;
    const double tv = (double)th_raw[t * NP + k];
    run += angle ? tv : tv * (double)tb.dt[t];
    loc[i] = run;
  }
  tb.seg[sg * NP + k] = run;
  __syncthreads();
  double base = 0.0;
  for (int s = 0; s < sg; ++s) base += tb.seg[s * NP + k];
  if (sg == NSEG - 1) tb.phi_end[k] = base + run;
  __syncthreads();
  const double pe = tb.phi_end[k];
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = sg * SEG + i;
    if (t < Lc) {
      const double ph = base + loc[i];
      float sn, cn;
      sincosf(reduce_angle(mode == 0 ? ph : pe - ph), &sn, &cn);
      tb.rot[t][k] = f2{cn, sn};
    }
  }
  __syncthreads();
}

// Rows [v0, v0 + 64) of the chunk's B or C (virtual row v = t R + r),
// rotated by -Phi_t, into st[v - v0][n].  16-byte loads, all issued before
// any is used; rows past the chunk's end are zero.
template <class Pol, typename TI, int N, int R, int NT>
__device__ void stage_rows(typename Pol::template Store<kRB, N>& st, const TI* __restrict__ src,
                           const PrefillArgs& a, int b, int h, int c0, int Lc, int v0,
                           const f2 (*rot)[N / 2]) {
  constexpr int E = N * R;
  constexpr int VPT = E / 8;
  constexpr int NTOK = kRB / R;
  constexpr int NV = NTOK * VPT;
  constexpr int IT = (NV + NT - 1) / NT;
  constexpr int NPAIR = 4 / R;              // complex pairs per vector
  const int tid = threadIdx.x;
  const int t0 = v0 / R;
  float v[IT][8];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    const int tl = vi / VPT, e0 = (vi % VPT) * 8;
    if (vi < NV && t0 + tl < Lc) {
      ld8(src, token_index(a, b, c0 + t0 + tl, h) * E + e0, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    if (vi >= NV) continue;
    const int tl = vi / VPT, e0 = (vi % VPT) * 8;
    const int t = t0 + tl;
    const bool ok = t < Lc;
    float o[8];
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
      const int n = e0 / R + 2 * pi;
      const f2 cs = ok ? rot[t][n / 2] : f2{1.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float u0 = v[i][(2 * pi) * R + r], u1 = v[i][(2 * pi + 1) * R + r];
        o[(2 * pi) * R + r] = cs.x * u0 + cs.y * u1;        // rotate by -Phi_t
        o[(2 * pi + 1) * R + r] = -cs.y * u0 + cs.x * u1;
      }
    }
    if constexpr (R == 1) {
      Pol::put8(st, tl, e0, o);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) Pol::put(st, tl * R + j % R, e0 / R + j / R, o[j]);
    }
  }
}

// Rows [v0, v0 + 64) of B rotated by +(Phi_end - Phi_t) and scaled by the
// chunk-state weight W_t, stored transposed: st[n][v - v0].  Consecutive
// lanes take consecutive tokens so the transposed LDS writes do not collide.
template <class Pol, typename TI, int N, int R, int NT>
__device__ void stage_rows_T(typename Pol::template Store<N, kRB>& st, const TI* __restrict__ src,
                             const PrefillArgs& a, int b, int h, int c0, int Lc, int v0,
                             const f2 (*rot)[N / 2], const float* w) {
  constexpr int E = N * R;
  constexpr int VPT = E / 8;
  constexpr int NTOK = kRB / R;
  constexpr int NV = NTOK * VPT;
  constexpr int IT = (NV + NT - 1) / NT;
  constexpr int NPAIR = 4 / R;
  const int tid = threadIdx.x;
  const int t0 = v0 / R;
  float v[IT][8];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    const int tl = vi % NTOK, e0 = (vi / NTOK) * 8;
    if (vi < NV && t0 + tl < Lc) {
      ld8(src, token_index(a, b, c0 + t0 + tl, h) * E + e0, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    if (vi >= NV) continue;
    const int tl = vi % NTOK, e0 = (vi / NTOK) * 8;
    const int t = t0 + tl;
    const bool ok = t < Lc;
    const float wt = ok ? w[t] : 0.0f;
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
      const int n = e0 / R + 2 * pi;
      const f2 cs = ok ? rot[t][n / 2] : f2{1.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float u0 = v[i][(2 * pi) * R + r], u1 = v[i][(2 * pi + 1) * R + r];
        Pol::put(st, n, tl * R + r, wt * (cs.x * u0 - cs.y * u1));   // rotate by +angle
        Pol::put(st, n + 1, tl * R + r, wt * (cs.y * u0 + cs.x * u1));
      }
    }
  }
}

// x rows [v0, v0 + 64) transposed: xs[p][v - v0]
template <class Pol, typename TI, int P, int R, int NT>
__device__ void stage_x_T(typename Pol::template XStore<P, kRB>& xs, const TI* __restrict__ src,
                          const PrefillArgs& a, int b, int h, int c0, int Lc, int v0) {
  constexpr int E = P * R;
  constexpr int VPT = E / 8;
  constexpr int NTOK = kRB / R;
  constexpr int NV = NTOK * VPT;
  constexpr int IT = (NV + NT - 1) / NT;
  const int tid = threadIdx.x;
  const int t0 = v0 / R;
  float v[IT][8];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    const int tl = vi % NTOK, e0 = (vi / NTOK) * 8;
    if (vi < NV && t0 + tl < Lc) {
      ld8(src, token_index(a, b, c0 + t0 + tl, h) * E + e0, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int vi = tid + NT * i;
    if (vi >= NV) continue;
    const int tl = vi % NTOK, e0 = (vi / NTOK) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) Pol::putx(xs, (e0 + j) / R, tl * R + (e0 + j) % R, v[i][j]);
  }
}

// --------------------------------------------------------------------------
// K1: the chunk's own end state S_c (from a zero entry state), rotated into
// the frame of the chunk's end, plus the next chunk's trapezoid
// left-endpoint term (1 - lam_{c1}) dt_{c1} x_{c1-1} B_{c1-1}^T; the chunk's
// total decay and phase go to the workspace.
template <class Pol, typename TI, int P, int N, int R>
struct K1Smem {
  Tables<Geo<P, N, R>::NT, N> tb;
  union U {
    typename Pol::template Store<N, kRB> bw;   // (W_u R(Phi_end - Phi_u) B_u)^T  [n][v]
    float th_raw[kQ * (N / 2)];
  } u;
  typename Pol::template XStore<P, kRB> xs;    // x^T  [p][v]
};

template <class Pol, typename TI, int P, int N, int R>
__global__ __launch_bounds__((Geo<P, N, R>::NT)) void k_chunk_state(PrefillArgs a) {
  using G = Geo<P, N, R>;
  __shared__ K1Smem<Pol, TI, P, N, R> sm;
  constexpr int NQ = G::PT * G::NTL;              // output tiles (p-tile, n-tile)
  constexpr int QPW = (NQ + G::NW - 1) / G::NW;   // per wave
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c0 = c * kQ;
  const int Lc = min(kQ, a.T - c0);
  const int rows = Lc * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t chunk_id = ((int64_t)b * a.H + h) * a.nchunk + c;

  chunk_tables<TI, N, G::NT>(a, b, h, c0, Lc, sm.tb, sm.u.th_raw, 1);
  const double cs_end = sm.tb.cs[Lc - 1];
  if (tid < kQ) {
    float w = 0.0f;
    if (tid < Lc) {
      const float wt = sm.tb.gam[tid] + (tid < Lc - 1 ? sm.tb.bpr[tid + 1] : 0.0f);
      w = expf((float)(cs_end - sm.tb.cs[tid])) * wt;
    }
    sm.tb.aux[tid] = w;
  }
  if (tid < G::NP) {
    float sn, cn;
    sincosf(reduce_angle(sm.tb.phi_end[tid]), &sn, &cn);
    reinterpret_cast<f2*>(a.rot_end)[chunk_id * G::NP + tid] = f2{cn, sn};
  }
  if (tid == 0) a.decay[chunk_id] = expf((float)cs_end);

  f4 acc[QPW];
#pragma unroll
  for (int q = 0; q < QPW; ++q) acc[q] = f4{0, 0, 0, 0};

  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  for (int ub = 0; ub < G::NUB; ++ub) {
    if (ub * kRB >= rows) break;
    __syncthreads();
    stage_rows_T<Pol, TI, N, R, G::NT>(sm.u.bw, Bg, a, b, h, c0, Lc, ub * kRB, sm.tb.rot, sm.tb.aux);
    stage_x_T<Pol, TI, P, R, G::NT>(sm.xs, Xg, a, b, h, c0, Lc, ub * kRB);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRB; kk += Pol::KS) {
#pragma unroll
      for (int q = 0; q < QPW; ++q) {
        const int qq = wave * QPW + q;
        if (qq < NQ) {
          const int pt = qq / G::NTL, nt = qq % G::NTL;
          acc[q] = Pol::mma_x(Pol::frag(sm.u.bw, 16 * nt, kk, lane),
                              Pol::fragx_c(sm.xs, 16 * pt, kk, lane), acc[q]);
        }
      }
    }
  }

  // the next chunk's left-endpoint term, then S_c[p][n..n+3]
  float bpn = 0.0f;
  const TI* xe = nullptr;
  const TI* Be = nullptr;
  if (c + 1 < a.nchunk) {
    const int64_t nx = token_index(a, b, c0 + kQ, h);
    const float d = ld1(static_cast<const TI*>(a.dt), nx);
    const float l = ld1(static_cast<const TI*>(a.lam), nx);
    bpn = (1.0f - l) * d;
    const int64_t last = token_index(a, b, c0 + kQ - 1, h);
    xe = Xg + last * P * R;
    Be = Bg + last * N * R;
  }
  float* __restrict__ S = a.S + chunk_id * P * N;
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    const int qq = wave * QPW + q;
    if (qq < NQ) {
      const int pt = qq / G::NTL, nt = qq % G::NTL;
      const int p = 16 * pt + l16, n = 16 * nt + 4 * g;
      f4 s = acc[q];
      if (xe) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xv = bpn * ld1(xe, (int64_t)p * R + r);
          s.x += xv * ld1(Be, (int64_t)(n + 0) * R + r);
          s.y += xv * ld1(Be, (int64_t)(n + 1) * R + r);
          s.z += xv * ld1(Be, (int64_t)(n + 2) * R + r);
          s.w += xv * ld1(Be, (int64_t)(n + 3) * R + r);
        }
      }
      *reinterpret_cast<f4*>(S + (int64_t)p * N + n) = s;
    }
  }
}

// --------------------------------------------------------------------------
// K2: serial pass over the chunks of one (batch, head), 16 state rows per
// block.  Entering chunk c the state (plus that chunk's left-endpoint term)
// is Shat_c; Shat_{c+1} = decay_c R(Phi_end,c) Shat_c + S_c, where S_c
// already carries the next chunk's left-endpoint term.  Shat_c replaces S_c
// in the workspace.  The loads of chunk c + D are issued while chunk c is
// processed.
template <typename TI, int N, int R>
__global__ __launch_bounds__(256) void k_state_pass(PrefillArgs a) {
  constexpr int VPR = N / 4;
  constexpr int NV = 16 * VPR;
  constexpr int VPT = (NV + 255) / 256;
  constexpr int D = 4;
  const int P = a.P;
  const int slices = P / 16;
  const int bh = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;

  int pv[VPT], nv[VPT];
  bool ok[VPT];
  f4 S[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = tid + 256 * i;
    ok[i] = v < NV;
    pv[i] = 16 * sl + (ok[i] ? v / VPR : 0);
    nv[i] = ok[i] ? 4 * (v % VPR) : 0;
    S[i] = f4{0, 0, 0, 0};
    if (ok[i] && a.h0) S[i] = *reinterpret_cast<const f4*>(a.h0 + ((int64_t)bh * P + pv[i]) * N + nv[i]);
  }
  if (a.has_prev) {  // left-endpoint term of token 0
    const int64_t t0 = token_index(a, b, 0, h);
    const float d = ld1(static_cast<const TI*>(a.dt), t0);
    const float l = ld1(static_cast<const TI*>(a.lam), t0);
    const float bp0 = (1.0f - l) * d;
    const TI* xh = static_cast<const TI*>(a.xp) + (int64_t)bh * P * R;
    const TI* Bh = static_cast<const TI*>(a.Bp) + (int64_t)bh * N * R;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (!ok[i]) continue;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float xv = bp0 * ld1(xh, (int64_t)pv[i] * R + r);
        S[i].x += xv * ld1(Bh, (int64_t)(nv[i] + 0) * R + r);
        S[i].y += xv * ld1(Bh, (int64_t)(nv[i] + 1) * R + r);
        S[i].z += xv * ld1(Bh, (int64_t)(nv[i] + 2) * R + r);
        S[i].w += xv * ld1(Bh, (int64_t)(nv[i] + 3) * R + r);
      }
    }
  }
  const int64_t cbase = (int64_t)bh * a.nchunk;
  const int nch = a.nchunk;
  f4 bs[D][VPT];
  f2 br0[D][VPT], br1[D][VPT];
  float bd[D];
  auto load = [&](int c, int q) {
    if (c < nch) {
      const int64_t cid = cbase + c;
      const float* Sc = a.S + cid * P * N;
      const f2* re = reinterpret_cast<const f2*>(a.rot_end) + cid * (N / 2);
      bd[q] = a.decay[cid];
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        if (!ok[i]) continue;
        bs[q][i] = *reinterpret_cast<const f4*>(Sc + (int64_t)pv[i] * N + nv[i]);
        br0[q][i] = re[nv[i] / 2];
        br1[q][i] = re[nv[i] / 2 + 1];
      }
    }
  };
#pragma unroll
  for (int q = 0; q < D; ++q) load(q, q);
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int c = c0 + q;
      if (c < nch) {
        float* Sc = a.S + (cbase + c) * P * N;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
          if (!ok[i]) continue;
          *reinterpret_cast<f4*>(Sc + (int64_t)pv[i] * N + nv[i]) = S[i];   // Shat_c
          S[i] = bd[q] * rot2pairs(S[i], br0[q][i], br1[q][i]) + bs[q][i];
        }
        load(c + D, q);
      }
    }
  }
  if (a.hT) {
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (ok[i]) *reinterpret_cast<f4*>(a.hT + ((int64_t)bh * P + pv[i]) * N + nv[i]) = S[i];
  }
}

// --------------------------------------------------------------------------
// K3: all outputs of one chunk
template <class Pol, typename TI, int P, int N, int R>
struct K3Smem {
  Tables<Geo<P, N, R>::NT, N> tb;
  union U {
    typename Pol::template Store<kRB, N> st;   // rotated C or B rows   [v][n]
    typename Pol::template Store<P, N> sh;     // Shat                  [p][n]
    float th_raw[kQ * (N / 2)];
  } u;
  typename Pol::template XStore<P, kRB> xs;    // x^T block             [p][v]
};

template <class Pol, typename TI, typename TO, int P, int N, int R>
__global__ __launch_bounds__((Geo<P, N, R>::NT)) void k_chunk_output(PrefillArgs a) {
  using G = Geo<P, N, R>;
  __shared__ K3Smem<Pol, TI, P, N, R> sm;
  constexpr int NKS = N / Pol::KS;
  constexpr int UG = 16 * Pol::DT;          // u rows per A fragment built from D tiles
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c0 = c * kQ;
  const int Lc = min(kQ, a.T - c0);
  const int rows = Lc * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t chunk_id = ((int64_t)b * a.H + h) * a.nchunk + c;

  chunk_tables<TI, N, G::NT>(a, b, h, c0, Lc, sm.tb, sm.u.th_raw, 0);
  if (tid < kQ) sm.tb.aux[tid] = tid < Lc ? expf((float)sm.tb.cs[tid]) : 0.0f;

  int tile[G::TPW];
  tile[0] = wave;
  if constexpr (G::TPW == 2) tile[1] = 2 * G::NW - 1 - wave;

  const TI* __restrict__ Cg = static_cast<const TI*>(a.C);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);

  // own rotated C rows -> MFMA fragments in registers
  typename Pol::Frag cf[G::TPW][NKS];
#pragma unroll
  for (int j = 0; j < G::TPW; ++j)
#pragma unroll
    for (int s = 0; s < NKS; ++s) cf[j][s] = typename Pol::Frag{};
  for (int blk = 0; blk < G::NUB; ++blk) {
    if (blk * kRB >= rows) break;
    __syncthreads();
    stage_rows<Pol, TI, N, R, G::NT>(sm.u.st, Cg, a, b, h, c0, Lc, blk * kRB, sm.tb.rot);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G::TPW; ++j)
      if (tile[j] / 4 == blk) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) cf[j][s] = Pol::frag(sm.u.st, 16 * (tile[j] % 4), s * Pol::KS, lane);
      }
  }

  // Y_off = e^{cs_t} Ct Shat^T
  __syncthreads();
  {
    const float* __restrict__ Sh = a.S + chunk_id * P * N;
    constexpr int NV = P * N / 8;
    constexpr int IT = (NV + G::NT - 1) / G::NT;
    float v[IT][8];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = tid + G::NT * i;
      if (vi < NV) ld8(Sh, (int64_t)vi * 8, v[i]);
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int vi = tid + G::NT * i;
      if (vi < NV) Pol::put8(sm.u.sh, (vi * 8) / N, (vi * 8) % N, v[i]);
    }
  }
  __syncthreads();
  f4 acc[G::TPW][G::PT];
#pragma unroll
  for (int j = 0; j < G::TPW; ++j) {
#pragma unroll
    for (int ct = 0; ct < G::PT; ++ct) {
      f4 d = f4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s) d = Pol::mma(cf[j][s], Pol::frag(sm.u.sh, 16 * ct, s * Pol::KS, lane), d);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int vv = 16 * tile[j] + 4 * g + jj;
        d[jj] *= vv < rows ? sm.tb.aux[vv / R] : 0.0f;
      }
      acc[j][ct] = d;
    }
  }

  // Y_diag: Gram tiles Bt Ct^T (D rows = u, columns = own rows), decay mask,
  // then the masked tile is the A operand of the product with x
  for (int ub = 0; ub < G::NUB; ++ub) {
    if (ub * kRB >= rows) break;
    __syncthreads();
    stage_rows<Pol, TI, N, R, G::NT>(sm.u.st, Bg, a, b, h, c0, Lc, ub * kRB, sm.tb.rot);
    stage_x_T<Pol, TI, P, R, G::NT>(sm.xs, Xg, a, b, h, c0, Lc, ub * kRB);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G::TPW; ++j) {
      const int i = tile[j];
      const int vrow = 16 * i + l16;
      const int tt = vrow / R;
      const bool row_ok = vrow < rows;
      const int tmax = min(Lc - 1, (16 * i + 15) / R);
      const double cst = sm.tb.cs[min(tt, kQ - 1)];
      for (int ug = 0; ug < kRB; ug += UG) {
        const int ubase = ub * kRB + ug;
        if (ubase / R > tmax) break;
        f4 d[Pol::DT];
#pragma unroll
        for (int dt = 0; dt < Pol::DT; ++dt) {
          f4 gt = f4{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            gt = Pol::mma(Pol::frag(sm.u.st, ug + 16 * dt, s * Pol::KS, lane), cf[j][s], gt);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int tu = (ubase + 16 * dt + 4 * g + jj) / R;
            float m = 0.0f;
            if (row_ok && tu <= tt) {
              const float w = sm.tb.gam[tu] + (tu < tt ? sm.tb.bpr[tu + 1] : 0.0f);
              m = __expf((float)(cst - sm.tb.cs[tu])) * w;
            }
            gt[jj] *= m;
          }
          d[dt] = gt;
        }
        const typename Pol::Frag af = Pol::frag_from_d(d);
#pragma unroll
        for (int ct = 0; ct < G::PT; ++ct)
          acc[j][ct] = Pol::mma_x(af, Pol::fragx_d(sm.xs, 16 * ct, ug, lane), acc[j][ct]);
      }
    }
  }

  // y[b, c0 + t, h, p, r] for D rows v = 16 tile + 4g + jj, column p
  TO* __restrict__ Y = static_cast<TO*>(a.y);
#pragma unroll
  for (int j = 0; j < G::TPW; ++j) {
#pragma unroll
    for (int ct = 0; ct < G::PT; ++ct) {
      const int p = 16 * ct + l16;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int v = 16 * tile[j] + 4 * g + jj;
        if (v < rows)
          st1(Y, (token_index(a, b, c0 + v / R, h) * P + p) * R + v % R, acc[j][ct][jj]);
      }
    }
  }
}

// --------------------------------------------------------------------------
template <class Pol, typename TI, typename TO, int P, int N, int R>
static hipError_t run_prefill(const PrefillArgs& a, hipStream_t s) {
  using G = Geo<P, N, R>;
  hipLaunchKernelGGL((k_chunk_state<Pol, TI, P, N, R>), dim3(a.nchunk, a.H, a.Bsz), dim3(G::NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_state_pass<TI, N, R>), dim3(a.Bsz * a.H * (P / 16)), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_chunk_output<Pol, TI, TO, P, N, R>), dim3(a.nchunk, a.H, a.Bsz), dim3(G::NT),
                     0, s, a);
  return hipGetLastError();
}

template <class Pol, typename TI, typename TO>
static int dispatch_shape(const PrefillArgs& a, hipStream_t s, hipError_t* e) {
#define M3_SHAPE(PP, NN, RR)                                  \
  if constexpr (NN % Pol::KS == 0) {                          \
    if (a.P == PP && a.N == NN && a.R == RR) {                \
      *e = run_prefill<Pol, TI, TO, PP, NN, RR>(a, s);        \
      return 0;                                               \
    }                                                         \
  }
  M3_SHAPE(16, 16, 1)
  M3_SHAPE(64, 128, 1)
  M3_SHAPE(64, 128, 4)
  M3_SHAPE(64, 128, 2)
  M3_SHAPE(32, 64, 1)
  M3_SHAPE(32, 64, 4)
#undef M3_SHAPE
  return -1;
}

bool prefill_supported(int P, int N, int R, int Q, int in_bf16) {
  if (Q != kQ) return false;
  const bool shape = (P == 16 && N == 16 && R == 1) ||
                     (P == 64 && N == 128 && (R == 1 || R == 2 || R == 4)) ||
                     (P == 32 && N == 64 && (R == 1 || R == 4));
  if (!shape) return false;
  if (in_bf16 && N % 32 != 0) return false;  // fp16 fragments span 32 state columns
  return true;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t prefill_workspace_bytes(int Bsz, int T, int H, int P, int N, int Q) {
  const size_t nchunk = (size_t)(T + Q - 1) / Q;
  const size_t units = (size_t)Bsz * H * nchunk;
  return align256(units * P * N * 4) + align256(units * N * 4) + align256(units * 4);
}

void prefill_carve(PrefillArgs& a, void* ws) {
  const size_t units = (size_t)a.Bsz * a.H * a.nchunk;
  char* p = static_cast<char*>(ws);
  a.S = reinterpret_cast<float*>(p);
  p += align256(units * a.P * a.N * 4);
  a.rot_end = reinterpret_cast<float*>(p);
  p += align256(units * a.N * 4);
  a.decay = reinterpret_cast<float*>(p);
}

int launch_prefill(const PrefillArgs& a, int in_bf16, int out_bf16, hipStream_t s, hipError_t* e) {
  if (in_bf16) {
    return out_bf16 ? dispatch_shape<PolF16, bf16_t, bf16_t>(a, s, e)
                    : dispatch_shape<PolF16, bf16_t, float>(a, s, e);
  }
  return out_bf16 ? dispatch_shape<PolF32, float, bf16_t>(a, s, e)
                  : dispatch_shape<PolF32, float, float>(a, s, e);
}

}  // namespace m3
