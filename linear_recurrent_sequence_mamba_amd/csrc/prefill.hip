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
// per-chunk token tables: chunk-local cumulative log-decay (double), gamma,
// beta' = (1 - lam) dt
template <typename TI>
__device__ __forceinline__ void token_tables(const PrefillArgs& a, int b, int h, int c0, int Lc,
                                             double* cs, float* gam, float* bpr) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    double v = 0.0;
    float gm = 0.0f, bp = 0.0f;
    if (tid < Lc) {
      const int64_t bth = ((int64_t)b * a.T + c0 + tid) * a.H + h;
      const float d = ld1(static_cast<const TI*>(a.dt), bth);
      const float l = ld1(static_cast<const TI*>(a.lam), bth);
      const float A = (a.flags & kAPerToken) ? a.A[bth] : a.A[h];
      v = (double)d * (double)A;
      gm = l * d;
      bp = (1.0f - l) * d;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(v, off, 64);
      if (tid >= off) v += o;
    }
    cs[tid] = v;
    gam[tid] = gm;
    bpr[tid] = bp;
  }
}

__device__ __forceinline__ float reduce_angle(double phi) {
  return (float)(phi - kTwoPi * rint(phi / kTwoPi));
}

// Chunk-local cumulative phases Phi[t][k] (double), for all t < Lc and
// k < N/2.  Each thread owns one pair k and a segment of tokens.  On return
// phi_end[k] holds Phi[Lc-1][k]; when `store` is true, rot[t][k] receives
// (cos, sin) of Phi[t][k] (mode 0) or of Phi_end - Phi[t] (mode 1).
template <typename TI, int N>
__device__ void phase_tables(const PrefillArgs& a, int b, int h, int c0, int Lc, f2* rot,
                             double* seg_sum, double* phi_end, int mode) {
  constexpr int NP = N / 2;
  constexpr int NSEG = 256 / NP;     // token segments per pair
  constexpr int SEG = kQ / NSEG;     // tokens per segment
  const int tid = threadIdx.x;
  const int k = tid % NP, seg = tid / NP;
  const TI* __restrict__ th = static_cast<const TI*>(a.theta);
  const TI* __restrict__ dtp = static_cast<const TI*>(a.dt);
  const bool angle = (a.flags & kThetaIsAngle) != 0;
  double loc[SEG];
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = seg * SEG + i;
    double p = 0.0;
    if (t < Lc) {
      const int64_t bth = ((int64_t)b * a.T + c0 + t) * a.H + h;
      const double tv = (double)ld1(th, bth * NP + k);
      p = angle ? tv : tv * (double)ld1(dtp, bth);
    }
    run += p;
    loc[i] = run;
  }
  seg_sum[seg * NP + k] = run;
  __syncthreads();
  double base = 0.0;
  for (int s = 0; s < seg; ++s) base += seg_sum[s * NP + k];
  if (seg == NSEG - 1) {
    double tot = base + run;
    phi_end[k] = tot;
  }
  __syncthreads();
  const double pe = phi_end[k];
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int t = seg * SEG + i;
    if (t < Lc) {
      const double ph = base + loc[i];
      const float r = reduce_angle(mode == 0 ? ph : pe - ph);
      float s, c;
      sincosf(r, &s, &c);
      rot[t * NP + k] = f2{c, s};
    }
  }
}

// --------------------------------------------------------------------------
// K1: per-chunk state S_c and the chunk's decay / phase totals
template <class Pol, typename TI, int P, int N, int R>
struct K1Smem {
  double cs[kQ];
  float gam[kQ], bpr[kQ], wu[kQ];
  double seg_sum[256];
  double phi_end[N / 2];
  f2 rot[kQ * (N / 2)];
  typename Pol::template Store<N, kRB> bw;   // (W_u R(Phi_end - Phi_u) B_u)^T  [n][u]
  typename Pol::template XStore<P, kRB> xs;  // x^T  [p][u]
};

template <class Pol, typename TI, int P, int N, int R>
__global__ __launch_bounds__(256) void k_chunk_state(PrefillArgs a) {
  __shared__ K1Smem<Pol, TI, P, N, R> sm;
  constexpr int NP = N / 2;
  constexpr int NT = N / 16;
  constexpr int PT = P / 16;
  constexpr int PTW = (PT + 3) / 4;  // p-tiles per wave
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c0 = c * kQ;
  const int Lc = min(kQ, a.T - c0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk_id = ((int64_t)b * a.H + h) * a.nchunk + c;

  token_tables<TI>(a, b, h, c0, Lc, sm.cs, sm.gam, sm.bpr);
  phase_tables<TI, N>(a, b, h, c0, Lc, sm.rot, sm.seg_sum, sm.phi_end, 1);
  // (phase_tables synchronises, so the token tables are visible here)
  const double cs_end = sm.cs[Lc - 1];
  if (tid < kQ) {
    float w = 0.0f;
    if (tid < Lc) {
      const float wt = sm.gam[tid] + (tid < Lc - 1 ? sm.bpr[tid + 1] : 0.0f);
      w = expf((float)(cs_end - sm.cs[tid])) * wt;
    }
    sm.wu[tid] = w;
  }
  if (tid < NP) {
    float s, co;
    sincosf(reduce_angle(sm.phi_end[tid]), &s, &co);
    a.rot_end[chunk_id * N + 2 * tid] = co;
    a.rot_end[chunk_id * N + 2 * tid + 1] = s;
  }
  if (tid == 0) a.decay[chunk_id] = expf((float)cs_end);

  f4 acc[PTW][NT];
#pragma unroll
  for (int i = 0; i < PTW; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f4{0, 0, 0, 0};

  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  const int rows = Lc * R;
  for (int ub = 0; ub * kRB < rows; ++ub) {
    __syncthreads();
    // stage (W_u R(Phi_end - Phi_u) B_u)^T: thread -> (virtual row, pair)
    for (int idx = tid; idx < kRB * NP; idx += 256) {
      const int k = idx % NP, ul = idx / NP;
      const int v = ub * kRB + ul;
      float o0 = 0.0f, o1 = 0.0f;
      if (v < rows) {
        const int t = v / R, r = v % R;
        const int64_t base = (((int64_t)b * a.T + c0 + t) * a.H + h) * N * R;
        const float u0 = ld1(Bg, base + (2 * k) * R + r);
        const float u1 = ld1(Bg, base + (2 * k + 1) * R + r);
        const f2 cs = sm.rot[t * NP + k];
        const float w = sm.wu[t];
        o0 = w * (cs.x * u0 - cs.y * u1);
        o1 = w * (cs.y * u0 + cs.x * u1);
      }
      Pol::put(sm.bw, 2 * k, ul, o0);
      Pol::put(sm.bw, 2 * k + 1, ul, o1);
    }
    // stage x^T: thread -> (virtual row, p)
    for (int idx = tid; idx < kRB * P; idx += 256) {
      const int p = idx % P, ul = idx / P;
      const int v = ub * kRB + ul;
      float xv = 0.0f;
      if (v < rows) {
        const int t = v / R, r = v % R;
        xv = ld1(Xg, ((((int64_t)b * a.T + c0 + t) * a.H + h) * P + p) * R + r);
      }
      Pol::putx(sm.xs, p, ul, xv);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PTW; ++i) {
      const int pt = wave + 4 * i;
      if (pt < PT) {
#pragma unroll
        for (int kk = 0; kk < kRB; kk += Pol::KS) {
          const typename Pol::XFrag xf = Pol::fragx_c(sm.xs, 16 * pt, kk, lane);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[i][nt] = Pol::mma_x(Pol::frag(sm.bw, 16 * nt, kk, lane), xf, acc[i][nt]);
        }
      }
    }
  }
  // S_c[p][n..n+3]: D rows are n (16nt + 4g + j), columns p (16pt + lane%16)
  float* __restrict__ S = a.S + chunk_id * P * N;
#pragma unroll
  for (int i = 0; i < PTW; ++i) {
    const int pt = wave + 4 * i;
    if (pt < PT) {
      const int p = 16 * pt + (lane & 15);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f4*>(S + (int64_t)p * N + 16 * nt + 4 * (lane >> 4)) = acc[i][nt];
    }
  }
}

// --------------------------------------------------------------------------
// K2: serial pass over the chunks of one (batch, head), 16 state rows per block
template <typename TI, int N, int R>
__global__ __launch_bounds__(256) void k_state_pass(PrefillArgs a) {
  constexpr int VPR = N / 4;               // float4 vectors per state row
  constexpr int NV = 16 * VPR;             // vectors per block
  constexpr int VPT = (NV + 255) / 256;    // vectors per thread
  const int P = a.P;
  const int slices = P / 16;
  const int bh = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);

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
  const int64_t cbase = (int64_t)bh * a.nchunk;
  for (int c = 0; c < a.nchunk; ++c) {
    const int c0 = c * kQ;
    const int64_t cid = cbase + c;
    // trapezoid left-endpoint term of the chunk's first token
    float bp0 = 0.0f;
    const TI* xh = nullptr;
    const TI* Bh = nullptr;
    {
      const int64_t bth = ((int64_t)b * a.T + c0) * a.H + h;
      const float d = ld1(static_cast<const TI*>(a.dt), bth);
      const float l = ld1(static_cast<const TI*>(a.lam), bth);
      bp0 = (1.0f - l) * d;
      if (c == 0) {
        if (a.has_prev) {
          xh = static_cast<const TI*>(a.xp) + (int64_t)bh * P * R;
          Bh = static_cast<const TI*>(a.Bp) + (int64_t)bh * N * R;
        }
      } else {
        const int64_t prev = ((int64_t)b * a.T + c0 - 1) * a.H + h;
        xh = Xg + prev * P * R;
        Bh = Bg + prev * N * R;
      }
    }
    const float dec = a.decay[cid];
    float* __restrict__ Sc = a.S + cid * P * N;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (!ok[i]) continue;
      float* ptr = Sc + (int64_t)pv[i] * N + nv[i];
      const f4 sc = *reinterpret_cast<const f4*>(ptr);
      f4 sh = S[i];
      if (xh) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xv = bp0 * ld1(xh, (int64_t)pv[i] * R + r);
          sh.x += xv * ld1(Bh, (int64_t)(nv[i] + 0) * R + r);
          sh.y += xv * ld1(Bh, (int64_t)(nv[i] + 1) * R + r);
          sh.z += xv * ld1(Bh, (int64_t)(nv[i] + 2) * R + r);
          sh.w += xv * ld1(Bh, (int64_t)(nv[i] + 3) * R + r);
        }
      }
      *reinterpret_cast<f4*>(ptr) = sh;   // state entering chunk c
      const f2* re = reinterpret_cast<const f2*>(a.rot_end + cid * N);
      S[i] = dec * rot2pairs(sh, re[nv[i] / 2], re[nv[i] / 2 + 1]) + sc;
    }
  }
  if (a.hT) {
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (ok[i]) *reinterpret_cast<f4*>(a.hT + ((int64_t)bh * P + pv[i]) * N + nv[i]) = S[i];
  }
}

// --------------------------------------------------------------------------
// K3: outputs of one 64-virtual-row block of one chunk
template <class Pol, typename TI, int P, int N, int R>
struct K3Smem {
  double cs[kQ];
  float gam[kQ], bpr[kQ], ecs[kQ];
  double seg_sum[256];
  double phi_end[N / 2];
  f2 rot[kQ * (N / 2)];
  float mtok[kRB / R + 1][kQ];
  union U {
    typename Pol::template Store<kRB, N> bt;  // rotated B block  [u][n]
    typename Pol::template Store<P, N> sh;    // Shat             [p][n]
    float craw[kRB][N + 4];                   // own C rows (before rotation)
  } u;
  typename Pol::template XStore<P, kRB> xs;   // x^T block        [p][u]
};

template <class Pol, typename TI, typename TO, int P, int N, int R>
__global__ __launch_bounds__(256) void k_chunk_output(PrefillArgs a) {
  __shared__ K3Smem<Pol, TI, P, N, R> sm;
  constexpr int NP = N / 2;
  constexpr int PT = P / 16;
  constexpr int NKS = N / Pol::KS;
  constexpr int NRB = (kQ * R + kRB - 1) / kRB;
  constexpr int UG = 16 * Pol::DT;    // u rows per A fragment built from D tiles
  // block -> (chunk, row block); the row blocks of one chunk share an XCD
  const int bid = blockIdx.x;
  const int grp = bid / (8 * NRB), rem = bid % (8 * NRB);
  const int c = grp * 8 + rem % 8, rb = rem / 8;
  const int h = blockIdx.y, b = blockIdx.z;
  if (c >= a.nchunk) return;
  const int c0 = c * kQ;
  const int Lc = min(kQ, a.T - c0);
  const int rows = Lc * R;
  const int row0 = rb * kRB;
  if (row0 >= rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t chunk_id = ((int64_t)b * a.H + h) * a.nchunk + c;
  const int tok0 = row0 / R;                                // first own token
  const int tok1 = min(Lc - 1, (row0 + kRB - 1) / R);       // last own token

  token_tables<TI>(a, b, h, c0, Lc, sm.cs, sm.gam, sm.bpr);
  // own C rows -> craw (before the phase tables overwrite nothing: separate)
  {
    const TI* __restrict__ Cg = static_cast<const TI*>(a.C);
    for (int idx = tid; idx < kRB * N; idx += 256) {
      const int n = idx % N, vl = idx / N;
      const int v = row0 + vl;
      float cv = 0.0f;
      if (v < rows) {
        const int t = v / R, r = v % R;
        cv = ld1(Cg, (((int64_t)b * a.T + c0 + t) * a.H + h) * N * R + (int64_t)n * R + r);
      }
      sm.u.craw[vl][n] = cv;
    }
  }
  phase_tables<TI, N>(a, b, h, c0, Lc, sm.rot, sm.seg_sum, sm.phi_end, 0);
  if (tid < kQ) sm.ecs[tid] = tid < Lc ? expf((float)sm.cs[tid]) : 0.0f;
  // decay mask for the own tokens: M[t][u] = e^{cs_t - cs_u} w_{t,u}, u <= t
  for (int idx = tid; idx < (tok1 - tok0 + 1) * kQ; idx += 256) {
    const int tl = idx / kQ, u = idx % kQ;
    const int t = tok0 + tl;
    float m = 0.0f;
    if (u <= t) {
      const float w = sm.gam[u] + (u < t ? sm.bpr[u + 1] : 0.0f);
      m = expf((float)(sm.cs[t] - sm.cs[u])) * w;
    }
    sm.mtok[tl][u] = m;
  }
  __syncthreads();

  // own rotated C rows -> fragments in registers: row v = row0 + 16*wave + l16
  const int vrow = row0 + 16 * wave + l16;
  const int trow = min(vrow / R, Lc - 1);
  typename Pol::Frag cf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    constexpr int KPL = Pol::KS / 4;
    float v[KPL];
    const int n0 = s * Pol::KS + KPL * g;
#pragma unroll
    for (int j = 0; j < KPL; j += 2) {
      const float u0 = sm.u.craw[16 * wave + l16][n0 + j];
      const float u1 = sm.u.craw[16 * wave + l16][n0 + j + 1];
      const f2 cs = sm.rot[trow * NP + (n0 + j) / 2];
      v[j] = cs.x * u0 + cs.y * u1;       // rotate by -Phi
      v[j + 1] = -cs.y * u0 + cs.x * u1;
    }
    cf[s] = Pol::make(v);
  }
  __syncthreads();

  // Y_off = e^{cs_t} Ct Shat^T
  f4 acc[PT];
  {
    const float* __restrict__ Sh = a.S + chunk_id * P * N;
    for (int idx = tid; idx < P * N / 4; idx += 256) {
      const int p = idx / (N / 4), n = 4 * (idx % (N / 4));
      const f4 v = *reinterpret_cast<const f4*>(Sh + (int64_t)p * N + n);
      Pol::put(sm.u.sh, p, n, v.x);
      Pol::put(sm.u.sh, p, n + 1, v.y);
      Pol::put(sm.u.sh, p, n + 2, v.z);
      Pol::put(sm.u.sh, p, n + 3, v.w);
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < PT; ++ct) {
      f4 d = f4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s) d = Pol::mma(cf[s], Pol::frag(sm.u.sh, 16 * ct, s * Pol::KS, lane), d);
      // D rows are virtual rows 16*wave + 4g + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vv = row0 + 16 * wave + 4 * g + j;
        const float e = vv < rows ? sm.ecs[vv / R] : 0.0f;
        d[j] *= e;
      }
      acc[ct] = d;
    }
  }

  // Y_diag over the u blocks that reach the own rows
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  const int my_tmax = min(Lc - 1, (row0 + 16 * wave + 15) / R);  // last token of own tile
  const int ulim = min(rows, (tok1 + 1) * R);                      // u rows needed by the block
  for (int ub = 0; ub * kRB < ulim; ++ub) {
    __syncthreads();
    for (int idx = tid; idx < kRB * NP; idx += 256) {
      const int k = idx % NP, ul = idx / NP;
      const int v = ub * kRB + ul;
      float o0 = 0.0f, o1 = 0.0f;
      if (v < rows) {
        const int t = v / R, r = v % R;
        const int64_t base = (((int64_t)b * a.T + c0 + t) * a.H + h) * N * R;
        const float u0 = ld1(Bg, base + (2 * k) * R + r);
        const float u1 = ld1(Bg, base + (2 * k + 1) * R + r);
        const f2 cs = sm.rot[t * NP + k];
        o0 = cs.x * u0 + cs.y * u1;
        o1 = -cs.y * u0 + cs.x * u1;
      }
      Pol::put(sm.u.bt, ul, 2 * k, o0);
      Pol::put(sm.u.bt, ul, 2 * k + 1, o1);
    }
    for (int idx = tid; idx < kRB * P; idx += 256) {
      const int p = idx % P, ul = idx / P;
      const int v = ub * kRB + ul;
      float xv = 0.0f;
      if (v < rows) {
        const int t = v / R, r = v % R;
        xv = ld1(Xg, ((((int64_t)b * a.T + c0 + t) * a.H + h) * P + p) * R + r);
      }
      Pol::putx(sm.xs, p, ul, xv);
    }
    __syncthreads();
    for (int ug = 0; ug < kRB; ug += UG) {
      const int ubase = ub * kRB + ug;
      if (ubase / R > my_tmax) break;   // causal: nothing left for this tile
      f4 d[Pol::DT];
#pragma unroll
      for (int dt = 0; dt < Pol::DT; ++dt) {
        f4 gt = f4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NKS; ++s)
          gt = Pol::mma(Pol::frag(sm.u.bt, ug + 16 * dt, s * Pol::KS, lane), cf[s], gt);
        // gt: rows u = ubase + 16dt + 4g + j, column t-row = own row l16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int uv = ubase + 16 * dt + 4 * g + j;
          const int tu = uv / R;
          const int tt = vrow / R;
          float m = 0.0f;
          if (vrow < rows && uv < rows && tu <= tt) m = sm.mtok[tt - tok0][tu];
          gt[j] *= m;
        }
        d[dt] = gt;
      }
      const typename Pol::Frag af = Pol::frag_from_d(d);
#pragma unroll
      for (int ct = 0; ct < PT; ++ct)
        acc[ct] = Pol::mma_x(af, Pol::fragx_d(sm.xs, 16 * ct, ug, lane), acc[ct]);
    }
  }

  // y[b, c0 + t, h, p, r] for D rows v = row0 + 16*wave + 4g + j, column p
  TO* __restrict__ Y = static_cast<TO*>(a.y);
#pragma unroll
  for (int ct = 0; ct < PT; ++ct) {
    const int p = 16 * ct + l16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = row0 + 16 * wave + 4 * g + j;
      if (v < rows) {
        const int t = v / R, r = v % R;
        st1(Y, ((((int64_t)b * a.T + c0 + t) * a.H + h) * P + p) * R + r, acc[ct][j]);
      }
    }
  }
}

// --------------------------------------------------------------------------
template <class Pol, typename TI, typename TO, int P, int N, int R>
static hipError_t run_prefill(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_state<Pol, TI, P, N, R>), dim3(a.nchunk, a.H, a.Bsz), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_state_pass<TI, N, R>), dim3(a.Bsz * a.H * (P / 16)), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NRB = (kQ * R + kRB - 1) / kRB;
  const int groups = (a.nchunk + 7) / 8;
  hipLaunchKernelGGL((k_chunk_output<Pol, TI, TO, P, N, R>), dim3(groups * 8 * NRB, a.H, a.Bsz),
                     dim3(256), 0, s, a);
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
  const bool shape = (P == 16 && N == 16 && R == 1) || (P == 64 && N == 128 && (R == 1 || R == 2 || R == 4)) ||
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
