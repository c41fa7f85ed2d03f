// decode_tokens.hip -- several decode steps in one launch on gfx950.
//
// K consecutive tokens advance the fp32 state h [Bsz,H,P,N] in place, the
// recurrence of the Mamba-3 article [xxxxx.co.kr, sections 1.1-1.3] applied
// token after token:
//   h <- R(phi_k) (alpha_k h + beta_k X_{k-1} B_{k-1}^T) + gamma_k X_k B_k^T,
//   y_k = h C_k.
// The state of a (batch, head) stays in registers for all K tokens, so it
// crosses HBM once in and once out per call instead of once per token; the
// per-token inputs stream past it, the next token's loads in flight while
// the current token is applied.
//
//  * k_decode_siso_tok (R = 1): the thread layout of the single-step kernel
//    (a state row over N/4 lanes, 4 consecutive columns per lane); a block
//    holds up to 8 rows per lane for all K tokens, and a unit with more rows
//    is split over several blocks.
//  * k_decode_mimo_grp (R = 4): the group form.  Over a group of four
//    tokens the recurrence unrolls into the chunked form of the prefill, so
//    the state is decayed and rotated once per group and its products (the
//    group's outputs, its rank-4 terms) are MFMA contractions with the
//    state's own registers as operands.
//  * k_decode_mimo_tok (R = 2, 3, 8): token after token.  One 16-row block
//    of the state per wave, P <= 64, in the MFMA D layout (the rank-R terms
//    are MFMA products with K = R, as in the single-step kernel), loaded in
//    that layout and stored through a per-wave LDS transpose (whole lines
//    per store); the token tables of a group of tokens are built once per
//    block.  Both MIMO kernels store the state that way.
#include "m3_device.h"
#include "m3_launch.h"

#ifndef M3_MONEG_WAVES
#define M3_MONEG_WAVES 4
#endif
#ifndef M3_ONEG_WAVES
#define M3_ONEG_WAVES 6
#endif
namespace m3 {

namespace {

// token k of the unit bh = (b, h): per-head tensors [Bsz, K, H, ...] and
// per-group tensors [Bsz, K, G, ...]
__device__ __forceinline__ int64_t tok_head(const DecodeArgs& a, int bh, int k) {
  return ((int64_t)(bh / a.H) * a.K + k) * a.H + bh % a.H;
}
__device__ __forceinline__ int64_t tok_group(const DecodeArgs& a, int bh, int k) {
  return ((int64_t)(bh / a.H) * a.K + k) * a.G + (bh % a.H) / (a.H / a.G);
}
__device__ __forceinline__ int64_t unit_group(const DecodeArgs& a, int bh) {
  return (int64_t)(bh / a.H) * a.G + (bh % a.H) / (a.H / a.G);
}

// the token scalars; pair phases of token k into cs (threads < N/2)
template <typename TI, int N>
struct TokScalars {
  Raw1<TI> d_, l_, th_;   // as loaded; converted where used
  float A;
  __device__ __forceinline__ void load(const DecodeArgs& a, int bh, int k) {
    const int64_t t = tok_head(a, bh, k);
    d_.load(static_cast<const TI*>(a.dt), t);
    l_.load(static_cast<const TI*>(a.lam), t);
    A = (a.flags & kAPerToken) ? a.A[t] : a.A[bh % a.H];
    // every thread reads (threads past the pairs re-read the last pair and
    // never use it): no branch around the load
    const int kk = min(static_cast<int>(threadIdx.x), N / 2 - 1);
    th_.load(static_cast<const TI*>(a.theta), tok_group(a, bh, k) * (N / 2) + kk);
  }
  __device__ __forceinline__ float d() const { return d_.f(); }
  __device__ __forceinline__ void finish(const DecodeArgs& a, float& alpha, float& beta,
                                         float& gamma, f2* cs) const {
    const float d = d_.f(), l = l_.f(), th = th_.f();
    alpha = expf(d * A);
    beta = (1.0f - l) * d * alpha;
    gamma = l * d;
    const int kk = threadIdx.x;
    if (kk < N / 2) cs[kk] = cos_sin_turns((a.flags & kThetaIsAngle) ? th : d * th);
  }
};

// One halving exchange of a reduce-scatter over lanes: of W values a lane
// keeps the lower half (bit O of its lane index clear) or the upper half,
// each summed with its partner's (lane ^ O).
template <int O, int W>
__device__ __forceinline__ void rs_step(float* v, int j) {
  const bool hi = (j & O) != 0;
#pragma unroll
  for (int i = 0; i < W / 2; ++i) {
    const float send = hi ? v[i] : v[i + W / 2];
    const float keep = hi ? v[i + W / 2] : v[i];
    v[i] = keep + __shfl_xor(send, O, 64);
  }
}

// The sums of UNR values over each aligned group of LPR lanes (UNR <= LPR,
// both powers of two), one per lane: log2(UNR) halving exchanges, then plain
// sums.  Lane j of a group ends with the sum of value j / (LPR / UNR).
template <int LPR, int UNR>
__device__ __forceinline__ float rows_sum(float* v, int j) {
  static_assert(UNR <= LPR && UNR <= 8, "rows per lane group");
  if constexpr (UNR >= 2) rs_step<LPR / 2, UNR>(v, j);
  if constexpr (UNR >= 4) rs_step<LPR / 4, UNR / 2>(v, j);
  if constexpr (UNR >= 8) rs_step<LPR / 8, UNR / 4>(v, j);
  float s = v[0];
#pragma unroll
  for (int o = LPR / UNR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  return s;
}

}  // namespace

// --------------------------------------------------------------------------
// Single input.  The token inputs of KG consecutive tokens (dt, lam, A, the
// phases, B and C rows, and x of the block's rows) are staged in LDS by the
// whole block in one round trip, double-buffered: group g + 1's loads are in
// flight while group g's tokens are applied.  Fetching each token's inputs
// one token ahead left every token waiting for a memory round trip, several
// per call, while the block's state stayed idle in registers.
constexpr int kTokGroup = 4;

template <typename TI, int N, int NR>
struct TokGroup {
  float d[kTokGroup], l[kTokGroup], A[kTokGroup];
  float th[kTokGroup][N / 2];
  f4 b[kTokGroup][N / 4];
  f4 c[kTokGroup][N / 4];
  float x[kTokGroup][NR];
};

// One group's inputs in registers, as loaded, spread over the block's 256
// threads: 8-element vectors of B and C (then of the phases), one x element
// and one token scalar per thread item.  Every lane loads from a valid
// address (tokens past K and rows past P read the last ones; items past the
// counts read the first) and the extra values are not stored.
template <typename TI, int N, int NR>
struct TokGroupLoad {
  static constexpr int NBC = kTokGroup * N / 4;        // B and C vectors
  static constexpr int NTH = kTokGroup * (N / 2) / 8;  // phase vectors
  static constexpr int NX = kTokGroup * NR;            // x elements
  static constexpr int IBC = (NBC + 255) / 256, ITH = (NTH + 255) / 256, IX = (NX + 255) / 256;
  Vec8<TI> bc[IBC], th[ITH];
  Raw1<TI> x[IX], d, l;
  float A;
  __device__ __forceinline__ void load(const DecodeArgs& a, int bh, int k0, int prow0) {
    const int tid = threadIdx.x;
    const int klast = a.K - 1;
#pragma unroll
    for (int i = 0; i < IBC; ++i) {
      const int v = min(tid + 256 * i, NBC - 1);
      const int j = v / (N / 4), w = v % (N / 4);   // token, vector (B: w < N/8)
      const TI* src = static_cast<const TI*>(w < N / 8 ? a.Bt : a.Ct);
      bc[i].load(src + tok_group(a, bh, min(k0 + j, klast)) * N + 8 * (w % (N / 8)));
    }
#pragma unroll
    for (int i = 0; i < ITH; ++i) {
      const int v = min(tid + 256 * i, NTH - 1);
      const int j = v / (N / 16), w = v % (N / 16);
      th[i].load(static_cast<const TI*>(a.theta) + tok_group(a, bh, min(k0 + j, klast)) * (N / 2) +
                 8 * w);
    }
#pragma unroll
    for (int i = 0; i < IX; ++i) {
      const int e = min(tid + 256 * i, NX - 1);
      const int j = e / NR, r = e % NR;
      x[i].load(static_cast<const TI*>(a.x),
                tok_head(a, bh, min(k0 + j, klast)) * a.P + min(prow0 + r, a.P - 1));
    }
    const int j = min(tid % kTokGroup, kTokGroup - 1);
    const int64_t t = tok_head(a, bh, min(k0 + j, klast));
    d.load(static_cast<const TI*>(a.dt), t);
    l.load(static_cast<const TI*>(a.lam), t);
    A = (a.flags & kAPerToken) ? a.A[t] : a.A[bh % a.H];
  }
  __device__ __forceinline__ void store(TokGroup<TI, N, NR>& g) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IBC; ++i) {
      const int v = tid + 256 * i;
      if (v < NBC) {
        const int j = v / (N / 4), w = v % (N / 4);
        float e[8];
        bc[i].get(e);
        f4* dst = w < N / 8 ? &g.b[j][2 * w] : &g.c[j][2 * (w - N / 8)];
        dst[0] = f4{e[0], e[1], e[2], e[3]};
        dst[1] = f4{e[4], e[5], e[6], e[7]};
      }
    }
#pragma unroll
    for (int i = 0; i < ITH; ++i) {
      const int v = tid + 256 * i;
      if (v < NTH) {
        const int j = v / (N / 16), w = v % (N / 16);
        float e[8];
        th[i].get(e);
#pragma unroll
        for (int q = 0; q < 8; ++q) g.th[j][8 * w + q] = e[q];
      }
    }
#pragma unroll
    for (int i = 0; i < IX; ++i) {
      const int e = tid + 256 * i;
      if (e < NX) g.x[e / NR][e % NR] = x[i].f();
    }
    if (tid < kTokGroup) {
      g.d[tid] = d.f();
      g.l[tid] = l.f();
      g.A[tid] = A;
    }
  }
};

// four waves per SIMD (at most 128 registers) for the 8-row blocks; the
// B/C preparation needs more registers than that
// ONEG: a call of at most kTokGroup tokens (one group), which needs no
// registers for the next group's inputs
template <typename TI, typename TO, int N, int UNR, bool PREV, bool PREP, bool ONEG = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONEG ? M3_ONEG_WAVES : UNR == 8 && !PREP ? 4 : 1))) void k_decode_siso_tok(
    DecodeArgs a) {
  constexpr int LPR = N / 4;      // lanes per state row
  constexpr int RPW = 64 / LPR;   // rows per wave per pass
  constexpr int RPB = 4 * RPW;    // rows per block per pass
  constexpr int NR = UNR * RPB;   // rows per block
  static_assert(N % 16 == 0, "whole phase vectors per token");
  __shared__ TokGroup<TI, N, NR> grp[2];
  // a unit's rows may be split over several blocks (NR rows each)
  const int nblk = (a.P + NR - 1) / NR;
  const int bh = blockIdx.x / nblk;
  const int P = a.P;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = 4 * (lane % LPR);
  const int prow0 = (blockIdx.x % nblk) * NR;     // the block's first row
  const int rloc = wave * RPW + lane / LPR;        // this lane's first row, within the block
  const int rsub = prow0 + rloc;
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  TO* __restrict__ Y = static_cast<TO*>(a.y);
  const int ngrp = ONEG ? 1 : (a.K + kTokGroup - 1) / kTokGroup;

  // the first group's inputs go out first, then the token before the first
  // one, then the block's state
  TokGroupLoad<TI, N, NR> gl;
  gl.load(a, bh, 0, prow0);
  f4 bo = PREV ? ld4(static_cast<const TI*>(a.Bp), unit_group(a, bh) * N + n0) : f4{0, 0, 0, 0};
  float xo[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u)
    xo[u] = PREV ? ld1(static_cast<const TI*>(a.xp), (int64_t)bh * P + min(u * RPB + rsub, P - 1)) : 0.0f;
  // B/C preparation: weight and this head's bias of columns n0..n0+3
  f4 bw = f4{1, 1, 1, 1}, cw = bw, bbias = f4{0, 0, 0, 0}, cbias = bbias;
  if constexpr (PREP) {
    const int64_t hb0 = (int64_t)(bh % a.H) * N + n0;
    bw = ld4_or(a.bc.Bw, n0, bw);
    cw = ld4_or(a.bc.Cw, n0, cw);
    bbias = ld4_or(a.bc.Bb, hb0, bbias);
    cbias = ld4_or(a.bc.Cb, hb0, cbias);
  }
  // the token-side reads stay ahead of the state stream
  asm volatile("" ::: "memory");
  f4 v[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) v[u] = ld4_state(hb + (int64_t)min(u * RPB + rsub, P - 1) * N + n0);
  // a row's N/4 lanes hold a token's whole B and C
  auto prep = [&](f4 u, f4 w, f4 b) {
    const float inv = bc_inv_rms(a.bc, group_sum<LPR>(u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w), N);
    return u * inv * w + b;
  };
  if (PREP && PREV) bo = prep(bo, bw, bbias);   // bo always holds a prepared B
  gl.store(grp[0]);
  __syncthreads();

  const bool ang = (a.flags & kThetaIsAngle) != 0;
  for (int gi = 0; gi < ngrp; ++gi) {
    const TokGroup<TI, N, NR>& gc = grp[gi & 1];
    const bool more = !ONEG && gi + 1 < ngrp;   // block-uniform
    if (more) gl.load(a, bh, (gi + 1) * kTokGroup, prow0);
    const int kend = min(kTokGroup, a.K - gi * kTokGroup);
    for (int j = 0; j < kend; ++j) {
      const int k = gi * kTokGroup + j;
      const float dk = gc.d[j], lk = gc.l[j];
      const float alpha = expf(dk * gc.A[j]);
      const float beta = (1.0f - lk) * dk * alpha;
      const float gamma = lk * dk;
      const f2 thk = *reinterpret_cast<const f2*>(&gc.th[j][n0 / 2]);   // pairs n0/2, n0/2 + 1
      const f2 r0 = cos_sin_turns(ang ? thk.x : dk * thk.x);
      const f2 r1 = cos_sin_turns(ang ? thk.y : dk * thk.y);
      f4 bk = gc.b[j][n0 / 4], ck = gc.c[j][n0 / 4];
      if constexpr (PREP) {
        bk = prep(bk, bw, bbias);
        ck = prep(ck, cw, cbias);
      }
      const f4 bt = gamma * bk, bp = beta * bo;
      TO* __restrict__ yk = Y + tok_head(a, bh, k) * P;
      float part[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float xk = gc.x[j][u * RPB + rloc];
        f4 s = alpha * v[u] + xo[u] * bp;
        s = rot2pairs(s, r0, r1);
        s += xk * bt;
        v[u] = s;
        xo[u] = xk;
        part[u] = s.x * ck.x + s.y * ck.y + s.z * ck.z + s.w * ck.w;
      }
      bo = bk;
      // y of the lane's UNR rows: summed over the row's LPR lanes
      if constexpr (UNR <= LPR) {
        const float tot = rows_sum<LPR, UNR>(part, lane % LPR);
        const int jj = lane % LPR;
        const int p = (jj / (LPR / UNR)) * RPB + rsub;
        if (jj % (LPR / UNR) == 0 && p < P) st1(yk, p, tot);
      } else {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const float tot = group_sum<LPR>(part[u]);
          const int p = u * RPB + rsub;
          if ((lane % LPR) == 0 && p < P) st1(yk, p, tot);
        }
      }
    }
    if (more) {   // the buffer written here was last read by group gi - 1
      gl.store(grp[(gi + 1) & 1]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int p = u * RPB + rsub;
    if (p < P) st4_stream(hb + (int64_t)p * N + n0, v[u]);
  }
}

// --------------------------------------------------------------------------
// Rank R > 1.  Each wave holds one 16-row block of the state in the MFMA D
// layout for all K tokens: D row 4g + i of tile t is state column
// 16t + 4g + i and D column i16 is state row p, so a lane's accumulator is
// the 16-byte vector of columns 16t + 4g .. + 3 of its row, loaded in
// place.  The rank-R terms are MFMA products with K = R (as in the
// single-step kernel).
//
// The inputs of a group of KG tokens are prepared once per block and read
// by every wave: the pair rotations and the token scalars, B of the token
// before the group's first (row 0: B_prev for the call's first token, else
// the previous token's B, read again) and of the group's tokens, and C.
// With one group per call (K <= KG) the block passes one barrier before
// its first token and one before the rows go back through LDS; a longer
// call refills the tables between groups.
template <int N, int R>
struct MGroup {
  static constexpr int RP = (R + 3) & ~3;
  float al[kTokGroup], be[kTokGroup], ga[kTokGroup];
  f2 cs[kTokGroup][N / 2];
  float b[kTokGroup + 1][N * RP];   // [n][r], r padded to RP with zeros
  float c[kTokGroup][N * RP];
};

// One group's B and C rows (8-element vectors), phases and token scalars
// in registers, as loaded, spread over the block's 256 threads.  Vectors
// 0 .. (KG+1) VR - 1 are the B rows 0..KG, the rest the C rows.  Every lane
// reads a valid address (tokens past K re-read the last; items past the
// counts re-read the last item) and only stores what belongs to the group.
template <typename TI, int N, int R>
struct MGroupLoad {
  static constexpr int NE = N * R, VR = NE / 8;
  static constexpr int NB = (kTokGroup + 1) * VR, NV = NB + kTokGroup * VR;
  static constexpr int NA = kTokGroup * (N / 2);
  static constexpr int IV = (NV + 255) / 256, IA = (NA + 255) / 256;
  static_assert(NE % 8 == 0, "whole 8-element vectors per row");
  Vec8<TI> bc[IV];
  Raw1<TI> th[IA], dth[IA];
  Raw1<TI> d, l;
  float A;
  bool b0_zero;   // row 0 is the call's first token's B_{-1} and there is none
  template <bool PREV>
  __device__ __forceinline__ void load(const DecodeArgs& a, int bh, int k0) {
    load<PREV>(a, bh, k0, threadIdx.x);
  }
  template <bool PREV>
  __device__ __forceinline__ void load(const DecodeArgs& a, int bh, int k0, int tid) {
    const int klast = a.K - 1;
    const TI* Bt = static_cast<const TI*>(a.Bt);
    const TI* Ct = static_cast<const TI*>(a.Ct);
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int v = min(tid + 256 * i, NV - 1);
      const TI* src;
      if (v < NB) {
        const int k = k0 - 1 + v / VR;   // token of B row v / VR
        src = (k < 0 && PREV) ? static_cast<const TI*>(a.Bp) + unit_group(a, bh) * NE
                              : Bt + tok_group(a, bh, min(max(k, 0), klast)) * NE;
      } else {
        src = Ct + tok_group(a, bh, min(k0 + (v - NB) / VR, klast)) * NE;
      }
      bc[i].load(src + 8 * (v % VR));
    }
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int e = min(tid + 256 * i, NA - 1);
      const int k = min(k0 + e / (N / 2), klast);
      th[i].load(static_cast<const TI*>(a.theta), tok_group(a, bh, k) * (N / 2) + e % (N / 2));
      dth[i].load(static_cast<const TI*>(a.dt), tok_head(a, bh, k));
    }
    const int64_t t = tok_head(a, bh, min(k0 + min(tid, kTokGroup - 1), klast));
    d.load(static_cast<const TI*>(a.dt), t);
    l.load(static_cast<const TI*>(a.lam), t);
    A = (a.flags & kAPerToken) ? a.A[t] : a.A[bh % a.H];
    b0_zero = !PREV && k0 == 0;
  }
  // raw rows into the tables (row 0 zeroed when there is no B_{-1}),
  // rotations and scalars
  __device__ __forceinline__ void store(const DecodeArgs& a, MGroup<N, R>& G) const {
    constexpr int RP = MGroup<N, R>::RP;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) {
        float e[8];
        bc[i].get(e, !(b0_zero && v < VR));
        float* row = v < NB ? G.b[v / VR] : G.c[(v - NB) / VR];
        const int e0 = 8 * (v % VR);
        if constexpr (RP == R) {
          *reinterpret_cast<f4*>(row + e0) = f4{e[0], e[1], e[2], e[3]};
          *reinterpret_cast<f4*>(row + e0 + 4) = f4{e[4], e[5], e[6], e[7]};
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) row[((e0 + q) / R) * RP + (e0 + q) % R] = e[q];
        }
      }
    }
    const bool ang = (a.flags & kThetaIsAngle) != 0;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int e = tid + 256 * i;
      if (e < NA) {
        const float th_ = th[i].f();
        G.cs[e / (N / 2)][e % (N / 2)] = cos_sin_turns(ang ? th_ : dth[i].f() * th_);
      }
    }
    if (tid < kTokGroup) {
      const float dd = d.f(), ll = l.f();
      const float alpha = expf(dd * A);
      G.al[tid] = alpha;
      G.be[tid] = (1.0f - ll) * dd * alpha;
      G.ga[tid] = ll * dd;
    }
  }

  // for the group form (R a multiple of 4): the raw rows as loaded (row 0
  // zeroed when there is no B_{-1}), the phase of every (token, pair) and
  // the token scalars
  template <int SB, int SC>
  __device__ __forceinline__ void store_raw(const DecodeArgs& a, float (*b)[SB], float (*c)[SC],
                                            float (*ph)[N / 2], float* d_, float* l_, float* A_,
                                            int tid) const {
    static_assert(R % 4 == 0 && SB % 4 == 0 && SC % 4 == 0, "rows of whole 16-byte pieces");
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int v = tid + 256 * i;
      if (v < NV) {
        float e[8];
        bc[i].get(e, !(b0_zero && v < VR));
        float* row = v < NB ? b[v / VR] : c[(v - NB) / VR];
        const int e0 = 8 * (v % VR);
        *reinterpret_cast<f4*>(row + e0) = f4{e[0], e[1], e[2], e[3]};
        *reinterpret_cast<f4*>(row + e0 + 4) = f4{e[4], e[5], e[6], e[7]};
      }
    }
    const bool ang = (a.flags & kThetaIsAngle) != 0;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int e = tid + 256 * i;
      if (e < NA) {
        const float th_ = th[i].f();
        ph[e / (N / 2)][e % (N / 2)] = ang ? th_ : dth[i].f() * th_;
      }
    }
    if (tid < kTokGroup) {
      d_[tid] = d.f();
      l_[tid] = l.f();
      A_[tid] = A;
    }
  }
};

// The B/C preparation of a group's tables in place: the inverse RMS of
// every (row, rank column) over its N entries (four lanes per column, each
// adding its entries n = lane, lane + 4, ... in order, then two xor steps:
// a fixed order), then x * inv * w[n] + bias[n][r].  Barriers between the
// passes; the caller's barrier ends the last.
// (b: the B rows 0..KG, c: the C rows; rows of any stride, entry n * RP + r)
template <int N, int R, int SB, int SC>
__device__ __forceinline__ void mgroup_prep(const BCPrep& bc, float (*b)[SB], float (*c)[SC],
                                            float (*inv)[R], const float (*pw)[N],
                                            const float (*pb)[N * R]) {
  constexpr int RP = MGroup<N, R>::RP;
  constexpr int ROWS = 2 * kTokGroup + 1;   // B rows 0..KG, then C rows
  constexpr int NC = ROWS * R;
  const int tid = threadIdx.x;
  __syncthreads();   // the raw rows are in place
  for (int c0 = 0; c0 < NC; c0 += 64) {   // 64 columns x 4 lanes per pass
    const int cc = c0 + tid / 4;
    const int col = min(cc, NC - 1);
    const int row = col / R, r = col % R;
    const float* src = row <= kTokGroup ? b[row] : c[row - kTokGroup - 1];
    float s = 0.0f;
    for (int n = tid % 4; n < N; n += 4) {
      const float v = src[n * RP + r];
      s += v * v;
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (cc < NC && tid % 4 == 0) inv[row][r] = bc_inv_rms(bc, s, N);
  }
  __syncthreads();
  for (int i = tid; i < ROWS * N * R; i += 256) {
    const int row = i / (N * R), j = i % (N * R), n = j / R, r = j % R;
    const bool isb = row <= kTokGroup;
    float* dst = isb ? &b[row][n * RP + r] : &c[row - kTokGroup - 1][n * RP + r];
    *dst = *dst * inv[row][r] * pw[isb ? 0 : 1][n] + pb[isb ? 0 : 1][j];
  }
}

// (four waves per SIMD at rank <= 4, at most 128 registers: the state's 32,
// the next group's inputs in flight and one tile's operands)
template <typename TI, typename TO, int N, int R, bool PREV, bool PREP, bool ONEG = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONEG ? M3_MONEG_WAVES : R <= 4 ? 4 : 1))) void k_decode_mimo_tok(DecodeArgs a) {
  constexpr int NT = N / 16;          // 16-column tiles of a row block
  constexpr int KB = (R + 3) / 4;     // K blocks of 4 for the MFMA
  constexpr int RP = (R + 3) & ~3;
  constexpr int NE = N * R;
  // the group tables, and at the end each wave's rows for the store (half
  // a row at a time, so that the buffer is no larger than the tables)
  constexpr int NHALF = NT >= 2 ? 2 : 1;
  constexpr int HC = N / NHALF;       // columns per transposed piece
  __shared__ union {
    MGroup<N, R> G;
    f4 tr[4][16][HC / 4 + 1];
  } sm;
  MGroup<N, R>& G = sm.G;
  // B/C preparation: this head's weights ([0] B, [1] C), biases, and the
  // inverse RMS of the group's rows
  __shared__ float pw_sh[PREP ? 2 : 1][PREP ? N : 1];
  __shared__ float pb_sh[PREP ? 2 : 1][PREP ? NE : 1];
  __shared__ float inv_sh[PREP ? 2 * kTokGroup + 1 : 1][R];

  const int bh = blockIdx.x;
  const int P = a.P;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const bool rows = wave * 16 < P;   // this wave's 16-row block exists
  const int p = wave * 16 + i16;
  const int prow = rows ? p : 0;     // a valid row for every lane's reads
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  TO* __restrict__ Y = static_cast<TO*>(a.y);
  const int ngrp = ONEG ? 1 : (a.K + kTokGroup - 1) / kTokGroup;

  // x of the lane's row and ranks 4kb + g for the token before the group's
  // first (j = 0) and the group's tokens (j = 1..KG), as loaded
  auto load_x = [&](int k0, Raw1<TI> (*xr)[KB]) {
#pragma unroll
    for (int j = 0; j <= kTokGroup; ++j) {
      const int k = k0 - 1 + j;
      const TI* src = (k < 0 && PREV) ? static_cast<const TI*>(a.xp) + (int64_t)bh * P * R
                                      : X + tok_head(a, bh, min(max(k, 0), a.K - 1)) * P * R;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int r = min(4 * kb + g, R - 1);
        xr[j][kb].load(src, (int64_t)prow * R + r);
      }
    }
  };
  // the value of x (j, kb) for this lane: zero with no row, no rank
  // 4kb + g, or no x_{-1}
  auto xval = [&](const Raw1<TI> (*xr)[KB], int j, int kb, int k0) {
    const bool live = rows && 4 * kb + g < R && (PREV || k0 + j > 0);
    return live ? xr[j][kb].f() : 0.0f;
  };

  // the first group's inputs go out first, then the state
  MGroupLoad<TI, N, R> gl;
  gl.template load<PREV>(a, bh, 0);
  Raw1<TI> xr[kTokGroup + 1][KB];
  load_x(0, xr);
  float wv[PREP ? 4 : 1][PREP ? (NE + 255) / 256 : 1];
  if constexpr (PREP) {   // weights and this head's biases (1 and 0 when absent)
    const int64_t hb0 = (int64_t)(bh % a.H) * NE;
#pragma unroll
    for (int q = 0; q < (NE + 255) / 256; ++q) {
      const int i = min(tid + 256 * q, NE - 1);
      wv[0][q] = ld_or(a.bc.Bw, min(i, N - 1), 1.0f);
      wv[1][q] = ld_or(a.bc.Cw, min(i, N - 1), 1.0f);
      wv[2][q] = ld_or(a.bc.Bb, hb0 + i, 0.0f);
      wv[3][q] = ld_or(a.bc.Cb, hb0 + i, 0.0f);
    }
  }
  asm volatile("" ::: "memory");   // the token-side reads stay ahead of the state stream
  f4 v[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) v[t] = ld4_state(hb + (int64_t)prow * N + 16 * t + 4 * g);

  if constexpr (RP != R) {   // the padding columns stay zero for every group
    for (int i = tid; i < (2 * kTokGroup + 1) * N; i += 256) {
      float* row = i < (kTokGroup + 1) * N ? G.b[i / N] : G.c[i / N - kTokGroup - 1];
#pragma unroll
      for (int r = R; r < RP; ++r) row[(i % N) * RP + r] = 0.0f;
    }
  }
  if constexpr (PREP) {
#pragma unroll
    for (int q = 0; q < (NE + 255) / 256; ++q) {
      const int i = tid + 256 * q;
      if (i < N) {
        pw_sh[0][i] = wv[0][q];
        pw_sh[1][i] = wv[1][q];
      }
      if (i < NE) {
        pb_sh[0][i] = wv[2][q];
        pb_sh[1][i] = wv[3][q];
      }
    }
  }
  gl.store(a, G);
  if constexpr (PREP) mgroup_prep<N, R>(a.bc, G.b, G.c, inv_sh, pw_sh, pb_sh);
  __syncthreads();

  // lane bases of the LDS operands: A-operand row i16 is state column
  // 16t + i16 (k lane group g), D rows 4g .. 4g + 3 are columns 16t + 4g ..
  const float* __restrict__ b_l = &G.b[0][0] + i16 * RP + g;
  const float* __restrict__ c_l = &G.c[0][0] + 4 * g * RP;
  const f2* __restrict__ cs_l = &G.cs[0][0] + 2 * g;
  for (int gi = 0; gi < ngrp; ++gi) {
    const int k0 = gi * kTokGroup;
    const bool more = !ONEG && gi + 1 < ngrp;   // block-uniform
    Raw1<TI> xn[kTokGroup + 1][KB];
    if (more) {
      gl.template load<PREV>(a, bh, k0 + kTokGroup);
      load_x(k0 + kTokGroup, xn);
    }
    const int kend = min(kTokGroup, a.K - k0);
#pragma unroll
    for (int j = 0; j < kTokGroup; ++j) {   // unrolled: xr indexed by constants
      if (j >= kend) break;
      const float alpha = G.al[j];
      float xo[KB], xk[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        xo[kb] = G.be[j] * xval(xr, j, kb, k0);
        xk[kb] = G.ga[j] * xval(xr, j + 1, kb, k0);
      }
      float yp[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) yp[r] = 0.0f;
      if (rows) {   // wave-uniform
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // every LDS operand is a lane base plus a constant offset
          const int tb = j * (N * RP) + 16 * t * RP;
          f4 acc = alpha * v[t];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b_l[tb + 4 * kb], xo[kb], acc, 0, 0, 0);
          acc = rot2pairs(acc, cs_l[j * (N / 2) + 8 * t], cs_l[j * (N / 2) + 8 * t + 1]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b_l[tb + N * RP + 4 * kb], xk[kb], acc, 0, 0, 0);
          v[t] = acc;
#pragma unroll
          for (int rb = 0; rb < RP; rb += 4) {
            const f4 c0 = *reinterpret_cast<const f4*>(c_l + tb + 0 * RP + rb);
            const f4 c1 = *reinterpret_cast<const f4*>(c_l + tb + 1 * RP + rb);
            const f4 c2 = *reinterpret_cast<const f4*>(c_l + tb + 2 * RP + rb);
            const f4 c3 = *reinterpret_cast<const f4*>(c_l + tb + 3 * RP + rb);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              yp[rb + q] += acc.x * c0[q] + acc.y * c1[q] + acc.z * c2[q] + acc.w * c3[q];
          }
          // one tile's LDS operands at a time (registers and occupancy)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        yp[r] += __shfl_xor(yp[r], 16, 64);
        yp[r] += __shfl_xor(yp[r], 32, 64);
      }
      if (rows && g == 0) {
        TO* __restrict__ yk = Y + tok_head(a, bh, k0 + j) * P * R;
#pragma unroll
        for (int r = 0; r < R; ++r) st1(yk, (int64_t)p * R + r, yp[r]);
      }
    }
    if (more) {   // every wave is past the group's tokens before its tables change
      __syncthreads();
      gl.store(a, G);
      if constexpr (PREP) mgroup_prep<N, R>(a.bc, G.b, G.c, inv_sh, pw_sh, pb_sh);
      __syncthreads();
#pragma unroll
      for (int j = 0; j <= kTokGroup; ++j)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) xr[j][kb] = xn[j][kb];
    }
  }

  // the wave's rows back to HBM through LDS, row-contiguous, so that each
  // store instruction covers whole lines (direct stores from the D layout
  // write half lines, which the counters show costing about a quarter more
  // write traffic)
  __syncthreads();   // every wave is past the last group's tables
  if (rows) {
    constexpr int V4 = HC / 4, LV = 16 * V4 / 64, TH = NT / NHALF;
#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf) {
#pragma unroll
      for (int t = 0; t < TH; ++t) sm.tr[wave][i16][(16 * t + 4 * g) / 4] = v[hf * TH + t];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < LV; ++j) {
        const int q = lane + 64 * j;
        st4_stream(hb + (int64_t)(wave * 16 + q / V4) * N + hf * HC + 4 * (q % V4),
                   sm.tr[wave][q / V4][q % V4]);
      }
      // this half's reads are done before the next half's writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// --------------------------------------------------------------------------
// Rank 4 in group form.  Unrolling the recurrence over a group of KG tokens
// (local tokens 1..KG; local token 0 is the one before the group) gives, with
// the cumulative log-decay cs_j = sum_{i<=j} dt_i A_i and the cumulative phase
// Phi_j = sum_{i<=j} phi_i of every pair (cs_0 = Phi_0 = 0),
//   y_j = e^{cs_j} h_0 Ct_j + sum_{u=0..j} e^{cs_j - cs_u} w_{j,u} X_u (Bt_u^T Ct_j),
//   h_K = rot(e^{cs_K} h_0 + sum_{u=0..K} e^{cs_K - cs_u} w_{K,u} X_u Bt_u^T, Phi_K),
// where Bt_u and Ct_j are B_u and C_j with every pair rotated by -Phi_u and
// -Phi_j, w_{j,0} = (1 - lam_1) dt_1 (the left-endpoint term of the group's
// first token) and w_{j,u} = lam_u dt_u + [u < j] (1 - lam_{u+1}) dt_{u+1}:
// the chunked form of the prefill, with a chunk of KG tokens [xxxxx.co.kr,
// sections 1.1-1.3].  So the state is rotated and decayed once per group, and
// its products are MFMA contractions with the state's own registers as
// operands:
//  * the group's outputs: the 16 x 16 block (rows p, columns (token, rank))
//    of h_0 times the rotated C columns, K = N (v_mfma_f32_16x16x4f32 with
//    the state's D-layout registers as the A operand), then the columns
//    scaled by e^{cs_j} and the terms inside the group added as one more
//    product, X (the lane's own x values) times the masked Gram of the
//    group's rotated B and C rows (computed once per block on the MFMA, the
//    four waves taking a quarter of N each);
//  * the state update: the rank-4 terms of the KG + 1 tokens as MFMA
//    products with K = 4 per token, then one rotation by Phi_K.
// The token work per group is about a third of the token-by-token kernel's;
// what is left of a call's time is mostly each block's memory round trips
// (its group inputs, then its state).
constexpr double kTwoPiD = 6.283185307179586476925286766559;

template <int N>
struct alignas(16) GTab {
  static constexpr int R = 4, NE = N * R;
  static constexpr int SB = NE + 16;   // B row stride: the Gram's four rows start in different banks
  static constexpr int SCT = N + 4;    // row stride of the transposed C
  float b[kTokGroup + 1][SB];          // B rows of local tokens 0..KG, [n][s]: raw, then rotated
  union {
    float c[kTokGroup][NE];            // raw C rows [n][r]
    float gp[4][32][16];               // the four waves' Gram partials
  } u;
  float ct[kTokGroup * R][SCT];        // rotated C, transposed: [(j - 1) R + r][n]
  float ph[kTokGroup][N / 2];          // phase of each token and pair
  f2 cph[kTokGroup + 1][N / 2];        // (cos, sin) of Phi_j, j = 0..KG
  float gm[(kTokGroup + 1) * R][16];   // masked Gram [(u, s)][(j - 1, r)]
  float msk[kTokGroup][kTokGroup + 1]; // e^{cs_j - cs_u} w_{j,u}, zero where u > j
  float ecs[kTokGroup * R];            // e^{cs_j} of each output column
  float coef[kTokGroup + 1];           // e^{cs_K - cs_u} w_{K,u}
  float ecsK;
  float d[kTokGroup], l[kTokGroup], A[kTokGroup];
};

#ifndef M3_GRP_WAVES
#define M3_GRP_WAVES 5
#endif

// (one group: five waves per SIMD, 32 KB of LDS at N = 128 and at most 96
// registers; four with the B/C preparation's tables or with several groups,
// whose loop needs a few more registers)
template <typename TI, typename TO, int N, bool PREV, bool PREP, bool ONEG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONEG && !PREP ? M3_GRP_WAVES : 4))) void k_decode_mimo_grp(DecodeArgs a) {
  constexpr int R = 4, KG = kTokGroup, NT = N / 16, NE = N * R;
  // threads 0 .. N/2 - 1 build the phases and threads 64 .. 93 the decay
  // tables, side by side; one 16-row block per wave (P <= 64)
  static_assert(N % 16 == 0 && N <= 128, "group-form state width");
  using TB = GTab<N>;
  constexpr int NHALF = NT >= 2 ? 2 : 1;
  constexpr int HC = N / NHALF;       // columns per transposed piece of the final store
  __shared__ union {
    TB t;
    f4 tr[4][16][HC / 4 + 1];
  } sm;
  TB& T = sm.t;
  __shared__ float pw_sh[PREP ? 2 : 1][PREP ? N : 1];
  __shared__ float pb_sh[PREP ? 2 : 1][PREP ? NE : 1];
  __shared__ float inv_sh[PREP ? 2 * KG + 1 : 1][R];

  const int bh = blockIdx.x;
  const int P = a.P;
  const bool rows = (int)(threadIdx.x >> 6) * 16 < P;   // this wave's 16-row block exists
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  TO* __restrict__ Y = static_cast<TO*>(a.y);
  const int ngrp = ONEG ? 1 : (a.K + KG - 1) / KG;

  // x of row prow (a valid row for every lane's reads) and rank g for local
  // tokens 0..KG, as loaded
  auto load_x = [&](int k0, Raw1<TI>* xr, int prow, int g) {
#pragma unroll
    for (int j = 0; j <= KG; ++j) {
      const int k = k0 - 1 + j;
      const TI* src = (k < 0 && PREV) ? static_cast<const TI*>(a.xp) + (int64_t)bh * P * R
                                      : X + tok_head(a, bh, min(max(k, 0), a.K - 1)) * P * R;
      xr[j].load(src, (int64_t)prow * R + g);
    }
  };

  f4 v[NT];   // this wave's 16 rows of the state, in the MFMA D layout
  for (int gi = 0; gi < ngrp; ++gi) {
    const int k0 = gi * KG;
    const bool more = !ONEG && gi + 1 < ngrp;   // block-uniform
    const int ke = min(KG, a.K - k0);           // tokens in this group
    // the thread index, opaque to the compiler once per group: the group's
    // addresses are then formed inside the loop instead of being hoisted out
    // of it and held in registers across all groups
    int tid = threadIdx.x;
    if constexpr (!ONEG) asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6, i16 = lane & 15, g = lane >> 4;
    const int prow = rows ? wave * 16 + i16 : 0;

    // the group's inputs: a later group's after the previous group's last
    // barrier (held in flight across a group they would cost the registers
    // of a fifth wave per SIMD, and the other resident blocks cover the
    // wait); at the first group they go out ahead of the state
    MGroupLoad<TI, N, R> gl;
    gl.template load<PREV>(a, bh, k0, tid);
    Raw1<TI> xr[KG + 1];
    load_x(k0, xr, prow, g);
    if (gi == 0) {
      float wv[PREP ? 4 : 1][PREP ? (NE + 255) / 256 : 1];
      if constexpr (PREP) {   // weights and this head's biases (1 and 0 when absent)
        const int64_t hb0 = (int64_t)(bh % a.H) * NE;
#pragma unroll
        for (int q = 0; q < (NE + 255) / 256; ++q) {
          const int i = min(tid + 256 * q, NE - 1);
          wv[0][q] = ld_or(a.bc.Bw, min(i, N - 1), 1.0f);
          wv[1][q] = ld_or(a.bc.Cw, min(i, N - 1), 1.0f);
          wv[2][q] = ld_or(a.bc.Bb, hb0 + i, 0.0f);
          wv[3][q] = ld_or(a.bc.Cb, hb0 + i, 0.0f);
        }
      }
      asm volatile("" ::: "memory");   // the token-side reads stay ahead of the state stream
#pragma unroll
      for (int t = 0; t < NT; ++t) v[t] = ld4_state(hb + (int64_t)prow * N + 16 * t + 4 * g);
      if constexpr (PREP) {
#pragma unroll
        for (int q = 0; q < (NE + 255) / 256; ++q) {
          const int i = tid + 256 * q;
          if (i < N) {
            pw_sh[0][i] = wv[0][q];
            pw_sh[1][i] = wv[1][q];
          }
          if (i < NE) {
            pb_sh[0][i] = wv[2][q];
            pb_sh[1][i] = wv[3][q];
          }
        }
      }
    }

    // (1) raw rows, phases and scalars (B/C preparation in place)
    gl.store_raw(a, T.b, T.u.c, T.ph, T.d, T.l, T.A, tid);
    if constexpr (PREP) mgroup_prep<N, R>(a.bc, T.b, T.u.c, inv_sh, pw_sh, pb_sh);
    __syncthreads();

    // (2) cumulative phases (double sums, reduced in turns) and the
    // decay/weight tables
    if (tid < N / 2) {
      double run = 0.0;
      T.cph[0][tid] = f2{1.0f, 0.0f};
#pragma unroll
      for (int j = 1; j <= KG; ++j) {
        run += (double)T.ph[j - 1][tid];
        double tu = run * (1.0 / kTwoPiD);
        tu -= rint(tu);
        const float tf = (float)tu;
        T.cph[j][tid] = f2{__builtin_amdgcn_cosf(tf), __builtin_amdgcn_sinf(tf)};
      }
    } else if (tid >= 64 && tid < 64 + KG * (KG + 1) + (KG + 1) + 1 + KG) {
      const int e = tid - 64;
      // log-decay of local tokens u+1..j and the weight w_{j,u}
      auto seg = [&](int u, int j) {
        float s = 0.0f;
        for (int i = u + 1; i <= j; ++i) s += T.d[i - 1] * T.A[i - 1];
        return s;
      };
      auto wgt = [&](int j, int u) {
        if (u == 0) return (1.0f - T.l[0]) * T.d[0];
        const float gam = T.l[u - 1] * T.d[u - 1];
        return u < j ? gam + (1.0f - T.l[u]) * T.d[u] : gam;
      };
      if (e < KG * (KG + 1)) {
        const int j = e / (KG + 1) + 1, u = e % (KG + 1);
        T.msk[j - 1][u] = (u <= j && j <= ke) ? expf(seg(u, j)) * wgt(j, u) : 0.0f;
      } else if (e < KG * (KG + 1) + KG + 1) {
        const int u = e - KG * (KG + 1);
        T.coef[u] = u <= ke ? expf(seg(u, ke)) * wgt(ke, u) : 0.0f;
      } else if (e == KG * (KG + 1) + KG + 1) {
        T.ecsK = expf(seg(0, ke));
      } else {
        const int j = e - (KG * (KG + 1) + KG + 1);   // 1..KG
        const float ec = expf(seg(0, j));
#pragma unroll
        for (int r = 0; r < R; ++r) T.ecs[(j - 1) * R + r] = ec;
      }
    }
    __syncthreads();

    // (3) B rows of tokens 1..KG rotated by -Phi_u in place; C rows rotated
    // by -Phi_j into the transposed table.  One item is one pair of one
    // token: its two columns for the four ranks.
    for (int it = tid; it < 2 * KG * (N / 2); it += 256) {
      const bool isb = it < KG * (N / 2);
      const int jt = (isb ? it : it - KG * (N / 2)) / (N / 2) + 1;
      const int k = it % (N / 2);
      const f2 cs = T.cph[jt][k];   // rotation by -Phi: (cos, -sin)
      const float* src = isb ? &T.b[jt][8 * k] : &T.u.c[jt - 1][8 * k];
      const f4 c0 = *reinterpret_cast<const f4*>(src);       // column 2k, ranks 0..3
      const f4 c1 = *reinterpret_cast<const f4*>(src + 4);   // column 2k + 1
      f4 o0, o1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        o0[r] = cs.x * c0[r] + cs.y * c1[r];
        o1[r] = -cs.y * c0[r] + cs.x * c1[r];
      }
      if (isb) {
        *reinterpret_cast<f4*>(&T.b[jt][8 * k]) = o0;
        *reinterpret_cast<f4*>(&T.b[jt][8 * k + 4]) = o1;
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
          *reinterpret_cast<f2*>(&T.ct[(jt - 1) * R + r][2 * k]) = f2{o0[r], o1[r]};
      }
    }
    __syncthreads();

    // (4) Gram partials: rows (u, s) of Bt (tile 0: u = 0..3, tile 1: u = 4),
    // columns (j, r) of Ct; wave w sums n over [w N/4, (w + 1) N/4)
    {
      f4 d0 = f4{0, 0, 0, 0}, d1 = f4{0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < N / 16; ++q) {
        const int n = wave * (N / 4) + 4 * q + g;
        const float a0 = T.b[i16 / 4][n * R + i16 % 4];
        const float a1 = i16 < 4 ? T.b[KG][n * R + i16] : 0.0f;
        const float bv = T.ct[i16][n];
        d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bv, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bv, d1, 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        T.u.gp[wave][4 * g + jj][i16] = d0[jj];
        T.u.gp[wave][16 + 4 * g + jj][i16] = d1[jj];
      }
    }
    __syncthreads();
    // (5) the sum over the waves, masked: gm[(u, s)][(j - 1, r)]
    for (int e = tid; e < (KG + 1) * R * 16; e += 256) {
      const int row = e / 16, col = e % 16;
      const float s = T.u.gp[0][row][col] + T.u.gp[1][row][col] + T.u.gp[2][row][col] +
                      T.u.gp[3][row][col];
      T.gm[row][col] = row / R <= col / R + 1 ? s * T.msk[col / R][row / R] : 0.0f;
    }
    __syncthreads();

    // (6) this wave's 16 rows: the group's outputs and the state update
    if (rows) {   // wave-uniform
      float xs[KG + 1], xc[KG + 1];
#pragma unroll
      for (int u = 0; u <= KG; ++u) {
        xs[u] = (PREV || k0 + u > 0) ? xr[u].f() : 0.0f;
        xc[u] = T.coef[u] * xs[u];
      }
      const float ecsK = T.ecsK;
      f4 yacc = f4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // h_0 against the rotated C columns: k = g is column 16t + 4g + i
        const f4 cv = *reinterpret_cast<const f4*>(&T.ct[i16][16 * t + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[t][i], cv[i], yacc, 0, 0, 0);
        // e^{cs_K} h_0 plus the group's rank-4 terms, then the rotation by Phi_K
        f4 acc = ecsK * v[t];
#pragma unroll
        for (int u = 0; u <= KG; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(T.b[u][(16 * t + i16) * R + g], xc[u], acc, 0, 0, 0);
        const f4 c2 = *reinterpret_cast<const f4*>(&T.cph[ke][8 * t + 2 * g]);
        v[t] = rot2pairs(acc, f2{c2.x, c2.y}, f2{c2.z, c2.w});
        __builtin_amdgcn_sched_barrier(0);   // one tile's operands at a time
      }
      // columns scaled by e^{cs_j}, then the terms inside the group, one
      // product per token u, added only to the columns of tokens j >= u (so
      // that a NaN in a later token's x never reaches an earlier token's y)
      yacc = yacc * T.ecs[i16];
#pragma unroll
      for (int u = 0; u <= KG; ++u) {
        const f4 tu = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[u], T.gm[u * R + g][i16], f4{0, 0, 0, 0}, 0, 0, 0);
        if (u <= i16 / R + 1) yacc = yacc + tu;
      }
      // lane: rows 16 wave + 4g + jj, column i16 = (token i16 / 4, rank i16 % 4)
      if (i16 / R < ke) {
        TO* __restrict__ yk = Y + tok_head(a, bh, k0 + i16 / R) * P * R;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int pp = wave * 16 + 4 * g + jj;
          if (pp < P) st1(yk, (int64_t)pp * R + i16 % R, yacc[jj]);
        }
      }
    }
    if (more) __syncthreads();   // every wave is past the group's tables before they change
  }

  // the wave's rows back to HBM through LDS, row-contiguous (whole lines per
  // store instruction)
  __syncthreads();   // every wave is past the last group's tables
  if (rows) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i16 = lane & 15, g = lane >> 4;
    constexpr int V4 = HC / 4, LV = 16 * V4 / 64, TH = NT / NHALF;
#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf) {
#pragma unroll
      for (int t = 0; t < TH; ++t) sm.tr[wave][i16][(16 * t + 4 * g) / 4] = v[hf * TH + t];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < LV; ++j) {
        const int q = lane + 64 * j;
        st4_stream(hb + (int64_t)(wave * 16 + q / V4) * N + hf * HC + 4 * (q % V4),
                   sm.tr[wave][q / V4][q % V4]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// --------------------------------------------------------------------------
namespace {

template <typename TI, typename TO, int N, int UNR>
hipError_t launch_siso_tok(const DecodeArgs& a, int units, hipStream_t s) {
  constexpr int RPB = 4 * (64 / (N / 4));
  const int nblk = (a.P + UNR * RPB - 1) / (UNR * RPB);
  const dim3 g(units * nblk), b(256);
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, false, true>), g, b, 0, s, a);
  } else if (UNR == 8 && a.K <= kTokGroup) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, true, false, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, false, false, true>), g, b, 0, s, a);
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

// rank 4: the group form (one group of tokens, or several)
template <typename TI, typename TO, int N>
hipError_t launch_mimo_grp(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 g(units), b(256);
  const bool one = a.K <= kTokGroup;
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, true, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, false, true, false>), g, b, 0, s, a);
  } else if (one) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, true, false, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, false, false, true>), g, b, 0, s, a);
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, true, false, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_grp<TI, TO, N, false, false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

template <typename TI, typename TO, int N, int R>
hipError_t launch_mimo_tok(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 g(units), b(256);
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, false, true>), g, b, 0, s, a);
  } else if (R <= 4 && a.K <= kTokGroup) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, true, false, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, false, false, true>), g, b, 0, s, a);
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

// rows per block pass of the single-input layout: 4 waves x 64 / (N/4) rows
constexpr int rows_per_pass(int N) { return 4 * (64 / (N / 4)); }

template <typename TI, typename TO, int N>
hipError_t siso_tok_n(const DecodeArgs& a, int units, hipStream_t s) {
  constexpr int RPB = rows_per_pass(N);
  const int passes = (a.P + RPB - 1) / RPB;
  // up to 8 row passes per block; more rows go to further blocks (measured:
  // one block of 8 passes beats two of 4 at P = 64, N = 128, since every
  // block loads the token inputs)
  switch (passes) {
    case 1: return launch_siso_tok<TI, TO, N, 1>(a, units, s);
    case 2: return launch_siso_tok<TI, TO, N, 2>(a, units, s);
    case 3:
    case 4: return launch_siso_tok<TI, TO, N, 4>(a, units, s);
    default: return launch_siso_tok<TI, TO, N, 8>(a, units, s);
  }
}

template <typename TI, typename TO>
int dispatch_tok(const DecodeArgs& a, int units, hipStream_t s, hipError_t* err) {
  if (a.R == 1) {
    switch (a.N) {
      case 16: *err = siso_tok_n<TI, TO, 16>(a, units, s); return 0;
      case 32: *err = siso_tok_n<TI, TO, 32>(a, units, s); return 0;
      case 64: *err = siso_tok_n<TI, TO, 64>(a, units, s); return 0;
      case 128: *err = siso_tok_n<TI, TO, 128>(a, units, s); return 0;
      case 256: *err = siso_tok_n<TI, TO, 256>(a, units, s); return 0;
      default: return -1;
    }
  }
#define M3_MIMO_N(NN)                                                       \
  case NN:                                                                  \
    switch (a.R) {                                                          \
      case 2: *err = launch_mimo_tok<TI, TO, NN, 2>(a, units, s); return 0; \
      case 3: *err = launch_mimo_tok<TI, TO, NN, 3>(a, units, s); return 0; \
      case 4: *err = launch_mimo_grp<TI, TO, NN>(a, units, s); return 0;    \
      case 8: *err = launch_mimo_tok<TI, TO, NN, 8>(a, units, s); return 0; \
      default: return -1;                                                   \
    }
  switch (a.N) {
    M3_MIMO_N(16)
    M3_MIMO_N(32)
    M3_MIMO_N(64)
    M3_MIMO_N(128)
    default: return -1;
  }
#undef M3_MIMO_N
}

}  // namespace

bool decode_tokens_supported(int P, int N, int R) {
  if (R == 1) return N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
  if (P % 16 != 0 || P > 64) return false;   // one 16-row block per wave
  if (!(N == 16 || N == 32 || N == 64 || N == 128)) return false;
  return R == 2 || R == 3 || R == 4 || R == 8;
}

int launch_decode_tokens(const DecodeArgs& a, int in_bf16, int out_bf16, int units,
                         hipStream_t s, hipError_t* err) {
  if (in_bf16) {
    return out_bf16 ? dispatch_tok<bf16_t, bf16_t>(a, units, s, err)
                    : dispatch_tok<bf16_t, float>(a, units, s, err);
  }
  return out_bf16 ? dispatch_tok<float, bf16_t>(a, units, s, err)
                  : dispatch_tok<float, float>(a, units, s, err);
}

}  // namespace m3
