// backward_mma.hip -- gradients of the rank-R chunked prefill scan on the
// matrix cores (gfx950).
//
// The gradients are those of backward.hip (the recurrence of the Mamba-3
// article [xxxxx.co.kr, sections 1.1-1.3], differentiated in the chunked
// form of prefill.hip).  With rank R every token is R virtual rows (t, r)
// of the chunk, and every contraction over them is a dense product of the
// chunk's Q R = 64 R rows, here on MFMA tiles (mfma_pol.h: fp32 operands
// for fp32 inputs, bf16 hi + lo splits for bf16 inputs):
//   K1 = Ct Bt^T,  K2 = dY X^T,  W1 = M o K1,  W2 = M o K2   (M: decay mask)
//   dx  = W1^T dY + diag(m_end) Bt Gt^T
//   dBt = W2^T Ct + diag(m_end) X Gt
//   dCt = W2 Bt + diag(e^{cs}) dY Shat
//   dM[t, u] = sum over the R x R rank pairs of K1 o K2
// Launches after the forward states (which launch_backward runs):
//  k_bwd_adjoint_mma (batch, head, chunk): sum_t e^{cs_t} dY_t Ct_t^T;
//  k_bwd_state_pass  (backward.hip): the reverse pass over chunks, with
//           each chunk's end-state sums;
//  k_bwd_u  (batch, head, chunk [x 2]): one wave per 16 u rows, walking the
//           t rows at or after them: dx, dB, the mask's column sums, the
//           u side of the phase gradient;
//  k_bwd_t  (batch, head, chunk [x 2]): one wave per 16 t rows, walking the
//           u rows at or before them: dC and the C side of the phase
//           gradient;
//  k_bwd_fin (batch, head, chunk): the per-token gradients of the chunk (dt,
//           lam, A, theta) from the token sums of both sides.
// Every sum runs in a fixed order (no atomics): equal calls give equal bits.
#include "chunk_common.h"
#include "mfma_pol.h"

namespace m3 {

namespace {

constexpr int kTB = 32;   // virtual rows of a staged block (two 16-row tiles)

// x or dy rows of a block as loaded, into st[v - v0][e] (split or fp32)
template <class Pol, typename TI, int E, int R, int NT, int ROWS>
__device__ __forceinline__ void put_rows(const RowBlock<TI, E * R, R, NT, false, ROWS>& rb,
                                         typename Pol::template Store<ROWS, E>& st) {
  using RBk = RowBlock<TI, E * R, R, NT, false, ROWS>;
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    float v[8];
    rb.get(i, v);
    if constexpr (R == 1) {
      Pol::put8(st, tl, e0, v);
    } else {
      constexpr int M = 8 / R;   // element j is (column e0/R + j/R, rank j%R)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float w[M];
#pragma unroll
        for (int m = 0; m < M; ++m) w[m] = v[m * R + r];
        Pol::template putn<M>(st, tl * R + r, e0 / R, w);
      }
    }
  }
}

// x rows of a block into an XStore, natural k order: xs[v - v0][p]
template <class Pol, typename TI, int P, int R, int NT, int ROWS>
__device__ __forceinline__ void put_xrows(const RowBlock<TI, P * R, R, NT, false, ROWS>& rb,
                                          typename Pol::template XStore<ROWS, P>& xs) {
  using RBk = RowBlock<TI, P * R, R, NT, false, ROWS>;
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    float v[8];
    rb.get(i, v);
    if constexpr (R == 1) {
      Pol::template putxn<4>(xs, tl, e0, v);
      Pol::template putxn<4>(xs, tl, e0 + 4, v + 4);
    } else {
      constexpr int M = 8 / R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float w[M];
#pragma unroll
        for (int m = 0; m < M; ++m) w[m] = v[m * R + r];
        Pol::template putxn<M>(xs, tl * R + r, e0 / R, w);
      }
    }
  }
}

// rows of a block transposed, st[e][v - v0]: B or C rotated by -Phi_t
// (ROT) and scaled by sc[t] (when given), or x / dy as loaded
template <class Pol, typename TI, int E, int R, int NT, int ROWS, bool ROT, class Tab>
__device__ __forceinline__ void put_rows_T(const RowBlock<TI, E * R, R, NT, false, ROWS>& rb,
                                           typename Pol::template Store<E, ROWS>& st, const Tab& tb,
                                           const float* sc, int t0, int Lc) {
  using RBk = RowBlock<TI, E * R, R, NT, false, ROWS>;
  constexpr int NPAIR = 4 / R;   // complex pairs per vector
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    const int t = t0 + tl;
    const bool ok = t < Lc;
    float v[8];
    rb.get(i, v);
    if constexpr (ROT) {
      f2 csr[NPAIR];
      tb.template cs_run<NPAIR>(t, e0 / R / 2, ok, csr);
      const float w = (sc && ok) ? sc[t] : 1.0f;
#pragma unroll
      for (int pi = 0; pi < NPAIR; ++pi) {
        const f2 cs = w * csr[pi];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float u0 = v[(2 * pi) * R + r], u1 = v[(2 * pi + 1) * R + r];
          v[(2 * pi) * R + r] = cs.x * u0 + cs.y * u1;
          v[(2 * pi + 1) * R + r] = -cs.y * u0 + cs.x * u1;
        }
      }
    }
    // the R virtual rows of token tl are consecutive columns of st
#pragma unroll
    for (int m = 0; m < 8 / R; ++m) Pol::template putn<R>(st, e0 / R + m, tl * R, v + m * R);
  }
}

// rows of a block into both layouts, st[v - v0][e] and stT[e][v - v0]: B or
// C rotated by -Phi_t (ROT; one rotation for both), or x / dy as loaded
template <class Pol, typename TI, int E, int R, int NT, int ROWS, bool ROT, class Tab>
__device__ __forceinline__ void put_rows_both(const RowBlock<TI, E * R, R, NT, false, ROWS>& rb,
                                              typename Pol::template Store<ROWS, E>& st,
                                              typename Pol::template Store<E, ROWS>& stT, const Tab& tb,
                                              int t0, int Lc) {
  using RBk = RowBlock<TI, E * R, R, NT, false, ROWS>;
  constexpr int NPAIR = 4 / R;
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi >= RBk::NV) continue;
    int tl, e0;
    RBk::where(vi, tl, e0);
    const int t = t0 + tl;
    float v[8];
    rb.get(i, v);
    if constexpr (ROT) {
      f2 csr[NPAIR];
      tb.template cs_run<NPAIR>(t, e0 / R / 2, t < Lc, csr);
#pragma unroll
      for (int pi = 0; pi < NPAIR; ++pi) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float u0 = v[(2 * pi) * R + r], u1 = v[(2 * pi + 1) * R + r];
          v[(2 * pi) * R + r] = csr[pi].x * u0 + csr[pi].y * u1;
          v[(2 * pi + 1) * R + r] = -csr[pi].y * u0 + csr[pi].x * u1;
        }
      }
    }
    if constexpr (R == 1) {
      Pol::put8(st, tl, e0, v);
    } else {
      constexpr int M = 8 / R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float w[M];
#pragma unroll
        for (int m = 0; m < M; ++m) w[m] = v[m * R + r];
        Pol::template putn<M>(st, tl * R + r, e0 / R, w);
      }
    }
#pragma unroll
    for (int m = 0; m < 8 / R; ++m) Pol::template putn<R>(stT, e0 / R + m, tl * R, v + m * R);
  }
}

// the R ranks of one (token, column) element: R consecutive values, one
// vector access (16-byte aligned arrays, so R * 4 or R * 2 bytes aligned)
template <int R>
__device__ __forceinline__ void ldr(const float* __restrict__ p, float* v) {
  if constexpr (R == 4) {
    const f4 q = *reinterpret_cast<const f4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (R == 2) {
    const f2 q = *reinterpret_cast<const f2*>(p);
    v[0] = q.x; v[1] = q.y;
  } else {
    v[0] = *p;
  }
}
template <int R>
__device__ __forceinline__ void ldr(const bf16_t* __restrict__ p, float* v) {
  if constexpr (R == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  } else if constexpr (R == 2) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(p);
    v[0] = __uint_as_float(q << 16); v[1] = __uint_as_float(q & 0xffff0000u);
  } else {
    v[0] = ld1(p, 0);
  }
}
template <int R>
__device__ __forceinline__ void str(float* __restrict__ p, const float* v) {
  if constexpr (R == 4) {
    *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
  } else if constexpr (R == 2) {
    *reinterpret_cast<f2*>(p) = f2{v[0], v[1]};
  } else {
    *p = v[0];
  }
}

// the R ranks of one (token, column) element as loaded (bf16 stays packed),
// held in registers from an early load until use
template <typename TI, int R>
struct RankRaw;
template <int R>
struct RankRaw<float, R> {
  float v[R];
  __device__ __forceinline__ void load(const float* __restrict__ p) { ldr<R>(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = 0.0f;
  }
  __device__ __forceinline__ void get(float* o) const {
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] = v[r];
  }
  __device__ __forceinline__ void get(float* o, bool keep) const {
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] = keep ? v[r] : 0.0f;
  }
};
template <int R>
struct RankRaw<bf16_t, R> {
  static_assert(R == 1 || R == 2 || R == 4, "ranks per element");
  uint32_t u[(R + 1) / 2];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p) {
    if constexpr (R == 4) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      u[0] = q.x;
      u[1] = q.y;
    } else if constexpr (R == 2) {
      u[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      u[0] = p->bits;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < (R + 1) / 2; ++i) u[i] = 0u;
  }
  __device__ __forceinline__ void get(float* o) const {
    if constexpr (R == 1) {
      o[0] = __uint_as_float(u[0] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < R / 2; ++i) {
        o[2 * i] = __uint_as_float(u[i] << 16);
        o[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  }
  // the values, or zeros when keep is false
  __device__ __forceinline__ void get(float* o, bool keep) const {
    RankRaw k = *this;
#pragma unroll
    for (int i = 0; i < (R + 1) / 2; ++i) k.u[i] = keep ? u[i] : 0u;
    k.get(o);
  }
};

// the rotated value (by -Phi) of element n of a (column n, partner n ^ 1)
// pair, from both raw elements
__device__ __forceinline__ float rot_own(float own, float oth, bool odd, f2 cs) {
  return odd ? -cs.y * oth + cs.x * own : cs.x * own + cs.y * oth;
}

// sum of a lane's four D rows by token (rows 4g .. 4g + 3 hold whole tokens
// when R divides 4) into out[token]: out gets one write per token
template <int R, class F>
__device__ __forceinline__ void rows_by_token(const float* v, int row0, F&& put) {
  float s = 0.0f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    s += v[jj];
    if (jj % R == R - 1) {
      put((row0 + jj) / R, s);
      s = 0.0f;
    }
  }
}

// --------------------------------------------------------------------------
// sum_{t,r} e^{cs_t} dy_{t,r} Ct_{t,r}^T of one chunk (P x N) into dS: the
// P x N output tiles over four waves, t in blocks of 32 virtual rows
template <int P, int N>
struct AdjGeo {
  static constexpr int NW = 4, NT = 256;
  static constexpr int NTN = N / 16, TILES = (P / 16) * NTN, TPW = TILES / NW;
  static_assert(TPW >= 1 && NTN % TPW == 0, "one output row of tiles per wave");
};

template <class Pol, int P, int N>
struct AdjSmem {
  Tables<N, false> tb;
  union U {
    TableScratch<N, AdjGeo<P, N>::NT> scr;
    struct S {
      typename Pol::template Store<P, kTB> y;   // dy^T     [p][v]
      typename Pol::template Store<N, kTB> c;   // e^cs Ct^T [n][v]
    } st;
  } u;
};

template <class Pol, typename TI, typename TY, int P, int N, int R>
__global__ __launch_bounds__(256) void k_bwd_adjoint_mma(BackwardArgs g) {
  const PrefillArgs& a = g.f;
  using AG = AdjGeo<P, N>;
  constexpr int NT = AG::NT;
  __shared__ AdjSmem<Pol, P, N> sm;
  const int h = blockIdx.y;
  ChunkRef ck;
  if (!chunk_ref(a, blockIdx.x, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, gq = lane >> 4, l16 = lane & 15;
  const int rows = Lc * R, nkb = (rows + kTB - 1) / kTB;
  const TI* __restrict__ Cg = static_cast<const TI*>(a.C);
  const TY* __restrict__ Yg = static_cast<const TY*>(g.dy);
  ThetaBlock<TI, N, NT> thb;
  thb.load(a, b, h, c0, Lc);
  RowBlock<TY, P * R, R, NT, false, kTB> yb;
  RowBlock<TI, N * R, R, NT, false, kTB> cb;
  yb.template load<false>(Yg, a, b, h, c0, Lc, 0);
  cb.template load<true>(Cg, a, b, h, c0, Lc, 0);
  chunk_tables<TI, N, NT>(a, thb, Lc, sm.tb, sm.u.scr, 0);
  if (tid < kQ) sm.tb.aux[tid] = tid < Lc ? __expf((float)sm.tb.cs[tid]) : 0.0f;

  const int tile0 = wave * AG::TPW, pt = tile0 / AG::NTN, nt0 = tile0 % AG::NTN;
  f4 acc[AG::TPW];
#pragma unroll
  for (int i = 0; i < AG::TPW; ++i) acc[i] = f4{0, 0, 0, 0};
  for (int k = 0; k < nkb; ++k) {
    __syncthreads();   // the tables are built; the previous block is read
    put_rows_T<Pol, TY, P, R, NT, kTB, false>(yb, sm.u.st.y, sm.tb, nullptr, k * kTB / R, Lc);
    put_rows_T<Pol, TI, N, R, NT, kTB, true>(cb, sm.u.st.c, sm.tb, sm.tb.aux, k * kTB / R, Lc);
    if (k + 1 < nkb) {
      yb.template load<false>(Yg, a, b, h, c0, Lc, (k + 1) * kTB);
      cb.template load<true>(Cg, a, b, h, c0, Lc, (k + 1) * kTB);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTB; kk += Pol::KS) {
      const typename Pol::Frag af = Pol::frag(sm.u.st.y, 16 * pt, kk, lane);
#pragma unroll
      for (int i = 0; i < AG::TPW; ++i)
        acc[i] = Pol::mma(af, Pol::frag(sm.u.st.c, 16 * (nt0 + i), kk, lane), acc[i]);
    }
  }
  // D[p][n]: column n = 16 nt + l16, rows p = 16 pt + 4 g + jj
  float* __restrict__ out = g.dS + ck.id * (P * N);
#pragma unroll
  for (int i = 0; i < AG::TPW; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[(16 * pt + 4 * gq + jj) * N + 16 * (nt0 + i) + l16] = acc[i][jj];
}

// --------------------------------------------------------------------------
// The u side.  One wave per 16-row u tile; a rank-4 chunk (16 tiles) is
// split over two blocks of 8 waves, the u rows 0..127 and 128..255.
template <int P, int N, int R>
struct GeoU {
  static constexpr int ROWS = kQ * R, TILES = ROWS / 16;
  static constexpr int NW = TILES > 8 ? 8 : TILES;
  static constexpr int SPLIT = TILES / NW;
  static constexpr int NT = 64 * NW;
  static constexpr int BROWS = ROWS / SPLIT;   // u rows per block
  static_assert((SPLIT == 1 || SPLIT == 2) && BROWS % 64 == 0, "u-side geometry");
};

// per-chunk token sums in the workspace: [units][kTokSums][Q]
enum TokSum {
  kMcol = 0, kEcol = 1, kEdiag = 2, kRrow0 = 3, kRrow1 = 4, kDmend = 5, kDe = 6, kTokSums = 7
};
static_assert(kTokSums == kBwdTokSums, "token sum slots");

template <class Pol, int P, int N, int R>
struct USmem {
  using G = GeoU<P, N, R>;
  Tables<N, false> tb;
  float rowpart[G::NW][kQ];   // each wave's row sums of dM o M
  float part[G::NT];          // per-thread parts of the end-state sums
  float red[G::NW];
  union U {
    TableScratch<N, G::NT> scr;
    struct O {
      typename Pol::template Store<64, N> b;    // own rotated B rows
      typename Pol::template XStore<64, P> x;   // own x rows
    } own;
    struct S {
      typename Pol::template Store<kTB, N> c;   // Ct rows   [v][n]
      typename Pol::template Store<kTB, P> y;   // dy rows   [v][p]
      typename Pol::template Store<N, kTB> ct;  // Ct^T      [n][v]
      typename Pol::template Store<P, kTB> yt;  // dy^T      [p][v]
    } st[2];                                    // double-buffered
    struct E {
      typename Pol::template Store<P, N> gt;    // Gt        [p][n]
      typename Pol::template Store<N, P> gtt;   // Gt^T      [n][p]
    } e;
  } u;
};

template <class Pol, typename TI, typename TY, int P, int N, int R>
__global__ __launch_bounds__((GeoU<P, N, R>::NT)) void k_bwd_u(BackwardArgs g) {
  const PrefillArgs& a = g.f;
  using G = GeoU<P, N, R>;
  constexpr int NT = G::NT, NW = G::NW, KS = Pol::KS;
  constexpr int NKS = N / KS, PKS = P / KS, PT = P / 16, NTL = N / 16, NP = N / 2;
  __shared__ USmem<Pol, P, N, R> sm;
  // the two blocks of a split chunk are 8 apart in launch order (same XCD)
  int c, half;
  if constexpr (G::SPLIT == 2) {
    c = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    half = (blockIdx.x >> 3) & 1;
  } else {
    c = blockIdx.x;
    half = 0;
  }
  const int h = blockIdx.y;
  ChunkRef ck;
  if (!chunk_ref(a, c, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc;
  const int rows = Lc * R;
  const int v0 = half * G::BROWS;
  if (v0 >= rows) return;   // k_bwd_t reads this half's row sums only when it exists
  const bool last = c + 1 >= a.nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4, l16 = lane & 15;
  // waves w and w + 4 share a SIMD: tiles w and 7 - w even out the causal work
  const int lt = (NW == 8) ? (wave < 4 ? wave : 11 - wave) : wave;
  const int utile = v0 / 16 + lt;
  const bool live = 16 * utile < rows;
  const int uv = 16 * utile + l16;   // this lane's u column in the Gram tiles
  const int utok = uv / R;

  const int G_ = a.G;
  const int64_t gi = group_index(a, b, c0, h), ti0 = token_index(a, b, c0, h);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Cg = static_cast<const TI*>(a.C);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  const TY* __restrict__ Yg = static_cast<const TY*>(g.dy);
  const TI* __restrict__ Bc = Bg + gi * N * R;   // this chunk's first token
  const TI* __restrict__ Xc = Xg + ti0 * P * R;

  // every prologue load goes out first: phase inputs and token scalars,
  // this block's own B and x rows, the first t block of C and dy
  constexpr int NPC = G::BROWS / 64;   // own-row pieces of 64 rows
  const int kb0 = v0 / kTB, nkb = (rows + kTB - 1) / kTB;
  ThetaBlock<TI, N, NT> thb;
  thb.load(a, b, h, c0, Lc);
  RowBlock<TI, N * R, R, NT, false, 64> rb[NPC];
  RowBlock<TI, P * R, R, NT, false, 64> rx[NPC];
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    if (v0 + 64 * pc < rows) {
      rb[pc].template load<true>(Bg, a, b, h, c0, Lc, v0 + 64 * pc);
      rx[pc].template load<false>(Xg, a, b, h, c0, Lc, v0 + 64 * pc);
    }
  }
  RowBlock<TI, N * R, R, NT, false, kTB> cb;
  RowBlock<TY, P * R, R, NT, false, kTB> yb;
  cb.template load<true>(Cg, a, b, h, c0, Lc, kb0 * kTB);
  yb.template load<false>(Yg, a, b, h, c0, Lc, kb0 * kTB);
  for (int i = tid; i < NW * kQ; i += NT) (&sm.rowpart[0][0])[i] = 0.0f;
  chunk_tables<TI, N, NT>(a, thb, Lc, sm.tb, sm.u.scr, 0);

  // own rotated B rows and x rows -> fragments in registers
  typename Pol::Frag bf[NKS];
  typename Pol::XFrag xf[PKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) bf[s] = typename Pol::Frag{};
#pragma unroll
  for (int s = 0; s < PKS; ++s) xf[s] = typename Pol::XFrag{};
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    const int pv0 = v0 + 64 * pc;
    if (pv0 >= rows) break;
    if (pc > 0) __syncthreads();   // the previous piece is read
    store_rows<Pol, TI, N, R, NT, 64>(rb[pc], sm.u.own.b, sm.tb, pv0 / R, Lc, NoPrep{});
    put_xrows<Pol, TI, P, R, NT, 64>(rx[pc], sm.u.own.x);
    __syncthreads();
    if (lt / 4 == pc) {
#pragma unroll
      for (int s = 0; s < NKS; ++s) bf[s] = Pol::frag(sm.u.own.b, 16 * (lt % 4), s * KS, lane);
#pragma unroll
      for (int s = 0; s < PKS; ++s) xf[s] = Pol::fragx_c(sm.u.own.x, 16 * (lt % 4), s * KS, lane);
    }
  }

  // the end-state and output operands go out now and arrive during the walk:
  // G_end (this thread's pairs of it), and the raw B and x of this lane's D
  // rows (u) and columns in the end-state products
  const float* __restrict__ Gend = last ? g.dhT ? g.dhT + ((int64_t)b * a.H + h) * P * N : nullptr
                                        : g.dS + (ck.id + 1) * (P * N);
  constexpr int GPT = P * NP / NT;   // G_end pairs per thread
  static_assert(P * NP % NT == 0, "G_end pairs per thread");
  f2 gpre[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int e = tid + NT * i, p = e / NP, kp = e % NP;
    gpre[i] = Gend ? *reinterpret_cast<const f2*>(Gend + (int64_t)p * N + 2 * kp) : f2{0.0f, 0.0f};
  }
  const int urow0 = 16 * utile + 4 * gq;   // this lane's D rows (u) in the end-state products
  // (a row past the chunk re-reads its first token and reads as zeros)
  RankRaw<TI, R> bpre[NTL][4 / R], xpre[PT][4 / R];
  uint32_t uok = 0u;   // bit j0 / R: the D rows urow0 + j0 .. + R - 1 are rows of the chunk
#pragma unroll
  for (int j0 = 0; j0 < 4; j0 += R) {
    const int vr = urow0 + j0;
    const bool ok = live && vr < rows;
    const int ut = ok ? vr / R : 0;
    uok |= static_cast<uint32_t>(ok) << (j0 / R);
#pragma unroll
    for (int i = 0; i < NTL; ++i) bpre[i][j0 / R].load(Bc + (int64_t)ut * G_ * N * R + (int64_t)(16 * i + l16) * R);
#pragma unroll
    for (int i = 0; i < PT; ++i) xpre[i][j0 / R].load(Xc + (int64_t)ut * a.H * P * R + (int64_t)(16 * i + l16) * R);
  }
  // this thread's end rotation (the pair tid % NP of every G_end pair it
  // holds) and the next chunk's left-endpoint weight, also for after the walk
  static_assert(NT % NP == 0, "a thread's G_end pairs share one column pair");
  const f2 rek = reinterpret_cast<const f2*>(a.rot_end)[ck.id * NP + tid % NP];
  const int64_t tnx = ti0 + (int64_t)(ck.next ? kQ : 0) * a.H;   // (a valid token when there is none)
  const float lam_n = ldy<TI>(a.lam, tnx), dt_n = ldy<TI>(a.dt, tnx);

  // ---- walk the t rows at or after this block's first u row
  f4 accx[PT], accb[NTL];
#pragma unroll
  for (int i = 0; i < PT; ++i) accx[i] = f4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NTL; ++i) accb[i] = f4{0, 0, 0, 0};
  float mcol = 0.0f, ecol = 0.0f, edg = 0.0f;
  const float gu = utok < kQ ? sm.tb.gam[utok] : 0.0f;
  const float bu = utok + 1 < kQ ? sm.tb.bpr[utok + 1] : 0.0f;
  const double csu = sm.tb.cs[min(utok, kQ - 1)];
  // t block k goes into buffer k & 1 while the MFMAs of block k - 1 run;
  // one barrier per block
  auto stage = [&](int k) {
    auto& st = sm.u.st[k & 1];
    put_rows_both<Pol, TI, N, R, NT, kTB, true>(cb, st.c, st.ct, sm.tb, k * kTB / R, Lc);
    put_rows_both<Pol, TY, P, R, NT, kTB, false>(yb, st.y, st.yt, sm.tb, k * kTB / R, Lc);
    if (k + 1 < nkb) {
      cb.template load<true>(Cg, a, b, h, c0, Lc, (k + 1) * kTB);
      yb.template load<false>(Yg, a, b, h, c0, Lc, (k + 1) * kTB);
    }
  };
  __syncthreads();   // the own-row buffers are read
  stage(kb0);
  __syncthreads();
  for (int k = kb0; k < nkb; ++k) {
    if (k + 1 < nkb) stage(k + 1);
    const auto& st = sm.u.st[k & 1];
    const int ttok_max = min(Lc - 1, (k * kTB + kTB - 1) / R);
    if (live && (16 * utile) / R <= ttok_max) {
      f4 w1[2], w2[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f4 d1 = f4{0, 0, 0, 0}, d2 = f4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NKS; ++s) d1 = Pol::mma(Pol::frag(st.c, 16 * dt, s * KS, lane), bf[s], d1);
#pragma unroll
        for (int s = 0; s < PKS; ++s) d2 = Pol::mma_x(Pol::frag(st.y, 16 * dt, s * KS, lane), xf[s], d2);
        // D[t][u]: column u = uv, rows t = k kTB + 16 dt + 4 g + jj; the R
        // rows of one t token share its mask value
        const int trow0 = k * kTB + 16 * dt + 4 * gq;
        float rv[4 / R];
#pragma unroll
        for (int j0 = 0; j0 < 4; j0 += R) {
          const int ttok = (trow0 + j0) / R;
          float em = 0.0f, mm = 0.0f;
          if (ttok < Lc && ttok >= utok && uv < rows) {
            em = __expf((float)(sm.tb.cs[ttok] - csu));
            mm = em * (gu + (utok < ttok ? bu : 0.0f));
          }
          float ps = 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int jj = j0 + r;
            ps += d1[jj] * d2[jj];
            w1[dt][jj] = d1[jj] * mm;
            w2[dt][jj] = d2[jj] * mm;
          }
          mcol += ps * mm;
          if (ttok > utok) ecol += ps * em;
          else edg += ps * em;
          rv[j0 / R] = group_sum<16>(ps * mm);   // over this tile's 16 u columns
        }
        if (l16 == 0) {
#pragma unroll
          for (int j0 = 0; j0 < 4; j0 += R) sm.rowpart[wave][(trow0 + j0) / R] = rv[j0 / R];
        }
      }
#pragma unroll
      for (int q = 0; q < 2 / Pol::DT; ++q) {
        const typename Pol::Frag a1 = Pol::frag_from_d(w1 + q * Pol::DT);
        const typename Pol::Frag a2 = Pol::frag_from_d(w2 + q * Pol::DT);
        const int kk = 16 * Pol::DT * q;
#pragma unroll
        for (int i = 0; i < PT; ++i) accx[i] = Pol::mma(a1, Pol::fragp(st.yt, 16 * i, kk, lane), accx[i]);
#pragma unroll
        for (int i = 0; i < NTL; ++i) accb[i] = Pol::mma(a2, Pol::fragp(st.ct, 16 * i, kk, lane), accb[i]);
      }
    }
    __syncthreads();
  }

  // ---- token sums: the mask's column sums (over the row groups, then the
  // ranks of a token) and the row sums of this block's u columns
  float* __restrict__ tk = g.tokw + ck.id * (kTokSums * kQ);
  mcol += __shfl_xor(mcol, 16, 64);
  mcol += __shfl_xor(mcol, 32, 64);
  ecol += __shfl_xor(ecol, 16, 64);
  ecol += __shfl_xor(ecol, 32, 64);
  edg += __shfl_xor(edg, 16, 64);
  edg += __shfl_xor(edg, 32, 64);
  mcol = group_sum<R>(mcol);
  ecol = group_sum<R>(ecol);
  edg = group_sum<R>(edg);
  if (live && gq == 0 && l16 % R == 0 && utok < Lc) {
    tk[kMcol * kQ + utok] = mcol;
    tk[kEcol * kQ + utok] = ecol;
    tk[kEdiag * kQ + utok] = edg;
  }
  __syncthreads();   // the row sums are in; the staging buffers are free
  if (tid < kQ) {
    float s = 0.0f;
    for (int w = 0; w < NW; ++w) s += sm.rowpart[w][tid];
    tk[(kRrow0 + half) * kQ + tid] = s;
  }

  // ---- the end state: Gt = rows of G_end rotated by -Phi_end, in both
  // layouts (the staging buffers are free: the row sums above are past a
  // barrier).  The chunk's end-state sums come from the reverse state pass.
  const float bpL = ck.next ? (1.0f - lam_n) * dt_n : 0.0f;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int e = tid + NT * i, p = e / NP, kp = e % NP;
    const f2 gt = rot_neg(gpre[i], rek);
    const float v2[2] = {gt.x, gt.y};
    Pol::template putn<2>(sm.u.e.gt, p, 2 * kp, v2);
    Pol::put(sm.u.e.gtt, 2 * kp, p, gt.x);
    Pol::put(sm.u.e.gtt, 2 * kp + 1, p, gt.y);
  }
  __syncthreads();
  const double cs_end = sm.tb.cs[Lc - 1];
  float mu[4], cu[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int ut = (urow0 + jj) / R;
    mu[jj] = cu[jj] = 0.0f;
    if (urow0 + jj < rows) {
      const float e = __expf((float)(cs_end - sm.tb.cs[ut]));
      mu[jj] = e * (sm.tb.gam[ut] + (ut < Lc - 1 ? sm.tb.bpr[ut + 1] : 0.0f));
      cu[jj] = mu[jj] + (ut == Lc - 1 ? bpL : 0.0f);
    }
  }
  // v = Bt Gt^T: dx += cu v, dm_end[u] = sum over p and ranks of x v
  {
    float dmv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      f4 v = f4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s) v = Pol::mma(bf[s], Pol::frag(sm.u.e.gt, 16 * i, s * KS, lane), v);
      float xv[4];
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += R) xpre[i][j0 / R].get(xv + j0, (uok >> (j0 / R)) & 1u);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        accx[i][jj] += cu[jj] * v[jj];
        dmv[jj] += xv[jj] * v[jj];
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dmv[jj] = group_sum<16>(dmv[jj]);
    if (live && l16 == 0)
      rows_by_token<R>(dmv, urow0, [&](int t, float v) {
        if (t < Lc) tk[kDmend * kQ + t] = v;
      });
  }

  // ---- outputs: dx; w = X Gt: dBt += m_end w, the crossing term of the
  // last token (raw frame, kept out of the phase gradient), dB back in the
  // raw frame and the u side of the phase gradient
  const bool shared_grp = G_ != a.H;
  if (live) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = 16 * i + l16;
      const float xo[4] = {accx[i][0], accx[i][1], accx[i][2], accx[i][3]};
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += R) {
        const int vr = urow0 + j0;
        if (vr < rows) str<R>(g.dx + (ti0 + (int64_t)(vr / R) * a.H) * P * R + p * R, xo + j0);
      }
    }
  }
  float* __restrict__ dBo = shared_grp ? g.dBh : g.dB;
  float* __restrict__ dph = g.dphiB + ck.id * (kQ * NP);
#pragma unroll
  for (int i = 0; i < NTL; ++i) {
    f4 w = f4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < PKS; ++s) w = Pol::mma_xa(xf[s], Pol::frag(sm.u.e.gtt, 16 * i, s * KS, lane), w);
    const int n = 16 * i + l16, kp = n >> 1;
    const bool odd = n & 1;
    // raw B of this lane's column (the pair partner's from the next lane)
    float bo[4], raw[4], ph[4];
    f2 cs[4];
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += R) {
      const int vr = urow0 + j0, ut = vr / R;
      const bool ok = live && vr < rows;
      bpre[i][j0 / R].get(bo + j0, (uok >> (j0 / R)) & 1u);
      const f2 c2 = ok ? sm.tb.cs_of(ut, kp) : f2{1.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < R; ++r) cs[j0 + r] = c2;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int ut = (urow0 + jj) / R;
      const float bq = __shfl_xor(bo[jj], 1, 64);
      const float dbt = accb[i][jj] + mu[jj] * w[jj];
      // cross(dBt, Bt) of pair kp: this lane's half
      ph[jj] = odd ? -dbt * rot_own(bq, bo[jj], false, cs[jj]) : dbt * rot_own(bq, bo[jj], true, cs[jj]);
      const float v = dbt + (ck.next && ut == Lc - 1 ? bpL * w[jj] : 0.0f);
      const float pv = __shfl_xor(v, 1, 64);
      raw[jj] = odd ? cs[jj].y * pv + cs[jj].x * v : cs[jj].x * v - cs[jj].y * pv;
    }
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += R) {
      const int vr = urow0 + j0;
      if (live && vr < rows) str<R>(dBo + (ti0 + (int64_t)(vr / R) * a.H) * N * R + (int64_t)n * R, raw + j0);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ph[jj] += __shfl_xor(ph[jj], 1, 64);
    if (live && !odd)
      rows_by_token<R>(ph, urow0, [&](int t, float v) {
        if (t < Lc) dph[t * NP + kp] = v;
      });
  }
}

// --------------------------------------------------------------------------
// The t side.  One wave per 16-row t tile, split over blocks as the u side.
template <class Pol, int P, int N, int R>
struct TSmem {
  using G = GeoU<P, N, R>;
  Tables<N, false> tb;
  float ecs[kQ];
  union alignas(16) U {
    TableScratch<N, G::NT> scr;
    typename Pol::template Store<64, P> own;   // own dy rows
    typename Pol::template Store<N, P> sht;    // Shat^T [n][p]
    struct S {
      typename Pol::template XStore<kTB, P> x;   // x rows [v][p]
      typename Pol::template Store<N, kTB> bt;   // Bt^T   [n][v]
    } stg[2];
  } u;
};

// a single input's t-side block is 64 KB of LDS: two fit on a CU once the
// registers allow two waves per SIMD (a few spill; the call measured 2-3% faster)
template <class Pol, int R>
constexpr int t_min_waves() { return R == 1 && std::is_same<Pol, PolHalf>::value ? 2 : 1; }

template <class Pol, typename TI, typename TY, int P, int N, int R>
__global__ __launch_bounds__((GeoU<P, N, R>::NT)) __attribute__((amdgpu_waves_per_eu(t_min_waves<Pol, R>()))) void k_bwd_t(BackwardArgs g) {
  const PrefillArgs& a = g.f;
  using G = GeoU<P, N, R>;
  constexpr int NT = G::NT, NW = G::NW, KS = Pol::KS;
  constexpr int PKS = P / KS, NTL = N / 16, NP = N / 2;
  __shared__ TSmem<Pol, P, N, R> sm;
  int c, half;
  if constexpr (G::SPLIT == 2) {
    c = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    half = (blockIdx.x >> 3) & 1;
  } else {
    c = blockIdx.x;
    half = 0;
  }
  const int h = blockIdx.y;
  ChunkRef ck;
  if (!chunk_ref(a, c, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc;
  const int rows = Lc * R;
  const int v0 = half * G::BROWS;
  if (v0 >= rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 4, l16 = lane & 15;
  // waves w and w + 4 share a SIMD: tiles w and 7 - w even out the causal work
  const int lt = (NW == 8) ? (wave < 4 ? wave : 11 - wave) : wave;
  const int ttile = v0 / 16 + lt;
  const bool live = 16 * ttile < rows;
  const int tv = 16 * ttile + l16;   // this lane's t column in the Gram tiles
  const int ttok = tv / R;
  const int G_ = a.G;
  const bool shared_grp = G_ != a.H;
  const int64_t gi = group_index(a, b, c0, h), ti0 = token_index(a, b, c0, h);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  const TY* __restrict__ Yg = static_cast<const TY*>(g.dy);
  const TI* __restrict__ Cc = static_cast<const TI*>(a.C) + gi * N * R;

  // every prologue load goes out first: phase inputs and token scalars,
  // this block's own dy rows, the entry state, the first u block of B and x
  constexpr int NPC = G::BROWS / 64;   // own-row pieces of 64 rows
  ThetaBlock<TI, N, NT> thb;
  thb.load(a, b, h, c0, Lc);
  RowBlock<TY, P * R, R, NT, false, 64> ybp[NPC];
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc)
    if (v0 + 64 * pc < rows) ybp[pc].template load<false>(Yg, a, b, h, c0, Lc, v0 + 64 * pc);
  StateBlock<P, N, NT> sb;
  sb.load(a.S + ck.id * (P * N));
  const int nkb = (min(rows, v0 + G::BROWS) + kTB - 1) / kTB;
  RowBlock<TI, N * R, R, NT, false, kTB> bb;
  RowBlock<TI, P * R, R, NT, false, kTB> xb;
  bb.template load<true>(Bg, a, b, h, c0, Lc, 0);
  xb.template load<false>(Xg, a, b, h, c0, Lc, 0);
  chunk_tables<TI, N, NT>(a, thb, Lc, sm.tb, sm.u.scr, 0);
  if (tid < kQ) sm.ecs[tid] = tid < Lc ? expf((float)sm.tb.cs[tid]) : 0.0f;

  // own dy rows -> fragments
  typename Pol::Frag yf[PKS];
#pragma unroll
  for (int s = 0; s < PKS; ++s) yf[s] = typename Pol::Frag{};
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) {
    if (v0 + 64 * pc >= rows) break;
    if (pc > 0) __syncthreads();   // the previous piece is read
    put_rows<Pol, TY, P, R, NT, 64>(ybp[pc], sm.u.own);
    __syncthreads();
    if (lt / 4 == pc) {
#pragma unroll
      for (int s = 0; s < PKS; ++s) yf[s] = Pol::frag(sm.u.own, 16 * (lt % 4), s * KS, lane);
    }
  }
  // the raw C of this lane's D rows (t) and columns, for the entry-state
  // and phase products: loaded once, now
  const int trow0 = 16 * ttile + 4 * gq;   // this lane's D rows (t) in the dC tiles
  // (a row past the chunk re-reads its first token and reads as zeros)
  RankRaw<TI, R> cpre[NTL][4 / R];
  uint32_t tok_rows = 0u;   // bit j0 / R: the D rows trow0 + j0 .. + R - 1 are rows of the chunk
#pragma unroll
  for (int j0 = 0; j0 < 4; j0 += R) {
    const int vr = trow0 + j0;
    const bool ok = live && vr < rows;
    const int t = ok ? vr / R : 0;
    tok_rows |= static_cast<uint32_t>(ok) << (j0 / R);
#pragma unroll
    for (int i = 0; i < NTL; ++i) cpre[i][j0 / R].load(Cc + (int64_t)t * G_ * N * R + (int64_t)(16 * i + l16) * R);
  }
  // the entry state: q = dY Shat, dCt = e^{cs_t} q, de_t = sum Ct . q
  __syncthreads();   // the own-row buffer is read
#pragma unroll
  for (int i = 0; i < StateBlock<P, N, NT>::IT; ++i) {
    const int vi = tid + NT * i;
    if (vi < StateBlock<P, N, NT>::NV) {
      float v[8];
      sb.raw[i].get(v);
      const int p = (8 * vi) / N, n = (8 * vi) % N;
#pragma unroll
      for (int j = 0; j < 8; ++j) Pol::put(sm.u.sht, n + j, p, v[j]);
    }
  }
  __syncthreads();
  float* __restrict__ tk = g.tokw + ck.id * (kTokSums * kQ);
  f4 acc[NTL];
  {
    float dev[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NTL; ++i) {
      f4 q = f4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < PKS; ++s) q = Pol::mma(yf[s], Pol::frag(sm.u.sht, 16 * i, s * KS, lane), q);
      const int n = 16 * i + l16;
      const bool odd = n & 1;
      float co[4], sc[4];
      f2 cs[4];
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += R) {
        const int vr = trow0 + j0, t = vr / R;
        const bool ok = live && vr < rows;
        cpre[i][j0 / R].get(co + j0, (tok_rows >> (j0 / R)) & 1u);
        const f2 c2 = ok ? sm.tb.cs_of(t, n >> 1) : f2{1.0f, 0.0f};
        const float e = ok ? sm.ecs[t] : 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          cs[j0 + r] = c2;
          sc[j0 + r] = e;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float cq = __shfl_xor(co[jj], 1, 64);
        dev[jj] += rot_own(co[jj], cq, odd, cs[jj]) * q[jj];
        acc[i][jj] = sc[jj] * q[jj];
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) dev[jj] = group_sum<16>(dev[jj]);
    if (live && l16 == 0)
      rows_by_token<R>(dev, trow0, [&](int t, float v) {
        if (t < Lc) tk[kDe * kQ + t] = v;
      });
  }

  // the u side's phase gradients of this lane's (token, pair) entries (k_bwd_u
  // wrote them before this kernel): with few ranks per lane (R >= 2) they are
  // read now and arrive during the walk
  float* __restrict__ dCo = shared_grp ? g.dCh : g.dC;
  float* __restrict__ dph = g.dphiB + ck.id * (kQ * NP);
  float dpre[NTL][4 / R];
  auto read_dph = [&]() {
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += R) {
      const bool ok = live && trow0 + j0 < rows;
      const int t = ok ? (trow0 + j0) / R : 0;
#pragma unroll
      for (int i = 0; i < NTL; ++i) dpre[i][j0 / R] = dph[t * NP + ((16 * i + l16) >> 1)];
    }
  };
  constexpr bool kEarlyDph = R >= 2;
  if constexpr (kEarlyDph) read_dph();

  // ---- walk the u rows at or before this wave's t rows: dCt += W2 Bt
  const int ttok_max = min(Lc - 1, (16 * ttile + 15) / R);
  auto stage = [&](int k) {
    put_rows_T<Pol, TI, N, R, NT, kTB, true>(bb, sm.u.stg[k & 1].bt, sm.tb, nullptr, k * kTB / R, Lc);
    put_xrows<Pol, TI, P, R, NT, kTB>(xb, sm.u.stg[k & 1].x);
    if (k + 1 < nkb) {
      bb.template load<true>(Bg, a, b, h, c0, Lc, (k + 1) * kTB);
      xb.template load<false>(Xg, a, b, h, c0, Lc, (k + 1) * kTB);
    }
  };
  __syncthreads();   // Shat^T is read
  stage(0);
  __syncthreads();
  const double cst = sm.tb.cs[min(ttok, kQ - 1)];
  for (int k = 0; k < nkb; ++k) {
    if (k + 1 < nkb) stage(k + 1);
    if (live && (k * kTB) / R <= ttok_max) {
      f4 w[2];
#pragma unroll
      for (int du = 0; du < 2; ++du) {
        f4 d = f4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < PKS; ++s)
          d = Pol::mma_xa(Pol::fragx_c(sm.u.stg[k & 1].x, 16 * du, s * KS, lane), yf[s], d);
        // D[u][t]: column t = tv, rows u = k kTB + 16 du + 4 g + jj; the R
        // rows of one u token share its mask value
#pragma unroll
        for (int j0 = 0; j0 < 4; j0 += R) {
          const int ut = (k * kTB + 16 * du + 4 * gq + j0) / R;
          float mm = 0.0f;
          if (ttok < Lc && ut <= ttok)
            mm = __expf((float)(cst - sm.tb.cs[ut])) * (sm.tb.gam[ut] + (ut < ttok ? sm.tb.bpr[ut + 1] : 0.0f));
#pragma unroll
          for (int r = 0; r < R; ++r) w[du][j0 + r] = d[j0 + r] * mm;
        }
      }
#pragma unroll
      for (int q = 0; q < 2 / Pol::DT; ++q) {
        const typename Pol::Frag af = Pol::frag_from_d(w + q * Pol::DT);
#pragma unroll
        for (int i = 0; i < NTL; ++i)
          acc[i] = Pol::mma(af, Pol::fragp(sm.u.stg[k & 1].bt, 16 * i, 16 * Pol::DT * q, lane), acc[i]);
      }
    }
    __syncthreads();
  }

  // ---- dC back in the raw frame; the phase gradient of every (token, pair)
  // = the u side (from k_bwd_u, in place) + the C side.  The u side's values
  // of this lane's (token, pair) entries are read in one batch first (every
  // lane reads; an odd column or a row past the chunk re-reads a valid entry
  // and drops it).  All values are formed (in acc and dpre, in place) before
  // the first store: a use of a loaded value after a store would wait for
  // the store too.
  // A single input (one token per row, the whole chunk in the block) moves
  // these per-lane scalars through LDS, which is free after the walk: the
  // chunk's phase-gradient rows come in, and dC and the phase gradients go
  // out, as 16-byte row vectors (a fifth of the memory instructions)
  constexpr bool kLdsIo = R == 1;
  constexpr int CS = N + 4, DS = NP + 4;   // LDS row strides (16-byte aligned rows)
  static_assert(!kLdsIo || (G::BROWS == kQ && sizeof(sm.u) >= sizeof(float) * kQ * CS &&
                            sizeof(sm.u) >= sizeof(float) * kQ * DS),
                "the staging space holds a chunk's dC and phase-gradient rows");
  static_assert(alignof(decltype(sm.u)) >= 16, "16-byte LDS rows");
  float* __restrict__ lio = reinterpret_cast<float*>(&sm.u);
  if constexpr (kLdsIo) {
    for (int q = tid; q < Lc * (NP / 4); q += NT) {
      const int t = q / (NP / 4), k4 = 4 * (q % (NP / 4));
      *reinterpret_cast<f4*>(lio + t * DS + k4) = *reinterpret_cast<const f4*>(dph + t * NP + k4);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NTL; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = trow0 + jj;   // < kQ
        dpre[i][jj] = t < Lc ? lio[t * DS + ((16 * i + l16) >> 1)] : 0.0f;
      }
    __syncthreads();   // the rows are read before dC takes the space
  } else if constexpr (!kEarlyDph) {
    read_dph();
  }
#pragma unroll
  for (int i = 0; i < NTL; ++i) {
    const int n = 16 * i + l16, kp = n >> 1;
    const bool odd = n & 1;
    float co[4], ph[4];
    f2 cs[4];
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += R) {
      const int vr = trow0 + j0, t = vr / R;
      const bool ok = live && vr < rows;
      cpre[i][j0 / R].get(co + j0, (tok_rows >> (j0 / R)) & 1u);
      const f2 c2 = ok ? sm.tb.cs_of(t, kp) : f2{1.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < R; ++r) cs[j0 + r] = c2;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float dct = acc[i][jj];
      const float cq = __shfl_xor(co[jj], 1, 64);
      ph[jj] = odd ? -dct * rot_own(cq, co[jj], false, cs[jj]) : dct * rot_own(cq, co[jj], true, cs[jj]);
      const float pv = __shfl_xor(dct, 1, 64);
      acc[i][jj] = odd ? cs[jj].y * pv + cs[jj].x * dct : cs[jj].x * dct - cs[jj].y * pv;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ph[jj] += __shfl_xor(ph[jj], 1, 64);
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += R) {
      float v = dpre[i][j0 / R];
#pragma unroll
      for (int r = 0; r < R; ++r) v += ph[j0 + r];
      dpre[i][j0 / R] = v;
    }
  }
  if constexpr (kLdsIo) {
#pragma unroll
    for (int i = 0; i < NTL; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) lio[(trow0 + jj) * CS + 16 * i + l16] = acc[i][jj];
    __syncthreads();
    for (int q = tid; q < Lc * (N / 4); q += NT) {
      const int t = q / (N / 4), n4 = 4 * (q % (N / 4));
      *reinterpret_cast<f4*>(dCo + (ti0 + (int64_t)t * a.H) * N + n4) = *reinterpret_cast<const f4*>(lio + t * CS + n4);
    }
    __syncthreads();   // dC is read before the phase gradients take the space
#pragma unroll
    for (int i = 0; i < NTL; ++i) {
      if (!(l16 & 1)) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) lio[(trow0 + jj) * DS + ((16 * i + l16) >> 1)] = dpre[i][jj];
      }
    }
    __syncthreads();
    for (int q = tid; q < Lc * (NP / 4); q += NT) {
      const int t = q / (NP / 4), k4 = 4 * (q % (NP / 4));
      *reinterpret_cast<f4*>(dph + t * NP + k4) = *reinterpret_cast<const f4*>(lio + t * DS + k4);
    }
  } else if (live) {
#pragma unroll
    for (int i = 0; i < NTL; ++i) {
      const int n = 16 * i + l16;
      const float raw[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += R) {
        const int vr = trow0 + j0;
        if (vr < rows) str<R>(dCo + (ti0 + (int64_t)(vr / R) * a.H) * N * R + (int64_t)n * R, raw + j0);
      }
      if (!(n & 1)) {
#pragma unroll
        for (int j0 = 0; j0 < 4; j0 += R) {
          const int t = (trow0 + j0) / R;
          if (trow0 + j0 < rows) dph[t * NP + (n >> 1)] = dpre[i][j0 / R];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// The chunk's per-token gradients from the token sums of both sides:
// suffix sums over the chunk, dt, lam, A, theta and the token before the
// sequence.  1024 threads per chunk.
constexpr int kFinNT = 1024;
template <int P, int N>
struct FinSmem {
  static constexpr int NT = kFinNT, NP = N / 2;
  double cs[kQ];
  float dt[kQ], lam[kQ], Av[kQ], gam[kQ], bpr[kQ];
  float dcs[kQ], dgam[kQ], dbpr[kQ], part[NT];
  float dphi_end[NP + 2];   // the end rotation's phase gradient per pair, then two sums
  float red[NT / 64];
  float dphi[kQ][NP + 1];
};

template <typename TI, int P, int N, int R>
__global__ __launch_bounds__(kFinNT) void k_bwd_fin(BackwardArgs g) {
  const PrefillArgs& a = g.f;
  constexpr int NT = kFinNT, NP = N / 2;
  __shared__ FinSmem<P, N> sm;
  const int h = blockIdx.y;
  ChunkRef ck;
  if (!chunk_ref(a, blockIdx.x, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc, tid = threadIdx.x;
  const int c = blockIdx.x;
  const int G_ = a.G;
  const bool shared_grp = G_ != a.H;
  const int64_t gi = group_index(a, b, c0, h), ti0 = token_index(a, b, c0, h);
  // every global read of the token phase goes out first, from every thread
  // (thread tid reads token tid % 64; a token past the chunk reads token 0
  // and drops it): no branch around a load
  const int ut = tid & 63;
  const bool uok = ut < Lc;
  const int64_t bth = ti0 + (int64_t)(uok ? ut : 0) * a.H;
  const float d_in = ld1(static_cast<const TI*>(a.dt), bth);
  const float l_in = ld1(static_cast<const TI*>(a.lam), bth);
  const float A_in = (a.flags & kAPerToken) ? a.A[bth] : a.A[h];
  const float* __restrict__ tk = g.tokw + ck.id * (kTokSums * kQ);
  using GU = GeoU<P, N, R>;
  const bool both_rows = GU::SPLIT == 2 && Lc * R > GU::BROWS;
  const float t_dmend = tk[kDmend * kQ + ut], t_rr0 = tk[kRrow0 * kQ + ut];
  const float t_rr1 = both_rows ? tk[kRrow1 * kQ + ut] : 0.0f;
  const float t_ecol = tk[kEcol * kQ + ut], t_mcol = tk[kMcol * kQ + ut];
  const float t_de = tk[kDe * kQ + ut], t_edg = tk[kEdiag * kQ + ut];
  // token scalars and the chunk-local log-decay prefix (double)
  if (tid < 64) {
    const float d = uok ? d_in : 0.0f, l = uok ? l_in : 0.0f, A = uok ? A_in : 0.0f;
    double lv = (double)d * (double)A;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(lv, off, 64);
      if (tid >= off) lv += o;
    }
    sm.cs[tid] = lv;
    sm.dt[tid] = d;
    sm.lam[tid] = l;
    sm.Av[tid] = A;
    sm.gam[tid] = l * d;
    sm.bpr[tid] = (1.0f - l) * d;
  }
  // the phase gradients of both sides
  const float* __restrict__ dph = g.dphiB + ck.id * (kQ * NP);
  for (int i = tid; i < Lc * NP; i += NT) sm.dphi[i / NP][i % NP] = dph[i];

  // the end state's sums: the state pass waves' parts, in wave order
  {
    constexpr int WPB = P * N / 256, EW = NP + 2;
    const float* __restrict__ ep = g.endp + ck.id * (WPB * EW);
    if (tid < EW) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WPB; ++w) v += ep[w * EW + tid];
      sm.dphi_end[tid] = v;   // pairs, then <Gt, Shat> and the previous token's sum
    }
  }
  __syncthreads();   // the tables, dphi and the end sums are in
  const float e_end = sm.dphi_end[NP], h_end = sm.dphi_end[NP + 1];

  // ---- the token sums: log-decay (cs), trapezoid weights (gamma, beta')
  const double cs_end = sm.cs[Lc - 1];
  if (tid < kQ) {
    const int u = tid;
    float dc = 0.0f, dg = 0.0f, dbn = 0.0f, pm = 0.0f;
    if (u < Lc) {
      const float e = expf((float)(cs_end - sm.cs[u]));
      const float m = e * (sm.gam[u] + (u < Lc - 1 ? sm.bpr[u + 1] : 0.0f));
      const float d = t_dmend;
      const float rr = t_rr0 + t_rr1;
      const float ec = t_ecol;
      dc = rr - t_mcol + expf((float)sm.cs[u]) * t_de;
      dg = ec + t_edg + d * e;
      dbn = ec;
      if (u < Lc - 1) {
        pm = d * m;
        dc -= pm;
        dbn += d * e;
      }
    }
    sm.dcs[u] = dc;
    sm.dgam[u] = dg;
    if (u + 1 < kQ) sm.dbpr[u + 1] = dbn;
    if (u == 0) sm.dbpr[0] = h_end;
    sm.part[u] = pm;
  }
  __syncthreads();
  if (tid == 0) {   // the chunk's last token: the end state's decay and weights
    float v = expf((float)cs_end) * e_end;
    for (int u = 0; u < Lc - 1; ++u) v += sm.part[u];
    sm.dcs[Lc - 1] += v;
  }
  __syncthreads();
  // suffix sums over the chunk's tokens (one lane per token, a wave per
  // column): phase (from the end rotation) and log-decay
  {
    const int lane = tid & 63, wave = tid >> 6;
    auto suffix = [&](float v) {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(v, off, 64);
        if (lane + off < 64) v += o;
      }
      return v;
    };
    for (int k = wave; k < NP; k += NT / 64) {
      const float v = suffix(lane < Lc ? sm.dphi[lane][k] : 0.0f);
      if (lane < Lc) sm.dphi[lane][k] = v + sm.dphi_end[k];
    }
    if (wave == (NP % (NT / 64))) {
      const float v = suffix(lane < Lc ? sm.dcs[lane] : 0.0f);
      if (lane < Lc) sm.dcs[lane] = v;
    }
  }
  __syncthreads();

  // ---- per-token outputs: theta, dt, lam, A
  constexpr int TPT = NT / kQ, KPT = NP / TPT;
  static_assert(KPT >= 1 && NP % TPT == 0, "pairs per thread");
  const bool angle = (a.flags & kThetaIsAngle) != 0;
  const int tt = tid / TPT, cg = tid % TPT;
  float dt_theta = 0.0f;
  if (tt < Lc) {
    const int64_t tok = ti0 + (int64_t)tt * a.H, grp = gi + (int64_t)tt * G_;
    const TI* __restrict__ th = static_cast<const TI*>(a.theta) + grp * NP;
    const float dtt = sm.dt[tt];
    float* __restrict__ dth = shared_grp ? g.dthh + tok * NP : g.dtheta + grp * NP;
    float thv[KPT];   // read before the stores below (a read after a store waits for it)
#pragma unroll
    for (int j = 0; j < KPT; ++j) thv[j] = ld1(th, cg * KPT + j);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int k = cg * KPT + j;
      const float dphv = sm.dphi[tt][k];
      if (!angle) dt_theta += thv[j] * dphv;
      dth[k] = angle ? dphv : dtt * dphv;
    }
  }
  dt_theta = group_sum<TPT>(dt_theta);
  float da_part = 0.0f;
  if (tt < Lc && cg == 0) {
    const int64_t tok = ti0 + (int64_t)tt * a.H;
    const float dtt = sm.dt[tt], lm = sm.lam[tt], da = sm.dcs[tt];
    g.ddt[tok] = sm.Av[tt] * da + lm * sm.dgam[tt] + (1.0f - lm) * sm.dbpr[tt] + dt_theta;
    g.dlam[tok] = dtt * (sm.dgam[tt] - sm.dbpr[tt]);
    if (a.flags & kAPerToken) g.dA[tok] = dtt * da;
    else da_part = dtt * da;
  }
  if (!(a.flags & kAPerToken)) {   // per chunk; a final pass sums them per head
    const float sA = block_sum<NT>(da_part, sm.red);
    if (tid == 0) g.dApart[ck.id] = sA;
  }
  // the token before the sequence: dx_prev = beta'_0 dShat_0 B_prev,
  // dB_prev = beta'_0 dShat_0^T x_prev
  if (c == 0 && a.has_prev && (g.dx_prev || g.dB_prev)) {
    const TI* __restrict__ xprev = static_cast<const TI*>(a.xp) + ((int64_t)b * a.H + h) * P * R;
    const TI* __restrict__ bprev = static_cast<const TI*>(a.Bp) + ((int64_t)b * G_ + head_group(a, h)) * N * R;
    const float bp0 = sm.bpr[0];
    const float* __restrict__ dSc = g.dS + ck.id * (P * N);
    if (g.dx_prev) {
      for (int i = tid; i < P * R; i += NT) {
        const int p = i / R, r = i % R;
        float v = 0.0f;
#pragma unroll 8
        for (int n = 0; n < N; ++n) v += dSc[(int64_t)p * N + n] * ld1(bprev, (int64_t)n * R + r);
        g.dx_prev[((int64_t)b * a.H + h) * P * R + i] = bp0 * v;
      }
    }
    if (g.dB_prev) {
      for (int i = tid; i < N * R; i += NT) {
        const int n = i / R, r = i % R;
        float v = 0.0f;
#pragma unroll 8
        for (int p = 0; p < P; ++p) v += dSc[(int64_t)p * N + n] * ld1(xprev, (int64_t)p * R + r);
        if (shared_grp) g.dBph[((int64_t)b * a.H + h) * N * R + i] = bp0 * v;
        else g.dB_prev[((int64_t)b * G_ + head_group(a, h)) * N * R + i] = bp0 * v;
      }
    }
  }
}

// --------------------------------------------------------------------------
template <class Pol, typename TI, typename TY, int P, int N, int R>
hipError_t run_mma(const BackwardArgs& g, hipStream_t s) {
  const PrefillArgs& a = g.f;
  const dim3 grid(a.nchunk, a.H, a.Bsz);
  hipLaunchKernelGGL((k_bwd_adjoint_mma<Pol, TI, TY, P, N, R>), grid, dim3(AdjGeo<P, N>::NT), 0, s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_bwd_state_pass(g, std::is_same<TI, bf16_t>::value, s)) != hipSuccess) return e;
  using GU = GeoU<P, N, R>;
  const int nx = GU::SPLIT == 1 ? a.nchunk : GU::SPLIT * ((a.nchunk + 7) / 8) * 8;
  hipLaunchKernelGGL((k_bwd_u<Pol, TI, TY, P, N, R>), dim3(nx, a.H, a.Bsz), dim3(GU::NT), 0, s, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_t<Pol, TI, TY, P, N, R>), dim3(nx, a.H, a.Bsz), dim3(GU::NT), 0, s, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_fin<TI, P, N, R>), grid, dim3(kFinNT), 0, s, g);
  return hipGetLastError();
}

template <class Pol, typename TI, typename TY>
int dispatch_mma(const BackwardArgs& g, hipStream_t s, hipError_t* e) {
  const PrefillArgs& a = g.f;
#define M3_MMA_SHAPE(PP, NN, RR)                                    \
  if (a.P == PP && a.N == NN && a.R == RR) {                        \
    *e = run_mma<Pol, TI, TY, PP, NN, RR>(g, s);                    \
    return 0;                                                       \
  }
  M3_MMA_SHAPE(64, 128, 1)
  M3_MMA_SHAPE(32, 64, 1)
  M3_MMA_SHAPE(64, 64, 1)
  M3_MMA_SHAPE(64, 128, 2)
  M3_MMA_SHAPE(64, 128, 4)
  M3_MMA_SHAPE(32, 64, 4)
  M3_MMA_SHAPE(64, 64, 4)
#undef M3_MMA_SHAPE
  return -1;
}

}  // namespace

int launch_backward_mma(const BackwardArgs& g, int in_bf16, int dy_bf16, hipStream_t s, hipError_t* e) {
  if (in_bf16)
    return dy_bf16 ? dispatch_mma<PolHalf, bf16_t, bf16_t>(g, s, e) : dispatch_mma<PolHalf, bf16_t, float>(g, s, e);
  return dy_bf16 ? dispatch_mma<PolF32, float, bf16_t>(g, s, e) : dispatch_mma<PolF32, float, float>(g, s, e);
}

}  // namespace m3
