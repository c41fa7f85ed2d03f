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
// masked Gram, the state) is split into bf16 hi + lo parts and each product
// is hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 (about fp32 accuracy
// and fp32's exponent range); x, a bf16 input, is exact and used unsplit.
#include "chunk_common.h"
#include "mfma_pol.h"

#include <algorithm>
#include <type_traits>

namespace m3 {

// --------------------------------------------------------------------------
// launch geometry: one block per chunk; each wave owns TPW 16-row tiles of
// the chunk's Q*R virtual rows (two tiles w and 2NW-1-w when TPW = 2, which
// balances the causal work across waves).  Up to 16 waves per block, so the
// rank-4 chunk (16 tiles) has one tile per wave.
template <int P, int N, int R, int MAXW = 16, int Q = kQ>
struct Geo {
  static constexpr int ROWS = Q * R;
  static constexpr int TILES = ROWS / 16;
  static constexpr int NW = (TILES >= 16 && MAXW >= 16) ? 16 : (TILES >= 8 ? 8 : 4);
  static constexpr int TPW = TILES / NW;
  static constexpr int NT = NW * 64;
  static constexpr int NP = N / 2;
  static constexpr int PT = P / 16;
  static constexpr int NTL = N / 16;
  static constexpr int NUB = ROWS / kRB;
  static_assert(TPW >= 1 && TILES % NW == 0, "tile split");
};

// B/C preparation tables of one block: the weight [N], one head's bias
// [N][R] and the inverse RMS [t][r] of the chunk's tokens.  NoTab stands in
// when the preparation is off.
template <int N, int R, int Q = kQ>
struct alignas(16) PrepTab {
  float w[N];
  float b[N * R];
  float inv[Q * R];
};
struct NoTab {};
template <bool PREP, int N, int R, int Q>
using PrepTabT = typename std::conditional<PREP, PrepTab<N, R, Q>, NoTab>::type;

// weight and bias of head h (1 and 0 where the arrays are absent), loaded
// into registers early and stored into a PrepTab once the tables exist
template <int N, int R, int NT>
struct PrepLoad {
  static constexpr int NE = N + N * R;
  static constexpr int IT = (NE + NT - 1) / NT;
  float v[IT];
  // every lane reads a valid address (see ld_or) and selects after
  __device__ __forceinline__ void load(const float* w, const float* bias, int h) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e = threadIdx.x + NT * i;
      const bool isw = e < N;
      const float r = isw ? ld_or(w, min(e, N - 1), 1.0f)
                          : ld_or(bias, (int64_t)h * N * R + min(e - N, N * R - 1), 0.0f);
      v[i] = e < NE ? r : 0.0f;
    }
  }
  template <int Q>
  __device__ __forceinline__ void store(PrepTab<N, R, Q>& t) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int e = threadIdx.x + NT * i;
      if (e < N) t.w[e] = v[i];
      else if (e < NE) t.b[e - N] = v[i];
    }
  }
};

// the preparation of one vector of eight elements (e0 .. e0 + 7 of token t's
// N x R row) in place from the block's tables (NoPrep: left as loaded)
template <int N, int R, int Q>
struct TabPrep {
  const PrepTab<N, R, Q>* tab;
  // the vector's R inverse RMS, 8/R weights and 8 biases in 16-byte (or
  // smaller) LDS reads
  __device__ __forceinline__ void operator()(int t, int e0, float* v) const {
    static_assert(8 % R == 0, "a vector holds whole rank groups");
    float iv[R], wv[8 / R], bv[8];
    if constexpr (R == 4) {
      const f4 q = *reinterpret_cast<const f4*>(&tab->inv[t * 4]);
      iv[0] = q.x; iv[1] = q.y; iv[2] = q.z; iv[3] = q.w;
    } else if constexpr (R == 2) {
      const f2 q = *reinterpret_cast<const f2*>(&tab->inv[t * 2]);
      iv[0] = q.x; iv[1] = q.y;
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) iv[r] = tab->inv[t * R + r];
    }
    if constexpr (8 / R >= 4) {
#pragma unroll
      for (int m = 0; m < 8 / R; m += 4) {
        const f4 q = *reinterpret_cast<const f4*>(&tab->w[e0 / R + m]);
        wv[m] = q.x; wv[m + 1] = q.y; wv[m + 2] = q.z; wv[m + 3] = q.w;
      }
    } else if constexpr (8 / R == 2) {
      const f2 q = *reinterpret_cast<const f2*>(&tab->w[e0 / R]);
      wv[0] = q.x; wv[1] = q.y;
    } else {
      wv[0] = tab->w[e0 / R];
    }
    const f4 b0 = *reinterpret_cast<const f4*>(&tab->b[e0]);
    const f4 b1 = *reinterpret_cast<const f4*>(&tab->b[e0 + 4]);
    bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
    bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * (iv[j % R] * wv[j / R]) + bv[j];
  }
};

// Sums of squares over the N channels of each rank column for the tokens
// of a row block of B or C (t = t0 + tl < Lc), when one token's vectors sit
// on VPT consecutive lanes: they are summed with lane shuffles and the
// token's first lane stores the inverse RMS into out[t][r].
template <typename TI, int E, int R, int NT, int ROWS>
__device__ __forceinline__ void row_sumsq(const RowBlock<TI, E, R, NT, false, ROWS>& rb,
                                          const BCPrep& bc, int N, int t0, int Lc, float* out) {
  using RBk = RowBlock<TI, E, R, NT, false, ROWS>;
  static_assert(RBk::VPT <= 64 && 64 % RBk::VPT == 0 && NT % RBk::VPT == 0,
                "a token's vectors on one aligned lane group");
#pragma unroll
  for (int i = 0; i < RBk::IT; ++i) {
    const int vi = threadIdx.x + NT * i;
    int tl, e0;
    RBk::where(vi, tl, e0);
    const int t = t0 + tl;
    float v[8], part[R];
    rb.get(i, v);
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j % R] += v[j] * v[j];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = group_sum<RBk::VPT>(part[r]);
    if (vi < RBk::NV && t < Lc && vi % RBk::VPT == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) out[t * R + r] = bc_inv_rms(bc, part[r], N);
    }
  }
}

// The same sums for a token-per-lane single-rank block (TF: token tl's
// vectors sit on threads tl + NTOK j), in a fixed order so that equal
// inputs give equal bits: each thread adds its own vectors in index order,
// then the lanes of a wave that hold one token are added by xor steps (the
// two operands of each step are the same on both lanes), and this wave's
// sum of token t0 + tl goes to part[wave][t0 + tl] (zero for a block that
// was not loaded, live false).  The caller adds the waves' parts in wave
// order after a barrier.
template <int Q, typename TI, int E, int NT, int ROWS>
__device__ __forceinline__ void row_sumsq_tf(const RowBlock<TI, E, 1, NT, true, ROWS>& rb, int t0,
                                             bool live, float* part) {
  using RBk = RowBlock<TI, E, 1, NT, true, ROWS>;
  constexpr int NTOK = RBk::NTOK;
  static_assert(NT % NTOK == 0 && 64 % NTOK == 0, "a token's vectors in fixed lanes of every wave");
  float s = 0.0f;
  if (live) {   // block-uniform
#pragma unroll
    for (int i = 0; i < RBk::IT; ++i) {
      float v[8];
      rb.get(i, v);   // zeros outside the chunk's rows
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) p += v[j] * v[j];
      s += p;
    }
  }
#pragma unroll
  for (int off = NTOK; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
  const int lane = threadIdx.x & 63;
  if (lane < NTOK) part[(threadIdx.x >> 6) * Q + t0 + lane] = s;
}

// --------------------------------------------------------------------------
// K1: the chunk's own end state S_c (from a zero entry state), rotated into
// the frame of the chunk's end, plus the next chunk's trapezoid
// left-endpoint term (1 - lam_{c1}) dt_{c1} x_{c1-1} B_{c1-1}^T; the chunk's
// total decay and phase go to the workspace.  With the B/C preparation the
// chunk's B rows are normalised, weighted and biased as they are staged, and
// their inverse RMS goes to the workspace for the output kernel.
// virtual rows per staged u-block: 32 for a single input (a smaller LDS
// footprint, three blocks per CU), 64 otherwise
template <int R>
constexpr int k1_rows() { return R == 1 ? 32 : kRB; }

template <class Pol, typename TI, int P, int N, int R, bool PREP, int Q>
struct K1Smem {
  static constexpr int UBR = k1_rows<R>();
  Tables<N, false, true, Q> tb;
  union U {
    typename Pol::template Store<N, UBR> bw;   // (W_u R(Phi_end - Phi_u) B_u)^T  [n][v]
    TableScratch<N, Geo<P, N, R, 8, Q>::NT, Q> scr;
    // single rank with the preparation: each wave's part of every token's
    // sum of squares [wave][t] (between the tables and the first staging)
    float sq[(PREP && R == 1) ? Geo<P, N, R, 8, Q>::NW * Q : 1];
  } u;
  typename Pol::template XStore<P, UBR> xs;    // x^T  [p][v]
  PrepTabT<PREP, N, R, Q> pb;                  // B preparation
};

template <class Pol, typename TI, int P, int N, int R, bool PREP, int Q>
__global__ __launch_bounds__((Geo<P, N, R, 8, Q>::NT)) void k_chunk_state(PrefillArgs a) {
  using G = Geo<P, N, R, 8, Q>;
  __shared__ K1Smem<Pol, TI, P, N, R, PREP, Q> sm;
  constexpr int UBR = k1_rows<R>(), NUB = G::ROWS / UBR;   // staged u-blocks
  constexpr int NQ = G::PT * G::NTL;              // output tiles (p-tile, n-tile)
  constexpr int QPW = (NQ + G::NW - 1) / G::NW;   // per wave
  const int h = blockIdx.y;
  ChunkRef ck;
  if (!chunk_ref<Q>(a, blockIdx.x, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc;
  const int rows = Lc * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t chunk_id = ck.id;

  // every load goes out first (the load counter retires in order): phase
  // inputs and token scalars, then all u-blocks of B and x, so that the
  // block waits for HBM once
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);
  constexpr bool TFK1 = R < 2;
  PrepLoad<N, R, G::NT> pl;
  if constexpr (PREP) {
    pl.load(a.bc.Bw, a.bc.Bb, h);
  }
  ThetaBlock<TI, N, G::NT, Q> thb;
  thb.load(a, b, h, c0, Lc);
  // with R >= 2 a token's row of B (N R values) or x (P R) is long enough
  // for lanes to walk it (whole lines per load); single-rank rows are
  // spread one token per lane, so the transposed stores pair up lanes
  RowBlock<TI, N * R, R, G::NT, TFK1, UBR> bb[NUB];
  RowBlock<TI, P * R, R, G::NT, TFK1, UBR> xb[NUB];
#pragma unroll
  for (int ub = 0; ub < NUB; ++ub) {
    if (ub * UBR < rows) {
      bb[ub].template load<true>(Bg, a, b, h, c0, Lc, ub * UBR);
      xb[ub].template load<false>(Xg, a, b, h, c0, Lc, ub * UBR);
    }
  }

  if (a.tp.on) project_theta<TI, N, G::NT, Q>(a, b, h, c0, Lc, sm.tb);
  chunk_tables<TI, N, G::NT>(a, thb, Lc, sm.tb, sm.u.scr, 1);
  const double cs_end = sm.tb.cs[Lc - 1];
  if (tid < Q) {
    float w = 0.0f;
    if (tid < Lc) {
      const float wt = sm.tb.gam[tid] + (tid < Lc - 1 ? sm.tb.bpr[tid + 1] : 0.0f);
      w = expf((float)(cs_end - sm.tb.cs[tid])) * wt;
    }
    sm.tb.aux[tid] = w;
  }
  if (tid < G::NP)
    reinterpret_cast<f2*>(a.rot_end)[chunk_id * G::NP + tid] = cos_sin_reduced(reduce_angle(sm.tb.phi_end[tid]));
  if (tid == 0) a.decay[chunk_id] = expf((float)cs_end);
  float* __restrict__ rsB = nullptr;
  if constexpr (PREP) {
    rsB = a.rsB + chunk_id * (Q * R);
    pl.store(sm.pb);
#pragma unroll
    for (int ub = 0; ub < NUB; ++ub) {
      if constexpr (TFK1) {   // every u-block writes its tokens' parts (zeros past the chunk)
        row_sumsq_tf<Q>(bb[ub], ub * UBR, ub * UBR < rows, sm.u.sq);
      } else {
        if (ub * UBR < rows) row_sumsq(bb[ub], a.bc, N, ub * UBR / R, Lc, sm.pb.inv);
      }
    }
  }
  __syncthreads();   // W_t visible (and the B preparation tables)
  if constexpr (PREP) {
    if constexpr (TFK1) {   // the waves' parts in wave order -> inverse RMS
      if (tid < Q) {
        float ss = 0.0f;
#pragma unroll
        for (int w = 0; w < G::NW; ++w) ss += sm.u.sq[w * Q + tid];
        sm.pb.inv[tid] = bc_inv_rms(a.bc, ss, N);
      }
      __syncthreads();
    }
    if (tid < Q * R) rsB[tid] = sm.pb.inv[tid];
  }

  f4 acc[QPW];
#pragma unroll
  for (int q = 0; q < QPW; ++q) acc[q] = f4{0, 0, 0, 0};

#pragma unroll
  for (int ub = 0; ub < NUB; ++ub) {
    if (ub * UBR >= rows) break;
    if (ub > 0) __syncthreads();   // the previous block's LDS reads are done
    if constexpr (PREP)
      store_rows_T<Pol, TI, N, R, G::NT, TFK1, UBR>(bb[ub], sm.u.bw, sm.tb, sm.tb.aux, ub * UBR / R, Lc,
                                                    TabPrep<N, R, Q>{&sm.pb});
    else
      store_rows_T<Pol, TI, N, R, G::NT, TFK1, UBR>(bb[ub], sm.u.bw, sm.tb, sm.tb.aux, ub * UBR / R, Lc,
                                                    NoPrep{});
    store_x_T<Pol, TI, P, R, G::NT, UBR, TFK1>(xb[ub], sm.xs);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
      const int qq = wave * QPW + q;
      if (NQ % G::NW == 0 || qq < NQ) {
        const int pt = qq / G::NTL, nt = qq % G::NTL;
#pragma unroll
        for (int kk = 0; kk < UBR; kk += Pol::KS)
          acc[q] = Pol::mma_x(Pol::frag(sm.u.bw, 16 * nt, kk, lane),
                              Pol::fragx_c(sm.xs, 16 * pt, kk, lane), acc[q]);
      }
    }
  }

  // the next chunk's left-endpoint term, then S_c[p][n..n+3].  Every read
  // of the term (this chunk's last x and B rows for each tile, the next
  // chunk's first dt and lam) goes out before any is used, kept as loaded,
  // with no branch around it: a chunk with no next one reads its own tokens
  // and drops the term.
  const bool nxt = ck.next;
  const int64_t nx = token_index(a, b, nxt ? c0 + Q : c0, h);
  Raw1<TI> dnr, lnr;
  dnr.load(static_cast<const TI*>(a.dt), nx);
  lnr.load(static_cast<const TI*>(a.lam), nx);
  const TI* __restrict__ xe = Xg + token_index(a, b, c0 + Lc - 1, h) * P * R;
  const TI* __restrict__ Be = Bg + group_index(a, b, c0 + Lc - 1, h) * N * R;
  RawVec<TI, R> xraw[QPW];
  RawVec<TI, 4 * R> braw[QPW];
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    const int qq = min(wave * QPW + q, NQ - 1);
    const int pt = qq / G::NTL, nt = qq % G::NTL;
    xraw[q].load(xe + (int64_t)(16 * pt + l16) * R);
    braw[q].load(Be + (int64_t)(16 * nt + 4 * g) * R);
  }
  const float bpn = nxt ? (1.0f - lnr.f()) * dnr.f() : 0.0f;
  float* __restrict__ S = a.S + chunk_id * P * N;
#pragma unroll
  for (int q = 0; q < QPW; ++q) {
    const int qq = wave * QPW + q;
    if (qq < NQ) {
      const int pt = qq / G::NTL, nt = qq % G::NTL;
      const int p = 16 * pt + l16, n = 16 * nt + 4 * g;
      f4 s = acc[q];
      if (nxt) {
        // x[p][0..R) and B[n..n+3][0..R) of the chunk's last token
        float xr[R], br[4 * R];
        xraw[q].get(xr);
        braw[q].get(br);
        if constexpr (PREP) {   // the last token's B, prepared like the staged rows
#pragma unroll
          for (int e = 0; e < 4 * R; ++e)
            br[e] = br[e] * sm.pb.inv[(Q - 1) * R + e % R] * sm.pb.w[n + e / R] + sm.pb.b[n * R + e];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xv = bpn * xr[r];
          s.x += xv * br[0 * R + r];
          s.y += xv * br[1 * R + r];
          s.z += xv * br[2 * R + r];
          s.w += xv * br[3 * R + r];
        }
      }
      *reinterpret_cast<f4*>(S + (int64_t)p * N + n) = s;
    }
  }
}

// --------------------------------------------------------------------------
// K2: serial pass over the chunks of one (batch, head) or (sequence, head).  Entering chunk c
// the state (plus that chunk's left-endpoint term) is Shat_c;
// Shat_{c+1} = decay_c R(Phi_end,c) Shat_c + S_c, where S_c already carries
// the next chunk's left-endpoint term.  Shat_c replaces S_c in the
// workspace.  Every element is independent, so each thread carries one
// 16-byte vector of the state through all chunks (one wave per block, many
// waves per (batch, head)); the loads of chunk c + 8 are issued while chunk
// c is processed.
template <typename TI, int N, int R>
__global__ __launch_bounds__(64) void k_state_pass(PrefillArgs a) {
  constexpr int D = 8;
  const int P = a.P;
  const int wpb = P * N / 4 / 64;          // blocks (waves) per (batch, head)
  const int bh = blockIdx.x / wpb;
  const int vi = (blockIdx.x % wpb) * 64 + threadIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int p = vi / (N / 4), n = 4 * (vi % (N / 4));
  // this sequence's chunks are workspace slots cbase .. cbase + nch - 1
  int64_t cbase, t0;
  int nch;
  bool any;
  if (a.seqs) {
    const int4 q = a.seqs[b];
    cbase = (int64_t)h * a.nchunk + q.x;
    nch = q.y;
    t0 = token_index(a, 0, q.z, h);
    any = q.w > 0;
  } else {
    cbase = (int64_t)bh * a.nchunk;
    nch = a.nchunk;
    t0 = token_index(a, b, 0, h);
    any = true;
  }

  f4 S = f4{0, 0, 0, 0};
  if (a.h0) S = *reinterpret_cast<const f4*>(a.h0 + ((int64_t)bh * P + p) * N + n);
  if (a.has_prev && any) {  // left-endpoint term of token 0
    const float d = ld1(static_cast<const TI*>(a.dt), t0);
    const float l = ld1(static_cast<const TI*>(a.lam), t0);
    const float bp0 = (1.0f - l) * d;
    const TI* xh = static_cast<const TI*>(a.xp) + (int64_t)bh * P * R;
    const TI* Bh = static_cast<const TI*>(a.Bp) + ((int64_t)b * a.G + head_group(a, h)) * N * R;
    float bv[4][R];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) bv[j][r] = ld1(Bh, (int64_t)(n + j) * R + r);
    if (a.bc.on) {
      // B_prev prepared like every B: the N / 4 lanes of row p hold all of it
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += bv[j][r] * bv[j][r];
        const float inv = bc_inv_rms(a.bc, group_sum<N / 4>(ss), N);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[j][r] = bv[j][r] * inv * ld_or(a.bc.Bw, n + j, 1.0f) +
                     ld_or(a.bc.Bb, ((int64_t)h * N + n + j) * R + r, 0.0f);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float xv = bp0 * ld1(xh, (int64_t)p * R + r);
      S.x += xv * bv[0][r];
      S.y += xv * bv[1][r];
      S.z += xv * bv[2][r];
      S.w += xv * bv[3][r];
    }
  }
  const int64_t off = (int64_t)p * N + n;
  f4 bs[D];
  f2 br0[D], br1[D];
  float bd[D];
  auto load = [&](int c, int q) {
    if (c < nch) {
      const int64_t cid = cbase + c;
      const f2* re = reinterpret_cast<const f2*>(a.rot_end) + cid * (N / 2);
      bd[q] = a.decay[cid];
      bs[q] = *reinterpret_cast<const f4*>(a.S + cid * P * N + off);
      br0[q] = re[n / 2];
      br1[q] = re[n / 2 + 1];
    }
  };
#pragma unroll
  for (int q = 0; q < D; ++q) load(q, q);
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int c = c0 + q;
      if (c < nch) {
        *reinterpret_cast<f4*>(a.S + (cbase + c) * P * N + off) = S;   // Shat_c
        S = bd[q] * rot2pairs(S, br0[q], br1[q]) + bs[q];
        load(c + D, q);
      }
    }
  }
  if (a.hT) *reinterpret_cast<f4*>(a.hT + ((int64_t)bh * P + p) * N + n) = S;
}

// --------------------------------------------------------------------------
// K3: the outputs of one chunk.  One wave per 16-row output tile; a rank-4
// chunk (16 tiles) is split over two blocks of 8 waves (virtual rows 0..127
// and 128..255), so that two blocks fit on a CU and one block's loads and
// table work overlap the other's MFMA work.
template <int P, int N, int R, int Q = kQ>
struct Geo3 {
  static constexpr int ROWS = Q * R;             // virtual rows per chunk
  static constexpr int TILES = ROWS / 16;
  static constexpr int SPLIT = TILES > 8 ? TILES / 8 : 1;
  static constexpr int NW = TILES / SPLIT;       // waves (= tiles) per block
  static constexpr int NT = NW * 64;
  static constexpr int BROWS = ROWS / SPLIT;     // virtual rows per block
  static constexpr int NCB = BROWS / kRB;        // C row blocks per block
  static constexpr int NUB = ROWS / kRB;         // u-blocks of a whole chunk
  static constexpr int PT = P / 16;
  static_assert(BROWS % kRB == 0 && (SPLIT == 1 || SPLIT == 2) && (NW == 4 || NW == 8),
                "output block geometry");
};

template <class Pol, typename TI, int P, int N, int R, bool PREP, int Q>
struct K3Smem {
  // with R a multiple of 4 each token-pair mask value serves 16 virtual
  // (row, column) pairs, so the block's mask rows are tabulated once
  static constexpr int MT = R % 4 == 0 ? Geo3<P, N, R, Q>::BROWS / R : 1;
  static constexpr int UB = 32;                // virtual rows per staged u-block
  // a single-input chunk (one 4-wave block) keeps its LDS small enough for
  // three blocks per CU: C rows staged 32 at a time, Shat in two halves,
  // one u-block buffer
  static constexpr bool LEAN = R == 1;
  static constexpr int CRB = LEAN ? 32 : kRB;  // C rows per staged piece
  static constexpr int SHP = LEAN && P >= 32 ? P / 2 : P;  // Shat rows per staged part (whole tiles)
  static constexpr int NBUF = LEAN ? 1 : 2;    // u-block buffers
  Tables<N, false, false, Q> tb;
  union U {
    typename Pol::template Store<CRB, N> st;   // rotated C rows        [v][n]
    typename Pol::template Store<SHP, N> sh;   // Shat                  [p][n]
    typename Pol::template Store<UB, N> bst[NBUF];  // rotated B rows
    TableScratch<N, Geo3<P, N, R, Q>::NT, Q> scr;
  } u;
  typename Pol::template XStore<P, UB> xs[NBUF];  // x^T of a u-block   [p][v]
  float msk[MT][Q + 1];                       // M[t - t_lo][u]
  PrepTabT<PREP, N, R, Q> pb, pc;                 // B and C preparation
};

// four consecutive outputs (one token's four ranks) in one store
__device__ __forceinline__ void st4_out(float* __restrict__ p, int64_t i, f4 v) {
  *reinterpret_cast<f4*>(p + i) = v;
}
__device__ __forceinline__ void st4_out(bf16_t* __restrict__ p, int64_t i, f4 v) {
  const uint32_t lo = to_bf16(v.x).bits | (static_cast<uint32_t>(to_bf16(v.y).bits) << 16);
  const uint32_t hi = to_bf16(v.z).bits | (static_cast<uint32_t>(to_bf16(v.w).bits) << 16);
  *reinterpret_cast<uint2*>(p + i) = uint2{lo, hi};
}

// the rank-4 bf16 kernel runs two 8-wave blocks per CU (four waves per
// SIMD); the B/C preparation's few extra registers must not break that
template <class Pol, int R, bool PREP, int Q>
constexpr int k3_min_waves() {
  // (and an 8-wave single-input block of 128 tokens, likewise two per CU)
  return ((PREP && R % 4 == 0 && std::is_same<Pol, PolHalf>::value) || (R == 1 && Q > kQ)) ? 4 : 1;
}

template <class Pol, typename TI, typename TO, int P, int N, int R, bool PREP, int Q>
__global__ __launch_bounds__((Geo3<P, N, R, Q>::NT))
__attribute__((amdgpu_waves_per_eu(k3_min_waves<Pol, R, PREP, Q>()))) void k_chunk_output(PrefillArgs a) {
  using G = Geo3<P, N, R, Q>;
  using SMT = K3Smem<Pol, TI, P, N, R, PREP, Q>;
  __shared__ SMT sm;
  constexpr int NKS = N / Pol::KS;
  constexpr int UG = 16 * Pol::DT;          // u rows per A fragment built from D tiles
  // the two blocks of a split chunk are 8 apart in launch order: same XCD
  // (blocks go round-robin over the 8 XCDs), so the second one finds the
  // chunk's state, B and x in that XCD's L2
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
  if (!chunk_ref<Q>(a, c, h, blockIdx.z, ck)) return;
  const int b = ck.bt, c0 = ck.t0, Lc = ck.Lc;
  const int rows = Lc * R;
  const int v0 = half * G::BROWS;           // this block's rows: [v0, vend)
  if (v0 >= rows) return;
  const int vend = min(rows, v0 + G::BROWS);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t chunk_id = ck.id;
  // this wave's tile; with 8 waves, waves w and w + 4 share a SIMD and take
  // tiles w and 7 - w, which evens out the causal work per SIMD
  const int lt = (G::NW == 8) ? (wave < 4 ? wave : 11 - wave) : wave;
  const int tile = v0 / 16 + lt;

  const TI* __restrict__ Cg = static_cast<const TI*>(a.C);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.B);
  const TI* __restrict__ Xg = static_cast<const TI*>(a.x);

  // the B/C preparation's weights, biases and the chunk's B inverse RMS
  // (small, L2-resident) go straight into LDS, so that no register holds
  // them across the loads below
  if constexpr (PREP) {
    PrepLoad<N, R, G::NT> plb, plc;
    plb.load(a.bc.Bw, a.bc.Bb, h);
    plc.load(a.bc.Cw, a.bc.Cb, h);
    const float rsb_in = a.rsB[chunk_id * (Q * R) + min(tid, Q * R - 1)];   // (no branch around the read)
    const float rsb = tid < Q * R ? rsb_in : 0.0f;
    plb.store(sm.pb);
    plc.store(sm.pc);
    if (tid < Q * R) sm.pb.inv[tid] = rsb;
  }
  // all loads go out first (the load counter retires in order): phase
  // inputs and token scalars, this block's C rows, the entry state, and the
  // first u-blocks of B and x
  constexpr int CRB = SMT::CRB, NCB = G::BROWS / CRB, NBUF = SMT::NBUF;
  ThetaBlock<TI, N, G::NT, Q> thb;
  thb.load(a, b, h, c0, Lc);
  RowBlock<TI, N * R, R, G::NT, false, CRB> cb[NCB];
#pragma unroll
  for (int k = 0; k < NCB; ++k)
    if (v0 + k * CRB < rows) cb[k].template load<true>(Cg, a, b, h, c0, Lc, v0 + k * CRB);
  // the entry state (a single-input block loads it once its C rows are
  // staged, to stay within the registers of three blocks per CU)
  StateBlock<P, N, G::NT> sb;
  if constexpr (!SMT::LEAN) sb.load(a.S + chunk_id * P * N);
  // B and x move in u-blocks of 32 virtual rows, three in flight (two with
  // the B/C preparation, whose staging needs the registers of the third,
  // and for a single input)
  constexpr int NS = (PREP || SMT::LEAN) ? 2 : 3;
  constexpr int UB = SMT::UB;
  constexpr int NKB = G::ROWS / UB;
  const int nkb = (vend + UB - 1) / UB;
  RowBlock<TI, N * R, R, G::NT, false, UB> bb[NS];
  RowBlock<TI, P * R, R, G::NT, (R < 2), UB> xb[NS];   // x rows walked by lanes when R >= 2
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    if (q < nkb) {
      bb[q].template load<true>(Bg, a, b, h, c0, Lc, q * UB);
      xb[q].template load<false>(Xg, a, b, h, c0, Lc, q * UB);
    }
  }

  if (a.tp.on) project_theta<TI, N, G::NT, Q>(a, b, h, c0, Lc, sm.tb);
  chunk_tables<TI, N, G::NT>(a, thb, Lc, sm.tb, sm.u.scr, 0);
  if (tid < Q) sm.tb.aux[tid] = tid < Lc ? expf((float)sm.tb.cs[tid]) : 0.0f;
  // decay mask M[t][u] = e^{cs_t - cs_u} w_{t,u} of this block's tokens
  // (zero above the diagonal and past the chunk's end)
  const int tlo = v0 / R;
  if constexpr (R % 4 == 0) {
    for (int idx = tid; idx < SMT::MT * Q; idx += G::NT) {
      const int tr = idx / Q, u = idx % Q, t = tlo + tr;
      float m = 0.0f;
      if (t < Lc && u <= t) {
        const float w = sm.tb.gam[u] + (u < t ? sm.tb.bpr[u + 1] : 0.0f);
        m = __expf((float)(sm.tb.cs[t] - sm.tb.cs[u])) * w;
      }
      sm.msk[tr][u] = m;
    }
  }
  if constexpr (PREP) {
#pragma unroll
    for (int k = 0; k < NCB; ++k)
      if (v0 + k * CRB < rows) row_sumsq(cb[k], a.bc, N, (v0 + k * CRB) / R, Lc, sm.pc.inv);
    __syncthreads();
  }

  // own rotated C rows -> MFMA fragments in registers
  typename Pol::Frag cf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) cf[s] = typename Pol::Frag{};
  constexpr int TPC = CRB / 16;   // tiles per staged piece of C rows
#pragma unroll
  for (int k = 0; k < NCB; ++k) {
    if (v0 + k * CRB < rows) {
      if (k > 0) __syncthreads();
      if constexpr (PREP)
        store_rows<Pol, TI, N, R, G::NT, CRB>(cb[k], sm.u.st, sm.tb, (v0 + k * CRB) / R, Lc,
                                              TabPrep<N, R, Q>{&sm.pc});
      else
        store_rows<Pol, TI, N, R, G::NT, CRB>(cb[k], sm.u.st, sm.tb, (v0 + k * CRB) / R, Lc, NoPrep{});
      __syncthreads();
      if (lt / TPC == k) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) cf[s] = Pol::frag(sm.u.st, 16 * (lt % TPC), s * Pol::KS, lane);
      }
    }
  }
  if constexpr (SMT::LEAN) sb.load(a.S + chunk_id * P * N);

  // Y_off = e^{cs_t} Ct Shat^T (Shat staged in parts of SHP rows)
  constexpr int SHP = SMT::SHP, CPS = SHP / 16;   // output column tiles per part
  static_assert(SHP % 16 == 0 && P % SHP == 0, "Shat parts of whole tiles");
  f4 acc[G::PT];
#pragma unroll
  for (int hs = 0; hs < P / SHP; ++hs) {
    __syncthreads();   // the C rows (or the previous part) are read
    if constexpr (SHP == P) sb.template store<Pol>(sm.u.sh);
    else sb.template store_part<Pol, SHP>(sm.u.sh, hs * SHP);
    __syncthreads();
#pragma unroll
    for (int ct = hs * CPS; ct < (hs + 1) * CPS; ++ct) {
      f4 d = f4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        d = Pol::mma(cf[s], Pol::frag(sm.u.sh, 16 * (ct - hs * CPS), s * Pol::KS, lane), d);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int vv = 16 * tile + 4 * g + jj;
        d[jj] *= vv < rows ? sm.tb.aux[vv / R] : 0.0f;
      }
      acc[ct] = d;
    }
  }

  // Y_diag: Gram tiles Bt Ct^T (D rows = u, columns = own rows), decay mask,
  // then the masked tile is the A operand of the product with x.  u-block
  // k + 1 is staged into the other buffer while the MFMAs of u-block k run,
  // one barrier per u-block.
  const int vrow = 16 * tile + l16;
  const int tt = vrow / R;
  const bool row_ok = vrow < rows;
  const int tmax = min(Lc - 1, (16 * tile + 15) / R);
  const double cst = sm.tb.cs[min(tt, Q - 1)];
  auto stage = [&](int k) {
    if constexpr (PREP)
      store_rows<Pol, TI, N, R, G::NT, UB>(bb[k % NS], sm.u.bst[k % NBUF], sm.tb, k * UB / R, Lc,
                                           TabPrep<N, R, Q>{&sm.pb});
    else
      store_rows<Pol, TI, N, R, G::NT, UB>(bb[k % NS], sm.u.bst[k % NBUF], sm.tb, k * UB / R, Lc, NoPrep{});
    store_x_T<Pol, TI, P, R, G::NT, UB, (R < 2)>(xb[k % NS], sm.xs[k % NBUF]);
    if (k + NS < nkb) {   // the freed slot takes u-block k + NS
      bb[k % NS].template load<true>(Bg, a, b, h, c0, Lc, (k + NS) * UB);
      xb[k % NS].template load<false>(Xg, a, b, h, c0, Lc, (k + NS) * UB);
    }
  };
  __syncthreads();   // Shat's reads are done (the buffers share its space)
  if constexpr (NBUF == 2) {
    stage(0);
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < NKB; ++k) {
    if (k >= nkb) break;
    if constexpr (NBUF == 2) {
      if (k + 1 < nkb) stage(k + 1);
    } else {   // one buffer (the previous u-block's reads ended at the loop's barrier)
      stage(k);
      __syncthreads();
    }
    const int buf = k % NBUF;
    const int ubase = k * UB;
    if (ubase / R <= tmax) {
      // decay mask M[t][u] = e^{cs_t - cs_u} w_{t,u} for the token u of
      // each D row; with R a multiple of 4 a lane's 4 rows share one token
      f4 mk[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        if constexpr (R % 4 == 0) {
          const float m = sm.msk[tt - tlo][(ubase + 16 * dt + 4 * g) / R];
          mk[dt] = f4{m, m, m, m};
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int tu = (ubase + 16 * dt + 4 * g + jj) / R;
            float m = 0.0f;
            if (row_ok && tu <= tt) {
              const float w = sm.tb.gam[tu] + (tu < tt ? sm.tb.bpr[tu + 1] : 0.0f);
              m = __expf((float)(cst - sm.tb.cs[tu])) * w;
            }
            mk[dt][jj] = m;
          }
        }
      }
      f4 d[2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f4 gt = f4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NKS; ++s)
          gt = Pol::mma(Pol::frag(sm.u.bst[buf], 16 * dt, s * Pol::KS, lane), cf[s], gt);
        d[dt] = gt * mk[dt];
      }
#pragma unroll
      for (int ug = 0; ug < UB; ug += UG) {
        const typename Pol::Frag af = Pol::frag_from_d(d + ug / 16);
#pragma unroll
        for (int ct = 0; ct < G::PT; ++ct)
          acc[ct] = Pol::mma_x(af, Pol::fragx_d(sm.xs[buf], 16 * ct, ug, lane), acc[ct]);
      }
    }
    __syncthreads();
  }

  // y[b, c0 + t, h, p, r] for D rows v = 16 tile + 4g + jj, column p
  TO* __restrict__ Y = static_cast<TO*>(a.y) + token_index(a, b, c0, h) * (P * R);
  const int ystride = a.H * P * R;
#pragma unroll
  for (int ct = 0; ct < G::PT; ++ct) {
    const int p = 16 * ct + l16;
    if constexpr (R % 4 == 0) {
      // the four rows are ranks v%R .. v%R + 3 of one token
      const int v = 16 * tile + 4 * g;
      if (v < rows) st4_out(Y, (v / R) * ystride + p * R + v % R, acc[ct]);
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int v = 16 * tile + 4 * g + jj;
        if (v < rows) st1(Y, (v / R) * ystride + p * R + v % R, acc[ct][jj]);
      }
    }
  }
}

// --------------------------------------------------------------------------
template <class Pol, typename TI, typename TO, int P, int N, int R, bool PREP, int Q>
static hipError_t run_prefill(const PrefillArgs& a, hipStream_t s) {
  using G1 = Geo<P, N, R, 8, Q>;
  // packed sequences: one row of chunk slots per head
  const int nz = a.cmap ? 1 : a.Bsz;
  hipLaunchKernelGGL((k_chunk_state<Pol, TI, P, N, R, PREP, Q>), dim3(a.nchunk, a.H, nz), dim3(G1::NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static_assert(P * N % 256 == 0, "state pass: whole waves per (batch, head)");
  hipLaunchKernelGGL((k_state_pass<TI, N, R>), dim3(a.Bsz * a.H * (P * N / 256)), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.states_only) return e;
  using G3 = Geo3<P, N, R, Q>;
  // a split chunk's blocks are 8 apart in launch order: pad to whole groups of 8
  const int nx = G3::SPLIT == 1 ? a.nchunk : G3::SPLIT * ((a.nchunk + 7) / 8) * 8;
  hipLaunchKernelGGL((k_chunk_output<Pol, TI, TO, P, N, R, PREP, Q>), dim3(nx, a.H, nz), dim3(G3::NT), 0, s, a);
  return hipGetLastError();
}

template <class Pol, typename TI, typename TO>
static int dispatch_shape(const PrefillArgs& a, hipStream_t s, hipError_t* e) {
#define M3_SHAPE(PP, NN, RR, QQ)                                          \
  if constexpr (NN % Pol::KS == 0) {                                      \
    if (a.P == PP && a.N == NN && a.R == RR && a.Q == QQ) {               \
      *e = a.bc.on ? run_prefill<Pol, TI, TO, PP, NN, RR, true, QQ>(a, s)  \
                   : run_prefill<Pol, TI, TO, PP, NN, RR, false, QQ>(a, s); \
      return 0;                                                           \
    }                                                                     \
  }
  M3_SHAPE(16, 16, 1, 64)
  M3_SHAPE(64, 128, 1, 64)
  M3_SHAPE(64, 128, 4, 64)
  M3_SHAPE(64, 128, 2, 64)
  M3_SHAPE(32, 64, 1, 64)
  M3_SHAPE(32, 64, 4, 64)
  M3_SHAPE(64, 64, 1, 64)
  M3_SHAPE(64, 64, 4, 64)
  // 128-token chunks for a single input: half the chunk states
  M3_SHAPE(16, 16, 1, 128)
  M3_SHAPE(64, 128, 1, 128)
  M3_SHAPE(32, 64, 1, 128)
  M3_SHAPE(64, 64, 1, 128)
#undef M3_SHAPE
  return -1;
}

bool prefill_supported(int P, int N, int R, int Q, int in_bf16) {
  const bool shape = (P == 16 && N == 16 && R == 1) ||
                     (P == 64 && N == 128 && (R == 1 || R == 2 || R == 4)) ||
                     (P == 32 && N == 64 && (R == 1 || R == 4)) ||
                     (P == 64 && N == 64 && (R == 1 || R == 4));
  if (!shape) return false;
  if (!(Q == kQ || (Q == 128 && R == 1))) return false;
  if (in_bf16 && N % 32 != 0) return false;  // 16-bit fragments span 32 state columns
  return true;
}

int prefill_default_chunk(int P, int N, int R, int in_bf16) {
  (void)P, (void)N, (void)in_bf16;
  return R == 1 ? kPrefillChunkR1 : kQ;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// per chunk unit: the state (P N), the end phase (N) and the decay (1), and
// with the B/C preparation the inverse RMS of the chunk's B rows (Q R)
static size_t unit_bytes(size_t units, int P, int N, int R, int Q, bool prep) {
  return align256(units * P * N * 4) + align256(units * N * 4) + align256(units * 4) +
         (prep ? align256(units * Q * R * 4) : 0);
}

static char* carve_units(PrefillArgs& a, size_t units, char* p) {
  a.S = reinterpret_cast<float*>(p);
  p += align256(units * a.P * a.N * 4);
  a.rot_end = reinterpret_cast<float*>(p);
  p += align256(units * a.N * 4);
  a.decay = reinterpret_cast<float*>(p);
  p += align256(units * 4);
  a.rsB = nullptr;
  if (a.bc.on) {
    a.rsB = reinterpret_cast<float*>(p);
    p += align256(units * a.Q * a.R * 4);
  }
  return p;
}

size_t prefill_workspace_bytes(int Bsz, int T, int H, int P, int N, int R, int Q, bool prep) {
  const size_t nchunk = (size_t)(T + Q - 1) / Q;
  return unit_bytes((size_t)Bsz * H * nchunk, P, N, R, Q, prep);
}

void prefill_carve(PrefillArgs& a, void* ws) {
  carve_units(a, (size_t)a.Bsz * a.H * a.nchunk, static_cast<char*>(ws));
}

// --------------------------------------------------------------------------
// Packed sequences.  The caller's offsets cu[0..S] are read once on the
// device and made safe: each is clamped into [0, T] and raised to the
// largest offset before it, so the sequences are disjoint, ordered ranges
// of the T token rows whatever the array holds (rows outside every range
// are not written).  Sequence s has ceil(len_s / Q) chunks; its chunks take
// consecutive slots from first_s = sum of the earlier counts.

int64_t varlen_slots(int Bsz, int T, int Q) {
  // every chunk holds >= 1 token, and ceil(len / Q) <= (len + Q - 1) / Q
  return std::min<int64_t>(T, ((int64_t)T + (int64_t)Bsz * (Q - 1)) / Q);
}

size_t prefill_varlen_workspace_bytes(int Bsz, int T, int H, int P, int N, int R, int Q, bool prep) {
  const size_t slots = (size_t)varlen_slots(Bsz, T, Q);
  return unit_bytes((size_t)H * slots, P, N, R, Q, prep) + align256((size_t)Bsz * sizeof(int4)) +
         align256(slots * sizeof(int4));
}

void prefill_varlen_carve(PrefillArgs& a, void* ws) {
  char* p = carve_units(a, (size_t)a.H * a.nchunk, static_cast<char*>(ws));
  a.seqs = reinterpret_cast<int4*>(p);
  p += align256((size_t)a.Bsz * sizeof(int4));
  a.cmap = reinterpret_cast<int4*>(p);
}

// inclusive block scans over 1024 threads (sixteen waves)
template <class Op>
__device__ __forceinline__ int block_scan(int v, int* wtot, Op op) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v = op(v, o);
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v = op(v, wtot[w]);
  __syncthreads();   // wtot is reused by the next scan
  return v;
}

// seqs[s] = {first slot, chunks, first token, length}: one block of 1024
// threads walks the offsets in tiles, carrying the running maximum offset
// and the running chunk count from tile to tile
__global__ __launch_bounds__(1024) void k_varlen_seqs(const int32_t* __restrict__ cu, int S, int T,
                                                      int Q, int4* __restrict__ seqs) {
  __shared__ int wtot[16];
  __shared__ int edge[1025];
  __shared__ int tile_sum;
  const int tid = threadIdx.x;
  int carry_max = 0, carry_sum = 0;
  for (int base = 0; base <= S; base += 1024) {
    const int i = base + tid;
    const int v = i <= S ? min(max(cu[i], 0), T) : 0;
    const int m = max(block_scan(v, wtot, [](int x, int y) { return max(x, y); }), carry_max);
    edge[tid + 1] = m;
    if (tid == 0) edge[0] = carry_max;
    __syncthreads();
    const bool is_seq = i >= 1 && i <= S;   // offset i closes sequence i - 1
    const int len = is_seq ? edge[tid + 1] - edge[tid] : 0;
    const int nch = (len + Q - 1) / Q;
    const int incl = block_scan(nch, wtot, [](int x, int y) { return x + y; });
    if (is_seq) seqs[i - 1] = int4{carry_sum + incl - nch, nch, edge[tid], len};
    if (tid == 1023) tile_sum = incl;
    __syncthreads();
    carry_max = edge[1024];
    carry_sum += tile_sum;
    __syncthreads();   // edge and tile_sum are rewritten by the next tile
  }
}

// cmap[j] for every slot j: the sequence whose chunks cover slot j (the
// last one starting at or before j) or -1 past the last chunk
__global__ __launch_bounds__(256) void k_varlen_slots(const int4* __restrict__ seqs, int S, int nslot,
                                                      int Q, int4* __restrict__ cmap) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= nslot) return;
  int lo = 0, hi = S;   // seqs[lo].x <= j (seqs[0].x = 0); hi = S or seqs[hi].x > j
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seqs[mid].x <= j) lo = mid;
    else hi = mid;
  }
  const int4 q = seqs[lo];
  const int c = j - q.x;
  cmap[j] = c < q.y ? int4{lo, q.z + c * Q, q.z + q.w, c} : int4{-1, 0, 0, 0};
}

hipError_t launch_varlen_map(const PrefillArgs& a, const int32_t* cu, hipStream_t s) {
  hipLaunchKernelGGL(k_varlen_seqs, dim3(1), dim3(1024), 0, s, cu, a.Bsz, a.T, a.Q, a.seqs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_varlen_slots, dim3((a.nchunk + 255) / 256), dim3(256), 0, s, a.seqs, a.Bsz,
                     a.nchunk, a.Q, a.cmap);
  return hipGetLastError();
}

bool prefill_offsets_fit(int H, int P, int N, int R, int Q) {
  // in-chunk element offsets are 32-bit: Q tokens of the widest per-token row
  const int64_t row = (int64_t)H * std::max(N, P) * R;
  return (int64_t)Q * row < (int64_t(1) << 31);
}

int launch_prefill(const PrefillArgs& a, int in_bf16, int out_bf16, hipStream_t s, hipError_t* e) {
  if (!prefill_offsets_fit(a.H, a.P, a.N, a.R, a.Q)) return -1;
  if (in_bf16) {
    return out_bf16 ? dispatch_shape<PolHalf, bf16_t, bf16_t>(a, s, e)
                    : dispatch_shape<PolHalf, bf16_t, float>(a, s, e);
  }
  return out_bf16 ? dispatch_shape<PolF32, float, bf16_t>(a, s, e)
                  : dispatch_shape<PolF32, float, float>(a, s, e);
}

}  // namespace m3
