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
//  * k_decode_mimo_tok (R > 1): one 16-row block of the state per wave,
//    P <= 64, in the MFMA D layout (the rank-R terms are MFMA products with
//    K = R, as in the single-step kernel); rows enter and leave through a
//    per-wave LDS transpose so that loads and stores cover whole lines.
#include "m3_device.h"
#include "m3_launch.h"

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
// four waves per SIMD (at most 128 registers) for the 8-row blocks; the
// B/C preparation needs more registers than that
template <typename TI, typename TO, int N, int UNR, bool PREV, bool PREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(UNR == 8 && !PREP ? 4 : 1))) void k_decode_siso_tok(
    DecodeArgs a) {
  constexpr int LPR = N / 4;      // lanes per state row
  constexpr int RPW = 64 / LPR;   // rows per wave per pass
  constexpr int RPB = 4 * RPW;    // rows per block per pass
  // a unit's rows may be split over several blocks (UNR * RPB rows each)
  const int nblk = (a.P + UNR * RPB - 1) / (UNR * RPB);
  const int bh = blockIdx.x / nblk;
  const int P = a.P;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = 4 * (lane % LPR);
  const int rsub = (blockIdx.x % nblk) * UNR * RPB + wave * RPW + lane / LPR;
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.Bt);
  const TI* __restrict__ Cg = static_cast<const TI*>(a.Ct);
  TO* __restrict__ Y = static_cast<TO*>(a.y);

  // a lane's own two pairs (columns n0..n0+3) need their two phases only:
  // no table, no barrier between tokens
  const TI* __restrict__ Tg = static_cast<const TI*>(a.theta);
  const TI* __restrict__ Dg = static_cast<const TI*>(a.dt);
  const TI* __restrict__ Lg = static_cast<const TI*>(a.lam);
  auto scal = [&](int k, float& d, float& l, float& A, f2& th) {
    const int64_t t = tok_head(a, bh, k);
    d = ld1(Dg, t);
    l = ld1(Lg, t);
    A = (a.flags & kAPerToken) ? a.A[t] : a.A[bh % a.H];
    th = ld2(Tg, tok_group(a, bh, k) * (N / 2) + n0 / 2);
  };
  // token 0's inputs go out first, then the whole state of the unit
  float dk, lk, Ak;
  f2 thk;
  scal(0, dk, lk, Ak, thk);
  f4 bk = ld4(Bg, tok_group(a, bh, 0) * N + n0);
  f4 ck = ld4(Cg, tok_group(a, bh, 0) * N + n0);
  float xk[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) xk[u] = ld1(X, tok_head(a, bh, 0) * P + min(u * RPB + rsub, P - 1));
  // the token before the first one: x_prev, B_prev (or zero)
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
  // a row's N/4 lanes hold a token's whole B and C
  auto prep = [&](f4 u, f4 w, f4 b) {
    const float inv = bc_inv_rms(a.bc, group_sum<LPR>(u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w), N);
    return u * inv * w + b;
  };
  f4 v[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) v[u] = ld4_state(hb + (int64_t)min(u * RPB + rsub, P - 1) * N + n0);
  if (PREP && PREV) bo = prep(bo, bw, bbias);   // bo always holds a prepared B

  for (int k = 0; k < a.K; ++k) {
    // the next token's inputs fly, as loaded, while this one is applied (the
    // last token re-reads its own and drops them: no branch around a load)
    const int kn = min(k + 1, a.K - 1);
    const int64_t tn = tok_head(a, bh, kn);
    Raw1<TI> dn, ln, xn[UNR];
    dn.load(Dg, tn);
    ln.load(Lg, tn);
    const float An = (a.flags & kAPerToken) ? a.A[tn] : a.A[bh % a.H];
    RawVec<TI, 2> thn;
    RawVec<TI, 4> bn, cn;
    thn.load(Tg + tok_group(a, bh, kn) * (N / 2) + n0 / 2);
    bn.load(Bg + tok_group(a, bh, kn) * N + n0);
    cn.load(Cg + tok_group(a, bh, kn) * N + n0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) xn[u].load(X, tn * P + min(u * RPB + rsub, P - 1));
    const float alpha = expf(dk * Ak);
    const float beta = (1.0f - lk) * dk * alpha;
    const float gamma = lk * dk;
    const bool ang = (a.flags & kThetaIsAngle) != 0;
    const f2 r0 = cos_sin_turns(ang ? thk.x : dk * thk.x);
    const f2 r1 = cos_sin_turns(ang ? thk.y : dk * thk.y);
    if constexpr (PREP) {
      bk = prep(bk, bw, bbias);
      ck = prep(ck, cw, cbias);
    }
    const f4 bt = gamma * bk, bp = beta * bo;
    TO* __restrict__ yk = Y + tok_head(a, bh, k) * P;
    float part[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      f4 s = alpha * v[u] + xo[u] * bp;
      s = rot2pairs(s, r0, r1);
      s += xk[u] * bt;
      v[u] = s;
      part[u] = s.x * ck.x + s.y * ck.y + s.z * ck.z + s.w * ck.w;
    }
    // y of the lane's UNR rows: summed over the row's LPR lanes
    float tot[UNR];
    if constexpr (UNR <= LPR) {
      tot[0] = rows_sum<LPR, UNR>(part, lane % LPR);
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) tot[u] = group_sum<LPR>(part[u]);
    }
    // the next token's inputs come into use before this token's y stores: a
    // loaded value used after a store would wait for the store as well
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      xo[u] = xk[u];
      xk[u] = xn[u].f();
    }
    bo = bk;
    {
      float t4[4], t2[2];
      bn.get(t4);
      bk = f4{t4[0], t4[1], t4[2], t4[3]};
      cn.get(t4);
      ck = f4{t4[0], t4[1], t4[2], t4[3]};
      thn.get(t2);
      thk = f2{t2[0], t2[1]};
    }
    dk = dn.f();
    lk = ln.f();
    Ak = An;
    if constexpr (UNR <= LPR) {
      const int j = lane % LPR;
      const int p = (j / (LPR / UNR)) * RPB + rsub;
      if (j % (LPR / UNR) == 0 && p < P) st1(yk, p, tot[0]);
    } else {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int p = u * RPB + rsub;
        if ((lane % LPR) == 0 && p < P) st1(yk, p, tot[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int p = u * RPB + rsub;
    if (p < P) st4_stream(hb + (int64_t)p * N + n0, v[u]);
  }
}

// --------------------------------------------------------------------------
// D row 4g + i of tile t is state column 16t + 4g + i (as in the single-step
// kernel): a lane's accumulator is the 16-byte vector of 4 consecutive
// columns of its row.
template <typename TI, typename TO, int N, int R, bool PREV, bool PREP>
__global__ __launch_bounds__(256) void k_decode_mimo_tok(DecodeArgs a) {
  constexpr int NT = N / 16;
  constexpr int KB = (R + 3) / 4;
  constexpr int RP = (R + 3) & ~3;
  constexpr int NE = N * R;
  constexpr int PER = (NE + 255) / 256;
  constexpr int V4 = N / 4;
  constexpr int LV = 16 * V4 / 64;
  // per-token operands, double-buffered (token k + 1's are written while
  // token k is applied: one barrier per token); the row transposes at the
  // start and the end share the space
  struct Tok {
    f2 cs[N / 2];
    float bp[N * RP];     // beta_k * B_{k-1}   [n][r]
    float bt[N * RP];     // gamma_k * B_k      [n][r]
    float c[N * RP];      // C_k                [n][r]
  };
  __shared__ union {
    Tok tok[2];
    f4 tr[4][16][N / 4 + 1];
  } sm;
  // B/C preparation: this head's weights and biases ([0] B, [1] C), and
  // each wave's partial sums of squares per rank column of the B, C and
  // (first token) B_prev that a table build prepares
  __shared__ float pw_sh[PREP ? 2 : 1][PREP ? N : 1];
  __shared__ float pb_sh[PREP ? 2 : 1][PREP ? NE : 1];
  __shared__ float part_sh[4][3][R];

  const int bh = blockIdx.x;
  const int P = a.P;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const bool rows = wave * 16 < P;   // this wave's 16-row block exists
  const int p = wave * 16 + i16;
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ X = static_cast<const TI*>(a.x);
  const TI* __restrict__ Bg = static_cast<const TI*>(a.Bt);
  const TI* __restrict__ Cg = static_cast<const TI*>(a.Ct);
  TO* __restrict__ Y = static_cast<TO*>(a.y);

  auto load_bc = [&](int k, float* eb, float* ec) {
    const TI* __restrict__ Bk = Bg + tok_group(a, bh, k) * NE;
    const TI* __restrict__ Ck = Cg + tok_group(a, bh, k) * NE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = min(tid + 256 * q, NE - 1);
      eb[q] = ld1(Bk, i);
      ec[q] = ld1(Ck, i);
    }
  };
  // the next token's B and C elements, as loaded
  auto load_bc_raw = [&](int k, Raw1<TI>* eb, Raw1<TI>* ec) {
    const TI* __restrict__ Bk = Bg + tok_group(a, bh, k) * NE;
    const TI* __restrict__ Ck = Cg + tok_group(a, bh, k) * NE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = min(tid + 256 * q, NE - 1);
      eb[q].load(Bk, i);
      ec[q].load(Ck, i);
    }
  };
  // x of this lane's rank r = 4 kb + g, as loaded (lanes with no such row or
  // rank read element 0; xval zeroes them): no branch around the load
  auto load_x = [&](const TI* __restrict__ src, Raw1<TI>* xr) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = 4 * kb + g;
      xr[kb].load(src, (rows && r < R) ? (int64_t)p * R + r : 0);
    }
  };
  auto xval = [&](const Raw1<TI>* xr, float* xv) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xv[kb] = (rows && 4 * kb + g < R) ? xr[kb].f() : 0.0f;
  };
  // token operands into buffer tb: beta/gamma-scaled B, C, phases.  With
  // the preparation, eb and ec (and eo when prep_prev) are raw on entry and
  // prepared on return: each wave reduces its elements' squares per rank
  // column into part_sh, and after a barrier every thread sums the four
  // waves' parts (the sums' last readers are past the barrier that ends
  // each token, before the next build writes them).
  auto put_tables = [&](Tok& tb, const TokScalars<TI, N>& sc, float* eb, float* eo, float* ec,
                        bool prep_prev) {
    float alpha, beta, gamma;
    sc.finish(a, alpha, beta, gamma, tb.cs);
    if constexpr (PREP) {
      auto wave_parts = [&](const float* e, int arr) {
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = 0.0f;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int i = tid + 256 * q;
          const float v = i < NE ? e[q] : 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) part[r] += (i % R == r) ? v * v : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = group_sum<64>(part[r]);
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r) part_sh[wave][arr][r] = part[r];
        }
      };
      wave_parts(eb, 0);
      wave_parts(ec, 2);
      if (prep_prev) wave_parts(eo, 1);
      __syncthreads();
      auto inv = [&](int arr, int r) {
        return bc_inv_rms(a.bc, part_sh[0][arr][r] + part_sh[1][arr][r] + part_sh[2][arr][r] +
                                    part_sh[3][arr][r], N);
      };
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int i = min(tid + 256 * q, NE - 1);
        const int r = i % R, n = i / R;
        eb[q] = eb[q] * inv(0, r) * pw_sh[0][n] + pb_sh[0][i];
        ec[q] = ec[q] * inv(2, r) * pw_sh[1][n] + pb_sh[1][i];
        if (prep_prev) eo[q] = eo[q] * inv(1, r) * pw_sh[0][n] + pb_sh[0][i];
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = tid + 256 * q;
      if (i < NE) {
        const int j = (i / R) * RP + i % R;
        tb.bt[j] = gamma * eb[q];
        tb.bp[j] = beta * eo[q];
        tb.c[j] = ec[q];
      }
    }
  };

  TokScalars<TI, N> sc;
  sc.load(a, bh, 0);
  float eb[PER], ec[PER], eo[PER];
  load_bc(0, eb, ec);
  float xk[KB], xo[KB];
  Raw1<TI> xkr[KB], xor_[KB];
  load_x(X + tok_head(a, bh, 0) * P * R, xkr);
  if (PREV) {
    const TI* __restrict__ Bp = static_cast<const TI*>(a.Bp) + unit_group(a, bh) * NE;
#pragma unroll
    for (int q = 0; q < PER; ++q) eo[q] = ld1(Bp, min(tid + 256 * q, NE - 1));
    load_x(static_cast<const TI*>(a.xp) + (int64_t)bh * P * R, xor_);
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q) eo[q] = 0.0f;
  }

  // the wave's 16 state rows, row-contiguous, then into the D layout
  f4 v[NT];
  if (rows) {
    f4 raw[LV];
#pragma unroll
    for (int j = 0; j < LV; ++j) {
      const int q = lane + 64 * j;
      raw[j] = ld4_state(hb + (int64_t)(wave * 16 + q / V4) * N + 4 * (q % V4));
    }
#pragma unroll
    for (int j = 0; j < LV; ++j) {
      const int q = lane + 64 * j;
      sm.tr[wave][q / V4][q % V4] = raw[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = sm.tr[wave][i16][(16 * t + 4 * g) / 4];
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = f4{0, 0, 0, 0};
  }
  if constexpr (PREP) {   // this head's weights and biases (1 and 0 when absent)
    const int64_t hb0 = (int64_t)(bh % a.H) * NE;
    for (int i = tid; i < N; i += 256) {
      pw_sh[0][i] = ld_or(a.bc.Bw, i, 1.0f);
      pw_sh[1][i] = ld_or(a.bc.Cw, i, 1.0f);
    }
    for (int i = tid; i < NE; i += 256) {
      pb_sh[0][i] = ld_or(a.bc.Bb, hb0 + i, 0.0f);
      pb_sh[1][i] = ld_or(a.bc.Cb, hb0 + i, 0.0f);
    }
  }
  __syncthreads();   // every wave's transpose is read before the tables take the space
  if constexpr (RP != R) {
    for (int i = tid; i < N * RP; i += 256)
      sm.tok[0].bt[i] = sm.tok[0].bp[i] = sm.tok[0].c[i] = sm.tok[1].bt[i] = sm.tok[1].bp[i] =
          sm.tok[1].c[i] = 0.0f;
    __syncthreads();
  }
  put_tables(sm.tok[0], sc, eb, eo, ec, PREV);
  __syncthreads();
  xval(xkr, xk);
  if (PREV) {
    xval(xor_, xo);
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xo[kb] = 0.0f;
  }

  for (int k = 0; k < a.K; ++k) {
    // token k + 1's inputs, as loaded (the last token re-reads its own and
    // drops them): no branch around the loads, no conversion before the
    // state update below
    const int kn = min(k + 1, a.K - 1);
    TokScalars<TI, N> scn;
    scn.load(a, bh, kn);
    Raw1<TI> ebn[PER], ecn[PER], xn[KB];
    load_bc_raw(kn, ebn, ecn);
    load_x(X + tok_head(a, bh, kn) * P * R, xn);
    const Tok& tb = sm.tok[k & 1];
    const float alpha = expf(sc.d() * sc.A);
    float yp[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) yp[r] = 0.0f;
    if (rows) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f4 acc = alpha * v[t];
        const int nA = 16 * t + 4 * (i16 >> 2) + (i16 & 3);   // state column of A-operand row i16
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tb.bp[nA * RP + 4 * kb + g], xo[kb], acc, 0, 0, 0);
        const int n = 16 * t + 4 * g;
        acc = rot2pairs(acc, tb.cs[n / 2], tb.cs[n / 2 + 1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tb.bt[nA * RP + 4 * kb + g], xk[kb], acc, 0, 0, 0);
        v[t] = acc;
#pragma unroll
        for (int rb = 0; rb < RP; rb += 4) {
          const f4 c0 = *reinterpret_cast<const f4*>(&tb.c[(n + 0) * RP + rb]);
          const f4 c1 = *reinterpret_cast<const f4*>(&tb.c[(n + 1) * RP + rb]);
          const f4 c2 = *reinterpret_cast<const f4*>(&tb.c[(n + 2) * RP + rb]);
          const f4 c3 = *reinterpret_cast<const f4*>(&tb.c[(n + 3) * RP + rb]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            yp[rb + q] += acc.x * c0[q] + acc.y * c1[q] + acc.z * c2[q] + acc.w * c3[q];
        }
        // one tile's LDS operands at a time (registers and occupancy)
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        yp[r] += __shfl_xor(yp[r], 16, 64);
        yp[r] += __shfl_xor(yp[r], 32, 64);
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      eo[q] = eb[q];
      eb[q] = ebn[q].f();
      ec[q] = ecn[q].f();
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xo[kb] = xk[kb];
    xval(xn, xk);
    sc = scn;
    // token k + 1's operands into the other buffer (last read at token k - 1,
    // before the previous barrier), before token k's y stores: a loaded value
    // used after a store would wait for the store as well
    if (k + 1 < a.K) put_tables(sm.tok[(k + 1) & 1], sc, eb, eo, ec, false);
    if (rows && g == 0) {
      TO* __restrict__ yk = Y + tok_head(a, bh, k) * P * R;
#pragma unroll
      for (int r = 0; r < R; ++r) st1(yk, (int64_t)p * R + r, yp[r]);
    }
    __syncthreads();
  }

  // the wave's rows back to HBM, row-contiguous (every wave is past the
  // last token's tables: the loop ends with a barrier)
  if (rows) {
#pragma unroll
    for (int t = 0; t < NT; ++t) sm.tr[wave][i16][(16 * t + 4 * g) / 4] = v[t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < LV; ++j) {
      const int q = lane + 64 * j;
      st4_stream(hb + (int64_t)(wave * 16 + q / V4) * N + 4 * (q % V4), sm.tr[wave][q / V4][q % V4]);
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
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, true, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso_tok<TI, TO, N, UNR, false, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

template <typename TI, typename TO, int N, int R>
hipError_t launch_mimo_tok(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 g(units), b(256);
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, true, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo_tok<TI, TO, N, R, false, true>), g, b, 0, s, a);
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
      case 4: *err = launch_mimo_tok<TI, TO, NN, 4>(a, units, s); return 0; \
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
