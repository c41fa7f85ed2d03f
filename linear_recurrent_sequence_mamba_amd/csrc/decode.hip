// decode.hip -- fused Mamba-3 decode step on gfx950.
//
// One token advances the fp32 state h [Bsz,H,P,N] in place:
//   h <- R(phi_t) (alpha h + beta X_{t-1} B_{t-1}^T) + gamma X_t B_t^T,
//   y_t = h C_t,
// the exponential-trapezoidal update [xxxxx.co.kr Mamba-3 article, section
// 1.1] with the complex (pairwise rotating) state of section 1.2 and the
// rank-R inputs/outputs of section 1.3.  Decode is bound by HBM traffic: the
// state is streamed once in and once out with 16-byte non-temporal accesses,
// everything else is a few KB per (batch, head).
//
// Two kernels:
//  * k_decode_siso (R = 1): each row of the state (N floats) is spread over
//    N/4 lanes holding 4 consecutive columns (two complex pairs), so a wave
//    moves whole 512-byte rows; the trapezoid terms and the rotation are
//    applied in registers and y_t is a shuffle reduction over those lanes.
//  * k_decode_mimo (R > 1): the rank-R input terms X B^T are 16x16 tiles of
//    v_mfma_f32_16x16x4_f32 with K = R (zero-padded to a multiple of 4).  The
//    MFMA row axis is the state column n, so each lane's accumulator holds 4
//    consecutive n of one row p -- the same 16-byte vector it loads and
//    stores -- and the decayed state is fed in as the accumulator.
#include "m3_device.h"
#include "m3_launch.h"

namespace m3 {

// --------------------------------------------------------------------------
// The per-token scalars and the phase of one pair are loaded before the
// state stream is issued: the load counter retires in order, so waiting for
// a small load issued after the state loads would wait for the whole stream.
// They are kept as loaded (bf16 bit patterns) until token_finish, and every
// thread reads a phase (threads past the pairs re-read the last one): with
// no conversion and no branch at the loads, nothing waits for them there.
template <typename TI, int N>
struct TokenIn {
  Raw1<TI> d, l, th;
  float A;
  float thp;   // with the angle projection: the projected phase input of pair threadIdx.x / TPP
};

// with the angle projection, TPP consecutive threads make one pair's phase
// input between them
template <int N>
constexpr int proj_tpp() { return 256 / (N / 2); }

// (batch, group) slot of B, C and theta for the unit bh = (batch, head)
__device__ __forceinline__ int64_t group_slot(const DecodeArgs& a, int bh) {
  return (int64_t)(bh / a.H) * a.G + (bh % a.H) / (a.H / a.G);
}

template <typename TI, int N, bool PROJ>
__device__ __forceinline__ TokenIn<TI, N> token_load(const DecodeArgs& a, int bh) {
  TokenIn<TI, N> in;
  const int head = bh % a.H;
  in.d.load(static_cast<const TI*>(a.dt), bh);
  in.l.load(static_cast<const TI*>(a.lam), bh);
  in.A = (a.flags & kAPerToken) ? a.A[bh] : a.A[head];
  if constexpr (PROJ) {
    // the angle projection [xxxxx.co.kr Mamba-3 article, section 1.2]:
    // theta_k = sum_j W[g][k][j] u[b][j], each of TPP threads summing every
    // TPP-th 16-byte piece of the row, then a lane-group sum (before the
    // state stream, which waits for nothing issued after it)
    constexpr int TPP = proj_tpp<N>();
    constexpr int VPV = 16 / sizeof(TI);
    static_assert(TPP >= 1 && TPP <= 64 && (TPP & (TPP - 1)) == 0, "pair groups of lanes");
    const int D = a.tp.dim;
    const int k = threadIdx.x / TPP, part = threadIdx.x % TPP;
    const TI* __restrict__ ur = static_cast<const TI*>(a.tp.u) + (int64_t)(bh / a.H) * D;
    const TI* __restrict__ wr = static_cast<const TI*>(a.tp.W) +
                                ((group_slot(a, bh) % a.G) * (N / 2) + k) * (int64_t)D;
    float s = 0.0f;
    for (int v = part; v < D / VPV; v += TPP) {
      if constexpr (VPV == 8) {
        float uv[8], wv[8];
        ld8(ur, (int64_t)v * 8, uv);
        ld8(wr, (int64_t)v * 8, wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += uv[e] * wv[e];
      } else {
        const f4 uv = ld4(ur, (int64_t)v * 4), wv = ld4(wr, (int64_t)v * 4);
        s += uv.x * wv.x + uv.y * wv.y + uv.z * wv.z + uv.w * wv.w;
      }
    }
    in.thp = group_sum<TPP>(s);
  } else {
    const int k = min(static_cast<int>(threadIdx.x), N / 2 - 1);
    in.th.load(static_cast<const TI*>(a.theta), group_slot(a, bh) * (N / 2) + k);
  }
  // the compiler may not move these loads past this point (towards their
  // uses, which come after the state stream)
  asm volatile("" ::: "memory");
  return in;
}

// alpha, beta, gamma; (cos, sin) of the token's phase per pair into LDS
template <typename TI, int N, bool PROJ>
__device__ __forceinline__ void token_finish(const DecodeArgs& a, const TokenIn<TI, N>& in,
                                             float& alpha, float& beta, float& gamma, f2* cs_sh) {
  const float d = in.d.f(), l = in.l.f();
  alpha = expf(d * in.A);
  beta = (1.0f - l) * d * alpha;
  gamma = l * d;
  constexpr int TPP = PROJ ? proj_tpp<N>() : 1;
  const int k = threadIdx.x / TPP;
  if (k < N / 2 && threadIdx.x % TPP == 0) {
    const float th = PROJ ? in.thp : in.th.f();
    const float phi = (a.flags & kThetaIsAngle) ? th : d * th;
    float s, c;
    sincosf(phi, &s, &c);
    cs_sh[k] = f2{c, s};
  }
}

// --------------------------------------------------------------------------
// single input / single output
template <typename TI, typename TO, int N, bool PREV, bool PREP, bool PROJ>
__global__ __launch_bounds__(256) void k_decode_siso(DecodeArgs a) {
  constexpr int LPR = N / 4;           // lanes per state row
  constexpr int RPW = 64 / LPR;        // rows per wave per pass
  constexpr int RPB = 4 * RPW;         // rows per block per pass
  constexpr int UNR = RPB >= 64 ? 1 : 64 / RPB;  // passes kept in flight
  static_assert(N / 2 <= 256, "one pair per thread");
  __shared__ f2 cs_sh[N / 2];

  const int bh = blockIdx.x;
  const int P = a.P;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = 4 * (lane % LPR);
  const int rsub = wave * RPW + lane / LPR;
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ x = static_cast<const TI*>(a.x) + (int64_t)bh * P;
  const TI* __restrict__ xp = static_cast<const TI*>(a.xp) + (int64_t)bh * P;
  TO* __restrict__ y = static_cast<TO*>(a.y) + (int64_t)bh * P;

  const TokenIn<TI, N> tin = token_load<TI, N, PROJ>(a, bh);
  const int64_t vec = group_slot(a, bh) * N + n0;
  f4 bt = ld4(static_cast<const TI*>(a.Bt), vec);
  f4 bp = PREV ? ld4(static_cast<const TI*>(a.Bp), vec) : f4{0, 0, 0, 0};
  f4 ct = ld4(static_cast<const TI*>(a.Ct), vec);
  // B/C preparation: weight and this head's bias of columns n0..n0+3
  f4 bw = f4{1, 1, 1, 1}, cw = bw, bb = f4{0, 0, 0, 0}, cb = bb;
  if constexpr (PREP) {
    const int64_t hb0 = (int64_t)(bh % a.H) * N + n0;
    // (read under branches: the branch-free form measured 4 us slower here)
    if (a.bc.Bw) bw = ld4(a.bc.Bw, n0);
    if (a.bc.Cw) cw = ld4(a.bc.Cw, n0);
    if (a.bc.Bb) bb = ld4(a.bc.Bb, hb0);
    if (a.bc.Cb) cb = ld4(a.bc.Cb, hb0);
  }

  // the token-side reads stay ahead of the state stream (the compiler may not
  // move them past it: a use would then wait for the whole stream)
  asm volatile("" ::: "memory");
  // the state stream; rows past P are clamped for the loads, masked for the stores
  f4 v[UNR];
  float xv[UNR], xpv[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int p = min(u * RPB + rsub, P - 1);
    v[u] = ld4_state(hb + (int64_t)p * N + n0);
    xv[u] = ld1(x, p);
    xpv[u] = PREV ? ld1(xp, p) : 0.0f;
  }

  float alpha, beta, gamma;
  token_finish<TI, N, PROJ>(a, tin, alpha, beta, gamma, cs_sh);
  if constexpr (PREP) {
    // a row's N/4 lanes hold the whole of B, B_prev and C
    auto prep = [&](f4 v, f4 w, f4 b) {
      const float inv = bc_inv_rms(a.bc, group_sum<LPR>(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w), N);
      return v * inv * w + b;
    };
    bt = prep(bt, bw, bb);
    if (PREV) bp = prep(bp, bw, bb);
    ct = prep(ct, cw, cb);
  }
  bt *= gamma;
  bp *= beta;
  __syncthreads();
  const f2 r0 = cs_sh[n0 / 2];
  const f2 r1 = cs_sh[n0 / 2 + 1];

  for (int pbase = 0;;) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pbase + u * RPB + rsub;
      f4 s = alpha * v[u] + xpv[u] * bp;
      s = rot2pairs(s, r0, r1);
      s += xv[u] * bt;
      if (p < P) st4_stream(hb + (int64_t)p * N + n0, s);
      const float part = group_sum<LPR>(s.x * ct.x + s.y * ct.y + s.z * ct.z + s.w * ct.w);
      if ((lane % LPR) == 0 && p < P) st1(y, p, part);
    }
    pbase += RPB * UNR;
    if (pbase >= P) break;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = min(pbase + u * RPB + rsub, P - 1);
      v[u] = ld4_state(hb + (int64_t)p * N + n0);
      xv[u] = ld1(x, p);
      xpv[u] = PREV ? ld1(xp, p) : 0.0f;
    }
  }
}

// --------------------------------------------------------------------------
// multi input / multi output, rank R (2 <= R <= 16)
//
// The MFMA row axis runs over state columns: D row 4g + i of tile t is
// column ncol(t, g) + i = 16t + 4g + i, so a lane's accumulator is the
// 16-byte vector of 4 consecutive columns it loads.  For the store the
// wave's 16 x N updated rows pass through a padded LDS buffer and leave as
// row-contiguous non-temporal 16-byte stores: every store instruction then
// writes whole 128-byte lines (stored straight from the D layout, each
// instruction would write half lines and HBM would see ~1.3x the bytes).
template <int NT>
__device__ __forceinline__ int ncol(int t, int g) { return 16 * t + 4 * g; }

// (the B/C preparation's prologue would otherwise cost the rank <= 4
// kernels a wave per SIMD: the register count is held to four waves)
template <typename TI, typename TO, int N, int R, bool PREV, bool PREP, bool PROJ>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(PREP && R <= 4 ? 4 : 1))) void k_decode_mimo(DecodeArgs a) {
  constexpr int NT = N / 16;          // 16-column tiles per state row block
  constexpr int KB = (R + 3) / 4;     // K blocks of 4 for the MFMA
  constexpr int RP = (R + 3) & ~3;    // rank padded to a multiple of 4 in LDS
  constexpr int NE = N * R;           // elements of one B or C
  constexpr int PER = (NE + 255) / 256;
  __shared__ f2 cs_sh[N / 2];
  __shared__ float bp_sh[N * RP];     // beta * B_{t-1}   [n][r]
  __shared__ float bt_sh[N * RP];     // gamma * B_t      [n][r]
  __shared__ float c_sh[N * RP];      // C_t              [n][r]
  __shared__ f4 tr_sh[4][16][N / 4 + 1];  // per-wave updated rows (one vector of padding)
  __shared__ float inv_sh[PREP ? 3 : 1][R];  // B/C preparation: inverse RMS per rank column

  const int bh = blockIdx.x;
  const int P = a.P;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i16 = lane & 15;   // MFMA column (state row p) / A-operand row
  const int g = lane >> 4;     // MFMA k lane group / D row group
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ x = static_cast<const TI*>(a.x) + (int64_t)bh * P * R;
  const TI* __restrict__ xp = static_cast<const TI*>(a.xp) + (int64_t)bh * P * R;
  TO* __restrict__ y = static_cast<TO*>(a.y) + (int64_t)bh * P * R;

  const TokenIn<TI, N> tin = token_load<TI, N, PROJ>(a, bh);
  float eb[PER], ep[PER], ec[PER];
  {
    const int64_t gs = group_slot(a, bh);
    const TI* __restrict__ Bt = static_cast<const TI*>(a.Bt) + gs * NE;
    const TI* __restrict__ Bp = static_cast<const TI*>(a.Bp) + gs * NE;
    const TI* __restrict__ Ct = static_cast<const TI*>(a.Ct) + gs * NE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = tid + 256 * q;
      const int ic = min(i, NE - 1);
      eb[q] = ld1(Bt, ic);
      ep[q] = PREV ? ld1(Bp, ic) : 0.0f;
      ec[q] = ld1(Ct, ic);
    }
  }
  // B/C preparation: weight and this head's bias of each element, loaded
  // before the state stream so that the preparation does not wait for it
  float wbv[PREP ? PER : 1], wcv[PREP ? PER : 1], bbv[PREP ? PER : 1], cbv[PREP ? PER : 1];
  if constexpr (PREP) {
    const int64_t hb0 = (int64_t)(bh % a.H) * NE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int ic = min(tid + 256 * q, NE - 1);
      wbv[q] = ld_or(a.bc.Bw, ic / R, 1.0f);
      wcv[q] = ld_or(a.bc.Cw, ic / R, 1.0f);
      bbv[q] = ld_or(a.bc.Bb, hb0 + ic, 0.0f);
      cbv[q] = ld_or(a.bc.Cb, hb0 + ic, 0.0f);
    }
  }

  // the token-side reads stay ahead of the state stream (as in the
  // single-input kernel)
  asm volatile("" ::: "memory");
  // the first row block's state stream, row-contiguous (whole 128-byte
  // lines per load instruction); it reaches the D layout through LDS
  constexpr int V4 = N / 4;            // 16-byte vectors per row
  constexpr int LV = 16 * V4 / 64;     // row vectors per lane per 16-row block
  int pb = wave;
  f4 raw[LV];
  if (pb * 16 < P) {
#pragma unroll
    for (int j = 0; j < LV; ++j) {
      const int q = lane + 64 * j;
      raw[j] = ld4_state(hb + (int64_t)(pb * 16 + q / V4) * N + 4 * (q % V4));
    }
  }

  float alpha, beta, gamma;
  token_finish<TI, N, PROJ>(a, tin, alpha, beta, gamma, cs_sh);
  if constexpr (RP != R) {
    for (int i = tid; i < N * RP; i += 256) bt_sh[i] = bp_sh[i] = c_sh[i] = 0.0f;
    __syncthreads();
  }
  // with the B/C preparation the tables first take the raw rows; waves 0-2
  // reduce one table each to inverse RMS per rank column, then every
  // element is normalised, weighted, biased and scaled in place
  const float sbt = PREP ? 1.0f : gamma, sbp = PREP ? 1.0f : beta;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + 256 * q;
    if (i < NE) {
      const int j = (i / R) * RP + i % R;
      bt_sh[j] = sbt * eb[q];
      bp_sh[j] = sbp * ep[q];
      c_sh[j] = ec[q];
    }
  }
  __syncthreads();
  if constexpr (PREP) {
    if (wave < 3 && (wave != 1 || PREV)) {
      const float* tab = wave == 0 ? bt_sh : (wave == 1 ? bp_sh : c_sh);
      float part[R];
#pragma unroll
      for (int r = 0; r < R; ++r) part[r] = 0.0f;
      for (int n = lane; n < N; n += 64) {
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] += tab[n * RP + r] * tab[n * RP + r];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) part[r] = group_sum<64>(part[r]);
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) inv_sh[wave][r] = bc_inv_rms(a.bc, part[r], N);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {   // each thread its own elements, from registers
      const int i = tid + 256 * q;
      if (i < NE) {
        const int r = i % R, j = (i / R) * RP + r;
        bt_sh[j] = gamma * (eb[q] * inv_sh[0][r] * wbv[q] + bbv[q]);
        if (PREV) bp_sh[j] = beta * (ep[q] * inv_sh[1][r] * wbv[q] + bbv[q]);
        c_sh[j] = ec[q] * inv_sh[2][r] * wcv[q] + cbv[q];
      }
    }
    __syncthreads();
  }

  for (; pb * 16 < P; pb += 4) {
    const int p = pb * 16 + i16;
    // rows -> LDS -> D layout (the buffer is private to the wave)
#pragma unroll
    for (int j = 0; j < LV; ++j) {
      const int q = lane + 64 * j;
      tr_sh[wave][q / V4][q % V4] = raw[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f4 v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = tr_sh[wave][i16][ncol<NT>(t, g) / 4];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float xo_p[KB], xo_t[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = 4 * kb + g;
      xo_t[kb] = (r < R) ? ld1(x, (int64_t)p * R + r) : 0.0f;
      xo_p[kb] = (r < R && PREV) ? ld1(xp, (int64_t)p * R + r) : 0.0f;
    }
    float yp[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) yp[r] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4 acc = alpha * v[t];
      const int nA = ncol<NT>(t, i16 >> 2) + (i16 & 3);   // state column of A-operand row i16
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bp_sh[nA * RP + 4 * kb + g], xo_p[kb], acc, 0, 0, 0);
      const int n = ncol<NT>(t, g);        // state columns n..n+3 of acc
      acc = rot2pairs(acc, cs_sh[n / 2], cs_sh[n / 2 + 1]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bt_sh[nA * RP + 4 * kb + g], xo_t[kb], acc, 0, 0, 0);
      tr_sh[wave][i16][n / 4] = acc;
#pragma unroll
      for (int rb = 0; rb < RP; rb += 4) {
        const f4 c0 = *reinterpret_cast<const f4*>(&c_sh[(n + 0) * RP + rb]);
        const f4 c1 = *reinterpret_cast<const f4*>(&c_sh[(n + 1) * RP + rb]);
        const f4 c2 = *reinterpret_cast<const f4*>(&c_sh[(n + 2) * RP + rb]);
        const f4 c3 = *reinterpret_cast<const f4*>(&c_sh[(n + 3) * RP + rb]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          yp[rb + q] += acc.x * c0[q] + acc.y * c1[q] + acc.z * c2[q] + acc.w * c3[q];
      }
      // keep each tile's LDS operands local to it (hoisting them all would
      // cost ~150 registers and halve the occupancy)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      yp[r] += __shfl_xor(yp[r], 16, 64);
      yp[r] += __shfl_xor(yp[r], 32, 64);
    }
    if (g == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) st1(y, (int64_t)p * R + r, yp[r]);
    }
    // the wave's 16 rows back to HBM, row-contiguous (the buffer is private
    // to the wave; a wave barrier orders the LDS writes before the reads)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
#pragma unroll
      for (int j = 0; j < LV; ++j) {
        const int q = lane + 64 * j;
        const int rr = q / V4, c4 = q % V4;
        st4_stream(hb + (int64_t)(pb * 16 + rr) * N + 4 * c4, tr_sh[wave][rr][c4]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((pb + 4) * 16 < P) {
#pragma unroll
      for (int j = 0; j < LV; ++j) {
        const int q = lane + 64 * j;
        raw[j] = ld4_state(hb + (int64_t)((pb + 4) * 16 + q / V4) * N + 4 * (q % V4));
      }
    }
  }
}

// --------------------------------------------------------------------------
template <typename TI, typename TO, int N, bool PROJ>
static hipError_t launch_siso_p(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 g(units), b(256);
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso<TI, TO, N, true, true, PROJ>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso<TI, TO, N, false, true, PROJ>), g, b, 0, s, a);
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_siso<TI, TO, N, true, false, PROJ>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_siso<TI, TO, N, false, false, PROJ>), g, b, 0, s, a);
  }
  return hipGetLastError();
}
template <typename TI, typename TO, int N>
static hipError_t launch_siso(const DecodeArgs& a, int units, hipStream_t s) {
  return a.tp.on ? launch_siso_p<TI, TO, N, true>(a, units, s)
                 : launch_siso_p<TI, TO, N, false>(a, units, s);
}

template <typename TI, typename TO, int N, int R, bool PROJ>
static hipError_t launch_mimo_p(const DecodeArgs& a, int units, hipStream_t s) {
  const dim3 g(units), b(256);
  if (a.bc.on) {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo<TI, TO, N, R, true, true, PROJ>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo<TI, TO, N, R, false, true, PROJ>), g, b, 0, s, a);
  } else {
    if (a.has_prev) hipLaunchKernelGGL((k_decode_mimo<TI, TO, N, R, true, false, PROJ>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_decode_mimo<TI, TO, N, R, false, false, PROJ>), g, b, 0, s, a);
  }
  return hipGetLastError();
}
template <typename TI, typename TO, int N, int R>
static hipError_t launch_mimo(const DecodeArgs& a, int units, hipStream_t s) {
  return a.tp.on ? launch_mimo_p<TI, TO, N, R, true>(a, units, s)
                 : launch_mimo_p<TI, TO, N, R, false>(a, units, s);
}

template <typename TI, typename TO>
static int dispatch_decode(const DecodeArgs& a, int units, hipStream_t s, hipError_t* err) {
  if (a.R == 1) {
    switch (a.N) {
      case 16: *err = launch_siso<TI, TO, 16>(a, units, s); return 0;
      case 32: *err = launch_siso<TI, TO, 32>(a, units, s); return 0;
      case 64: *err = launch_siso<TI, TO, 64>(a, units, s); return 0;
      case 128: *err = launch_siso<TI, TO, 128>(a, units, s); return 0;
      case 256: *err = launch_siso<TI, TO, 256>(a, units, s); return 0;
      default: return -1;
    }
  }
  if (a.P % 16 != 0) return -1;
#define M3_MIMO_N(NN)                                                   \
  case NN:                                                              \
    switch (a.R) {                                                      \
      case 2: *err = launch_mimo<TI, TO, NN, 2>(a, units, s); return 0; \
      case 3: *err = launch_mimo<TI, TO, NN, 3>(a, units, s); return 0; \
      case 4: *err = launch_mimo<TI, TO, NN, 4>(a, units, s); return 0; \
      case 8: *err = launch_mimo<TI, TO, NN, 8>(a, units, s); return 0; \
      default: return -1;                                               \
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

bool decode_supported(int P, int N, int R) {
  if (R == 1) return N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
  if (P % 16 != 0) return false;
  if (!(N == 16 || N == 32 || N == 64 || N == 128)) return false;
  return R == 2 || R == 3 || R == 4 || R == 8;
}

int launch_decode(const DecodeArgs& a, int in_bf16, int out_bf16, int units,
                  hipStream_t s, hipError_t* err) {
  if (in_bf16) {
    return out_bf16 ? dispatch_decode<bf16_t, bf16_t>(a, units, s, err)
                    : dispatch_decode<bf16_t, float>(a, units, s, err);
  }
  return out_bf16 ? dispatch_decode<float, bf16_t>(a, units, s, err)
                  : dispatch_decode<float, float>(a, units, s, err);
}

}  // namespace m3
