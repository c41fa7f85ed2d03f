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
// single input / single output
template <typename TI, typename TO, int N>
__global__ __launch_bounds__(256) void k_decode_siso(DecodeArgs a) {
  constexpr int LPR = N / 4;           // lanes per state row
  constexpr int RPW = 64 / LPR;        // rows per wave per pass
  constexpr int RPB = 4 * RPW;         // rows per block per pass
  constexpr int UNR = RPB >= 64 ? 1 : 64 / RPB;  // passes kept in flight
  __shared__ f2 cs_sh[N / 2];

  const int bh = blockIdx.x;
  const int head = bh % a.H;
  const int P = a.P;
  const TI* __restrict__ dt = static_cast<const TI*>(a.dt);
  const TI* __restrict__ lam = static_cast<const TI*>(a.lam);
  const TI* __restrict__ theta = static_cast<const TI*>(a.theta);

  const float d = ld1(dt, bh);
  const float l = ld1(lam, bh);
  const float A = (a.flags & kAPerToken) ? a.A[bh] : a.A[head];
  const float alpha = expf(d * A);
  const float beta = (1.0f - l) * d * alpha;
  const float gamma = l * d;

  for (int k = threadIdx.x; k < N / 2; k += blockDim.x) {
    const float th = ld1(theta, (int64_t)bh * (N / 2) + k);
    const float phi = (a.flags & kThetaIsAngle) ? th : d * th;
    float s, c;
    sincosf(phi, &s, &c);
    cs_sh[k] = f2{c, s};
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = 4 * (lane % LPR);
  const int64_t vec = (int64_t)bh * N + n0;
  const f4 bt = ld4(static_cast<const TI*>(a.Bt), vec) * gamma;
  const f4 bp = a.has_prev ? ld4(static_cast<const TI*>(a.Bp), vec) * beta : f4{0, 0, 0, 0};
  const f4 ct = ld4(static_cast<const TI*>(a.Ct), vec);
  __syncthreads();
  const f2 r0 = cs_sh[n0 / 2];
  const f2 r1 = cs_sh[n0 / 2 + 1];

  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ x = static_cast<const TI*>(a.x) + (int64_t)bh * P;
  const TI* __restrict__ xp = static_cast<const TI*>(a.xp) + (int64_t)bh * P;
  TO* __restrict__ y = static_cast<TO*>(a.y) + (int64_t)bh * P;
  const int rsub = wave * RPW + lane / LPR;

  for (int pbase = 0; pbase < P; pbase += RPB * UNR) {
    f4 v[UNR];
    float xv[UNR], xpv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pbase + u * RPB + rsub;
      if (p < P) {
        v[u] = ld4_stream(hb + (int64_t)p * N + n0);
        xv[u] = ld1(x, p);
        xpv[u] = a.has_prev ? ld1(xp, p) : 0.0f;
      } else {
        v[u] = f4{0, 0, 0, 0};
        xv[u] = xpv[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pbase + u * RPB + rsub;
      f4 s = alpha * v[u] + xpv[u] * bp;
      s = rot2pairs(s, r0, r1);
      s += xv[u] * bt;
      if (p < P) st4_stream(hb + (int64_t)p * N + n0, s);
      float part = s.x * ct.x + s.y * ct.y + s.z * ct.z + s.w * ct.w;
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      if ((lane % LPR) == 0 && p < P) st1(y, p, part);
    }
  }
}

// --------------------------------------------------------------------------
// multi input / multi output, rank R (2 <= R <= 16)
template <typename TI, typename TO, int N, int R>
__global__ __launch_bounds__(256) void k_decode_mimo(DecodeArgs a) {
  constexpr int NT = N / 16;          // 16-column tiles per state row block
  constexpr int KB = (R + 3) / 4;     // K blocks of 4 for the MFMA
  __shared__ f2 cs_sh[N / 2];
  __shared__ float bp_sh[N * R];      // beta * B_{t-1}
  __shared__ float bt_sh[N * R];      // gamma * B_t
  __shared__ float c_sh[N * R];       // C_t

  const int bh = blockIdx.x;
  const int head = bh % a.H;
  const int P = a.P;
  const TI* __restrict__ dt = static_cast<const TI*>(a.dt);
  const TI* __restrict__ lam = static_cast<const TI*>(a.lam);
  const TI* __restrict__ theta = static_cast<const TI*>(a.theta);

  const float d = ld1(dt, bh);
  const float l = ld1(lam, bh);
  const float A = (a.flags & kAPerToken) ? a.A[bh] : a.A[head];
  const float alpha = expf(d * A);
  const float beta = (1.0f - l) * d * alpha;
  const float gamma = l * d;

  for (int k = threadIdx.x; k < N / 2; k += blockDim.x) {
    const float th = ld1(theta, (int64_t)bh * (N / 2) + k);
    const float phi = (a.flags & kThetaIsAngle) ? th : d * th;
    float s, c;
    sincosf(phi, &s, &c);
    cs_sh[k] = f2{c, s};
  }
  {
    const TI* __restrict__ Bt = static_cast<const TI*>(a.Bt) + (int64_t)bh * N * R;
    const TI* __restrict__ Bp = static_cast<const TI*>(a.Bp) + (int64_t)bh * N * R;
    const TI* __restrict__ Ct = static_cast<const TI*>(a.Ct) + (int64_t)bh * N * R;
    for (int i = threadIdx.x; i < N * R; i += blockDim.x) {
      bt_sh[i] = gamma * ld1(Bt, i);
      bp_sh[i] = a.has_prev ? beta * ld1(Bp, i) : 0.0f;
      c_sh[i] = ld1(Ct, i);
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i16 = lane & 15;   // MFMA column (state row p) / A-operand row
  const int g = lane >> 4;     // MFMA k lane group / D row group
  float* __restrict__ hb = a.h + (int64_t)bh * P * N;
  const TI* __restrict__ x = static_cast<const TI*>(a.x) + (int64_t)bh * P * R;
  const TI* __restrict__ xp = static_cast<const TI*>(a.xp) + (int64_t)bh * P * R;
  TO* __restrict__ y = static_cast<TO*>(a.y) + (int64_t)bh * P * R;

  for (int pb = wave; pb * 16 < P; pb += 4) {
    const int p = pb * 16 + i16;
    f4 v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = ld4_stream(hb + (int64_t)p * N + 16 * t + 4 * g);
    float xo_p[KB], xo_t[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = 4 * kb + g;
      xo_t[kb] = (r < R) ? ld1(x, (int64_t)p * R + r) : 0.0f;
      xo_p[kb] = (r < R && a.has_prev) ? ld1(xp, (int64_t)p * R + r) : 0.0f;
    }
    float yp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) yp[r] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4 acc = alpha * v[t];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int r = 4 * kb + g;
        const float aop = (r < R) ? bp_sh[(16 * t + i16) * R + r] : 0.0f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, xo_p[kb], acc, 0, 0, 0);
      }
      const int k0 = 8 * t + 2 * g;    // pair index of acc.x/acc.y
      acc = rot2pairs(acc, cs_sh[k0], cs_sh[k0 + 1]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int r = 4 * kb + g;
        const float aop = (r < R) ? bt_sh[(16 * t + i16) * R + r] : 0.0f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, xo_t[kb], acc, 0, 0, 0);
      }
      st4_stream(hb + (int64_t)p * N + 16 * t + 4 * g, acc);
      const int n = 16 * t + 4 * g;
#pragma unroll
      for (int r = 0; r < R; ++r)
        yp[r] += acc.x * c_sh[n * R + r] + acc.y * c_sh[(n + 1) * R + r] +
                 acc.z * c_sh[(n + 2) * R + r] + acc.w * c_sh[(n + 3) * R + r];
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
  }
}

// --------------------------------------------------------------------------
template <typename TI, typename TO, int N>
static hipError_t launch_siso(const DecodeArgs& a, int units, hipStream_t s) {
  hipLaunchKernelGGL((k_decode_siso<TI, TO, N>), dim3(units), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TI, typename TO, int N, int R>
static hipError_t launch_mimo(const DecodeArgs& a, int units, hipStream_t s) {
  hipLaunchKernelGGL((k_decode_mimo<TI, TO, N, R>), dim3(units), dim3(256), 0, s, a);
  return hipGetLastError();
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
