// api.cpp -- the C ABI of libm3ssm (include/m3ssm.h): argument checks,
// workspace sizing and dispatch to the gfx950 kernels.  Every check runs on
// the host before anything is launched.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/m3ssm.h"
#include "m3_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

m3_status hip_status(hipError_t e) {
  if (e == hipSuccess) return M3_OK;
  g_last_hip_error = static_cast<int>(e);
  return M3_ERR_HIP;
}

m3_status check_dims(const m3_dims* d, bool need_seqlen) {
  if (!d) return M3_ERR_NULL;
  if (d->batch <= 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->rank <= 0)
    return M3_ERR_SHAPE;
  if (need_seqlen && d->seqlen <= 0) return M3_ERR_SHAPE;
  if (d->dstate % 2 != 0) return M3_ERR_SHAPE;
  if (d->chunk < 0) return M3_ERR_SHAPE;
  if (d->in_dtype != M3_F32 && d->in_dtype != M3_BF16) return M3_ERR_DTYPE;
  if (d->out_dtype != M3_F32 && d->out_dtype != M3_BF16) return M3_ERR_DTYPE;
  if (d->flags & ~(M3_THETA_IS_ANGLE | M3_A_PER_TOKEN)) return M3_ERR_SHAPE;
  if (d->ngroups < 0 || d->ngroups > d->nheads) return M3_ERR_SHAPE;
  if (d->ngroups > 0 && d->nheads % d->ngroups != 0) return M3_ERR_SHAPE;
  return M3_OK;
}

int groups_of(const m3_dims* d) { return d->ngroups > 0 ? d->ngroups : d->nheads; }

// the B/C preparation of dims->bc into kernel arguments (off when absent)
m3_status bc_args(const m3_dims* d, m3::BCPrep* out) {
  *out = m3::BCPrep{};
  const m3_bc_prep* bc = d->bc;
  if (!bc) return M3_OK;
  if (!isfinite(bc->eps) || bc->eps < 0.0f) return M3_ERR_SHAPE;
  const void* ptrs[] = {bc->B_weight, bc->C_weight, bc->B_bias, bc->C_bias};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  out->Bw = bc->B_weight;
  out->Cw = bc->C_weight;
  out->Bb = bc->B_bias;
  out->Cb = bc->C_bias;
  out->eps = bc->eps;
  out->rms = bc->rms != 0;
  out->on = 1;
  return M3_OK;
}

// the angle projection of dims->tp into kernel arguments (off when absent)
m3_status tp_args(const m3_dims* d, m3::ThetaProj* out) {
  *out = m3::ThetaProj{};
  const m3_theta_proj* tp = d->tp;
  if (!tp) return M3_OK;
  if (tp->dim <= 0 || tp->dim % 32 != 0) return M3_ERR_SHAPE;
  if (!tp->u || !tp->W) return M3_ERR_NULL;
  if (misaligned(tp->u) || misaligned(tp->W)) return M3_ERR_ALIGN;
  out->u = tp->u;
  out->W = tp->W;
  out->dim = tp->dim;
  out->on = 1;
  return M3_OK;
}

// the backward's chunk length (64 unless the caller asks)
int chunk_of(const m3_dims* d) { return d->chunk > 0 ? d->chunk : 64; }
// a forward prefill's chunk length: the caller's, or the library's default
// for the shape
int prefill_chunk_of(const m3_dims* d) {
  return d->chunk > 0 ? d->chunk
                      : m3::prefill_default_chunk(d->headdim, d->dstate, d->rank,
                                                  d->in_dtype == M3_BF16);
}

// ---------------------------------------------------------------------------
// The scratch buffer of m3_scan_prefill_noalloc: one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host
// stand-in, not device memory, so every host use goes through the device
// address that hipGetSymbolAddress returns for the current device, looked up
// once per device and kept.
static __device__ __align__(256) unsigned char scratch[M3_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // this device's copy of `scratch`, or null until looked up

// the device address of `scratch` on the device of `stream` (the current
// device for the null stream), which must be the current device
hipError_t scratch_of_stream_device(void* stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// m3_scan_prefill with the caller's workspace, or (noalloc) with this
// device's copy of `scratch`
m3_status scan_prefill(const m3_dims* d, const void* x, const void* dt, const float* A,
                       const void* lam, const void* theta, const void* B, const void* C,
                       const float* h0, const void* x_prev, const void* B_prev, void* y,
                       float* hT, void* ws, size_t ws_bytes, bool noalloc, void* stream) {
  m3_status st = check_dims(d, true);
  if (st != M3_OK) return st;
  m3::BCPrep bcp;
  if ((st = bc_args(d, &bcp)) != M3_OK) return st;
  m3::ThetaProj tpa;
  if ((st = tp_args(d, &tpa)) != M3_OK) return st;
  if (!x || !dt || !A || !lam || (!theta && !tpa.on) || !B || !C || !y) return M3_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_NULL;
  const void* ptrs[] = {x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y, hT, ws};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  const int Q = prefill_chunk_of(d);
  const int in_bf16 = d->in_dtype == M3_BF16;
  if (!m3::prefill_supported(d->headdim, d->dstate, d->rank, Q, in_bf16))
    return M3_ERR_UNSUPPORTED;
  const size_t need = m3::prefill_workspace_bytes(d->batch, d->seqlen, d->nheads, d->headdim,
                                                  d->dstate, d->rank, Q, bcp.on != 0);
  if (noalloc) {
    if (need > M3_NOALLOC_SCRATCH_BYTES) return M3_ERR_TOO_LARGE;
    hipError_t e = scratch_of_stream_device(stream, &ws);
    if (e != hipSuccess) return hip_status(e);
    ws_bytes = M3_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < need) return M3_ERR_WORKSPACE;

  m3::PrefillArgs a{};
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.B = B;
  a.C = C;
  a.h0 = h0;
  a.xp = x_prev;
  a.Bp = B_prev;
  a.y = y;
  a.hT = hT;
  a.Bsz = d->batch;
  a.T = d->seqlen;
  a.H = d->nheads;
  a.P = d->headdim;
  a.N = d->dstate;
  a.R = d->rank;
  a.Q = Q;
  a.nchunk = (d->seqlen + Q - 1) / Q;
  a.G = groups_of(d);
  a.flags = d->flags;
  a.has_prev = x_prev != nullptr;
  a.bc = bcp;
  a.tp = tpa;
  m3::prefill_carve(a, ws);
  hipError_t err = hipSuccess;
  if (m3::launch_prefill(a, in_bf16, d->out_dtype == M3_BF16,
                         static_cast<hipStream_t>(stream), &err) != 0)
    return M3_ERR_UNSUPPORTED;
  return hip_status(err);
}


}  // namespace

extern "C" {

const char* m3_status_str(m3_status s) {
  // a C caller may pass any int; read its bits as an int, since a C++ load
  // of an enum value outside the enumerators' range is undefined
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "required pointer is NULL";
    case M3_ERR_SHAPE: return "invalid shape or flags";
    case M3_ERR_DTYPE: return "unsupported dtype";
    case M3_ERR_UNSUPPORTED: return "no kernel for this (headdim, dstate, rank, chunk)";
    case M3_ERR_ALIGN: return "pointer not 16-byte aligned";
    case M3_ERR_WORKSPACE: return "workspace missing or too small";
    case M3_ERR_HIP: return "HIP launch failed";
    case M3_ERR_TOO_LARGE: return "call needs more than the built-in scratch buffer";
  }
  return "unknown status";
}

int m3_last_hip_error(void) { return g_last_hip_error; }

size_t m3_prefill_workspace_size(const m3_dims* d) {
  if (check_dims(d, true) != M3_OK) return 0;
  return m3::prefill_workspace_bytes(d->batch, d->seqlen, d->nheads, d->headdim, d->dstate,
                                     d->rank, prefill_chunk_of(d), d->bc != nullptr);
}

m3_status m3_scan_prefill(const m3_dims* d, const void* x, const void* dt, const float* A,
                          const void* lam, const void* theta, const void* B, const void* C,
                          const float* h0, const void* x_prev, const void* B_prev, void* y,
                          float* hT, void* ws, size_t ws_bytes, void* stream) {
  return scan_prefill(d, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y, hT, ws, ws_bytes,
                      false, stream);
}

m3_status m3_scan_prefill_noalloc(const m3_dims* d, const void* x, const void* dt,
                                  const float* A, const void* lam, const void* theta,
                                  const void* B, const void* C, const float* h0,
                                  const void* x_prev, const void* B_prev, void* y, float* hT,
                                  void* stream) {
  return scan_prefill(d, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y, hT, nullptr, 0, true,
                      stream);
}

size_t m3_prefill_backward_workspace_size(const m3_dims* d) {
  if (check_dims(d, true) != M3_OK) return 0;
  return m3::backward_workspace_bytes(d->batch, d->seqlen, d->nheads, d->headdim, d->dstate,
                                      d->rank, groups_of(d), chunk_of(d));
}

m3_status m3_scan_prefill_backward(const m3_dims* d, const void* x, const void* dt,
                                   const float* A, const void* lam, const void* theta,
                                   const void* B, const void* C, const float* h0,
                                   const void* x_prev, const void* B_prev, const void* dy,
                                   const float* dhT, float* dx, float* ddt, float* dA,
                                   float* dlam, float* dtheta, float* dB, float* dC, float* dh0,
                                   float* dx_prev, float* dB_prev, void* ws, size_t ws_bytes,
                                   void* stream) {
  m3_status st = check_dims(d, true);
  if (st != M3_OK) return st;
  if (d->bc || d->tp) return M3_ERR_UNSUPPORTED;
  if (!x || !dt || !A || !lam || !theta || !B || !C || !dy) return M3_ERR_NULL;
  if (!dx || !ddt || !dA || !dlam || !dtheta || !dB || !dC) return M3_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_NULL;
  const void* ptrs[] = {x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, dy, dhT, dx, ddt, dA,
                        dlam, dtheta, dB, dC, dh0, dx_prev, dB_prev, ws};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  const int Q = chunk_of(d);
  const int in_bf16 = d->in_dtype == M3_BF16;
  if (!m3::prefill_supported(d->headdim, d->dstate, d->rank, Q, in_bf16) ||
      !m3::backward_supported(d->headdim, d->dstate, d->rank, Q))
    return M3_ERR_UNSUPPORTED;
  const size_t need = m3::backward_workspace_bytes(d->batch, d->seqlen, d->nheads, d->headdim,
                                                   d->dstate, d->rank, groups_of(d), Q);
  if (!ws || ws_bytes < need) return M3_ERR_WORKSPACE;

  m3::BackwardArgs g{};
  m3::PrefillArgs& a = g.f;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.B = B;
  a.C = C;
  a.h0 = h0;
  a.xp = x_prev;
  a.Bp = B_prev;
  a.Bsz = d->batch;
  a.T = d->seqlen;
  a.H = d->nheads;
  a.P = d->headdim;
  a.N = d->dstate;
  a.R = d->rank;
  a.Q = Q;
  a.nchunk = (d->seqlen + Q - 1) / Q;
  a.G = groups_of(d);
  a.flags = d->flags;
  a.has_prev = x_prev != nullptr;
  g.dy = dy;
  g.dhT = dhT;
  g.dx = dx;
  g.ddt = ddt;
  g.dA = dA;
  g.dlam = dlam;
  g.dtheta = dtheta;
  g.dB = dB;
  g.dC = dC;
  g.dh0 = dh0;
  g.dx_prev = x_prev ? dx_prev : nullptr;
  g.dB_prev = x_prev ? dB_prev : nullptr;
  m3::backward_carve(g, ws);
  hipError_t err = hipSuccess;
  if (m3::launch_backward(g, in_bf16, d->out_dtype == M3_BF16, static_cast<hipStream_t>(stream),
                          &err) != 0)
    return M3_ERR_UNSUPPORTED;
  return hip_status(err);
}

size_t m3_prefill_varlen_workspace_size(const m3_dims* d) {
  if (check_dims(d, true) != M3_OK) return 0;
  return m3::prefill_varlen_workspace_bytes(d->batch, d->seqlen, d->nheads, d->headdim, d->dstate,
                                            d->rank, prefill_chunk_of(d), d->bc != nullptr);
}

m3_status m3_scan_prefill_varlen(const m3_dims* d, const int32_t* cu_seqlens, const void* x,
                                 const void* dt, const float* A, const void* lam,
                                 const void* theta, const void* B, const void* C,
                                 const float* h0, const void* x_prev, const void* B_prev, void* y,
                                 float* hT, void* ws, size_t ws_bytes, void* stream) {
  m3_status st = check_dims(d, true);
  if (st != M3_OK) return st;
  m3::BCPrep bcp;
  if ((st = bc_args(d, &bcp)) != M3_OK) return st;
  m3::ThetaProj tpa;
  if ((st = tp_args(d, &tpa)) != M3_OK) return st;
  if (!cu_seqlens || !x || !dt || !A || !lam || (!theta && !tpa.on) || !B || !C || !y)
    return M3_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_NULL;
  const void* ptrs[] = {x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y, hT, ws};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return M3_ERR_ALIGN;
  const int Q = prefill_chunk_of(d);
  const int in_bf16 = d->in_dtype == M3_BF16;
  if (!m3::prefill_supported(d->headdim, d->dstate, d->rank, Q, in_bf16) ||
      !m3::prefill_offsets_fit(d->nheads, d->headdim, d->dstate, d->rank, Q))
    return M3_ERR_UNSUPPORTED;
  const size_t need = m3::prefill_varlen_workspace_bytes(d->batch, d->seqlen, d->nheads,
                                                         d->headdim, d->dstate, d->rank, Q,
                                                         bcp.on != 0);
  if (!ws || ws_bytes < need) return M3_ERR_WORKSPACE;

  m3::PrefillArgs a{};
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.B = B;
  a.C = C;
  a.h0 = h0;
  a.xp = x_prev;
  a.Bp = B_prev;
  a.y = y;
  a.hT = hT;
  a.Bsz = d->batch;
  a.T = d->seqlen;
  a.H = d->nheads;
  a.P = d->headdim;
  a.N = d->dstate;
  a.R = d->rank;
  a.Q = Q;
  a.nchunk = static_cast<int>(m3::varlen_slots(d->batch, d->seqlen, Q));
  a.G = groups_of(d);
  a.flags = d->flags;
  a.has_prev = x_prev != nullptr;
  a.bc = bcp;
  a.tp = tpa;
  m3::prefill_varlen_carve(a, ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = m3::launch_varlen_map(a, cu_seqlens, s);
  if (err != hipSuccess) return hip_status(err);
  if (m3::launch_prefill(a, in_bf16, d->out_dtype == M3_BF16, s, &err) != 0)
    return M3_ERR_UNSUPPORTED;
  return hip_status(err);
}

m3_status m3_decode_step(const m3_dims* d, float* h, const void* x_t, const void* x_prev,
                         const void* B_t, const void* B_prev, const void* C_t, const void* dt_t,
                         const float* A, const void* lam_t, const void* theta_t, void* y_t,
                         void* stream) {
  m3_status st = check_dims(d, false);
  if (st != M3_OK) return st;
  m3::BCPrep bcp;
  if ((st = bc_args(d, &bcp)) != M3_OK) return st;
  m3::ThetaProj tpa;
  if ((st = tp_args(d, &tpa)) != M3_OK) return st;
  if (!h || !x_t || !B_t || !C_t || !dt_t || !A || !lam_t || (!theta_t && !tpa.on) || !y_t)
    return M3_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_NULL;
  const void* ptrs[] = {h, x_t, x_prev, B_t, B_prev, C_t, dt_t, A, lam_t, theta_t, y_t};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  if (!m3::decode_supported(d->headdim, d->dstate, d->rank)) return M3_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(d->batch) * d->nheads;
  if (units > 0x7fffffff) return M3_ERR_SHAPE;

  m3::DecodeArgs a{};
  a.h = h;
  a.x = x_t;
  a.xp = x_prev;
  a.Bt = B_t;
  a.Bp = B_prev;
  a.Ct = C_t;
  a.dt = dt_t;
  a.A = A;
  a.lam = lam_t;
  a.theta = theta_t;
  a.y = y_t;
  a.H = d->nheads;
  a.P = d->headdim;
  a.N = d->dstate;
  a.R = d->rank;
  a.G = groups_of(d);
  a.K = 1;
  a.flags = d->flags;
  a.has_prev = x_prev != nullptr;
  a.bc = bcp;
  a.tp = tpa;
  hipError_t err = hipSuccess;
  if (m3::launch_decode(a, d->in_dtype == M3_BF16, d->out_dtype == M3_BF16,
                        static_cast<int>(units), static_cast<hipStream_t>(stream), &err) != 0)
    return M3_ERR_UNSUPPORTED;
  return hip_status(err);
}

m3_status m3_decode_tokens(const m3_dims* d, float* h, const void* x, const void* x_prev,
                           const void* B, const void* B_prev, const void* C, const void* dt,
                           const float* A, const void* lam, const void* theta, void* y,
                           void* stream) {
  m3_status st = check_dims(d, true);
  if (st != M3_OK) return st;
  m3::BCPrep bcp;
  if ((st = bc_args(d, &bcp)) != M3_OK) return st;
  if (d->tp) return M3_ERR_UNSUPPORTED;
  if (!h || !x || !B || !C || !dt || !A || !lam || !theta || !y) return M3_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_NULL;
  const void* ptrs[] = {h, x, x_prev, B, B_prev, C, dt, A, lam, theta, y};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return M3_ERR_ALIGN;
  if (!m3::decode_tokens_supported(d->headdim, d->dstate, d->rank)) return M3_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(d->batch) * d->nheads;
  if (units > 0x7fffffff) return M3_ERR_SHAPE;

  m3::DecodeArgs a{};
  a.h = h;
  a.x = x;
  a.xp = x_prev;
  a.Bt = B;
  a.Bp = B_prev;
  a.Ct = C;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.y = y;
  a.H = d->nheads;
  a.P = d->headdim;
  a.N = d->dstate;
  a.R = d->rank;
  a.G = groups_of(d);
  a.K = d->seqlen;
  a.flags = d->flags;
  a.has_prev = x_prev != nullptr;
  a.bc = bcp;
  hipError_t err = hipSuccess;
  if (m3::launch_decode_tokens(a, d->in_dtype == M3_BF16, d->out_dtype == M3_BF16,
                               static_cast<int>(units), static_cast<hipStream_t>(stream), &err) != 0)
    return M3_ERR_UNSUPPORTED;
  return hip_status(err);
}

}  // extern "C"
