// m3_launch.h -- host-side launch interface between the C ABI layer and the
// kernels of libm3ssm.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

constexpr uint32_t kThetaIsAngle = 1u << 0;
constexpr uint32_t kAPerToken = 1u << 1;

// the preparation of B and C applied inside the kernels when `on`:
// B' = Bw[n] * B / rms + Bb[h][n][r], rms over the N channels of a rank
// column (1 when !rms); the same for C
struct BCPrep {
  const float* Bw;   // [N] or null (1)
  const float* Cw;
  const float* Bb;   // [H, N, R] or null (0)
  const float* Cb;
  float eps;
  int rms;
  int on;
};

// the angle projection applied inside the kernels when `on`:
// theta[.., g, k] = sum_j W[g][k][j] u[.., j] (u and W in the input dtype)
struct ThetaProj {
  const void* u;   // [tokens, D]
  const void* W;   // [G, N/2, D]
  int dim;         // D, a multiple of 32
  int on;
};

struct DecodeArgs {
  float* h;
  const void* x;
  const void* xp;
  const void* Bt;
  const void* Bp;
  const void* Ct;
  const void* dt;
  const float* A;
  const void* lam;
  const void* theta;
  void* y;
  int H, P, N, R;
  int G;           // groups sharing B, C and theta (G divides H)
  int K;           // tokens of a multi-token call (1 for a single step)
  uint32_t flags;
  int has_prev;
  BCPrep bc;
  ThetaProj tp;
};

bool decode_supported(int P, int N, int R);
bool decode_tokens_supported(int P, int N, int R);
// several tokens per launch, the state kept on chip between them
int launch_decode_tokens(const DecodeArgs& a, int in_bf16, int out_bf16, int units,
                         hipStream_t s, hipError_t* err);
// returns 0 when launched (err = hipGetLastError), -1 when no kernel fits
int launch_decode(const DecodeArgs& a, int in_bf16, int out_bf16, int units,
                  hipStream_t s, hipError_t* err);

struct PrefillArgs {
  const void* x;
  const void* dt;
  const float* A;
  const void* lam;
  const void* theta;
  const void* B;
  const void* C;
  const float* h0;
  const void* xp;
  const void* Bp;
  void* y;
  float* hT;
  // workspace carve-up
  float* S;        // [Bsz, H, nchunk, P, N]: chunk end states, then chunk entry states
  float* rot_end;  // [Bsz, H, nchunk, N/2, 2]: cos/sin of each chunk's total phase
  float* decay;    // [Bsz, H, nchunk]: exp of each chunk's total log-decay
  // packed sequences (null for [Bsz, T] inputs): the token rows are one
  // [T, ...] array holding Bsz sequences back to back; nchunk is then the
  // number of chunk slots per head, and the two tables are built on the
  // device from the caller's sequence offsets
  int4* seqs;      // [Bsz]: {first slot, chunks, first token, length}
  int4* cmap;      // [nchunk]: {sequence, first token, end token, chunk}, sequence -1 = unused
  int Bsz, T, H, P, N, R, Q, nchunk;
  int G;           // groups sharing B, C and theta (G divides H)
  uint32_t flags;
  int has_prev;
  BCPrep bc;
  ThetaProj tp;
  float* rsB;      // with bc.on: [units, Q, R] inverse RMS of the chunk's B rows
  int states_only; // stop after the chunk entry states (and h_T): no outputs
};

bool prefill_supported(int P, int N, int R, int Q, int in_bf16);
// the chunk length a prefill call with dims->chunk = 0 takes
constexpr int kPrefillChunkR1 = 128;
int prefill_default_chunk(int P, int N, int R, int in_bf16);
bool prefill_offsets_fit(int H, int P, int N, int R, int Q);
size_t prefill_workspace_bytes(int Bsz, int T, int H, int P, int N, int R, int Q, bool prep);
// carve-ups read a.bc.on, so set it first
void prefill_carve(PrefillArgs& a, void* ws);
// packed sequences: chunk slots per head (an upper bound of the chunk count
// for any split of T tokens into Bsz sequences), workspace and carve-up
int64_t varlen_slots(int Bsz, int T, int Q);
size_t prefill_varlen_workspace_bytes(int Bsz, int T, int H, int P, int N, int R, int Q, bool prep);
void prefill_varlen_carve(PrefillArgs& a, void* ws);
// gradients of the dense prefill (single input): the chunk entry states are
// recomputed into the workspace first
struct BackwardArgs {
  PrefillArgs f;      // forward inputs; workspace carved for the chunk states
  const void* dy;     // [Bsz, T, H, P, R], out dtype
  const float* dhT;   // [Bsz, H, P, N] or null
  float* dS;          // workspace [units, P, N]: chunk adjoints, then dL/dShat_c
  float* hTw;         // workspace [Bsz, H, P, N]: the forward's final state
  float *dx, *ddt, *dA, *dlam, *dtheta, *dB, *dC, *dh0, *dx_prev, *dB_prev;
  // workspace: per-chunk dA partials; with head groups, per-head gradients
  // of B, C, theta and B_prev before the fixed-order sum over each group
  float *dApart, *dBh, *dCh, *dthh, *dBph;
  // workspace of the matrix-core kernels: per-chunk token sums
  // [units, kBwdTokSums, Q], phase gradients [units, Q, N/2] and each state
  // pass wave's part of the end-state sums [units, P N / 256, N/2 + 2]
  float *tokw, *dphiB, *endp;
};
constexpr int kBwdTokSums = 7;
bool backward_supported(int P, int N, int R, int Q);
size_t backward_workspace_bytes(int Bsz, int T, int H, int P, int N, int R, int G, int Q);
void backward_carve(BackwardArgs& a, void* ws);
int launch_backward(const BackwardArgs& a, int in_bf16, int dy_bf16, hipStream_t s, hipError_t* e);
// the chunk kernels of the rank-R backward on matrix cores (after the
// forward states): 0 when launched (*e = the launch status), -1 when the
// shape has no such kernels
int launch_backward_mma(const BackwardArgs& a, int in_bf16, int dy_bf16, hipStream_t s, hipError_t* e);
// the reverse pass over chunks turning chunk adjoints into dL/dShat_c (and
// dh0); with a.endp also the end-state sums of every chunk
hipError_t launch_bwd_state_pass(const BackwardArgs& a, int in_bf16, hipStream_t s);

// builds seqs and cmap from the sequence offsets cu [Bsz + 1] (device)
hipError_t launch_varlen_map(const PrefillArgs& a, const int32_t* cu, hipStream_t s);
// returns 0 when launched (err = first launch error), -1 when no kernel fits
int launch_prefill(const PrefillArgs& a, int in_bf16, int out_bf16,
                   hipStream_t s, hipError_t* err);

}  // namespace m3
