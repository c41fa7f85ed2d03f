/*
 * m3ssm.h -- C ABI of libm3ssm: the Mamba-3 SSM core recurrence on gfx950.
 *
 * The library computes, for every (batch, head) pair independently, the
 * exponential-trapezoidal three-term update
 *
 *     h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t,
 *     alpha_t = exp(dt_t A_t), beta_t = (1 - lam_t) dt_t alpha_t,
 *     gamma_t = lam_t dt_t
 *
 * [xxxxx.co.kr Mamba-3 article ("2배 작은 상태 크기와 향상된 MIMO 디코딩 하드웨어
 * 효율..."), section 1.1, the h_t equation], with the complex-valued state
 * of section 1.2 of the same article (pairs of state columns (2k, 2k+1) form
 * one complex number whose transition has modulus alpha_t and phase
 * phi_{t,k} = dt_t theta_{t,k}; the decayed state and the beta term carry the
 * phase, the gamma term does not; computed in the "RoPE" frame, where B and
 * C are rotated by minus the cumulative phase), and the MIMO rank-R form of
 * section 1.3 (x_t is P x R, B_t and C_t are N x R, the output is P x R).
 * The output of a token is y_t = h_t C_t (a real dot product over N).
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer, owned by the caller, dense
 *    and row-major (last index fastest), 16-byte aligned.
 *  - The library never allocates, frees or synchronises (the one buffer it
 *    holds, that of m3_scan_prefill_noalloc, is static device memory that
 *    comes with the loaded code).  Work is queued on
 *    `stream` (a hipStream_t passed as void*; NULL = the default stream) and
 *    the call returns at once.  Argument checks run on the host before any
 *    launch; a failed check returns its status and launches nothing.
 *  - ngroups outside [0, nheads] or not dividing nheads is M3_ERR_SHAPE.
 *  - Launch failures return M3_ERR_HIP (m3_last_hip_error() gives the HIP
 *    code).  Faults inside a kernel surface at the caller's next
 *    synchronisation.  NaN/Inf inputs propagate; they are not checked.
 *  - Calls are stateless and re-entrant; concurrent calls on different
 *    streams must not share output or workspace buffers.
 *
 * Layouts (Bsz = batch, T = seqlen, H = nheads, P = headdim, N = dstate,
 * R = rank, G = ngroups or H when ngroups is 0):
 *     x, y           [Bsz, T, H, P, R]      in_dtype / out_dtype
 *     B, C           [Bsz, T, G, N, R]      in_dtype
 *     dt, lam        [Bsz, T, H]            in_dtype (already activated)
 *     theta          [Bsz, T, G, N/2]       in_dtype (one angle per pair)
 *     A              [H] fp32, or [Bsz, T, H] fp32 with M3_A_PER_TOKEN
 *     h0, hT, h      [Bsz, H, P, N]         fp32
 *     x_prev         [Bsz, H, P, R]         in_dtype
 *     B_prev         [Bsz, G, N, R]         in_dtype
 * Head h reads B, C and theta of group h / (H / G): the groups of heads
 * that share one B, C and phase projection (G = H: one per head).
 * The decode step drops the T axis.  With R = 1 the trailing axis has size 1.
 */
#ifndef M3SSM_H
#define M3SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  M3_OK = 0,
  M3_ERR_NULL = 1,        /* a required pointer is NULL                    */
  M3_ERR_SHAPE = 2,       /* a size is <= 0, N is odd, ...                 */
  M3_ERR_DTYPE = 3,       /* in_dtype / out_dtype not one of m3_dtype      */
  M3_ERR_UNSUPPORTED = 4, /* valid, but no kernel for this (P, N, R, Q)    */
  M3_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned              */
  M3_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required       */
  M3_ERR_HIP = 7,         /* a HIP launch failed                           */
  M3_ERR_TOO_LARGE = 8    /* m3_scan_prefill_noalloc: the call needs more
                             than M3_NOALLOC_SCRATCH_BYTES of workspace    */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

/* flags */
#define M3_THETA_IS_ANGLE (1u << 0) /* phase phi_t = theta_t, not dt_t*theta_t */
#define M3_A_PER_TOKEN (1u << 1)    /* A is [Bsz,T,H] fp32 instead of [H]      */

/* Optional preparation of B and C inside the kernels [the same article,
 * section 2: B and C are RMS-normalised, as attention normalises Q and K,
 * and get a learned bias per head and channel].  With dims->bc set, every
 * call reads B_t, C_t and B_prev as the raw projections and uses, for head
 * h of group g and rank column r,
 *     B'[n][r] = B_weight[n] * B[g][n][r] / rms_r + B_bias[h][n][r],
 *     rms_r    = sqrt(mean over n of B[g][n][r]^2 + eps)   (rms != 0; else 1)
 * and the same for C, before the phase rotation.  Readings: the
 * normalisation runs over the N channels of each rank column; the weight is
 * per channel, shared by heads and ranks; the bias is per head, so heads
 * that share a group's B and C differ after it.  All four arrays are
 * optional DEVICE pointers (NULL: weight 1, bias 0), 16-byte aligned.  A
 * raw column of zeros with eps = 0 gives NaN.  eps must be finite and >= 0
 * (else M3_ERR_SHAPE). */
typedef struct {
  const float* B_weight; /* [N] fp32 or NULL                               */
  const float* C_weight; /* [N] fp32 or NULL                               */
  const float* B_bias;   /* [H, N, R] fp32 or NULL                         */
  const float* C_bias;   /* [H, N, R] fp32 or NULL                         */
  float eps;             /* added to the mean square                       */
  int32_t rms;           /* nonzero: RMS-normalise over N                  */
} m3_bc_prep;

/* Optional angle projection inside the kernels [the same article, section
 * 1.2: the rotation angles are data-dependent, a projection of the layer's
 * input like B and C].  With dims->tp set, the theta argument is not read
 * (it may be NULL) and every call uses, for token row i and head group g,
 *     theta[i][g][k] = sum_j W[g][k][j] * u[i][j],   k < N/2, j < dim,
 * in fp32 (bf16 products are exact), then interprets theta as usual (a rate
 * multiplied by dt_t, or the angle itself with M3_THETA_IS_ANGLE).  Reading:
 * one linear map per head group, no bias, no activation.  u has the token
 * layout of the call without the head axis: [Bsz, T, dim] (prefill),
 * [T, dim] (packed prefill), [Bsz, dim] (decode step); W is [G, N/2, dim].
 * Both are DEVICE pointers in in_dtype, 16-byte aligned; dim must be a
 * positive multiple of 32 (else M3_ERR_SHAPE).  Supported by
 * m3_scan_prefill, m3_scan_prefill_noalloc, m3_scan_prefill_varlen and
 * m3_decode_step; m3_decode_tokens and m3_scan_prefill_backward return
 * M3_ERR_UNSUPPORTED. */
typedef struct {
  const void* u;   /* token rows of the projection's input                 */
  const void* W;   /* [G, N/2, dim]                                        */
  int32_t dim;     /* projection width                                     */
} m3_theta_proj;

typedef struct {
  int32_t batch;     /* Bsz >= 1                                           */
  int32_t seqlen;    /* T >= 1 (ignored by the decode step)                */
  int32_t nheads;    /* H >= 1                                             */
  int32_t headdim;   /* P                                                  */
  int32_t dstate;    /* N, even                                            */
  int32_t rank;      /* R >= 1; 1 = single input / single output           */
  int32_t chunk;     /* prefill chunk length Q; 0 = library default        */
  int32_t in_dtype;  /* m3_dtype of x, B, C, dt, lam, theta, x_prev, B_prev */
  int32_t out_dtype; /* m3_dtype of y                                      */
  uint32_t flags;    /* M3_THETA_IS_ANGLE | M3_A_PER_TOKEN                 */
  int32_t ngroups;   /* G, groups sharing B, C, theta; 0 = nheads; G | H   */
  const m3_bc_prep* bc; /* host pointer; NULL = B and C are used as given */
  const m3_theta_proj* tp; /* host pointer; NULL = theta is read as given */
} m3_dims;

/* Bytes of device workspace m3_scan_prefill needs for `dims` (0 if dims is
 * invalid).  The workspace holds per-chunk end states and per-chunk decay
 * and phase totals; its contents on entry do not matter. */
size_t m3_prefill_workspace_size(const m3_dims* dims);

/* Chunked prefill scan over T tokens [the same article, sections 1.1-1.3;
 * the pages name prefill kernels without giving their algorithm, and this
 * one is the exact chunked evaluation of the recurrence]:
 *   y  <- outputs y_t for t = 0..T-1
 *   hT <- state after the last token (not written when NULL)
 * h0 NULL means a zero initial state.  x_prev/B_prev give the token before
 * t = 0 for the beta term of the first step (both NULL = zero); passing the
 * previous call's last x and B makes a split scan equal the whole scan.
 * h0 may alias hT; no other argument may alias an output.  A NaN or Inf in
 * one token's inputs stays in its (batch, head) and in its chunk and later
 * chunks, but may also reach the outputs of the earlier tokens of its own
 * chunk (masked products multiply it by zero).
 * Precision: fp32 inputs run their chunk contractions on fp32 matrix-core
 * operands.  bf16 inputs run them on bf16 hi + lo splits of every operand
 * computed in fp32 (rotated B and C, masked Gram tiles, chunk states; about
 * 2^-17 relative each; x is exact as one bf16 part).  bf16 keeps fp32's
 * exponent range, so there is no range limit beyond fp32's own.
 * Chunk length: dims->chunk = 0 takes 128 for a single input and 64
 * otherwise; 64 and, at R = 1, 128 may be asked for (else
 * M3_ERR_UNSUPPORTED).  It changes only the summation order.
 * ws must be at least m3_prefill_workspace_size(dims) bytes. */
m3_status m3_scan_prefill(const m3_dims* dims, const void* x, const void* dt,
                          const float* A, const void* lam, const void* theta,
                          const void* B, const void* C, const float* h0,
                          const void* x_prev, const void* B_prev, void* y,
                          float* hT, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): m3_scan_prefill without the ws/ws_bytes arguments.  Its
 * workspace is a buffer inside the library, M3_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held by each GPU the library runs on until the process
 * ends; the call itself allocates nothing.  A call whose
 * m3_prefill_workspace_size(dims) is larger returns M3_ERR_TOO_LARGE and
 * launches nothing (at P = 64, N = 128: about 2000 chunk-heads, e.g.
 * Bsz * H * ceil(T / Q) <= 2000).  Every call on one GPU uses that GPU's one
 * buffer, which keeps the last call's contents (the prefill workspace needs
 * no particular contents on entry): calls that overlap in time on one GPU,
 * on different streams or from different threads, race and give wrong
 * results; calls queued on one stream do not overlap.  `stream` must
 * belong to the current device (else M3_ERR_HIP).  The first call on a
 * device looks up that device's copy of the buffer (hipGetSymbolAddress),
 * so a caller that captures graphs makes one call on each device before
 * capturing.  Results are bit-identical to m3_scan_prefill with the same
 * arguments. */
#define M3_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
m3_status m3_scan_prefill_noalloc(const m3_dims* dims, const void* x, const void* dt,
                                  const float* A, const void* lam, const void* theta,
                                  const void* B, const void* C, const float* h0,
                                  const void* x_prev, const void* B_prev, void* y,
                                  float* hT, void* stream);

/* Bytes of device workspace m3_scan_prefill_backward needs for `dims` (0
 * if dims is invalid). */
size_t m3_prefill_backward_workspace_size(const m3_dims* dims);

/* Gradients of the prefill scan [the recurrence of the same article,
 * sections 1.1-1.3, differentiated; the pages do not describe a backward
 * pass]: for the loss L = <y, dy> + <hT, dhT> (dhT NULL = 0) over the
 * outputs of m3_scan_prefill with the same inputs, writes dL/d of each
 * input, all fp32 in the layout of that input:
 *   dx [Bsz,T,H,P,R], ddt and dlam [Bsz,T,H], dA [H] (or [Bsz,T,H] with
 *   M3_A_PER_TOKEN), dtheta [Bsz,T,G,N/2], dB and dC [Bsz,T,G,N,R],
 *   dh0 [Bsz,H,P,N] (NULL: not written), dx_prev [Bsz,H,P,R] and dB_prev
 *   [Bsz,G,N,R] (written when x_prev/B_prev are given and the pointers are
 *   not NULL).
 * dy has out_dtype and the layout of y.  dA and, with head groups, dB, dC,
 * dtheta and dB_prev are sums over heads (and tokens), taken in a fixed
 * order in ws (no atomics), so equal calls return equal bits.  The forward
 * chunk states are recomputed into ws.  Supported: Q = 64 and (P, N, R) in
 * (16, 16, 1), (64, 128, 1 | 2 | 4), (32, 64, 1 | 4), (64, 64, 1 | 4), the
 * shapes of m3_scan_prefill; dims->bc must be NULL; otherwise
 * M3_ERR_UNSUPPORTED. */
m3_status m3_scan_prefill_backward(const m3_dims* dims, const void* x, const void* dt,
                                   const float* A, const void* lam, const void* theta,
                                   const void* B, const void* C, const float* h0,
                                   const void* x_prev, const void* B_prev, const void* dy,
                                   const float* dhT, float* dx, float* ddt, float* dA,
                                   float* dlam, float* dtheta, float* dB, float* dC,
                                   float* dh0, float* dx_prev, float* dB_prev, void* ws,
                                   size_t ws_bytes, void* stream);

/* Bytes of device workspace m3_scan_prefill_varlen needs for `dims`
 * (dims->batch = number of sequences S, dims->seqlen = total tokens T); 0
 * if dims is invalid.  Besides the per-chunk totals it holds two small
 * tables built from cu_seqlens on every call. */
size_t m3_prefill_varlen_workspace_size(const m3_dims* dims);

/* Chunked prefill of S = dims->batch independent sequences packed back to
 * back into T = dims->seqlen token rows [the recurrence of the same
 * article, sections 1.1-1.3, run separately for each sequence; packing is a
 * serving layout that the pages do not describe].  cu_seqlens is a DEVICE
 * array of S + 1 int32 offsets, 4-byte aligned: sequence s is rows
 * [cu_seqlens[s], cu_seqlens[s+1]).  Layouts are those of m3_scan_prefill
 * with Bsz = 1 for the token rows and Bsz = S for the per-sequence arrays:
 *     x, y           [T, H, P, R]       B, C     [T, G, N, R]
 *     dt, lam        [T, H]             theta    [T, G, N/2]
 *     A              [H] fp32, or [T, H] fp32 with M3_A_PER_TOKEN
 *     h0, hT         [S, H, P, N] fp32  x_prev   [S, H, P, R]
 *     B_prev         [S, G, N, R]
 * Each sequence starts from its own h0 row (NULL = zero) and token before
 * (x_prev/B_prev rows; NULL = zero) and ends in its own hT row, so the
 * result equals one m3_scan_prefill per sequence.  A sequence may be empty
 * (its hT row is then its h0 row).  The offsets are meant to rise from
 * cu_seqlens[0] = 0 to cu_seqlens[S] = T; they cannot be checked on the
 * host, so the kernels clamp each one into [0, T] and raise it to the
 * largest offset before it: no access leaves the buffers whatever the array
 * holds, and y rows that no sequence covers are left unwritten.  The rest
 * of m3_scan_prefill's contract applies; ws must be at least
 * m3_prefill_varlen_workspace_size(dims) bytes. */
m3_status m3_scan_prefill_varlen(const m3_dims* dims, const int32_t* cu_seqlens,
                                 const void* x, const void* dt, const float* A,
                                 const void* lam, const void* theta, const void* B,
                                 const void* C, const float* h0, const void* x_prev,
                                 const void* B_prev, void* y, float* hT, void* ws,
                                 size_t ws_bytes, void* stream);

/* One decode step [the same article, sections 1.1-1.3]: the state h
 * [Bsz,H,P,N] fp32 is advanced in place by the token (x_t, B_t, C_t, dt_t,
 * lam_t, theta_t), with (x_prev, B_prev) the token before it (both NULL =
 * zero), and y_t [Bsz,H,P,R] receives h_t C_t.  dims->seqlen is ignored;
 * A is [H] (or [Bsz,H] with M3_A_PER_TOKEN).  h is read once and written
 * once. */
m3_status m3_decode_step(const m3_dims* dims, float* h, const void* x_t,
                         const void* x_prev, const void* B_t,
                         const void* B_prev, const void* C_t, const void* dt_t,
                         const float* A, const void* lam_t,
                         const void* theta_t, void* y_t, void* stream);

/* K = dims->seqlen consecutive decode steps in one call [the same article,
 * sections 1.1-1.3; the recurrence applied token after token]: the state h
 * [Bsz,H,P,N] fp32 is advanced in place by the K tokens and y receives y_k
 * for each of them.  The inputs use the prefill layouts with T = K: x, y
 * [Bsz,K,H,P,R]; B, C [Bsz,K,G,N,R]; dt, lam [Bsz,K,H]; theta [Bsz,K,G,N/2];
 * A [H] (or [Bsz,K,H] with M3_A_PER_TOKEN); x_prev [Bsz,H,P,R] and B_prev
 * [Bsz,G,N,R] are the token before the first (both NULL = zero).  The
 * result equals K calls of m3_decode_step up to the order of fp32 sums (at
 * R = 4 the tokens are applied four at a time in the prefill's chunked
 * form), and h crosses HBM once in and once out.  Supported: R = 1 with N in {16, 32, 64, 128, 256}, or R in
 * {2, 3, 4, 8} with P a multiple of 16 up to 64 and N in {16, 32, 64, 128};
 * otherwise M3_ERR_UNSUPPORTED. */
m3_status m3_decode_tokens(const m3_dims* dims, float* h, const void* x,
                           const void* x_prev, const void* B,
                           const void* B_prev, const void* C, const void* dt,
                           const float* A, const void* lam, const void* theta,
                           void* y, void* stream);

/* Static, human-readable name of a status. */
const char* m3_status_str(m3_status status);

/* The HIP error code of the last M3_ERR_HIP returned on this thread (0 if
 * none). */
int m3_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* M3SSM_H */
