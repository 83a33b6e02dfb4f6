/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Two forward operations of selective state-space models, each one call that
 * enqueues hand-written HIP kernels on the caller's stream:
 *
 *   ssm_selective_scan_fwd  -- the S6 selective scan (Mamba-1 layer scan)
 *   ssm_ssd_chunk_fwd       -- the scalar-decay-per-head SSD form (Mamba-2)
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major
 *     and contiguous in the stated shape (last axis fastest).  The library
 *     never allocates, frees or retains them; scratch space is the caller's
 *     `workspace` whose size comes from the matching *_workspace_bytes query.
 *   - Large operands (u, delta, z, y, B, C, X, Y) must be 16-byte aligned;
 *     fp32 parameter vectors 4-byte aligned.  Outputs must not overlap inputs.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls return as
 *     soon as the kernels are enqueued; they never synchronise.  They keep no
 *     state between calls and may be issued concurrently on different streams
 *     with different workspaces.
 *   - Arithmetic is fp32 throughout (state, accumulation, discretisation);
 *     storage dtype `dtype` applies to the activation tensors (see each call).
 *     bf16 outputs are rounded to nearest even from fp32.
 *   - Validation happens on the host before any HIP call: a nonzero status is
 *     returned and nothing is launched.  A failed launch returns
 *     SSM_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - L = 0 is valid: nothing is written to y, and h_last (if given) receives
 *     h0 (or zeros).
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 1

/* storage dtype of the activation tensors */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* status codes */
enum {
    SSM_OK = 0,
    SSM_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    SSM_ERR_BAD_SHAPE = 2,     /* a size is negative/zero where it must not be, or overflows */
    SSM_ERR_BAD_DTYPE = 3,     /* dtype is not an ssm_dtype */
    SSM_ERR_UNSUPPORTED = 4,   /* valid request outside what the kernels implement */
    SSM_ERR_MISALIGNED = 5,    /* a pointer violates the alignment rule above */
    SSM_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than the query returned */
    SSM_ERR_HIP = 7            /* a HIP call or kernel launch failed */
};

/* flags */
#define SSM_FLAG_DELTA_SOFTPLUS 1u  /* delta <- softplus(delta + delta_bias) */
#define SSM_FLAG_ZOH            2u  /* exact zero-order-hold input term instead of delta*B */

int ssm_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* ssm_status_string(int status);

/*
 * ---------------------------------------------------------------- S6 scan
 * The selective scan, per batch row b and channel d, with an N-wide state h
 * carried over tokens t (the per-token discretisation and readout of the
 * "Discretization becomes a per-token operation" section of the
 * Transformer-math "Selective state space" article; the gate of section 4 of
 * the temporalbook "Selective State-Space Models (Mamba)" chapter):
 *
 *   dt     = softplus(delta[b,t,d] + delta_bias[d])   (flag set; else delta + bias)
 *   h[n]   = exp(dt * A[d,n]) * h[n] + dt * B[b,t,n] * u[b,t,d]
 *            (with SSM_FLAG_ZOH the input term is (exp(dt*A)-1)/A * B * u)
 *   y      = sum_n C[b,t,n] * h[n]  + Dskip[d] * u[b,t,d]
 *   y[b,t,d] = y * silu(z[b,t,d])                       (if z given)
 *
 * Arguments (shapes in elements):
 *   u, delta, z, y : [B, L, D]  dtype     (z may be NULL)
 *   A              : [D, N]     fp32      continuous-time diagonal, normally -exp(A_log)
 *   Bm, Cm         : [B, L, N]  dtype     shared by all D channels of row b
 *   Dskip, delta_bias : [D]     fp32 or NULL
 *   h0             : [B, D, N]  fp32 or NULL (zeros)
 *   h_last         : [B, D, N]  fp32 or NULL; receives the state after t = L-1
 *   1 <= N <= 64; B, D >= 1; L >= 0.
 * Two execution paths, chosen from the sizes:
 *   - state per lane (N = 16, D a multiple of 16, no ZOH; see
 *     ssm_selective_scan_lanes): one lane per (channel, state).  With at least
 *     two of its B*D/4 wavefronts per SIMD the whole sequence is one pass.
 *     With fewer the sequence is cut into segments of whole 128-token tiles,
 *     scanned in parallel (each after the first from a zero state); their
 *     (decay, end state) pairs are folded in segment order into each
 *     segment's incoming state and h_last, and a third launch adds to y the
 *     part of the incoming state that survives to each token,
 *     exp(A * cumsum dt) * h_in, in parallel over 1024-token chunks that
 *     start from the running sums of dt the scan stored, each stopping once
 *     that part is exactly zero in fp32 (with softplus, where dt >= 0).  No
 *     exponential is evaluated twice except in that fix-up's reach.  (Shapes
 *     whose fix-up would need 2^24 workgroups or more take the split path.)
 *   - split: one lane per channel (other N, ZOH, D not a multiple of 16, or
 *     the state-per-lane kernel turned off); long sequences are split into
 *     short segments whose (decay, offset) pairs are carried the same way,
 *     then every segment is rescanned from its incoming state.
 * The workspace holds the segment pairs, and on the state-per-lane path one
 * fp32 sum of dt per (segment, 1024-token chunk, batch row, channel); the
 * query returns the larger of the two paths' needs (it takes no flags, and
 * ZOH calls take the split path).
 * The plan (path, segment count, workspace size) is a pure function of the
 * sizes: it balances wavefronts over the 1024 SIMDs of an MI355X and makes no
 * HIP call.
 */
size_t ssm_selective_scan_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                          int dtype);

/* Number of sequence segments a forward call without SSM_FLAG_ZOH uses at
 * these sizes, on the path it takes (1 = one pass, no carry); 0 for invalid
 * sizes.  The environment variable SSM_S6_SEGMENTS (1..256) overrides the
 * choice, for both this query and the call (on the state-per-lane path
 * capped at one segment per 128 tokens). */
int ssm_selective_scan_segments(int64_t B, int64_t L, int64_t D, int64_t N);

/* 1 if a forward call at these sizes without SSM_FLAG_ZOH (with or without
 * the fused convolution) runs the state-per-lane kernel, else 0 (also for
 * invalid sizes).  The environment variable SSM_S6_LANES=0 turns that kernel
 * off, for both this query and the call. */
int ssm_selective_scan_lanes(int64_t B, int64_t L, int64_t D, int64_t N);

int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A,
                           const void* Bm, const void* Cm, const float* Dskip,
                           const void* z, const float* delta_bias, unsigned flags,
                           const float* h0, void* y, float* h_last,
                           int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * operation of ssm_selective_scan_fwd with no workspace argument.  Where the
 * plan needs scratch (the split path's segment pairs), it comes from a static
 * device array inside the library, SSM_NOALLOC_SCRATCH_BYTES on each GPU,
 * which the runtime sets up when it loads the library's code on that device
 * and holds until the process ends; the call itself allocates nothing (no
 * hipMalloc, no allocating library routine).  Sizes whose workspace query
 * exceeds SSM_NOALLOC_SCRATCH_BYTES return SSM_ERR_WORKSPACE before any HIP
 * call.  All calls on one GPU share that array and leave their contents in
 * it: calls that overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller.  The first call on a device looks up
 * the array's device address (hipGetSymbolAddress, after validation).
 * Arguments, results and errors are otherwise those of ssm_selective_scan_fwd.
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int ssm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                                   const void* Bm, const void* Cm, const float* Dskip,
                                   const void* z, const float* delta_bias, unsigned flags,
                                   const float* h0, void* y, float* h_last,
                                   int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                   void* stream);

/*
 * Variable-length batch: row b runs only its first seq_lens[b] tokens
 * (seq_lens: device int32 [B], values clamped to [0, L]); y at positions
 * t >= seq_lens[b] is left untouched and h_last is the state after the row's
 * last token.  Sequences of different lengths share one launch with the
 * layout [B, L, ...] right-padded to the longest.  Otherwise as
 * ssm_selective_scan_fwd (same workspace query).
 */
int ssm_selective_scan_fwd_varlen(const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* delta_bias, unsigned flags,
                                  const float* h0, void* y, float* h_last,
                                  const int32_t* seq_lens, int64_t B, int64_t L, int64_t D,
                                  int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Same operation, for measurement: `events` is NULL or points to 4 hipEvent_t
 * created by the caller; they are recorded on `stream` at the phase
 * boundaries.  State-per-lane path: before the scan of the segments, before
 * the carry, before the fix-up, after it (with one segment the last three
 * coincide).  Split path: before the segment reduce, before the carry, before
 * the segment rescan, after it (with one segment the first three coincide).
 * Recording is asynchronous; the caller reads the intervals after it has
 * synchronised.  The arguments and results are otherwise those of
 * ssm_selective_scan_fwd.
 */
int ssm_selective_scan_fwd_timed(const void* u, const void* delta, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip,
                                 const void* z, const float* delta_bias, unsigned flags,
                                 const float* h0, void* y, float* h_last,
                                 int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events);

/*
 * The same scan with the causal depthwise conv1d + SiLU of ssm_causal_conv1d_silu
 * fused in front of it: the call reads the convolution's input x [B, L, D]
 * and forms u = silu(bias + sum_k weight[d,k] x_{t-(K-1)+k}) per token in
 * registers, so u never round-trips through memory (the Mamba block applies
 * the short convolution and SiLU just before the selective SSM: temporalbook
 * "Selective State-Space Models (Mamba)", section 4).
 *   x              : [B, L, D] dtype (the place of u)
 *   conv_weight    : [D, K] fp32; conv_bias : [D] fp32 or NULL; 1 <= K <= 4
 *   conv_state_in  : [B, D, K-1] fp32 or NULL (zeros): inputs before t = 0
 *   conv_state_out : [B, D, K-1] fp32 or NULL: the last K-1 inputs
 *   u_out          : [B, L, D] dtype or NULL: the convolution's output u
 *                    (what the backward pass takes as u)
 * Everything else as ssm_selective_scan_fwd (same workspace query).
 * Supported: N = 16; flags SSM_FLAG_DELTA_SOFTPLUS only.
 */
int ssm_selective_scan_conv_fwd(const void* x, const float* conv_weight, const float* conv_bias,
                                const float* conv_state_in, float* conv_state_out, int64_t K,
                                void* u_out, const void* delta, const float* A, const void* Bm,
                                const void* Cm, const float* Dskip, const void* z,
                                const float* delta_bias, unsigned flags, const float* h0, void* y,
                                float* h_last, int64_t B, int64_t L, int64_t D, int64_t N,
                                int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------- SSD chunked
 * The Mamba-2 form with a scalar transition per head (section 3 "Mamba-2 and
 * State Space Duality" of "Mamba & Mamba-2 Architecture"): per (b, head h),
 * g = h / (H/G),
 *   dt   = softplus(delta[b,t,h] + delta_bias[h])       (flag set; else delta + bias)
 *   S    = exp(dt * A[h]) * S + dt * X[b,t,h,:] (outer) B[b,t,g,:]   (S is P x N)
 *   Y[b,t,h,:] = (S C[b,t,g,:] + Dskip[h] * X[b,t,h,:]) * silu(z[b,t,h,:])
 * computed chunk by chunk: within a chunk as the masked product
 * (M o (C B^T)) (dt o X) on the matrix cores, across chunks through the
 * carried P x N state.  The chunk length does not change the result beyond
 * rounding.
 *   X, Y, z : [B, L, H, P] dtype (z may be NULL)
 *   delta   : [B, L, H]    dtype
 *   A       : [H] fp32 (negative);  Dskip, delta_bias : [H] fp32 or NULL
 *   Bm, Cm  : [B, L, G, N] dtype;  H % G == 0
 *   h0, h_last : [B, H, P, N] fp32 or NULL
 *   supported: dtype SSM_BF16, P a multiple of 32, N in {32, 64, 96, 128},
 *   chunk in {64, 128, 256}, B * H * (P / 64, or P / 32 when P % 64 != 0)
 *   below 2^31,
 *   and one batch row within 32-bit byte offsets with two chunks to spare:
 *   (L + 512) * H * P * 2 and (L + 512) * G * N * 2 at most 2^32 - 1
 *   (else SSM_ERR_UNSUPPORTED).
 */
size_t ssm_ssd_chunk_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P,
                                     int64_t G, int64_t N, int64_t chunk, int dtype);

int ssm_ssd_chunk_fwd(const void* X, const void* delta, const float* A,
                      const void* Bm, const void* Cm, const float* Dskip,
                      const void* z, const float* delta_bias, unsigned flags,
                      const float* h0, void* Y, float* h_last,
                      int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                      int64_t N, int64_t chunk, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Variable-length batch for the SSD form, as ssm_selective_scan_fwd_varlen
 * for the scan: row b runs only its first seq_lens[b] tokens (seq_lens:
 * device int32 [B], values clamped to [0, L]) of the [B, L, ...] layout
 * right-padded to the longest; Y at t >= seq_lens[b] is left untouched, the
 * padding is never read, and h_last is the state after the row's last token.
 * Otherwise as ssm_ssd_chunk_fwd.
 */
int ssm_ssd_chunk_fwd_varlen(const void* X, const void* delta, const float* A,
                             const void* Bm, const void* Cm, const float* Dskip,
                             const void* z, const float* delta_bias, unsigned flags,
                             const float* h0, void* Y, float* h_last, const int32_t* seq_lens,
                             int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                             int64_t N, int64_t chunk, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------- S6 backward
 * Gradients of the selective scan (the operation of ssm_selective_scan_fwd,
 * Euler input term) for L = sum(dy * y) + sum(dh_last * h_last).  The states
 * are not stored by the forward call: they are recomputed from the saved
 * inputs (the backward pass by recomputation of the Transformer-math
 * "Selective state space" article, "Why the fused kernel is the real
 * contribution").
 *
 * Inputs: those of the forward call (u, delta, A, Bm, Cm, Dskip, z,
 * delta_bias, flags, h0; same shapes and dtype), plus
 *   dy       : [B, L, D]  dtype       gradient of y
 *   dh_last  : [B, D, N]  fp32 or NULL (zeros)
 * Outputs (all written, never accumulated into):
 *   du, ddelta     : [B, L, D] dtype  (ddelta is the gradient of the raw delta)
 *   dz             : [B, L, D] dtype, required when z is given
 *   dA             : [D, N]    fp32
 *   dB, dC         : [B, L, N] fp32   (summed over the D channels)
 *   dDskip, ddelta_bias : [D]  fp32 or NULL (not computed)
 *   dh0            : [B, D, N] fp32 or NULL
 * Supported: 1 <= N <= 16; flags SSM_FLAG_DELTA_SOFTPLUS only (no ZOH).
 * Both sweeps (a forward one storing the state every 16 tokens, then the
 * adjoint one) run one workgroup per channel group and batch row.  When
 * there are fewer than 128 adjoint-sweep workgroups (B * ceil(D/48)) and at
 * least 2048 tokens, the sequence is cut into segments (whole 128-token
 * multiples of at least 1024 tokens, at most 64, as many as keep the
 * adjoint-sweep workgroups within four per CU over the call; see
 * ssm_selective_scan_bwd_segments): each segment's
 * forward pair (its end state from zero) and adjoint pair (its adjoint from
 * zero at its end) are computed in parallel, folded in segment order into
 * every segment's incoming state and adjoint (both decaying over a segment by
 * exp(A * its sum of dt)), and then all segments are swept from those.
 * The workspace (query below; 256-byte aligned) holds per-channel-group
 * partial sums, the segment buffers and a state checkpoint every 16 tokens;
 * results are deterministic (no atomics).
 */
size_t ssm_selective_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                              int dtype);

/* Number of sequence segments a backward call uses at these sizes (1 = one
 * pass); 0 for sizes the backward does not take.  The environment variable
 * SSM_BWD_SEGMENTS (1..64) overrides the choice, for this query and the call
 * (capped at one segment per 16 tokens). */
int ssm_selective_scan_bwd_segments(int64_t B, int64_t L, int64_t D, int64_t N);

int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, const void* z,
                           const float* delta_bias, unsigned flags, const float* h0,
                           const void* dy, const float* dh_last, void* du, void* ddelta,
                           float* dA, float* dB, float* dC, float* dDskip, void* dz,
                           float* ddelta_bias, float* dh0, int64_t B, int64_t L, int64_t D,
                           int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Variable-length batch (the backward of ssm_selective_scan_fwd_varlen): row
 * b has only its first seq_lens[b] tokens (device int32 [B], values clamped
 * to [0, L]), dh_last is the gradient of the state after its last one, and
 * the padding of the [B, L, ...] inputs is never read.  The gradients at
 * t >= seq_lens[b] (du, ddelta, dz, dB, dC) are written as zeros.  Otherwise
 * as ssm_selective_scan_bwd (same workspace query).
 */
int ssm_selective_scan_bwd_varlen(const void* u, const void* delta, const float* A,
                                  const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* delta_bias, unsigned flags,
                                  const float* h0, const void* dy, const float* dh_last, void* du,
                                  void* ddelta, float* dA, float* dB, float* dC, float* dDskip,
                                  void* dz, float* ddelta_bias, float* dh0,
                                  const int32_t* seq_lens, int64_t B, int64_t L, int64_t D,
                                  int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * -------------------------------------------- S6 forward and backward, training
 * A training step runs the forward and then the backward over the same
 * inputs; the backward above starts with a forward sweep of its own that
 * recomputes the state entering every 16-token tile.  These two calls split
 * that work differently: the forward call saves those states as it passes
 * them, and the backward call takes them instead of recomputing them (the
 * chunk-boundary states of the recomputation scheme in the Transformer-math
 * "Selective state space" article, "Why the fused kernel is the real
 * contribution": the per-token states are still recomputed inside each tile,
 * never stored).
 *
 *   ckpt : [B, D, ceil(L/16), N] fp32; ckpt[b,d,k,:] = the state before token
 *          16k (h0, or zeros, for k = 0).  ssm_selective_scan_ckpt_bytes
 *          returns its size (0 for sizes the backward does not take).
 *
 * ssm_selective_scan_fwd_ckpt: ssm_selective_scan_fwd (same arguments,
 * results, workspace query and errors) that also writes ckpt.  Sizes, flags
 * and dtype: those of ssm_selective_scan_bwd (1 <= N <= 16; only
 * SSM_FLAG_DELTA_SOFTPLUS).  Where the state-per-lane scan runs, it stores
 * each checkpoint itself (one 4-byte store per lane and tile); when it runs
 * in segments, those after the first store their states from zero and the
 * fix-up pass adds exp(A * cumsum dt) * h_in to each, as it does to y.  On
 * the split path the call runs the backward's forward sweep after the scan,
 * as one segment.  The one-pass scan and that sweep give the values the
 * backward's own sweep computes when it runs as one segment, bit for bit;
 * the segmented scan's values round differently.  ckpt may be NULL only when
 * L = 0; 16-byte aligned.
 *
 * ssm_selective_scan_bwd_ckpt: ssm_selective_scan_bwd (same arguments,
 * results and errors) reading the checkpoints from ckpt, as written by
 * ssm_selective_scan_fwd_ckpt over the same inputs (or by any forward of the
 * same operation); its forward sweeps are skipped and its workspace
 * (ssm_selective_scan_bwd_ckpt_workspace_bytes) holds the partial sums and
 * the segment buffers.  Where ssm_selective_scan_bwd runs as one segment and
 * its checkpoints equal these, the gradients are equal bit for bit.  ckpt may
 * be NULL only when L = 0; 16-byte aligned.
 */
size_t ssm_selective_scan_ckpt_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int dtype);

int ssm_selective_scan_fwd_ckpt(const void* u, const void* delta, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip,
                                const void* z, const float* delta_bias, unsigned flags,
                                const float* h0, void* y, float* h_last, float* ckpt,
                                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

size_t ssm_selective_scan_bwd_ckpt_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                                   int dtype);

int ssm_selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* Bm,
                                const void* Cm, const float* Dskip, const void* z,
                                const float* delta_bias, unsigned flags, const float* h0,
                                const float* ckpt, const void* dy, const float* dh_last,
                                void* du, void* ddelta, float* dA, float* dB, float* dC,
                                float* dDskip, void* dz, float* ddelta_bias, float* dh0,
                                int64_t B, int64_t L, int64_t D, int64_t N, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---------------------------------------------------------------- S6 decode
 * One token of the selective scan against a resident state, for
 * autoregressive generation: the plain recurrence, one token at a time, with
 * a constant D x N state per sequence (Transformer-math "Selective state
 * space" article, section "What it costs at inference, and on a CPU").  Per
 * (b, d), with the formulas of ssm_selective_scan_fwd at a single t:
 *
 *   dt     = softplus(delta[b,d] + delta_bias[d])     (flag set; else delta + bias)
 *   state[b,d,n] = exp(dt * A[d,n]) * state[b,d,n] + dt * B[b,n] * u[b,d]
 *   y[b,d] = (sum_n C[b,n] * state[b,d,n] + Dskip[d] * u[b,d]) * silu(z[b,d])
 *
 * Arguments:
 *   state          : [B, D, N]  fp32, read and overwritten in place (owned by
 *                    the caller; a sequence's state after token t is its
 *                    input for token t + 1, as h_last / h0 of the scan)
 *   u, delta, z, y : [B, D]     dtype (z may be NULL)
 *   A              : [D, N]     fp32
 *   Bm, Cm         : [B, N]     dtype, shared by all D channels of row b
 *   Dskip, delta_bias : [D]     fp32 or NULL
 *   flags          : SSM_FLAG_DELTA_SOFTPLUS, SSM_FLAG_ZOH as for the scan
 *   1 <= N <= 64 (N in {4, 8, 16, 32, 64} takes the vectorised path).
 * Alignment: state, A and the dtype tensors 16 B; Dskip and delta_bias 4 B.
 * `state` must not overlap any input.  No workspace; asynchronous on stream.
 */
int ssm_selective_state_update(float* state, const void* u, const void* delta, const float* A,
                               const void* Bm, const void* Cm, const float* Dskip,
                               const void* z, const float* delta_bias, unsigned flags, void* y,
                               int64_t B, int64_t D, int64_t N, int dtype, void* stream);

/*
 * ---------------------------------------------------------------- conv1d + SiLU
 * The short causal depthwise convolution over tokens, then SiLU, that turns
 * the inner branch of a Mamba block into the scan input u (temporalbook
 * "Selective State-Space Models (Mamba)", section 4; width d_conv = 4 in the
 * block constructor of section 5).  Per (b, channel d):
 *
 *   s[b,t,d] = bias[d] + sum_{k<K} weight[d,k] * x[b, t-(K-1)+k, d]
 *   u[b,t,d] = silu(s) = s * sigmoid(s)        (silu != 0; else u = s)
 *
 * The last tap multiplies the current token.  Inputs before t = 0 come from
 * state_in (the previous chunk's last K-1 inputs, oldest first) or are zero;
 * state_out receives this call's last K-1 inputs, so chunked prefill is
 * exact when each call passes the previous state_out as its state_in.
 *   x, u      : [B, L, D] dtype (channels contiguous, the layout of the scan's u)
 *   weight    : [D, K] fp32;  bias : [D] fp32 or NULL
 *   state_in, state_out : [B, D, K-1] fp32 or NULL (must not overlap)
 *   1 <= K <= 4;  L >= 0 (L = 0 copies state_in, or zeros, to state_out).
 */
int ssm_causal_conv1d_silu(const void* x, const float* weight, const float* bias,
                           const float* state_in, int silu, void* u, float* state_out,
                           int64_t B, int64_t L, int64_t D, int64_t K, int dtype, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SSM_MI355X_H */
