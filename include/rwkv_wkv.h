/*
 * rwkv_wkv.h -- C ABI of the RWKV WKV time-mixing operators for AMD
 * Instinct MI355X (gfx950).
 *
 * The library computes the WKV recurrence of three RWKV generations:
 *
 *  RWKV-4: per-channel decayed weighted average (RWKV paper summary,
 *    cafeforensic.com zhuanlan/310315, section "Temporal structure for
 *    sequential data processing": decay e^{-w} and current-token bonus e^{u}
 *    of the WKV; section "Gradient stability and layer stacking": evaluated
 *    as a time-dependent softmax for numerical stability):
 *        y_t = (sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t)
 *            / (sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t})
 *
 *  Eagle (RWKV-5) and Finch (RWKV-6): per-head matrix-valued state
 *    (RWKV-5/6 summary, blob.wenxiaobai.com, section 4 notation: per-head row
 *    vectors, matrices act on the right; 4.1.2 "Eagle time mixing":
 *    w = exp(-exp(omega)) per key channel, bonus u on the current token's
 *    k^T v, r used like a query; 4.2.2 "Finch time mixing": w_t varies per
 *    token and channel):
 *        o_t = r_t (S_{t-1} + diag(u) k_t^T v_t)
 *        S_t = diag(w_t) S_{t-1} + k_t^T v_t,     w_t = exp(-exp(x_t))
 *    with S[i][j], i = key channel, j = value channel.
 *
 * Both modes the pages describe are provided: the time-parallel (chunked)
 * mode for prefill / training forward (RWKV paper summary, section
 * "Transformer-like parallelization"), and the serial RNN mode for decoding
 * (section "RNN-like sequential decoding": each output depends only on the
 * latest state, so speed and memory per token are constant in sequence
 * length).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, frees nothing and never synchronises a stream inside
 *    a call; its only state is a per-device cache of two attributes (compute
 *    units and XCDs) read on first use, and the device address of the static
 *    scratch array of rwkv6_wkv_fwd_noalloc (part of the code object, one per
 *    device), looked up on that entry point's first call on a device.
 *  - Layouts are row-major, channel fastest: [B][T][H][N] is the same memory
 *    as [B][T][D] with D = H*N and head h owning channels [h*N, (h+1)*N).
 *  - bf16 tensors hold raw bfloat16 bits (rwkv_bf16); outputs are rounded to
 *    nearest, ties to even.
 *  - `stream` is the hipStream_t the work is enqueued on (NULL = the default
 *    stream).  Errors raised by a running kernel surface at the caller's next
 *    synchronisation.  Every call may be made during HIP graph capture.
 *  - Return value: RWKV_OK, or a negative status.  Arguments are validated on
 *    the host before any HIP call; on a validation error nothing is
 *    launched and no output is touched.
 *  - Inputs containing Inf or NaN give unspecified results (they are not
 *    scanned for).
 *  - T == 0 is valid: the state is copied from state_in to state_out (or set
 *    to the empty / zero state when state_in is NULL); r, k, v, x, y, o may
 *    then be NULL.
 *
 * Workspaces.  Entry points whose kernels need device scratch take a
 * `workspace` pointer and its size in bytes; a matching *_workspace_bytes()
 * call gives the size needed for a shape on the current device (0: the call
 * needs none, and workspace may be NULL).  The caller owns the workspace; it
 * must be 16-byte aligned, must not overlap any other argument of the call,
 * and, where the entry point says so, must be ZERO-FILLED before its first
 * use.  Such a workspace carries hand-offs between workgroups: its first
 * 16 KiB are a control block (an epoch advanced by every launch, and an
 * error word), and the kernels leave it valid for the next call, so it is
 * zero-filled once and then reused for any number of calls of the same
 * family (rwkv4_wkv_fwd; or the Eagle/Finch chunked entry points), also as
 * replays of a captured HIP graph.  Two calls that use one workspace must
 * not run concurrently (different streams, or two graphs replayed at once).
 * A hand-off wait is bounded (about a second) so that every kernel ends; it
 * is never reached in normal operation, since a producer always has a lower
 * workgroup index than its consumer and runs before or beside it.  A
 * consumer that gave up continues from a NaN state, so the affected outputs
 * read NaN, and it sets the error word (rwkv_wkv_workspace_status).
 */
#ifndef RWKV_WKV_H
#define RWKV_WKV_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared as HIP declares it (a pointer to an opaque
 * struct), so that this header compiles with or without the HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

typedef uint16_t rwkv_bf16; /* raw bfloat16 bits */

enum rwkv_status {
    RWKV_OK = 0,
    RWKV_E_NULL = -1,        /* a required pointer is NULL */
    RWKV_E_DIM = -2,         /* B, H or N < 1, T < 0, or a size overflows */
    RWKV_E_UNSUPPORTED = -3, /* a valid shape this build does not implement */
    RWKV_E_ALIGN = -4,       /* a pointer is not 16-byte aligned where required */
    RWKV_E_ALIAS = -5,       /* an output overlaps an input or another output */
    RWKV_E_HIP = -6,         /* the HIP runtime rejected a launch or copy */
    RWKV_E_TIMEOUT = -7      /* a workgroup gave up waiting for another's
                                hand-off (rwkv_wkv_workspace_status) */
};

/* Static, human-readable text of a status code. */
const char *rwkv_wkv_strerror(int status);

/* Whether a kernel that used `workspace` (a zero-filled workspace of one of
 * the entry points with hand-offs: rwkv4_wkv_fwd, the chunked Eagle/Finch
 * forwards and backwards) gave up a hand-off wait since the last check.
 * It synchronises `stream`, reads the workspace's error word, and returns
 * RWKV_E_TIMEOUT if it was set (then clears it), RWKV_OK if not, RWKV_E_HIP
 * if the runtime fails, RWKV_E_NULL / RWKV_E_DIM / RWKV_E_ALIGN for a NULL,
 * shorter than 16 KiB or misaligned workspace.  A diagnostic: call it after
 * a batch of work, outside graph capture.  It allocates nothing.
 */
int rwkv_wkv_workspace_status(void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * RWKV-4 WKV forward, fp32.  Channels are independent: C = H*N and any
 * factorisation of C gives identical results.
 *
 *   k, v       [B][T][C] fp32 keys and values
 *   w          [C] fp32 decay RATE, w >= 0; the per-step factor is e^{-w}
 *   u          [C] fp32 bonus of the current token
 *   state_in   [B][3][C] fp32 history (a, b, p), or NULL for an empty one.
 *              The history's numerator and denominator are a*e^p and b*e^p
 *              (p is a running maximum exponent that keeps a and b finite);
 *              the empty history is a = b = 0, p = -1e38.
 *   state_out  [B][3][C] fp32 state after token T, or NULL.  It may equal
 *              state_in exactly (in-place update) but not partially overlap.
 *   y          [B][T][C] fp32 output
 *
 *   workspace  rwkv4_wkv_fwd_workspace_bytes(B, T, H, N) bytes, ZERO-FILLED
 *              before first use (see Workspaces above); NULL when that is 0
 *              (T <= 256).  RWKV_E_NULL if NULL, RWKV_E_DIM if shorter,
 *              RWKV_E_ALIGN / RWKV_E_ALIAS as for the tensors.
 *
 * Pointers need 4-byte alignment (the workspace 16).  C = H*N must be at
 * most 2^20 and B * C below 2^36, else RWKV_E_UNSUPPORTED.  Values of v up
 * to about 1e25 in magnitude are handled: where every channel of a wave's
 * 32-channel block has |u - w| <= 30, a token's output is formed with its
 * value scaled by e^{u-w}.
 *
 * The 256-token passes of a sequence's block of 32 channels run in separate
 * workgroups that hand the state on through the workspace (1.5 KiB of
 * records per workgroup of a launch, at most 8192 workgroups per launch;
 * longer inputs take several launches, the state carried between them in
 * the workspace).  Outputs of sequences longer than one pass may differ from
 * run to run in the last bits: how far back a pass finds a finished
 * predecessor depends on timing, and so does the order in which the carried
 * state is combined.
 */
size_t rwkv4_wkv_fwd_workspace_bytes(int B, int T, int H, int N);

int rwkv4_wkv_fwd(int B, int T, int H, int N,
                  const float *k, const float *v,
                  const float *w, const float *u,
                  const float *state_in, float *state_out,
                  float *y, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * RWKV-4 WKV, serial (RNN) mode (RWKV paper summary, section "RNN-like
 * sequential decoding": an output needs only the latest state).  Tokens are
 * applied one at a time; decoding calls it with T == 1.  Arguments as
 * rwkv4_wkv_fwd, except:
 *
 *   state      [B][3][C] fp32 (a, b, p), read as the history and overwritten
 *              with the state after token T (required, never NULL; it must
 *              not overlap any other argument).
 *
 * Within a call the running exponent p is recomputed from the key that last
 * set it and the steps since, so its rounding does not build up over the
 * call's tokens; the stored p is rounded once per call.  Splitting a
 * sequence therefore changes results in the last bits only.  B * C must be
 * at most 2^38, else RWKV_E_UNSUPPORTED.
 */
int rwkv4_wkv_step(int B, int T, int H, int N,
                   const float *k, const float *v,
                   const float *w, const float *u,
                   float *state, float *y, hipStream_t stream);

/*
 * Eagle (RWKV-5) WKV forward, time-parallel (chunked) mode.  N must be 64.
 *
 *   r, k, v    [B][T][H][N] bf16 receptance, key, value
 *   x          [H][N] fp32 decay logit omega, shared by all tokens and
 *              sequences: w = exp(-exp(x)) lies in (0, 1)
 *   u          [H][N] fp32 bonus
 *   state_in   [B][H][N][N] fp32 initial state S_0 (key-major: row i is key
 *              channel i), or NULL for zeros
 *   state_out  [B][H][N][N] fp32 state after token T, or NULL.  It may equal
 *              state_in exactly, but not partially overlap it.
 *   o          [B][T][H][N] bf16 output
 *
 *   workspace  rwkv_wkv_fwd_workspace_bytes(B, T, H, N) bytes, ZERO-FILLED
 *              before first use (see Workspaces above); NULL when that is 0.
 *              It is 0 unless B*H exceeds the device's compute units and
 *              T >= 256: then each workgroup runs its own head plus a segment
 *              of an extra head, and the segments hand the state on through
 *              the workspace (16 KiB per hand-off, at most 4096; past twice
 *              the compute units also 16 KiB per workgroup, where a
 *              workgroup's own state waits meanwhile).  The size depends on
 *              the current device: query it with the device current.
 *
 * All pointers need 16-byte alignment.  H must be at most 65536 and B*H below
 * 2^31, else RWKV_E_UNSUPPORTED.
 */
size_t rwkv_wkv_fwd_workspace_bytes(int B, int T, int H, int N);

int rwkv5_wkv_fwd(int B, int T, int H, int N,
                  const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                  const float *x, const float *u,
                  const float *state_in, float *state_out,
                  rwkv_bf16 *o, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * Finch (RWKV-6) WKV forward, time-parallel (chunked) mode.  N must be 64.
 * As rwkv5_wkv_fwd, except that the decay logit is per token and channel:
 *
 *   x          [B][T][H][N] fp32: token t decays the state by
 *              w_t = exp(-exp(x_t)) after producing o_t, so x at the last
 *              token only affects state_out.
 */
int rwkv6_wkv_fwd(int B, int T, int H, int N,
                  const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                  const float *x, const float *u,
                  const float *state_in, float *state_out,
                  rwkv_bf16 *o, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * rwkv6_wkv_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): the same
 * arguments, outputs and status codes without the workspace.  The hand-off
 * area of the balanced split lives in a file-scope device array of 8 MiB,
 * one per GPU, held until the process ends; a shape that needs more
 * (rwkv_wkv_fwd_workspace_bytes(B, T, H, N) > 8 MiB: on 256 compute units,
 * more than 512 heads with T >= 256) returns RWKV_E_UNSUPPORTED and
 * launches nothing.  Every call on one GPU shares that GPU's array; it
 * starts zero-filled and the kernels leave it valid for the next call, so
 * nothing is cleared between calls, but calls that overlap in time on one
 * GPU (two streams, or two graphs replayed at once) race.  It allocates
 * nothing; its first call on a device looks up the array's address.
 */
int rwkv6_wkv_fwd_noalloc(int B, int T, int H, int N,
                          const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                          const float *x, const float *u,
                          const float *state_in, float *state_out,
                          rwkv_bf16 *o, hipStream_t stream);

/*
 * Finch (RWKV-6) WKV, serial (RNN) mode: tokens are applied one at a time to
 * a state that stays in registers.  Decoding calls it with T == 1.  N must
 * be 64.  Arguments as rwkv6_wkv_fwd, except:
 *
 *   state      [B][H][N][N] fp32, read as S_0 and overwritten with S_T
 *              (required, never NULL).
 *
 * Splitting a sequence at any token and handing the state over gives
 * bit-identical outputs and state.
 */
int rwkv6_wkv_step(int B, int T, int H, int N,
                   const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                   const float *x, const float *u,
                   float *state, rwkv_bf16 *o, hipStream_t stream);

/*
 * Eagle (RWKV-5) WKV, serial (RNN) mode.  As rwkv6_wkv_step, except that x
 * is the static decay logit omega, [H][N] fp32, shared by all tokens and
 * sequences (as in rwkv5_wkv_fwd).
 */
int rwkv5_wkv_step(int B, int T, int H, int N,
                   const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                   const float *x, const float *u,
                   float *state, rwkv_bf16 *o, hipStream_t stream);

/*
 * Eagle / Finch time-parallel forward with the time-mixing epilogue fused
 * into the output write (RWKV-5/6 summary, 4.1.2 "Eagle time mixing": a
 * LayerNorm on each of the h heads, equivalently a GroupNorm over h groups,
 * and a SiLU gate on the attention output before the output weights):
 *
 *   y = ((o - mean) / sqrt(var + eps) * ln_w + ln_b) * g / (1 + e^-g)
 *
 * with o the output of rwkv5/6_wkv_fwd for the same arguments, and the mean
 * and biased variance over the N = 64 channels of one head of one token
 * (taken from the fp32 accumulators, before rounding).
 *
 *   g          [B][T][H][N] bf16 gate
 *   ln_w, ln_b [H][N] fp32 per-channel weight and bias of the norm
 *   eps        added to the variance; finite and >= 0, else RWKV_E_DIM
 *   y          [B][T][H][N] bf16 output (in place of o)
 * Other arguments, the state, the workspace (rwkv_wkv_fwd_workspace_bytes)
 * and the error codes as rwkv6_wkv_fwd (rwkv5: x is [H][N]).  All pointers
 * need 16-byte alignment.
 */
int rwkv5_wkv_fwd_gated(int B, int T, int H, int N,
                        const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                        const float *x, const float *u,
                        const float *state_in, float *state_out,
                        const rwkv_bf16 *g, const float *ln_w, const float *ln_b,
                        float eps, rwkv_bf16 *y, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

int rwkv6_wkv_fwd_gated(int B, int T, int H, int N,
                        const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                        const float *x, const float *u,
                        const float *state_in, float *state_out,
                        const rwkv_bf16 *g, const float *ln_w, const float *ln_b,
                        float eps, rwkv_bf16 *y, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Eagle / Finch backward of the time-parallel forward (rwkv5_wkv_fwd,
 * rwkv6_wkv_fwd): the gradients of a loss L with respect to every input,
 * given dL/do and dL/dS_T.  Reverse-mode differentiation of the recurrence
 * in the RWKV-5/6 summary, 4.1.2 "Eagle time mixing" and 4.2.2 "Finch time
 * mixing"; RWKV paper summary, "Transformer-like parallelization" (the
 * training pass runs time-parallel).  N must be 64.
 *
 *   r, k, v, x, u, state_in   the forward's inputs, as in rwkv6_wkv_fwd
 *              (rwkv5_wkv_bwd: x is [H][N]); state_in may be NULL (zeros)
 *   d_o        [B][T][H][N] bf16, dL/do
 *   d_state_out  [B][H][N][N] fp32 dL/dS_T, or NULL for zero
 *   d_r, d_k, d_v  [B][T][H][N] bf16 outputs
 *   d_x        fp32 output: [B][T][H][N] (rwkv6), or [H][N] summed over
 *              sequences and tokens (rwkv5)
 *   d_u        [H][N] fp32 output, summed over sequences and tokens
 *   d_state_in [B][H][N][N] fp32 output dL/dS_0, or NULL; it may equal
 *              d_state_out exactly (in place)
 *   workspace  rwkv_wkv_bwd_workspace_bytes(B, T, H, N) bytes, 16-byte
 *              aligned, ZERO-FILLED before first use (see Workspaces above),
 *              not overlapping any other argument (RWKV_E_DIM if too small).
 *              It holds the hand-off area of the balanced splits (the
 *              recomputation's and the reverse sweep's, when B*H exceeds the
 *              compute units and T >= 256: 48 KiB per hand-off and per
 *              workgroup for the sweep), the state entering every 64-token
 *              chunk, recomputed by the forward (16 KiB per chunk and head),
 *              and the per-sequence partial sums of d_u and Eagle's d_x.
 *              The size depends on the current device.
 * When B*H exceeds the device's compute units and T >= 256, a workgroup per
 * compute unit sweeps whole heads in rounds; when the last round's remainder
 * is at most half the compute units, each workgroup sweeps its own head of
 * that round plus a segment of an extra head, and the segments hand the
 * sweep's state on through the workspace.
 *
 * All pointers need 16-byte alignment; outputs may not overlap inputs or
 * each other.  H must be at most 65536.  T = 0 sets d_u (and rwkv5's d_x)
 * to zero and d_state_in to d_state_out.  Sums over sequences are taken in
 * a fixed order (results do not depend on scheduling).
 */
size_t rwkv_wkv_bwd_workspace_bytes(int B, int T, int H, int N);

int rwkv5_wkv_bwd(int B, int T, int H, int N,
                  const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                  const float *x, const float *u, const float *state_in,
                  const rwkv_bf16 *d_o, const float *d_state_out,
                  rwkv_bf16 *d_r, rwkv_bf16 *d_k, rwkv_bf16 *d_v,
                  float *d_x, float *d_u, float *d_state_in,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);

int rwkv6_wkv_bwd(int B, int T, int H, int N,
                  const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                  const float *x, const float *u, const float *state_in,
                  const rwkv_bf16 *d_o, const float *d_state_out,
                  rwkv_bf16 *d_r, rwkv_bf16 *d_k, rwkv_bf16 *d_v,
                  float *d_x, float *d_u, float *d_state_in,
                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Training pair that saves the backward's recomputation.  rwkv5/6_wkv_fwd_save
 * is rwkv5/6_wkv_fwd (same arguments, outputs and errors) that also stores,
 * in `workspace`, the state entering every 64-token chunk and the final
 * state, as the backward's first pass would; rwkv5/6_wkv_bwd_saved is
 * rwkv5/6_wkv_bwd without that pass, reading the states a matching
 * *_fwd_save call (same r, k, v, x, u, state_in, B, T, H) left in the same
 * workspace.  The pair gives bit for bit the gradients of the *_fwd and
 * *_bwd pair.
 *   workspace  rwkv_wkv_bwd_workspace_bytes(B, T, H, N) bytes, 16-byte
 *              aligned, zero-filled before first use, overlapping no other
 *              argument (RWKV_E_DIM if too small; RWKV_E_NULL if NULL with
 *              T > 0).
 * The backward's other arguments as rwkv5/6_wkv_bwd (it takes no state_in:
 * the saved states hold it).
 */
int rwkv5_wkv_fwd_save(int B, int T, int H, int N,
                       const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                       const float *x, const float *u,
                       const float *state_in, float *state_out, rwkv_bf16 *o,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
int rwkv6_wkv_fwd_save(int B, int T, int H, int N,
                       const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                       const float *x, const float *u,
                       const float *state_in, float *state_out, rwkv_bf16 *o,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
int rwkv5_wkv_bwd_saved(int B, int T, int H, int N,
                        const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                        const float *x, const float *u,
                        const rwkv_bf16 *d_o, const float *d_state_out,
                        rwkv_bf16 *d_r, rwkv_bf16 *d_k, rwkv_bf16 *d_v,
                        float *d_x, float *d_u, float *d_state_in,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);
int rwkv6_wkv_bwd_saved(int B, int T, int H, int N,
                        const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                        const float *x, const float *u,
                        const rwkv_bf16 *d_o, const float *d_state_out,
                        rwkv_bf16 *d_r, rwkv_bf16 *d_k, rwkv_bf16 *d_v,
                        float *d_x, float *d_u, float *d_state_in,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Finch decay producer (RWKV-5/6 summary, 4.1.1 "Eagle token shift",
 * 4.2.1 "Finch token shift" and 4.2.2 "Finch time mixing": the decay logit
 * of every token and channel from the block input by the data-dependent
 * interpolation (ddlerp) with a LoRA of rank 32, then LoRA_omega of rank 64).
 * Per sequence b and token t, with x_{-1} = shift[b] (zero when shift is
 * NULL) and act the identity (act = 0) or tanh (act = 1):
 *
 *   dx = x_{t-1} - x_t
 *   y  = x_t + dx * mu_x
 *   m  = lam + act(y A1) B1
 *   z  = x_t + dx * m
 *   d  = omega + act(z A2) B2,     w_t = exp(-exp(d)) is Finch's decay.
 *
 *   x          [B][T][D] bf16 block input (D = H N, a multiple of 64 and at
 *              most 64 * 65535, else RWKV_E_UNSUPPORTED)
 *   shift      [B][D] bf16, the token before x[b][0] (a previous segment's
 *              last token), or NULL
 *   mu_x, lam, omega [D] fp32
 *   A1 [D][32], B1 [32][D], A2 [D][64], B2 [64][D] bf16 (row-major, as the
 *              pages give their shapes)
 *   d          [B][T][D] fp32 output: the logits rwkv6_wkv_fwd takes as x
 *              (with D = H N in its [B][T][H][N] layout)
 *   workspace  rwkv6_decay_lora_workspace_bytes(B, T, D) bytes: act(z A2)
 *              of every token (rank 64, bf16, B T 128 bytes), then, for D up
 *              to 2560, the weights laid out as the products' operands (D/64
 *              x 16 KiB; the block input is then read once); 16-byte
 *              aligned, not overlapping any other argument; no zero-filling
 *              needed.
 * The products run on bf16 matrix cores with fp32 accumulation (the mixed
 * values and act(.) rounded to bf16 as operands).  B T must be below 2^31.
 * T = 0 does nothing.  All pointers need 16-byte alignment; d must not
 * overlap an input.
 */
size_t rwkv6_decay_lora_workspace_bytes(int B, int T, int D);

int rwkv6_decay_lora(int B, int T, int D, int act,
                     const rwkv_bf16 *x, const rwkv_bf16 *shift,
                     const float *mu_x, const float *lam,
                     const rwkv_bf16 *A1, const rwkv_bf16 *B1,
                     const float *omega, const rwkv_bf16 *A2, const rwkv_bf16 *B2,
                     float *d, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Finch time-parallel forward fed by the decay producer: the same output and
 * state as rwkv6_decay_lora followed by rwkv6_wkv_fwd with x = d, without
 * the fp32 logits ever going to memory.  The producer writes act(z A2)
 * (rank 64, bf16, B T 128 bytes of the workspace, beside its packed weights)
 * and the chunked kernel forms each head's logits omega + act(z A2) B2 on
 * the matrix cores.
 * Arguments: r, k, v, u, state_in, state_out, o as rwkv6_wkv_fwd; x (the
 * block input, [B][T][H N] bf16), shift, mu_x, lam, A1, B1, omega, A2, B2 and
 * act as rwkv6_decay_lora with D = H N.
 *   workspace  rwkv6_wkv_fwd_lora_workspace_bytes(B, T, H, N) bytes: the
 *              chunked forward's hand-off area (as rwkv_wkv_fwd_workspace_
 *              bytes) followed by the producer's factor.  16-byte aligned,
 *              ZERO-FILLED before first use, overlapping no other argument.
 */
size_t rwkv6_wkv_fwd_lora_workspace_bytes(int B, int T, int H, int N);

int rwkv6_wkv_fwd_lora(int B, int T, int H, int N,
                       const rwkv_bf16 *r, const rwkv_bf16 *k, const rwkv_bf16 *v,
                       const rwkv_bf16 *x, const rwkv_bf16 *shift,
                       const float *mu_x, const float *lam,
                       const rwkv_bf16 *A1, const rwkv_bf16 *B1,
                       const float *omega, const rwkv_bf16 *A2, const rwkv_bf16 *B2,
                       int act, const float *u,
                       const float *state_in, float *state_out,
                       rwkv_bf16 *o, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RWKV_WKV_H */
