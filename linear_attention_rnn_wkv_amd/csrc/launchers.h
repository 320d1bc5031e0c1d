// launchers.h -- host-side launch functions of the WKV kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

// Compute units of the current device (read once per device).
int device_cus();

// Device workspace of one kind for (current device, stream), at least `bytes`
// long and zero-filled when first allocated (on `stream`).  Launches on one
// stream run in order and may share it; a kernel that uses flags in it must
// leave them cleared.  A larger request reallocates (synchronising the
// stream first).  Kept until the process ends.
enum { kWsRwkv4Chain = 0, kWsChunkHandoff = 1, kWsDecayH = 2, kWsBwdSplit = 3 };
hipError_t stream_workspace(int kind, hipStream_t stream, size_t bytes, void **out);

// Byte offset, in the workspace of each kind, of the word a kernel sets when
// one of its bounded waits for another workgroup gives up (that workgroup's
// results were then never seen, and the call's outputs are invalid); -1 for
// a kind with no waits.  Only the host clears it (workspace_timed_out).
constexpr long kWsErrorWord[] = {128, 4096 * 4, -1, 4096 * 4};
// Waits for `stream`, then reads and clears the error words of its
// workspaces on the current device; *timed_out is set when any was set.
hipError_t workspace_timed_out(hipStream_t stream, bool *timed_out);

// RWKV-4 time-split scan: y and the (a, b, p) state for C = H*N channels.
hipError_t launch_rwkv4(int B, int T, int C, const float *k, const float *v,
                        const float *w, const float *u, const float *state_in,
                        float *state_out, float *y, hipStream_t stream);

// RWKV-4 serial (RNN-mode) path, (a, b, p) state updated in place.
hipError_t launch_rwkv4_step(int B, int T, int C, const float *k, const float *v,
                             const float *w, const float *u, float *state, float *y,
                             hipStream_t stream);

// Eagle (per_token_decay = false) / Finch serial (RNN-mode) path, N = 64,
// state updated in place.
hipError_t launch_wkv_step(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                           const uint16_t *k, const uint16_t *v, const float *x,
                           const float *u, float *state, uint16_t *o, hipStream_t stream);

// Eagle / Finch chunked (time-parallel) path, N = 64.  With chunk_states
// non-NULL it writes, instead of o and state_out, the state entering every
// chunk and the final state: [B H][ceil(T/64) + 1][64][64] fp32.
hipError_t launch_wkv_chunked(bool per_token_decay, int B, int T, int H,
                              const uint16_t *r, const uint16_t *k,
                              const uint16_t *v, const float *x, const float *u,
                              const float *state_in, float *state_out,
                              uint16_t *o, hipStream_t stream,
                              float *chunk_states = nullptr, const uint16_t *gate = nullptr,
                              const float *ln_w = nullptr, const float *ln_b = nullptr,
                              float eps = 0.0f, const uint16_t *lora_h = nullptr,
                              const uint16_t *lora_B2 = nullptr,
                              const float *lora_omega = nullptr);

// Finch decay producer (decay_lora.hip): h = act(z A2) per token, bf16
// [rows][64], from the block input x [rows][D] (rows = B T, T tokens per
// sequence), the shift row per sequence (NULL: zero), mu, lam [D] fp32,
// A1 [D][32], B1 [32][D], A2 [D][64] bf16.  D a multiple of 64.
hipError_t launch_decay_lora(int rows, int T, int D, bool tanh_act, const uint16_t *x,
                             const uint16_t *shift, const float *mu, const float *lam,
                             const uint16_t *A1, const uint16_t *B1, const uint16_t *A2,
                             uint16_t *h, hipStream_t stream);
// d = omega + h B2 [rows][D] fp32 (B2 [64][D] bf16, omega [D])
hipError_t launch_lora_logits(int rows, int D, const uint16_t *h, const uint16_t *B2,
                              const float *omega, float *d, hipStream_t stream);

// Eagle / Finch chunked forward with the time-mixing epilogue (LayerNorm per
// head, affine, SiLU gate) applied to the output: y instead of o.
hipError_t launch_wkv_chunked_gated(bool per_token_decay, int B, int T, int H,
                                    const uint16_t *r, const uint16_t *k, const uint16_t *v,
                                    const float *x, const float *u, const float *state_in,
                                    float *state_out, const uint16_t *gate, const float *ln_w,
                                    const float *ln_b, float eps, uint16_t *y,
                                    hipStream_t stream);

// Eagle / Finch chunked backward, N = 64: workspace size and launch (the
// forward's state recomputation, the reverse sweep, the sums over sequences).
size_t wkv_bwd_workspace_bytes(int B, int T, int H);
hipError_t launch_wkv_bwd(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                          const uint16_t *k, const uint16_t *v, const float *x, const float *u,
                          const float *state_in, const uint16_t *d_o, const float *d_sT,
                          uint16_t *d_r, uint16_t *d_k, uint16_t *d_v, float *d_x, float *d_u,
                          float *d_s0, void *workspace, hipStream_t stream,
                          bool states_saved = false);

// Fill n floats with `value` (used for empty / zero states when T == 0).
hipError_t launch_fill(float *dst, int64_t n, float value, hipStream_t stream);

// RWKV-4 empty history: a = b = 0, p = -1e38 for [B][3][C].
hipError_t launch_rwkv4_empty_state(int B, int C, float *state, hipStream_t stream);

}  // namespace wkv
