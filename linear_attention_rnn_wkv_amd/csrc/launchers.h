// launchers.h -- host-side launch functions of the WKV kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wkv {

// Compute units and XCDs (accelerator dies) of the current device, read once
// per device.  Workgroups of a launch are dealt to the XCDs round-robin.
int device_cus();
int device_xcds();

// Control block at the start of every workspace whose kernels hand a state
// from one workgroup to another.  Each word sits on a 128-byte line of its
// own:
//   epoch  advanced once per launch, after every workgroup of the launch has
//          read it.  A hand-off word is valid only while it carries the
//          launch's tag (epoch + 1), so nothing is cleared between launches
//          and a word written late by an earlier launch is never taken for
//          a current one.
//   err    set to 1 when a bounded wait for another workgroup gave up; that
//          consumer continued with a NaN state, so the affected outputs read
//          NaN.  Read and cleared by rwkv_wkv_workspace_status.
//   done   workgroups of the current launch that have finished (chunked
//          kernels), reset by the last one
//   total, group[]  the RWKV-4 chain's two-level count of finished chains
// A zero-filled block is a valid start (epoch 0, nothing pending).
constexpr int kWsGroups = 64;
struct WsCtrl {
    struct Line {
        unsigned n, pad[31];
    };
    Line epoch, err, done, total, group[kWsGroups];
};
constexpr size_t kWsCtrlBytes = 16384;  // the control block, rounded up
static_assert(sizeof(WsCtrl) <= kWsCtrlBytes, "control block");
constexpr size_t kWsErrOffset = offsetof(WsCtrl, err);

// Bytes of caller workspace each launcher below needs (0: none), for the
// current device.  A workspace is zero-filled by its owner before first use.
size_t rwkv4_workspace_bytes(int B, int T, int C);
size_t chunk_workspace_bytes(int B, int T, int H);   // chunked forward, gated forward
size_t bwd_workspace_bytes(int B, int T, int H);     // backward; forward + backward pair
size_t bwd_states_offset(int B, int T, int H);       // where the saved chunk states start
size_t lora_workspace_bytes(int B, int T, int D);    // decay producer: act(z A2), packed weights
size_t lora_packed_offset(int B, int T);             // where the packed weights start in it
size_t lora_packed_bytes(int D);                     // the packed weights (0: not used for D)
size_t lora_fwd_workspace_bytes(int B, int T, int H);  // producer + chunked forward
size_t lora_fwd_factor_offset(int B, int T, int H);  // where the producer's part starts in it

// RWKV-4 time-split scan: y and the (a, b, p) state for C = H*N channels.
// ws: rwkv4_workspace_bytes(B, T, C) bytes (may be NULL when that is 0).
hipError_t launch_rwkv4(int B, int T, int C, const float *k, const float *v,
                        const float *w, const float *u, const float *state_in,
                        float *state_out, float *y, void *ws, hipStream_t stream);

// RWKV-4 serial (RNN-mode) path, (a, b, p) state updated in place.
hipError_t launch_rwkv4_step(int B, int T, int C, const float *k, const float *v,
                             const float *w, const float *u, float *state, float *y,
                             hipStream_t stream);

// Eagle (per_token_decay = false) / Finch serial (RNN-mode) path, N = 64,
// state updated in place.
hipError_t launch_wkv_step(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                           const uint16_t *k, const uint16_t *v, const float *x,
                           const float *u, float *state, uint16_t *o, hipStream_t stream);

// Eagle / Finch chunked (time-parallel) path, N = 64.  ws: the hand-off area
// of the balanced split, chunk_workspace_bytes(B, T, H) bytes (NULL when
// that is 0).  With chunk_states non-NULL it writes, instead of o and
// state_out, the state entering every chunk and the final state:
// [B H][ceil(T/64) + 1][64][64] fp32.
hipError_t launch_wkv_chunked(bool per_token_decay, int B, int T, int H,
                              const uint16_t *r, const uint16_t *k,
                              const uint16_t *v, const float *x, const float *u,
                              const float *state_in, float *state_out,
                              uint16_t *o, void *ws, hipStream_t stream,
                              float *chunk_states = nullptr, const uint16_t *gate = nullptr,
                              const float *ln_w = nullptr, const float *ln_b = nullptr,
                              float eps = 0.0f, const uint16_t *lora_h = nullptr,
                              const uint16_t *lora_B2 = nullptr,
                              const float *lora_omega = nullptr);

// Finch decay producer (decay_lora.hip): h = act(z A2) per token, bf16
// [rows][64], from the block input x [rows][D] (rows = B T, T tokens per
// sequence), the shift row per sequence (NULL: zero), mu, lam [D] fp32,
// A1 [D][32], B1 [32][D], A2 [D][64] bf16.  D a multiple of 64.  packed:
// lora_packed_bytes(D) bytes of scratch for the weights laid out as product
// operands (unused when that is 0).
hipError_t launch_decay_lora(int rows, int T, int D, bool tanh_act, const uint16_t *x,
                             const uint16_t *shift, const float *mu, const float *lam,
                             const uint16_t *A1, const uint16_t *B1, const uint16_t *A2,
                             uint16_t *h, void *packed, hipStream_t stream);
// d = omega + h B2 [rows][D] fp32 (B2 [64][D] bf16, omega [D])
hipError_t launch_lora_logits(int rows, int D, const uint16_t *h, const uint16_t *B2,
                              const float *omega, float *d, hipStream_t stream);

// Eagle / Finch chunked forward with the time-mixing epilogue (LayerNorm per
// head, affine, SiLU gate) applied to the output: y instead of o.
hipError_t launch_wkv_chunked_gated(bool per_token_decay, int B, int T, int H,
                                    const uint16_t *r, const uint16_t *k, const uint16_t *v,
                                    const float *x, const float *u, const float *state_in,
                                    float *state_out, const uint16_t *gate, const float *ln_w,
                                    const float *ln_b, float eps, uint16_t *y, void *ws,
                                    hipStream_t stream);

// Eagle / Finch chunked backward, N = 64 (the forward's state recomputation,
// the reverse sweep, the sums over sequences).  ws: bwd_workspace_bytes(B,
// T, H) bytes: the hand-off area of both kernels' splits at offset 0, the
// chunk states at bwd_states_offset(B, T, H).
hipError_t launch_wkv_bwd(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                          const uint16_t *k, const uint16_t *v, const float *x, const float *u,
                          const float *state_in, const uint16_t *d_o, const float *d_sT,
                          uint16_t *d_r, uint16_t *d_k, uint16_t *d_v, float *d_x, float *d_u,
                          float *d_s0, void *ws, hipStream_t stream,
                          bool states_saved = false);

// Fill n floats with `value` (used for empty / zero states when T == 0).
hipError_t launch_fill(float *dst, int64_t n, float value, hipStream_t stream);

// RWKV-4 empty history: a = b = 0, p = -1e38 for [B][3][C].
hipError_t launch_rwkv4_empty_state(int B, int C, float *state, hipStream_t stream);

}  // namespace wkv
