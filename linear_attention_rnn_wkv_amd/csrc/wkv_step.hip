// wkv_step.hip -- Eagle (RWKV-5) and Finch (RWKV-6) WKV in serial (RNN) mode
// on gfx950.
//
// Operation, per head (RWKV-5/6 summary, blob.wenxiaobai.com, 4.1.2 "Eagle
// time mixing" and 4.2.2 "Finch time mixing"; RWKV paper summary, section
// "RNN-like sequential decoding"):
//   o_t[j] = sum_i r_t[i] S[i][j] + (sum_i r_t[i] u[i] k_t[i]) v_t[j]
//   S[i][j] <- w_t[i] S[i][j] + k_t[i] v_t[j],   w_t = exp(-exp(x_t))
// Finch reads a decay logit x_t per token; Eagle's x is one per channel of a
// head, shared by every token and sequence (so its decay is computed once).
//
// One wave64 owns one (sequence, head): its 64x64 fp32 state (16 KiB) is
// loaded once into registers, every token of the call is applied to it,
// and it is stored back once.  Lane l holds columns 4*(l%16)..+3 of rows
// i = 4*m + l/16 (m = 0..15), so each 16-byte load or store instruction of
// the wave covers 1 KiB of contiguous state.  Decoding (T == 1) is bound by
// that state traffic: 2 * 16 KiB per head and step.
//
// k_t[i] * v_t[j] is exact in fp32 for bf16 operands, so each state entry
// takes exactly one rounding per token (the fused multiply-add); splitting a
// sequence anywhere and handing the state over is bit-identical.
#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr int kN = 64;
constexpr int kHeadsPerBlock = 4;
// States larger than this are loaded and stored non-temporal.  A state that
// (mostly) fits the 256 MiB last-level cache is partly served from it on the
// next step, and the non-temporal accesses would forgo that; past about 1.4
// times the cache nothing of it survives until the next step, and they stream
// faster.  Measured per step at 64 heads: 320 MiB state 118.1 us plain against
// 121.3 us non-temporal, 384 MiB 151.9 against 146.0 us, 1 GiB 417 against
// 399 us.
constexpr size_t kStreamStateBytes = (size_t)352 << 20;

__device__ __forceinline__ float wave_sum(float s) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return s;
}

template <bool PT, bool NT>
__global__ __launch_bounds__(256) void wkv_step_kernel(
    int BH, int T, int H, const uint16_t *__restrict__ r, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ x, const float *__restrict__ u,
    float *state, uint16_t *__restrict__ o) {
    const int lane = threadIdx.x & 63;
    const int head = blockIdx.x * kHeadsPerBlock + (threadIdx.x >> 6);
    if (head >= BH) return;  // whole wave leaves; the kernel has no barriers
    const int b = head / H;
    const int h = head % H;
    const int g = lane >> 4;   // row group
    const int c4 = lane & 15;  // column quad

    float *sp = state + (size_t)head * kN * kN + g * kN + 4 * c4;
    f32x4 S[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const f32x4 *src = (const f32x4 *)(sp + m * 4 * kN);
        S[m] = NT ? __builtin_nontemporal_load(src) : *src;
    }

    const float uu = u[h * kN + lane];
    const float xo = PT ? 0.0f : x[h * kN + lane];
    // Eagle's per-channel decay: with a state streamed from HBM (NT) it is
    // formed before the first token's loads, which then wait for it and the
    // state (measured 390 against 401 us per step at 1024 sequences); with a
    // cached state, after them (see the loop: 84.1 against 80.8 us at 256)
    const float w_head = (PT || !NT) ? 0.0f : exp_fast(-exp_fast(xo));

    for (int t = 0; t < T; ++t) {
        const size_t base = (((size_t)b * T + t) * H + h) * kN;
        const float ri = bf16_to_f32(r[base + lane]);
        const float ki = bf16_to_f32(k[base + lane]);
        const u32x2 vp = *(const u32x2 *)(v + base + 4 * c4);
        const float vj[4] = {bf16_lo(vp.x), bf16_hi(vp.x), bf16_lo(vp.y), bf16_hi(vp.y)};
        float xt = PT ? x[base + lane] : xo;
        // Eagle with a cached state: the decay is formed here, after the
        // token's loads, and is not hoisted ahead of them (its wait, which
        // also waits for the state, would hold them back by a round trip)
        if (!PT && !NT) {
            __builtin_amdgcn_sched_barrier(0);
            __asm__ volatile("" : "+v"(xt));
        }
        const float wi = (PT || !NT) ? exp_fast(-exp_fast(xt)) : w_head;
        const float bonus = wave_sum(ri * uu * ki);

        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = 4 * m + g;
            const float rm = __shfl(ri, i, 64);
            const float km = __shfl(ki, i, 64);
            const float wm = __shfl(wi, i, 64);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[c] = fmaf(rm, S[m][c], acc[c]);
                S[m][c] = fmaf(wm, S[m][c], km * vj[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[c] += __shfl_xor(acc[c], 16, 64);
            acc[c] += __shfl_xor(acc[c], 32, 64);
        }
        if (g == 0) {
            u32x2 out;
            out.x = pack_bf16x2(fmaf(bonus, vj[0], acc[0]), fmaf(bonus, vj[1], acc[1]));
            out.y = pack_bf16x2(fmaf(bonus, vj[2], acc[2]), fmaf(bonus, vj[3], acc[3]));
            *(u32x2 *)(o + base + 4 * c4) = out;
        }
    }

#pragma unroll
    for (int m = 0; m < 16; ++m) {
        f32x4 *dst = (f32x4 *)(sp + m * 4 * kN);
        if (NT) __builtin_nontemporal_store(S[m], dst);
        else *dst = S[m];
    }
}

}  // namespace

hipError_t launch_wkv_step(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                           const uint16_t *k, const uint16_t *v, const float *x,
                           const float *u, float *state, uint16_t *o, hipStream_t stream) {
    const int64_t BH = (int64_t)B * H;
    const int64_t blocks = (BH + kHeadsPerBlock - 1) / kHeadsPerBlock;
    const bool nt = (size_t)BH * kN * kN * sizeof(float) > kStreamStateBytes;
    auto kernel = per_token_decay ? (nt ? wkv_step_kernel<true, true> : wkv_step_kernel<true, false>)
                                  : (nt ? wkv_step_kernel<false, true> : wkv_step_kernel<false, false>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (int)BH, T, H, r, k,
                       v, x, u, state, o);
    return hipGetLastError();
}

}  // namespace wkv
