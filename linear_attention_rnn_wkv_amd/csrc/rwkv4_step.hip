// rwkv4_step.hip -- RWKV-4 WKV in serial (RNN) mode on gfx950.
//
// Operation (RWKV paper summary, cafeforensic.com zhuanlan/310315, section
// "RNN-like sequential decoding": each output needs only the latest state;
// section "Gradient stability and layer stacking" for the stable form), per
// channel and token, on the state (a, b, p) with Num = a e^p, Den = b e^p:
//   output:  q = max(p, u + k);  y = (e^{p-q} a + e^{u+k-q} v) / (e^{p-q} b + e^{u+k-q})
//   update:  q' = max(p - w, k); a <- e^{p-w-q'} a + e^{k-q'} v;
//            b <- e^{p-w-q'} b + e^{k-q'};  p <- q'
// One of the two exponentials of each line is e^0 = 1, so each line takes a
// single exponential of a non-positive argument.  Within a call p is carried
// as (the key or incoming exponent that last set the maximum, steps since)
// and recomputed with one fused multiply-add, so its rounding does not
// accumulate over the tokens of the call.  The exponent stored at the end of
// a call is rounded, and its exact rounding residual r is folded into a and
// b (times e^r = 1 + r): decoding one token per call would otherwise shift
// the weight of the whole history by the rounding of p at every token, an
// error that grows like |p| 2^-25 sqrt(steps) (about 1e-5 after 1024 steps).
//
// One thread per (sequence, channel); consecutive threads take consecutive
// channels, so every load and store of a wave covers 256 contiguous bytes.
// Longer calls fetch the operands of kBlock tokens at once.  Decoding
// (T == 1) moves 36 bytes per channel: k, v, y and the state read and
// written; when C is a multiple of 4 and every pointer is 16-byte aligned a
// thread takes 4 channels with 16-byte accesses (a quarter of the
// instructions and of the waves).
#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr int kBlock = 8;

// Running state of a channel: Num = a e^p, Den = b e^p, p = kp - m w.
struct Run {
    float a, b, kp, m;
};

// output of token (k, v), then the update
__device__ __forceinline__ float token(Run &s, float w, float u, float k, float v) {
    const float p = fmaf(-s.m, w, s.kp);
    const float uk = u + k;
    const bool hist = p > uk;
    const float e = exp_fast(-fabsf(p - uk));
    const float eh = hist ? 1.0f : e, ec = hist ? e : 1.0f;
    const float y = fmaf(eh, s.a, ec * v) * __builtin_amdgcn_rcpf(fmaf(eh, s.b, ec));
    const float pw = fmaf(-(s.m + 1.0f), w, s.kp);
    const bool old = pw > k;
    const float f = exp_fast(-fabsf(pw - k));
    const float fo = old ? 1.0f : f, fn = old ? f : 1.0f;
    s.a = fmaf(fo, s.a, fn * v);
    s.b = fmaf(fo, s.b, fn);
    s.kp = old ? s.kp : k;
    s.m = old ? s.m + 1.0f : 0.0f;
    return y;
}

// The state to store: p = kp - m w rounded, and r = (kp - m w) - p exactly
// (up to a rounding of r itself; the product's error by a fused multiply-add,
// the difference's by the two-sum, with explicit roundings so that nothing is
// fused) folded into a and b as e^r = 1 + r.
__device__ __forceinline__ void store_state(const Run &s, float w, float &a, float &b,
                                            float &p) {
    const float mw = __fmul_rn(s.m, w);
    const float mw_err = fmaf(s.m, w, -mw);
    const float ps = __fsub_rn(s.kp, mw);
    const float bb = __fsub_rn(ps, s.kp);
    const float s_err = __fadd_rn(__fsub_rn(s.kp, __fsub_rn(ps, bb)), __fsub_rn(-mw, bb));
    const float r = __fsub_rn(s_err, mw_err);
    a = fmaf(s.a, r, s.a);
    b = fmaf(s.b, r, s.b);
    p = ps;
}

__global__ __launch_bounds__(256) void rwkv4_step_kernel(
    int B, int T, int C, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ w, const float *__restrict__ u, float *state,
    float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * C) return;  // no barriers in this kernel
    const int64_t b = i / C;
    const int c = (int)(i - b * C);
    float *sp = state + b * 3 * C + c;
    Run st{sp[0], sp[C], sp[2 * (int64_t)C], 0.0f};
    const float wc = w[c], uc = u[c];
    const float *kptr = k + b * (int64_t)T * C + c;
    const float *vptr = v + b * (int64_t)T * C + c;
    float *yptr = y + b * (int64_t)T * C + c;
    for (int t0 = 0; t0 < T; t0 += kBlock) {
        float kk[kBlock], vv[kBlock];
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            const bool in = t0 + j < T;
            kk[j] = in ? kptr[(int64_t)(t0 + j) * C] : 0.0f;
            vv[j] = in ? vptr[(int64_t)(t0 + j) * C] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            if (t0 + j >= T) break;
            yptr[(int64_t)(t0 + j) * C] = token(st, wc, uc, kk[j], vv[j]);
        }
    }
    store_state(st, wc, sp[0], sp[C], sp[2 * (int64_t)C]);
}

// One token, four channels per thread (C % 4 == 0, 16-byte aligned).
__global__ __launch_bounds__(256) void rwkv4_decode4_kernel(
    int B, int C4, const f32x4 *__restrict__ k, const f32x4 *__restrict__ v,
    const f32x4 *__restrict__ w, const f32x4 *__restrict__ u, f32x4 *state,
    f32x4 *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * C4) return;  // no barriers in this kernel
    const int64_t b = i / C4;
    const int c = (int)(i - b * C4);
    f32x4 *sp = state + b * 3 * C4 + c;
    const f32x4 sa = sp[0], sb = sp[C4], sq = sp[2 * (int64_t)C4];
    // k and v, read once per step, take non-temporal loads (7.2 -> 6.9 us per
    // step at 256 sequences x 4096 channels); the state, kept in the
    // last-level cache between steps, and w, u keep plain ones
    const f32x4 kk = __builtin_nontemporal_load(k + i), vv = __builtin_nontemporal_load(v + i);
    const f32x4 ww = w[c], uu = u[c];
    f32x4 yo, na, nb, np;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        Run st{sa[j], sb[j], sq[j], 0.0f};
        yo[j] = token(st, ww[j], uu[j], kk[j], vv[j]);
        float a_, b_, p_;
        store_state(st, ww[j], a_, b_, p_);
        na[j] = a_;
        nb[j] = b_;
        np[j] = p_;
    }
    y[i] = yo;
    sp[0] = na;
    sp[C4] = nb;
    sp[2 * (int64_t)C4] = np;
}

}  // namespace

hipError_t launch_rwkv4_step(int B, int T, int C, const float *k, const float *v,
                             const float *w, const float *u, float *state, float *y,
                             hipStream_t stream) {
    auto a16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (T == 1 && C % 4 == 0 && a16(k) && a16(v) && a16(w) && a16(u) && a16(state) &&
        a16(y)) {
        const int64_t n4 = (int64_t)B * (C / 4);
        hipLaunchKernelGGL(rwkv4_decode4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256),
                           0, stream, B, C / 4, (const f32x4 *)k, (const f32x4 *)v,
                           (const f32x4 *)w, (const f32x4 *)u, (f32x4 *)state, (f32x4 *)y);
        return hipGetLastError();
    }
    const int64_t n = (int64_t)B * C;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(rwkv4_step_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, B, T,
                       C, k, v, w, u, state, y);
    return hipGetLastError();
}

}  // namespace wkv
