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
// Decoding (T == 1) moves 36 bytes per channel: k, v, y and the state read
// and written.  Longer calls fetch the operands of kBlock tokens at once.
#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr int kBlock = 8;

__global__ __launch_bounds__(256) void rwkv4_step_kernel(
    int B, int T, int C, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ w, const float *__restrict__ u, float *state,
    float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * C) return;  // no barriers in this kernel
    const int64_t b = i / C;
    const int c = (int)(i - b * C);
    float *sp = state + b * 3 * C + c;
    float sa = sp[0], sb = sp[C], kp = sp[2 * (int64_t)C], m = 0.0f;
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
            const float kt = kk[j], vt = vv[j];
            // output
            const float p = fmaf(-m, wc, kp);
            const float uk = uc + kt;
            const bool hist = p > uk;
            const float e = exp_fast(-fabsf(p - uk));
            const float eh = hist ? 1.0f : e, ec = hist ? e : 1.0f;
            yptr[(int64_t)(t0 + j) * C] =
                fmaf(eh, sa, ec * vt) * __builtin_amdgcn_rcpf(fmaf(eh, sb, ec));
            // update
            const float pw = fmaf(-(m + 1.0f), wc, kp);
            const bool old = pw > kt;
            const float f = exp_fast(-fabsf(pw - kt));
            const float fo = old ? 1.0f : f, fn = old ? f : 1.0f;
            sa = fmaf(fo, sa, fn * vt);
            sb = fmaf(fo, sb, fn);
            kp = old ? kp : kt;
            m = old ? m + 1.0f : 0.0f;
        }
    }
    // p = kp - m w rounded, and r = (kp - m w) - p exactly (up to a rounding
    // of r itself): the product's error by a fused multiply-add, the
    // difference's by the two-sum; explicit roundings keep them unfused
    const float mw = __fmul_rn(m, wc);
    const float mw_err = fmaf(m, wc, -mw);
    const float ps = __fsub_rn(kp, mw);
    const float bb = __fsub_rn(ps, kp);
    const float s_err = __fadd_rn(__fsub_rn(kp, __fsub_rn(ps, bb)), __fsub_rn(-mw, bb));
    const float r = __fsub_rn(s_err, mw_err);
    sp[0] = fmaf(sa, r, sa);
    sp[C] = fmaf(sb, r, sb);
    sp[2 * (int64_t)C] = ps;
}

}  // namespace

hipError_t launch_rwkv4_step(int B, int T, int C, const float *k, const float *v,
                             const float *w, const float *u, float *state, float *y,
                             hipStream_t stream) {
    const int64_t n = (int64_t)B * C;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(rwkv4_step_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, B, T,
                       C, k, v, w, u, state, y);
    return hipGetLastError();
}

}  // namespace wkv
