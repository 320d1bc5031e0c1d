// rwkv4_scan.hip -- RWKV-4 WKV forward on gfx950.
//
// Operation (RWKV paper summary, cafeforensic.com zhuanlan/310315, section
// "Temporal structure for sequential data processing": decay e^{-w}, bonus
// e^{u}; section "Gradient stability and layer stacking": the WKV is a
// time-dependent softmax, evaluated in a numerically stable form):
//   y_t = (Num_{t-1} + e^{u+k_t} v_t) / (Den_{t-1} + e^{u+k_t})
//   Num_t = e^{-w} Num_{t-1} + e^{k_t} v_t,   Den_t = e^{-w} Den_{t-1} + e^{k_t}
// The state is kept as (a, b, p) with Num = a e^p, Den = b e^p, p the running
// maximum exponent, so every exponential taken is e^{-|d|} <= 1 and a, b
// stay finite for any k.
//
// Parallel form (section "Transformer-like parallelization": wkv_t is a
// serial scan).  The scan over time is associative: a block of n tokens
// acts on the state as X -> e^{-n w} X + (block summary).  One workgroup of
// 1024 lanes owns CB channels of one sequence and splits time into
// 1024/CB segments of SEG tokens each:
//   1. every lane loads its segment's k, v (kept in registers) and folds
//      them into a summary from the empty state;
//   2. summaries are scanned: inside a wave with cross-lane shuffles,
//      across waves through LDS, starting from the incoming state;
//   3. every lane replays its segment from its carry-in state, writing y.
// k and v are read from HBM once and y written once (12 bytes per
// token-channel), which is what bounds this kernel.  Longer sequences loop
// over passes of 1024/CB * SEG tokens with the state carried in LDS.
#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr float kEmptyP = -1e38f;  // exponent of the empty history

struct St {
    float a, b, p;
};

// Running state of a lane while it walks its tokens: Num = a e^p, Den = b e^p
// with p = kp - m w, where kp is the key (or incoming exponent) that last set
// the maximum and m the number of decay steps since.  Recomputing p with one
// fused multiply-add, instead of updating p -= w every step, keeps fp32
// rounding of large exponents from accumulating along the sequence.
struct Walk {
    float a, b, kp, m;
};

__device__ __forceinline__ Walk walk_from(const St &s) { return Walk{s.a, s.b, s.p, 0.0f}; }
__device__ __forceinline__ St walk_state(const Walk &s, float w) {
    return St{s.a, s.b, fmaf(-s.m, w, s.kp)};
}

// Fold one token (k, v) into the walk with per-step log-decay -w.
__device__ __forceinline__ void fold(Walk &s, float w, float k, float v) {
    const float pw = fmaf(-(s.m + 1.0f), w, s.kp);  // exponent of the decayed history
    const bool old_wins = pw > k;
    const float e = exp_fast(-fabsf(pw - k));  // e^{smaller - larger}
    const float e_old = old_wins ? 1.0f : e;
    const float e_new = old_wins ? e : 1.0f;
    s.a = e_old * s.a + e_new * v;
    s.b = e_old * s.b + e_new;
    s.kp = old_wins ? s.kp : k;
    s.m = old_wins ? s.m + 1.0f : 0.0f;
}

// Output of the current token (k, v) given the history walk s.
__device__ __forceinline__ float emit(const Walk &s, float w, float u, float k, float v) {
    const float p = fmaf(-s.m, w, s.kp);
    const float uk = u + k;
    const bool hist_wins = p > uk;
    const float e = exp_fast(-fabsf(p - uk));
    const float e_hist = hist_wins ? 1.0f : e;
    const float e_cur = hist_wins ? e : 1.0f;
    const float num = e_hist * s.a + e_cur * v;
    const float den = e_hist * s.b + e_cur;  // >= 1: one of the factors is 1
    return num * __builtin_amdgcn_rcpf(den);
}

// State after `first` followed by a block whose summary is `later` and whose
// total log-decay is -later_nw.
__device__ __forceinline__ St combine(const St &first, float later_nw, const St &later) {
    const float q = first.p - later_nw;
    const bool first_wins = q > later.p;
    const float e = exp_fast(-fabsf(q - later.p));
    const float e1 = first_wins ? 1.0f : e;
    const float e2 = first_wins ? e : 1.0f;
    St r;
    r.a = e1 * first.a + e2 * later.a;
    r.b = e1 * first.b + e2 * later.b;
    r.p = first_wins ? q : later.p;
    return r;
}

__device__ __forceinline__ St shfl_up_st(const St &s, int delta) {
    St r;
    r.a = __shfl_up(s.a, delta, 64);
    r.b = __shfl_up(s.b, delta, 64);
    r.p = __shfl_up(s.p, delta, 64);
    return r;
}

template <int CB, int SEG>
__global__ __launch_bounds__(1024) void rwkv4_scan_kernel(
    int T, int C, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ w, const float *__restrict__ u,
    const float *state_in, float *state_out, float *__restrict__ y) {
    constexpr int kThreads = 1024;
    constexpr int kWaves = kThreads / 64;
    constexpr int kSegs = kThreads / CB;  // segments per pass
    constexpr int kPass = kSegs * SEG;    // tokens per pass
    static_assert(64 % CB == 0, "a wave must hold whole segment groups");

    __shared__ St s_tot[kWaves][CB];
    __shared__ float s_totnw[kWaves][CB];
    __shared__ St s_pre[kWaves][CB];
    __shared__ St s_carry[CB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = tid % CB;
    const int seg = tid / CB;
    const int nblk = (C + CB - 1) / CB;
    const int c = (blockIdx.x % nblk) * CB + cl;
    const int b = blockIdx.x / nblk;
    const bool active = c < C;

    const float wc = active ? w[c] : 0.0f;
    const float uc = active ? u[c] : 0.0f;

    St carry;  // state entering the current pass
    if (state_in != nullptr && active) {
        const float *sp = state_in + (size_t)b * 3 * C + c;
        carry.a = sp[0];
        carry.b = sp[C];
        carry.p = sp[2 * (size_t)C];
    } else {
        carry.a = 0.0f;
        carry.b = 0.0f;
        carry.p = kEmptyP;
    }

    // Sequence base (uniform per workgroup) plus 32-bit per-lane offsets: one
    // sequence spans fewer than 2^31 elements (checked by the launcher).
    const size_t seq = (size_t)b * T * C;
    const float *kseq = k + seq;
    const float *vseq = v + seq;
    float *yseq = y + seq;
    for (int t0 = 0; t0 < T; t0 += kPass) {
        const int ts = t0 + seg * SEG;
        const int n = min(max(T - ts, 0), SEG);

        float kk[SEG], vv[SEG];
        int off = ts * C + c;
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            const bool ld = active && i < n;
            kk[i] = ld ? kseq[off] : 0.0f;
            vv[i] = ld ? vseq[off] : 0.0f;
            off += C;
        }

        // 1. segment summary from the empty state
        Walk wk = walk_from(St{0.0f, 0.0f, kEmptyP});
#pragma unroll
        for (int i = 0; i < SEG; ++i)
            if (i < n) fold(wk, wc, kk[i], vv[i]);
        const St sum = walk_state(wk, wc);
        const float nw = (float)n * wc;

        // 2a. inclusive scan over the segment groups of this wave
        St inc = sum;
        float incnw = nw;
#pragma unroll
        for (int off = CB; off < 64; off <<= 1) {
            const St prev = shfl_up_st(inc, off);
            const float prevnw = __shfl_up(incnw, off, 64);
            if (lane >= off) {
                inc = combine(prev, incnw, inc);
                incnw += prevnw;
            }
        }
        // exclusive prefix inside the wave
        St exc = shfl_up_st(inc, CB);
        float excnw = __shfl_up(incnw, CB, 64);
        if (lane < CB) {
            exc.a = 0.0f;
            exc.b = 0.0f;
            exc.p = kEmptyP;
            excnw = 0.0f;
        }
        if (lane >= 64 - CB) {
            s_tot[wave][cl] = inc;
            s_totnw[wave][cl] = incnw;
        }
        __syncthreads();

        // 2b. scan of the wave totals, seeded with the incoming state
        if (tid < CB) {
            St run = carry;
            for (int wv = 0; wv < kWaves; ++wv) {
                s_pre[wv][tid] = run;
                run = combine(run, s_totnw[wv][tid], s_tot[wv][tid]);
            }
            s_carry[tid] = run;
        }
        __syncthreads();

        // 3. replay the segment from its carry-in state
        Walk s = walk_from(combine(s_pre[wave][cl], excnw, exc));
        off = ts * C + c;
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            if (i < n) {
                const float yi = emit(s, wc, uc, kk[i], vv[i]);
                fold(s, wc, kk[i], vv[i]);
                if (active) yseq[off] = yi;
            }
            off += C;
        }
        carry = s_carry[cl];
        __syncthreads();  // s_pre / s_carry are rewritten by the next pass
    }

    if (state_out != nullptr && active && tid < CB) {
        float *sp = state_out + (size_t)b * 3 * C + c;
        sp[0] = carry.a;
        sp[C] = carry.b;
        sp[2 * (size_t)C] = carry.p;
    }
}

__global__ void rwkv4_empty_kernel(int B, int C, float *state) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)B * 3 * C;
    if (i < n) state[i] = ((i / C) % 3 == 2) ? kEmptyP : 0.0f;
}

__global__ void fill_kernel(float *dst, int64_t n, float value) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = value;
}

}  // namespace

hipError_t launch_rwkv4(int B, int T, int C, const float *k, const float *v,
                        const float *w, const float *u, const float *state_in,
                        float *state_out, float *y, hipStream_t stream) {
    constexpr int CB = 16, SEG = 16;
    dim3 grid((unsigned)(((C + CB - 1) / CB) * (int64_t)B));
    hipLaunchKernelGGL((rwkv4_scan_kernel<CB, SEG>), grid, dim3(1024), 0, stream,
                       T, C, k, v, w, u, state_in, state_out, y);
    return hipGetLastError();
}

hipError_t launch_rwkv4_empty_state(int B, int C, float *state, hipStream_t stream) {
    const int64_t n = (int64_t)B * 3 * C;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(rwkv4_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       B, C, state);
    return hipGetLastError();
}

hipError_t launch_fill(float *dst, int64_t n, float value, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n,
                       value);
    return hipGetLastError();
}

}  // namespace wkv
