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
// acts on the state as X -> e^{-n w} X + (block summary).  A workgroup of
// 512 lanes owns 32 channels (one 128-byte row of k, v, y per token) of one
// sequence and walks the sequence in passes of 16 segments x 16 tokens:
//   1. every lane folds its segment's k, v (held in registers) into a
//      summary from the empty state;
//   2. summaries are scanned: inside a wave with cross-lane shuffles,
//      across waves through LDS, starting from the state entering the pass;
//   3. every lane replays its segment from its carry-in state, writing y.
// The next pass's k and v are in flight while a pass computes.  k and v are
// read from HBM once and y written once (12 bytes per token-channel).
#include <type_traits>

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

template <int SEG>
struct Seg {  // one lane's tokens of a pass
    float k[SEG], v[SEG];
};

template <int NT, int CB, int SEG>
__global__ __launch_bounds__(NT) void rwkv4_scan_kernel(
    int T, int C, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ w, const float *__restrict__ u,
    const float *state_in, float *state_out, float *__restrict__ y) {
    constexpr int kWaves = NT / 64;
    constexpr int kSegs = NT / CB;     // segments per pass
    constexpr int kPass = kSegs * SEG; // tokens per pass
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
    const int c0 = (blockIdx.x % nblk) * CB;
    const int c = c0 + cl;
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

    // Each pass addresses its rows through a raw buffer resource (uniform,
    // 64-bit base) with 32-bit per-lane byte offsets.  Rows past T and lanes
    // past C fall outside the resource: their loads return zero and their
    // stores are dropped, so loads and stores need no branches and the next
    // pass's loads stay in flight while a pass computes.
    const size_t seq = (size_t)b * T * C;
    const uint32_t row_bytes = (uint32_t)C * 4u;
    const uint32_t lane_off = active ? (uint32_t)(seg * SEG) * row_bytes + (uint32_t)c * 4u
                                     : 0x80000000u;
    auto rsrc = [&](const float *base, int t0) {
        const uint32_t rows = (uint32_t)min(kPass, T - t0);
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + seq + (size_t)t0 * C), (short)0,
                                                 (int)(rows * row_bytes), 0x00020000);
    };

    auto load = [&](Seg<SEG> &d, int t0) {
        const auto rk = rsrc(k, t0), rv = rsrc(v, t0);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            d.k[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rk, lane_off + i * row_bytes, 0, 0));
            d.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rv, lane_off + i * row_bytes, 0, 0));
        }
    };

    // FULL: every row of the pass exists (uniform over the workgroup)
    auto pass_impl = [&](int t0, const Seg<SEG> &d, auto full_tag) {
        constexpr bool full = decltype(full_tag)::value;
        const int ts = t0 + seg * SEG;
        const int n = full ? SEG : min(max(T - ts, 0), SEG);

        // 1. segment summary from the empty state
        Walk wk = walk_from(St{0.0f, 0.0f, kEmptyP});
#pragma unroll
        for (int i = 0; i < SEG; ++i)
            if (full || i < n) fold(wk, wc, d.k[i], d.v[i]);
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
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                s_pre[wv][tid] = run;
                run = combine(run, s_totnw[wv][tid], s_tot[wv][tid]);
            }
            s_carry[tid] = run;
        }
        __syncthreads();

        // 3. replay the segment from its carry-in state
        Walk s = walk_from(combine(s_pre[wave][cl], excnw, exc));
        const auto ry = rsrc(y, t0);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            if (full || i < n) {
                const float yi = emit(s, wc, uc, d.k[i], d.v[i]);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yi), ry,
                                                      lane_off + i * row_bytes, 0, 0);
                fold(s, wc, d.k[i], d.v[i]);
            }
        }
        carry = s_carry[cl];
        __syncthreads();  // s_pre / s_carry are rewritten by the next pass
    };
    auto pass = [&](int t0, const Seg<SEG> &d) {
        if (t0 + kPass <= T) pass_impl(t0, d, std::true_type{});
        else pass_impl(t0, d, std::false_type{});
    };

    // passes, the next one's k and v in flight while the current one computes
    Seg<SEG> bufA, bufB;
    if (T > 0) load(bufA, 0);
    for (int t0 = 0; t0 < T; t0 += 2 * kPass) {
        if (t0 + kPass < T) load(bufB, t0 + kPass);
        pass(t0, bufA);
        if (t0 + kPass < T) {
            if (t0 + 2 * kPass < T) load(bufA, t0 + 2 * kPass);
            pass(t0 + kPass, bufB);
        }
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
    // 32 channels (128-byte rows) x 16 segments of 16 tokens per workgroup
    constexpr int NT = 512, CB = 32, SEG = 16;
    const int64_t blocks = (int64_t)B * ((C + CB - 1) / CB);
    hipLaunchKernelGGL((rwkv4_scan_kernel<NT, CB, SEG>), dim3((unsigned)blocks), dim3(NT), 0,
                       stream, T, C, k, v, w, u, state_in, state_out, y);
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
