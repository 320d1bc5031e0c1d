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
// acts on the state as X -> e^{-n w} X + (block summary).  A workgroup
// handles one pass of 256 tokens of 32 channels (one 128-byte row of k, v, y
// per token) of one sequence, as 16 segments x 16 tokens:
//   1. every lane folds its segment's k, v (held in registers) into a
//      summary from the empty state;
//   2. summaries are scanned: inside a wave with cross-lane shuffles, across
//      waves through LDS, giving the pass's own aggregate;
//   3. the state entering the pass comes from the passes before it (a
//      decoupled look-back: each workgroup publishes its aggregate, then its
//      inclusive state, and the next ones combine what they find);
//   4. every lane replays its segment from its carry-in state, writing y.
// All passes of a sequence run at once, so every CU has work even when the
// sequences x channel blocks alone would not fill the chip.  k and v are read
// from HBM once and y written once (12 bytes per token-channel).
#include <algorithm>
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

// Workspace record of one workgroup of a chain: the aggregate of its pass
// (state after the pass from the empty state) and its inclusive state, each
// (a, b, p) for CB channels, plus a flag: 0 nothing, 1 aggregate, 2 inclusive.
constexpr unsigned kAgg = 1u, kIncl = 2u;
// Bound on the polls of a predecessor's flag (about a second): predecessors
// have lower workgroup indices and are dispatched first, so the wait always
// ends; the bound only guarantees that the kernel terminates.
constexpr int kSpinLimit = 1 << 20;

template <int NT, int CB, int SEG>
__global__ __launch_bounds__(NT) void rwkv4_chain_kernel(
    int T, int t_begin, int nq, int C, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ w, const float *__restrict__ u,
    const float *state_in, float *state_out, float *__restrict__ y, float *recs,
    unsigned *flags, unsigned *err) {
    constexpr int kWaves = NT / 64;
    constexpr int kSegs = NT / CB;     // segments per pass
    constexpr int kPass = kSegs * SEG; // tokens per pass
    static_assert(64 % CB == 0, "a wave must hold whole segment groups");

    __shared__ St s_tot[kWaves][CB];
    __shared__ float s_totnw[kWaves][CB];
    __shared__ St s_pre[kWaves][CB];
    __shared__ float s_prenw[kWaves][CB];
    __shared__ St s_excl[CB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = tid % CB;
    const int seg = tid / CB;
    const int nblk = (C + CB - 1) / CB;
    const int units = gridDim.x / nq;        // (sequence, channel block) pairs
    const int unit = blockIdx.x % units;
    const int q = blockIdx.x / units;        // pass of this workgroup in the chain
    const int c = (unit % nblk) * CB + cl;
    const int b = unit / nblk;
    const bool active = c < C;
    const int t0 = t_begin + q * kPass;

    const float wc = active ? w[c] : 0.0f;
    const float uc = active ? u[c] : 0.0f;

    // Rows of the pass through a raw buffer resource (uniform 64-bit base,
    // 32-bit per-lane byte offsets): rows past T and lanes past C read zero
    // and drop their stores.
    const size_t seq = (size_t)b * T * C;
    const uint32_t row_bytes = (uint32_t)C * 4u;
    const uint32_t lane_off = active ? (uint32_t)(seg * SEG) * row_bytes + (uint32_t)c * 4u
                                     : 0x80000000u;
    auto rsrc = [&](const float *base) {
        const uint32_t rows = (uint32_t)min(kPass, T - t0);
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + seq + (size_t)t0 * C), (short)0,
                                                 (int)(rows * row_bytes), 0x00020000);
    };
    Seg<SEG> d;
    {
        const auto rk = rsrc(k), rv = rsrc(v);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            d.k[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rk, lane_off + i * row_bytes, 0, 0));
            d.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rv, lane_off + i * row_bytes, 0, 0));
        }
    }

    // Chain records and flags are only accessed with agent-scope relaxed
    // atomics, which read and write at the device's coherence point: they
    // need no cache write-back or invalidation (a release/acquire pair would
    // write back and invalidate the whole L2 on every poll and publish).
    // Order comes from waiting for the record stores to complete before the
    // flag is stored, and on the reading side from reading the records only
    // after the flag load has returned.
    auto ld = [](const void *p) {
        return __hip_atomic_load((unsigned *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto st = [](void *p, unsigned val) {
        __hip_atomic_store((unsigned *)p, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // wait until a predecessor's flag reaches `atleast`; returns the flag
    auto wait_flag = [&](const unsigned *f, unsigned atleast) -> unsigned {
        unsigned val;
        int polls = 0;
        while ((val = ld(f)) < atleast) {
            __builtin_amdgcn_s_sleep(4);
            if (++polls > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return atleast;
            }
        }
        return val;
    };
    auto publish = [&](int link, int slot, const St &s, unsigned flag) {
        float *rec = recs + (size_t)link * 6 * CB + slot * 3 * CB;
        st(rec + tid, __float_as_uint(s.a));
        st(rec + CB + tid, __float_as_uint(s.b));
        st(rec + 2 * CB + tid, __float_as_uint(s.p));
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the records have landed
        __asm__ volatile("" ::: "memory");
        if (tid == 0) st(flags + link, flag);
    };
    auto record = [&](int link, int slot) {
        const float *rec = recs + (size_t)link * 6 * CB + slot * 3 * CB;
        return St{__uint_as_float(ld(rec + tid)), __uint_as_float(ld(rec + CB + tid)),
                  __uint_as_float(ld(rec + 2 * CB + tid))};
    };

    // FULL: every row of the pass exists (uniform over the workgroup)
    auto pass = [&](auto full_tag) {
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

        // 2b. prefixes of the wave totals from the empty state, the pass's
        // aggregate, and the state entering the pass from the chain
        if (tid < CB) {
            St run{0.0f, 0.0f, kEmptyP};
            float rnw = 0.0f;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                s_pre[wv][tid] = run;
                s_prenw[wv][tid] = rnw;
                run = combine(run, s_totnw[wv][tid], s_tot[wv][tid]);
                rnw += s_totnw[wv][tid];
            }
            const int link = q * units + unit;
            St excl;
            if (q == 0) {
                excl = St{0.0f, 0.0f, kEmptyP};
                if (state_in != nullptr && active) {
                    const float *sp = state_in + (size_t)b * 3 * C + c;
                    excl = St{sp[0], sp[C], sp[2 * (size_t)C]};
                }
            } else {
                if (q + 1 < nq) publish(link, 0, run, kAgg);
                // walk back: aggregates until an inclusive state (pass 0
                // publishes only its inclusive state, so the walk ends there)
                St acc{0.0f, 0.0f, kEmptyP};
                float accnw = 0.0f;
                for (int j = q - 1;; --j) {
                    const int lj = j * units + unit;
                    if (wait_flag(flags + lj, kAgg) >= kIncl || j == 0) {
                        excl = combine(record(lj, 1), accnw, acc);
                        break;
                    }
                    acc = combine(record(lj, 0), accnw, acc);
                    accnw += (float)kPass * wc;  // predecessors are whole passes
                }
            }
            const St incl = combine(excl, rnw, run);
            if (q + 1 < nq) {
                publish(link, 1, incl, kIncl);
            } else {
                if (state_out != nullptr && active) {
                    float *sp = state_out + (size_t)b * 3 * C + c;
                    sp[0] = incl.a;
                    sp[C] = incl.b;
                    sp[2 * (size_t)C] = incl.p;
                }
                // A workgroup publishes its inclusive state only after its
                // walk, so once every flag of the chain is inclusive no walk
                // reads them any more: only then clear them for the next
                // launch (clearing one while a later walk may still pass it
                // would strand that walk).
                if (tid == 0) {
                    for (int j = 0; j + 1 < nq; ++j) wait_flag(flags + j * units + unit, kIncl);
                    for (int j = 0; j + 1 < nq; ++j) st(flags + j * units + unit, 0u);
                }
            }
            s_excl[tid] = excl;
        }
        __syncthreads();

        // 3. replay the segment from its carry-in state
        Walk s = walk_from(combine(s_excl[cl], s_prenw[wave][cl] + excnw,
                                   combine(s_pre[wave][cl], excnw, exc)));
        const auto ry = rsrc(y);
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            if (full || i < n) {
                const float yi = emit(s, wc, uc, d.k[i], d.v[i]);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yi), ry,
                                                      lane_off + i * row_bytes, 0, 0);
                fold(s, wc, d.k[i], d.v[i]);
            }
        }
    };
    if (t0 + kPass <= T) pass(std::true_type{});
    else pass(std::false_type{});
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
    // one pass of 32 channels (128-byte rows) x 16 segments of 16 tokens per
    // workgroup; the passes of a (sequence, channel block) form a chain
    constexpr int NT = 512, CB = 32, SEG = 16, kPass = (NT / CB) * SEG;
    const int64_t units = (int64_t)B * ((C + CB - 1) / CB);
    const int64_t passes = (T + kPass - 1) / kPass;
    // a launch covers at most kMaxLinks workgroups; longer sequences take
    // several launches, the state carried between them in the workspace
    constexpr int64_t kMaxLinks = 8192;
    const int64_t per_launch = std::max<int64_t>(1, std::min<int64_t>(passes, kMaxLinks / units));
    const bool windows = per_launch < passes;
    // layout: flags (a fixed region, so the cleared flags of one launch are
    // the cleared flags of the next whatever its shape), records, carry
    const int64_t links = per_launch * units;
    const size_t flag_bytes = (size_t)kMaxLinks * 4 + 256;
    const size_t rec_bytes = (size_t)links * 6 * CB * 4;
    const size_t carry_bytes = windows ? (size_t)B * 3 * C * 4 : 0;
    char *ws = nullptr;
    hipError_t e = stream_workspace(kWsRwkv4Chain, stream, flag_bytes + rec_bytes + carry_bytes,
                                    (void **)&ws);
    if (e != hipSuccess) return e;
    unsigned *flags = (unsigned *)ws;
    unsigned *err = flags + kMaxLinks;
    float *recs = (float *)(ws + flag_bytes);
    float *carry = (float *)(ws + flag_bytes + rec_bytes);
    for (int64_t q0 = 0; q0 < passes; q0 += per_launch) {
        const int64_t nq = std::min(per_launch, passes - q0);
        const float *si = q0 == 0 ? state_in : carry;
        float *so = q0 + nq == passes ? state_out : carry;
        hipLaunchKernelGGL((rwkv4_chain_kernel<NT, CB, SEG>), dim3((unsigned)(nq * units)),
                           dim3(NT), 0, stream, T, (int)(q0 * kPass), (int)nq, C, k, v, w, u,
                           si, so, y, recs, flags, err);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
