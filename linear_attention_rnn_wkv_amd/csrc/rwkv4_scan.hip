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
//   1. every lane sums its segment's k, v (held in registers) into a
//      summary from the empty state, relative to the segment's largest
//      exponent;
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
#include <cstddef>
#include <type_traits>

#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr float kEmptyP = -1e38f;  // exponent of the empty history
// cache policy of the k and v loads, each read once: non-temporal.  At
// B8 T1024 C768 this took the launch from 22.3 to 19.4 us, inputs from HBM.
constexpr int kReadOnce = 2;
// Largest |u - w| of a wave's channels for which the replay takes the
// output from the fold's exponential (fold_emit): E = e^{u-w} stays within
// [e^-30, e^30], so E v is finite for |v| < 3e25 and no term underflows
// before it is negligible.  Other waves take the output's own exponential.
constexpr float kFusedSpan = 30.0f;


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

// Output of token (k, v) and the fold of it into s, sharing the fold's one
// exponential.  With P = max(p - w, k) the fold's reference, the output's
// numerator and denominator multiplied by e^{-w-P} are
//   a e_old + E e_new v   and   b e_old + E e_new,   E = e^{u-w},
// where e_old = e^{p-w-P}, e_new = e^{k-P} are the fold's own factors (one of
// them is 1).  Every term is positive, so nothing cancels; E scales the
// current token's term, so the caller keeps |u - w| small enough that
// neither E nor E v leaves the fp32 range (see the replay).
__device__ __forceinline__ float fold_emit(Walk &s, float w, float E, float k, float v) {
    const float pw = fmaf(-(s.m + 1.0f), w, s.kp);
    const bool old_wins = pw > k;
    const float e = exp_fast(-fabsf(pw - k));
    const float e_old = old_wins ? 1.0f : e;
    const float e_new = old_wins ? e : 1.0f;
    const float ta = e_old * s.a, tb = e_old * s.b, ee = E * e_new;
    const float y = fmaf(ee, v, ta) * __builtin_amdgcn_rcpf(tb + ee);
    s.a = fmaf(e_new, v, ta);
    s.b = tb + e_new;
    s.kp = old_wins ? s.kp : k;
    s.m = old_wins ? s.m + 1.0f : 0.0f;
    return y;
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

// Workspace of the chains.  A record of one workgroup holds the aggregate of
// its pass (state after the pass from the empty state) and its inclusive
// state, each (a, b, p) for CB channels.  Every record word is 64 bits: the
// value in the low half and the tag epoch + 1 in the high half, so a word
// read with the current tag was written by this launch and needs no separate
// flag.  Once every workgroup of a launch holds the epoch it is advanced,
// which makes all records of the launch stale without clearing them.
//
// When that is: the last pass of a chain finishes its walk only after every
// pass of the chain has published a tagged record (walks reach back to an
// inclusive state, whose publisher walked before it, down to pass 0), i.e.
// after each of them has read the epoch.  The last passes of the chains then
// arrive at one of kWsGroups counters of the control block (WsCtrl), and
// the last arrival of each group at a total; the last arrival there advances
// the epoch.  Two levels keep any one counter to a few dozen atomics (a
// single counter hit by every workgroup serialises and stalls the memory
// system).
using Ctrl = WsCtrl;
constexpr int kGroups = kWsGroups;
// Bound on the polls of a predecessor's record (about a second):
// predecessors have lower workgroup indices and are dispatched first, so the
// wait always ends; the bound only guarantees that the kernel terminates.
constexpr int kSpinLimit = 1 << 20;

// Registers are capped so that three 512-thread workgroups (six waves per
// SIMD) share a CU: then every pass of the benchmark-sized launches is
// resident at once and no chain waits for a workgroup slot.
template <int NT, int CB, int SEG>
__global__ __launch_bounds__(NT, 3 * NT / 256) void rwkv4_chain_kernel(
    int T, int t_begin, int nq, int C, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ w, const float *__restrict__ u,
    const float *state_in, float *state_out, float *__restrict__ y,
    unsigned long long *recs, Ctrl *ctrl) {
    constexpr int kWaves = NT / 64;
    constexpr int kSegs = NT / CB;     // segments per pass
    constexpr int kPass = kSegs * SEG; // tokens per pass
    static_assert(64 % CB == 0, "a wave must hold whole segment groups");
    static_assert(kWaves >= 2, "waves 0 and 1 split the chain work");

    __shared__ St s_tot[kWaves][CB];
    __shared__ float s_totnw[kWaves][CB];
    __shared__ St s_excl[CB];
    __shared__ unsigned s_epoch;

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
                                                   rk, lane_off + i * row_bytes, 0, kReadOnce));
            d.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rv, lane_off + i * row_bytes, 0, kReadOnce));
        }
    }

    // The control block and the records are only accessed with agent-scope
    // relaxed atomics, which read and write at the device's coherence point,
    // so they need no cache write-back or invalidation.  A record word is
    // valid on its own (its tag), so a publisher never waits for its stores.
    using u64 = unsigned long long;
    auto ld32 = [](const unsigned *p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto ld64 = [](const u64 *p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto st64 = [](u64 *p, u64 val) {
        __hip_atomic_store(p, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // record words of channel cl: link, slot 0 aggregate / 1 inclusive
    auto word = [&](int link, int slot, int comp) {
        return recs + ((size_t)link * 6 + slot * 3 + comp) * CB + cl;
    };
    auto publish = [&](int link, int slot, const St &s, unsigned tag) {
        const u64 hi = (u64)tag << 32;
        st64(word(link, slot, 0), hi | __float_as_uint(s.a));
        st64(word(link, slot, 1), hi | __float_as_uint(s.b));
        st64(word(link, slot, 2), hi | __float_as_uint(s.p));
    };
    // the epoch is read with the operands
    unsigned epoch = 0;
    if (tid == 0 && nq > 1) epoch = ld32(&ctrl->epoch.n);

    // FULL: every row of the pass exists (uniform over the workgroup)
    auto pass = [&](auto full_tag) {
        constexpr bool full = decltype(full_tag)::value;
        const int ts = t0 + seg * SEG;
        const int n = full ? SEG : min(max(T - ts, 0), SEG);

        // 1. segment summary from the empty state: Num = sum_i e^{z_i} v_i
        // with z_i = k_i - (n-1-i) w, taken relative to the largest z (one
        // exponential per token, each term <= 1, no running rescale)
        St sum;
        {
            float z[SEG], zmax = kEmptyP;
#pragma unroll
            for (int i = 0; i < SEG; ++i)
                if (full || i < n) {
                    z[i] = fmaf(-(float)((full ? SEG : n) - 1 - i), wc, d.k[i]);
                    zmax = fmaxf(zmax, z[i]);
                }
            float sa = 0.0f, sb = 0.0f;
#pragma unroll
            for (int i = 0; i < SEG; ++i)
                if (full || i < n) {
                    const float e = exp_fast(z[i] - zmax);
                    sa = fmaf(e, d.v[i], sa);
                    sb += e;
                }
            sum = St{sa, sb, zmax};
        }
        const float nw = (float)n * wc;
        if (tid == 0) s_epoch = epoch;
        unsigned arrived = 0;  // thread 0 of a chain's last pass: its group's count

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

        // 2b. every lane: the prefix of the wave totals before its wave
        // (from the empty state) and the pass's aggregate
        St pre{0.0f, 0.0f, kEmptyP}, run = pre;
        float prenw = 0.0f, rnw = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
            if (wv == wave) {
                pre = run;
                prenw = rnw;
            }
            run = combine(run, s_totnw[wv][cl], s_tot[wv][cl]);
            rnw += s_totnw[wv][cl];
        }

        // 2c. the state entering the pass, from the chain.  Wave 1
        // publishes the aggregate and wave 0 walks back: stores count with
        // loads in a wave's memory counter, so a wave that waits for its
        // polls would also wait for its own stores to complete.
        const int link = q * units + unit;
        const unsigned tag = s_epoch + 1u;
        if (wave == 1 && lane < CB && q > 0 && q + 1 < nq) publish(link, 0, run, tag);
        if (tid < CB) {
            St excl;
            if (q == 0) {
                excl = St{0.0f, 0.0f, kEmptyP};
                if (state_in != nullptr && active) {
                    const float *sp = state_in + (size_t)b * 3 * C + c;
                    excl = St{sp[0], sp[C], sp[2 * (size_t)C]};
                }
            } else {
                // walk back: aggregates until an inclusive state (pass 0
                // publishes only its inclusive state, so the walk ends
                // there).  Every channel reads a predecessor's inclusive
                // state, then its aggregate; while neither is complete, lane
                // 0 alone polls its own two words (two loads per poll).
                auto ok = [&](u64 x) { return (unsigned)(x >> 32) == tag; };
                auto val = [](u64 x) { return __uint_as_float((unsigned)x); };
                St acc{0.0f, 0.0f, kEmptyP};
                float accnw = 0.0f;
                int polls = 0;
                auto give_up = [&]() {  // cannot happen: see kSpinLimit
                    if (++polls <= kSpinLimit) return false;
                    ws_fail(ctrl);
                    return true;
                };
                excl = acc;
                for (int j = q - 1;;) {
                    const int lj = j * units + unit;
                    {
                        const u64 xa = ld64(word(lj, 1, 0)), xb = ld64(word(lj, 1, 1)),
                                  xp = ld64(word(lj, 1, 2));
                        if (__all(ok(xa) && ok(xb) && ok(xp))) {
                            excl = combine(St{val(xa), val(xb), val(xp)}, accnw, acc);
                            break;
                        }
                    }
                    if (j > 0) {
                        const u64 xa = ld64(word(lj, 0, 0)), xb = ld64(word(lj, 0, 1)),
                                  xp = ld64(word(lj, 0, 2));
                        if (__all(ok(xa) && ok(xb) && ok(xp))) {
                            acc = combine(St{val(xa), val(xb), val(xp)}, accnw, acc);
                            accnw += (float)kPass * wc;  // predecessors are whole passes
                            --j;
                            continue;
                        }
                    }
                    bool late = false;
                    for (;;) {
                        __builtin_amdgcn_s_sleep(2);
                        int shown = 0;
                        if (tid == 0)
                            shown = ok(ld64(word(lj, 1, 2))) || (j > 0 && ok(ld64(word(lj, 0, 2))));
                        if (__shfl(shown, 0, 64) || (late = give_up())) break;
                    }
                    if (late) {  // go on from NaN: the pass's outputs show it
                        const float nan = __builtin_nanf("");
                        excl = St{nan, nan, nan};
                        break;
                    }
                }
            }
            const St incl = combine(excl, rnw, run);
            if (q + 1 < nq) {
                publish(link, 1, incl, tag);
            } else if (state_out != nullptr && active) {
                float *sp = state_out + (size_t)b * 3 * C + c;
                sp[0] = incl.a;
                sp[C] = incl.b;
                sp[2 * (size_t)C] = incl.p;
            }
            s_excl[tid] = excl;
            // after the walk (see Ctrl); the count is only read at the end
            if (tid == 0 && q > 0 && q + 1 == nq)
                arrived = __hip_atomic_fetch_add(&ctrl->group[unit % kGroups].n, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();

        // 3. replay the segment from its carry-in state
        Walk s = walk_from(combine(s_excl[cl], prenw + excnw, combine(pre, excnw, exc)));
        const auto ry = rsrc(y);
        if (!__any(!(fabsf(uc - wc) <= kFusedSpan))) {  // (uniform over the wave)
            const float E = exp_fast(uc - wc);
#pragma unroll
            for (int i = 0; i < SEG; ++i) {
                if (full || i < n) {
                    const float yi = fold_emit(s, wc, E, d.k[i], d.v[i]);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yi), ry,
                                                          lane_off + i * row_bytes, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < SEG; ++i) {
                if (full || i < n) {
                    const float yi = emit(s, wc, uc, d.k[i], d.v[i]);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, yi), ry,
                                                          lane_off + i * row_bytes, 0, 0);
                    fold(s, wc, d.k[i], d.v[i]);
                }
            }
        }

        // the last arrival of a group counts at the total, and the last
        // arrival there advances the epoch (tag 0 stays unused)
        if (tid == 0 && q > 0 && q + 1 == nq) {
            const int g = unit % kGroups;
            if (arrived == (unsigned)((units - 1 - g) / kGroups)) {
                __hip_atomic_store(&ctrl->group[g].n, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                const unsigned t = __hip_atomic_fetch_add(&ctrl->total.n, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                if (t + 1 == (unsigned)min(units, kGroups)) {
                    __hip_atomic_store(&ctrl->total.n, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    const unsigned next = s_epoch + 1u == 0xffffffffu ? 0u : s_epoch + 1u;
                    __hip_atomic_store(&ctrl->epoch.n, next, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
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

size_t rwkv4_workspace_bytes(int B, int T, int C) {
    constexpr int NT = 512, CB = 32, SEG = 16, kPass = (NT / CB) * SEG;
    const int64_t units = (int64_t)B * ((C + CB - 1) / CB);
    const int64_t passes = (T + kPass - 1) / kPass;
    const int64_t per_launch = std::max<int64_t>(1, std::min<int64_t>(passes, 8192 / units));
    if (passes <= 1) return 0;
    return kWsCtrlBytes + (size_t)(per_launch * units) * 6 * CB * 8 +
           (per_launch < passes ? (size_t)B * 3 * C * 4 : 0);
}

hipError_t launch_rwkv4(int B, int T, int C, const float *k, const float *v,
                        const float *w, const float *u, const float *state_in,
                        float *state_out, float *y, void *wsp, hipStream_t stream) {
    constexpr int NT = 512, CB = 32, SEG = 16, kPass = (NT / CB) * SEG;
    const int64_t units = (int64_t)B * ((C + CB - 1) / CB);
    const int64_t passes = (T + kPass - 1) / kPass;
    constexpr int64_t kMaxLinks = 8192;
    const int64_t per_launch = std::max<int64_t>(1, std::min<int64_t>(passes, kMaxLinks / units));
    const int64_t links = per_launch * units;
    const size_t rec_bytes = (size_t)links * 6 * CB * 8;
    char *ws = (char *)wsp;
    Ctrl *ctrl = (Ctrl *)ws;
    unsigned long long *recs = ws ? (unsigned long long *)(ws + kWsCtrlBytes) : nullptr;
    float *carry = ws ? (float *)(ws + kWsCtrlBytes + rec_bytes) : nullptr;
    for (int64_t q0 = 0; q0 < passes; q0 += per_launch) {
        const int64_t nq = std::min(per_launch, passes - q0);
        const float *si = q0 == 0 ? state_in : carry;
        float *so = q0 + nq == passes ? state_out : carry;
        hipLaunchKernelGGL((rwkv4_chain_kernel<NT, CB, SEG>), dim3((unsigned)(nq * units)),
                           dim3(NT), 0, stream, T, (int)(q0 * kPass), (int)nq, C, k, v, w, u,
                           si, so, y, recs, ctrl);
        hipError_t e = hipGetLastError();
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
