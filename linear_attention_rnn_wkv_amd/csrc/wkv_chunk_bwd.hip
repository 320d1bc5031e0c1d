// wkv_chunk_bwd.hip -- Eagle (RWKV-5) / Finch (RWKV-6) WKV backward in
// time-parallel (chunked) mode on gfx950, bf16 MFMA with fp32 accumulation.
//
// The forward (RWKV-5/6 summary, blob.wenxiaobai.com, section 4 notation;
// 4.1.2 "Eagle time mixing"; 4.2.2 "Finch time mixing"), per head:
//   o_t = r_t S_{t-1} + (r_t diag(u) k_t^T) v_t,  S_t = diag(w_t) S_{t-1} + k_t^T v_t,
//   w_t = exp(-exp(x_t)) = e^{g_t}.
// Given dL/do and dL/dS_T, the gradients are, with S_c the state entering a
// chunk of L = 64 tokens, dS_end the gradient of the state leaving it, Lam
// the chunk-relative cumulative log-decay (log2 units), r~ = r e^{Lam_{t-1} -
// Lam_L}, k^ = k e^{Lam_L - Lam_s}, A[t][s] = r~_t . k^_s and dA[t][s] =
// do_t . v_s for s < t (strictly causal), beta_t = r_t diag(u) k_t^T and
// dbeta_t = do_t . v_t:
//   dr_t = e^{Lam_{t-1}-Lam_L} [sum_s dA[t][s] k^_s + do_t (diag(e^{Lam_L}) S_c)^T]
//          + u k_t dbeta_t
//   dk_s = e^{Lam_L-Lam_s} [sum_t dA[t][s] r~_t + v_s dS_end^T] + u r_s dbeta_s
//   dv_s = sum_t A[t][s] do_t + k^_s dS_end + beta_s do_s
//   dS_c = diag(e^{Lam_L}) (dS_end + R~^T dO),   du = sum_t r_t k_t dbeta_t.
// The decay gradient needs no state: writing dr^a, dk^a for dr, dk without
// their bonus terms, every (query t, key s) pair with s < m < t carries the
// decay of token m, and summing over pairs gives
//   dg_m = sum_{t > m} r_t dr^a_t - sum_{s >= m} k_s dk^a_s + sum_j (dS_T o S_T)[.][j],
// the last term being the final state seen as a query after the last token.
// It is a suffix sum over the sequence, carried across chunks as the sweep
// runs backwards; dx = dg g (g = -e^x).
//
// Passes: the forward kernel first stores the state entering every chunk
// (and the final state) in the workspace; this kernel then runs one
// workgroup of eight waves (two per SIMD) per (sequence, head) over the
// chunks from last to first, carrying dS in registers.  Per chunk, products
// on the matrix cores (wave w owns token tile w % 4 and half w / 4 of the
// output columns; both halves form the dA^T, dA and A tiles they need):
//   dA^T (s <= t tiles), dA and A (t >= s tiles);
//   dr~^T = K^^T dA^T + S_c dO^T (scaled by e^{Lam_L} per row),
//   dk^^T = R~^T dA + dS_end V^T,  dv^T = dO^T A + dS_end^T K^^T,
//   dS   += (R~_hi + R~_lo)^T dO (then scaled by e^{Lam_L} per row).
// dr~ and dk^ go through LDS in fp32 to the staging threads, which apply the
// factors and the bonus terms and run the decay-gradient scan.  A chunk
// whose decay falls below the factorised range (as in the forward) is taken
// token by token on the VALU, with the states inside it recomputed from S_c.
#include <algorithm>
#include <type_traits>

#include "launchers.h"
#include "wkv_device.h"
#include "wkv_tiles.h"

namespace wkv {
namespace {

using namespace tiles;

constexpr int NW = 8;            // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * NW;
constexpr int kTW = 4;           // waves that take a fast-decay chunk token by token
constexpr int kMaxSlots = 4096;  // hand-off slots of the balanced split
constexpr int kMaxSegs = 16;     // segments per extra head
constexpr int TP = 16 / NW;      // tokens per staging thread
constexpr int kSF = 24;          // floats of the sweep's state per thread
constexpr int kPF = 68;          // pitch (floats) of the fp32 gradient tiles
constexpr float kLn2 = 0.69314718055994530942f;

// bf16 operand tiles, row-major with pitch kPC: r~ and k^ (hi, lo), v, do
// as [token][channel]; S_c (hi, lo) as [i][j]; dS_end (hi, lo) transposed,
// [j][i].  Every operand of the products that form dr~ and dk^ is split
// into bf16 hi + lo (and so are dA^T, dA): the decay gradient is a
// difference of suffix sums of r dr and k dk, which amplifies their
// relative error, and plain bf16 operands (2^-9) would leave it at ~1e-2.
enum { B_R = 0, B_RL, B_K, B_KL, B_V, B_DO, B_SC, B_SCL, B_DST, B_DSTL, B_COUNT };

// a = hi + lo with hi, lo bf16: the two halves of a product operand
__device__ __forceinline__ void split8(const f32x4 &a, const f32x4 &b, bf16x8 &hi, bf16x8 &lo) {
    hi = pack8(a, b);
    const u32x4 hb = __builtin_bit_cast(u32x4, hi);
    const f32x4 ra = {a[0] - bf16_lo(hb.x), a[1] - bf16_hi(hb.x), a[2] - bf16_lo(hb.y),
                      a[3] - bf16_hi(hb.y)};
    const f32x4 rb = {b[0] - bf16_lo(hb.z), b[1] - bf16_hi(hb.z), b[2] - bf16_lo(hb.w),
                      b[3] - bf16_hi(hb.w)};
    lo = pack8(ra, rb);
}
__device__ __forceinline__ u32x2 lo4(const f32x4 &a, u32x2 hi) {
    return pack4(a[0] - bf16_lo(hi.x), a[1] - bf16_hi(hi.x), a[2] - bf16_lo(hi.y),
                 a[3] - bf16_hi(hi.y));
}

// Balanced split of the reverse sweep (as the forward's, mirrored): with up
// to half as many heads again as CUs, workgroup i runs its own head and one
// segment of one of the `extra` remaining heads.  The segments of an extra
// head run on workgroups i, i + stride, ... (the same XCD, dispatched in
// order); segment s covers chunks [e(s+1), e(s)) with e(s) = n - s n / K, and
// runs after the workgroup's chunks [e(s), n) of its own head, by when
// segment s-1 is done.  The sweep's state (dS, the dg carry, the du and dx
// sums) goes between segments through `slots`, and the own head's waits in
// `park` meanwhile, kSF floats per thread.
struct BwdSplit {
    int extra, first_extra, K, stride, chains_per_xcd;
    int nfull;        // whole heads per workgroup before the split round
    WsCtrl *ctrl;     // control block of the hand-off workspace (epoch, error word)
    unsigned *flags;  // [extra * (K - 1)] slot flags: the launch's tag once a slot is full
    float *slots;     // [extra * (K - 1)][kThreads][kSF]
    float *park;      // [workgroups][kThreads][kSF]
};

template <bool PT>
__global__ __launch_bounds__(kThreads, 1) void wkv_bwd_kernel(
    int T, int H, const uint16_t *__restrict__ r, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ x, const float *__restrict__ u,
    const uint16_t *__restrict__ d_o, const float *__restrict__ d_sT,
    const float *__restrict__ chunk_states, uint16_t *__restrict__ d_r,
    uint16_t *__restrict__ d_k, uint16_t *__restrict__ d_v, float *__restrict__ d_x,
    float *__restrict__ du_part, float *__restrict__ dx_part, float *__restrict__ d_s0,
    BwdSplit sp) {
    __shared__ __align__(16) uint16_t sm[B_COUNT][kTile];
    __shared__ __align__(16) float sDR[kL * kPF];   // dr~ [token][channel]
    __shared__ __align__(16) float sDK[kL * kPF];   // dk^ [token][channel]
    __shared__ __align__(16) float sWave[NW][kN];   // per-wave log2-decay totals
    __shared__ __align__(16) float sDecay[kN];      // e^{Lam_L}
    __shared__ __align__(16) float sBonus[kL];      // beta_t
    __shared__ __align__(16) float sDBeta[kL];      // dbeta_t
    __shared__ __align__(16) float sScan[NW][kN];   // per-wave totals of the dg scan
    __shared__ __align__(16) float sCF[NW][kN];     // partial rows of sum_j dS_T S_T
    __shared__ int sBad[NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    int bh = 0, h = 0;  // (sequence, head) of the current job
    const int nchunks = (T + kL - 1) / kL;

    Ctx cx;
    cx.T = T;
    cx.cq = c;
    cx.tq = tid >> 4;  // = 4 w + g
    cx.vt = tid >> 3;
    cx.vo = tid & 7;
    cx.tok_stride = (size_t)H * kN;
    cx.tokb = (uint32_t)H * kN * 2;
    cx.off_rk = (uint32_t)(TP * cx.tq) * cx.tokb + 8 * cx.cq;
    cx.off_v = (uint32_t)cx.vt * cx.tokb + 16 * cx.vo;

    // dS block of this wave: key rows [16 (w/2), +16) x value columns
    // [32 (w%2), +32), two 16x16 tiles; dS[t][e] = dS[skey0 + 4 g + e][sval(t) + c]
    const int skey0 = 16 * (w >> 1), sval0 = 32 * (w & 1);
    auto skey = [&](int) { return skey0; };
    auto sval = [&](int t) { return sval0 + 16 * t; };
    auto sidx = [&](int t, int e) { return (skey(t) + 4 * g + e) * kN + sval(t) + c; };
    f32x4 dS[2];

    // per-head values of the current job
    f32x4 uq, a2e;  // u; Eagle: log2-decay per channel
    auto set_head = [&](int head) {
        bh = head;
        h = head % H;
        cx.seq_base = (size_t)(head / H) * T * cx.tok_stride + (size_t)h * kN;
        uq = *(const f32x4 *)(u + (size_t)h * kN + 4 * c);
        a2e = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!PT) {
            const f32x4 xs = *(const f32x4 *)(x + (size_t)h * kN + 4 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) a2e[q] = -exp2_fast(xs[q] * kLog2e) * kLog2e;
        }
    };

    // The sweep's state: dS; the carry of the dg suffix sum for this
    // thread's channels 4 c .. 4 c + 3 (the final-state term, then the totals
    // of the chunks already done); du and Eagle dx sums; threads < 64: Eagle
    // dx of channel tid from fast-decay chunks.
    f32x4 carry, du_acc, dx_acc;
    float fb_dx;
    // the state at the end of the sequence: dS = dL/dS_T and the final-state
    // term of dg
    auto init_state = [&]() {
        lds_barrier();  // (the previous job's last reads of sCF are done)
        const size_t sbase = (size_t)bh * kN * kN;
        const float *ST = chunk_states + ((size_t)bh * (nchunks + 1) + nchunks) * kN * kN;
        f32x4 part = {0.f, 0.f, 0.f, 0.f};  // rows skey0 + 4 g + e: sum over this wave's columns
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dS[t][e] = d_sT ? d_sT[sbase + sidx(t, e)] : 0.0f;
                part[e] += dS[t][e] * ST[sidx(t, e)];
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) part[e] = row_sum16(part[e]);
        if (c == 0) *(f32x4 *)&sCF[w][skey0 + 4 * g] = part;
        lds_barrier();
        const int wa = (4 * c) / 16 * 2;  // the two waves holding these key rows
        carry = *(const f32x4 *)&sCF[wa][4 * c] + *(const f32x4 *)&sCF[wa + 1][4 * c];
        du_acc = f32x4{0.f, 0.f, 0.f, 0.f};
        dx_acc = du_acc;
        fb_dx = 0.0f;
    };
    // the state to / from kSF floats per thread at p (plain or agent-scope
    // atomic accesses: slots between workgroups use the latter)
    auto put_state = [&](float *p, bool shared) {
        float v[kSF];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * t + e] = dS[t][e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[8 + q] = carry[q];
            v[12 + q] = du_acc[q];
            v[16 + q] = dx_acc[q];
        }
        v[20] = fb_dx;
        v[21] = v[22] = v[23] = 0.0f;
        float *dst = p + (size_t)tid * kSF;
#pragma unroll
        for (int i = 0; i < kSF; ++i) {
            if (shared)
                __hip_atomic_store((unsigned *)(dst + i), __float_as_uint(v[i]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            else
                dst[i] = v[i];
        }
    };
    // (poison: the hand-off never came; continue from NaN)
    auto get_state = [&](const float *p, bool shared, bool poison = false) {
        float v[kSF];
        const float *src = p + (size_t)tid * kSF;
#pragma unroll
        for (int i = 0; i < kSF; ++i)
            v[i] = poison   ? __builtin_nanf("")
                   : shared ? __uint_as_float(ld_agent((const unsigned *)(src + i)))
                            : src[i];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[t][e] = v[4 * t + e];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            carry[q] = v[8 + q];
            du_acc[q] = v[12 + q];
            dx_acc[q] = v[16 + q];
        }
        fb_dx = v[20];
    };

    // fixed thread mapping of the chunk-state tile: row tid/8, 8 columns
    const int sc_row = tid >> 3, sc_col = 8 * (tid & 7);

    // chunks [ch_lo, ch_hi) of the current head, from the last
    auto run = [&](int ch_hi, int ch_lo) {
    // Finch: the decay logits of the next chunk in sweep order are requested
    // a chunk ahead, after this chunk's operands and before its gradient
    // stores, so that stage A waits neither for them nor for the stores
    Raw<NW> xn;
    if (PT) load_x<NW>(xn, (ch_hi - 1) * kL, cx, x, ch_hi > ch_lo);
    for (int ch = ch_hi - 1; ch >= ch_lo; --ch) {
        const int c0 = ch * kL;
        // The lane indices, opaque to the compiler inside each chunk: the
        // LDS addresses derived from them are then formed where they are
        // used instead of all being hoisted out of the loop and held in
        // registers for the whole kernel.
        int c = lane & 15, g = lane >> 4;
        asm volatile("" : "+v"(c), "+v"(g));
        // ---- operands of the chunk ----------------------------------------
        Raw<NW> d;
        load_rkv<NW>(d, c0, cx, r, k, v);
        u32x4 dov[Raw<NW>::NV];
        {
            const Rsrc rd = rsrc(d_o + cx.base(c0), cx.span(c0));
#pragma unroll
            for (int j = 0; j < Raw<NW>::NV; ++j)
                dov[j] = __builtin_amdgcn_raw_buffer_load_b128(rd, cx.off_v + j * 8 * NW * cx.tokb,
                                                               0, kReadOnce);
        }
        f32x4 scv[2];
        {
            const float *Sc = chunk_states + ((size_t)bh * (nchunks + 1) + ch) * kN * kN;
#pragma unroll
            for (int q = 0; q < 2; ++q) scv[q] = *(const f32x4 *)(Sc + sc_row * kN + sc_col + 4 * q);
        }
        if (PT) {
#pragma unroll
            for (int e = 0; e < TP; ++e) d.x[e] = xn.x[e];
            load_x<NW>(xn, (ch - 1) * kL, cx, x, ch > ch_lo);
        }

        // ---- stage A: log2 decays and their in-wave scan -------------------
        float a2[TP][4], lower[4];
#pragma unroll
        for (int e = 0; e < TP; ++e) {
            const bool valid = c0 + TP * cx.tq + e < T;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a2[e][q] = !valid ? 0.0f : PT ? -exp2_fast(d.x[e][q] * kLog2e) * kLog2e : a2e[q];
        }
        {
            f32x4 wt;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = a2[0][q];
#pragma unroll
                for (int e = 1; e < TP; ++e) s += a2[e][q];
                const float s1 = __shfl_up(s, 16, 64);
                if (g >= 1) s += s1;
                const float s2 = __shfl_up(s, 32, 64);
                if (g >= 2) s += s2;
                const float ex = __shfl_up(s, 16, 64);
                lower[q] = (g == 0) ? 0.0f : ex;
                wt[q] = s;
            }
            if (g == 3) *(f32x4 *)&sWave[w][4 * c] = wt;
        }
        lds_barrier();  // (1) decay totals

        // ---- stage B: factors, operand tiles, bonus ------------------------
        f32x4 LL, before = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4 part = *(const f32x4 *)&sWave[0][4 * c];
#pragma unroll
            for (int j = 1; j < NW; ++j) {
                if (j == w) before = part;
                part += *(const f32x4 *)&sWave[j][4 * c];
            }
            LL = part;
        }
        bool bad = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) bad |= LL[q] < kSafeLog2;
        if (w == 0 && g == 0) {
            f32x4 dd;
#pragma unroll
            for (int q = 0; q < 4; ++q) dd[q] = exp2_fast(LL[q]);
            *(f32x4 *)&sDecay[4 * c] = dd;
        }
        float fr[TP][4], fk[TP][4];  // e^{Lam_{t-1} - Lam_L}, e^{Lam_L - Lam_t}
        {
            float wv[TP][4], f1[4], f2[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float pre = before[q] + lower[q];
                float run = pre;
#pragma unroll
                for (int e = 0; e < TP; ++e) {
                    run += a2[e][q];
                    wv[e][q] = exp2_fast(a2[e][q]);
                }
                f1[q] = exp2_fast(pre - LL[q]);
                f2[q] = exp2_fast(LL[q] - run);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                fk[TP - 1][q] = f2[q];
#pragma unroll
                for (int e = TP - 2; e >= 0; --e) fk[e][q] = fk[e + 1][q] * wv[e + 1][q];
#pragma unroll
                for (int e = 0; e < TP; ++e) {
                    fr[e][q] = f1[q];
                    f1[q] *= wv[e][q];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < TP; ++e) {
            const int tau = TP * cx.tq + e;
            const float rr[4] = {bf16_lo(d.r[e].x), bf16_hi(d.r[e].x), bf16_lo(d.r[e].y),
                                 bf16_hi(d.r[e].y)};
            const float kk[4] = {bf16_lo(d.k[e].x), bf16_hi(d.k[e].x), bf16_lo(d.k[e].y),
                                 bf16_hi(d.k[e].y)};
            float rt[4], rl[4], kh[4], sb = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                rt[q] = rr[q] * fr[e][q];
                kh[q] = kk[q] * fk[e][q];
                sb = fmaf(rr[q] * uq[q], kk[q], sb);
            }
            const u32x2 hi = pack4(rt[0], rt[1], rt[2], rt[3]);
            rl[0] = rt[0] - bf16_lo(hi.x);
            rl[1] = rt[1] - bf16_hi(hi.x);
            rl[2] = rt[2] - bf16_lo(hi.y);
            rl[3] = rt[3] - bf16_hi(hi.y);
            *(u32x2 *)(sm[B_R] + tau * kPC + 4 * c) = hi;
            *(u32x2 *)(sm[B_RL] + tau * kPC + 4 * c) = pack4(rl[0], rl[1], rl[2], rl[3]);
            const u32x2 khi = pack4(kh[0], kh[1], kh[2], kh[3]);
            *(u32x2 *)(sm[B_K] + tau * kPC + 4 * c) = khi;
            *(u32x2 *)(sm[B_KL] + tau * kPC + 4 * c) = lo4(f32x4{kh[0], kh[1], kh[2], kh[3]}, khi);
            const float bs = row_sum16(sb);
            if (c == 0) sBonus[tau] = bs;
        }
#pragma unroll
        for (int j = 0; j < Raw<NW>::NV; ++j) {
            *(u32x4 *)(sm[B_V] + (cx.vt + 8 * NW * j) * kPC + 8 * cx.vo) = d.v[j];
            *(u32x4 *)(sm[B_DO] + (cx.vt + 8 * NW * j) * kPC + 8 * cx.vo) = dov[j];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x2 hi = pack4(scv[q][0], scv[q][1], scv[q][2], scv[q][3]);
            *(u32x2 *)(sm[B_SC] + sc_row * kPC + sc_col + 4 * q) = hi;
            *(u32x2 *)(sm[B_SCL] + sc_row * kPC + sc_col + 4 * q) = lo4(scv[q], hi);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x2 hi = pack4(dS[t][0], dS[t][1], dS[t][2], dS[t][3]);
            *(u32x2 *)(sm[B_DST] + (sval(t) + c) * kPC + skey(t) + 4 * g) = hi;
            *(u32x2 *)(sm[B_DSTL] + (sval(t) + c) * kPC + skey(t) + 4 * g) = lo4(dS[t], hi);
        }
        // (2) operands staged; the range flag is uniform over the workgroup
        const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
        if (lane == 0) sBad[w] = any ? 1 : 0;
        lds_barrier();
        int anybad = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) anybad |= sBad[j];
        const bool unsafe = anybad != 0;
        if (unsafe) {
            // ---- fast-decay chunk: its tokens one at a time, backwards -----
            // Raw r, k (bf16) and w (fp32) are staged in the factor tiles,
            // whose products this chunk does not run.  Waves w < kTW hold
            // columns [16 w, +16) of dS and of the recomputed state:
            // X[m][e] = X[16 m + 4 g + e][16 w + c] (the other waves only
            // keep the barriers).  For each token the state before it is
            // recomputed from S_c (quadratic in the chunk length, exact at any
            // decay); the row sums over the columns are formed per wave and
            // added over the waves through LDS.
            uint16_t *tr = sm[B_R], *tk = sm[B_RL];
            float *tw = (float *)sm[B_SC];       // [64][64] fp32 over B_SC, B_SCL
            float *red = (float *)sm[B_K];       // [2][3][kTW][64] partial row sums
            float *xfer = sDR;                   // layout changes of dS
            const bool tbw = w < kTW;            // wave-uniform
            const int wc = w & (kTW - 1);
#pragma unroll
            for (int e = 0; e < TP; ++e) {
                const int tau = TP * cx.tq + e;
                *(u32x2 *)(tr + tau * kPC + 4 * c) = d.r[e];
                *(u32x2 *)(tk + tau * kPC + 4 * c) = d.k[e];
                f32x4 wv;
#pragma unroll
                for (int q = 0; q < 4; ++q) wv[q] = exp2_fast(a2[e][q]);
                *(f32x4 *)(tw + tau * kN + 4 * c) = wv;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) xfer[(skey(t) + 4 * g + e) * kPF + sval(t) + c] = dS[t][e];
            if (tid < kL) {  // dbeta of every token of the chunk
                float db = 0.0f;
                for (int j = 0; j < kN; ++j)
                    db = fmaf(bf16_to_f32(sm[B_DO][tid * kPC + j]), bf16_to_f32(sm[B_V][tid * kPC + j]), db);
                sDBeta[tid] = db;
            }
            lds_barrier();
            f32x4 dSc[4];
            const float *Sg = chunk_states + ((size_t)bh * (nchunks + 1) + ch) * kN * kN;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dSc[m][e] = xfer[(16 * m + 4 * g + e) * kPF + 16 * wc + c];
                }
            lds_barrier();  // xfer (sDR) is free again
            const int nvalid = min(kL, T - c0);
            const int j = 16 * wc + c;
#pragma unroll 1
            for (int tau = nvalid - 1; tau >= 0; --tau) {
                float *rb = red + (tau & 1) * 3 * kTW * kN;
                if (tbw) {
                f32x4 Sw[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sw[m][e] = Sg[(16 * m + 4 * g + e) * kN + j];
#pragma unroll 1
                for (int t2 = 0; t2 < tau; ++t2) {
                    const float vj = bf16_to_f32(sm[B_V][t2 * kPC + j]);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const f32x4 wv = *(const f32x4 *)(tw + t2 * kN + 16 * m + 4 * g);
                        const u32x2 kp = *(const u32x2 *)(tk + t2 * kPC + 16 * m + 4 * g);
                        const float k4[4] = {bf16_lo(kp.x), bf16_hi(kp.x), bf16_lo(kp.y), bf16_hi(kp.y)};
#pragma unroll
                        for (int e = 0; e < 4; ++e) Sw[m][e] = fmaf(wv[e], Sw[m][e], k4[e] * vj);
                    }
                }
                const float vj = bf16_to_f32(sm[B_V][tau * kPC + j]);
                const float doj = bf16_to_f32(sm[B_DO][tau * kPC + j]);
                float dvj = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x2 kp = *(const u32x2 *)(tk + tau * kPC + 16 * m + 4 * g);
                    const u32x2 rp = *(const u32x2 *)(tr + tau * kPC + 16 * m + 4 * g);
                    const f32x4 wv = *(const f32x4 *)(tw + tau * kN + 16 * m + 4 * g);
                    const float k4[4] = {bf16_lo(kp.x), bf16_hi(kp.x), bf16_lo(kp.y), bf16_hi(kp.y)};
                    const float r4[4] = {bf16_lo(rp.x), bf16_hi(rp.x), bf16_lo(rp.y), bf16_hi(rp.y)};
                    f32x4 pr, pk, pw;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pr[e] = row_sum16(doj * Sw[m][e]);        // dr^a: do . S row
                        pk[e] = row_sum16(dSc[m][e] * vj);        // dk^a: dS' row . v
                        pw[e] = row_sum16(dSc[m][e] * Sw[m][e]);  // dw
                        dvj = fmaf(dSc[m][e], k4[e], dvj);
                        dSc[m][e] = fmaf(wv[e], dSc[m][e], r4[e] * doj);
                    }
                    if (c == 0) {
                        *(f32x4 *)(rb + (0 * kTW + w) * kN + 16 * m + 4 * g) = pr;
                        *(f32x4 *)(rb + (1 * kTW + w) * kN + 16 * m + 4 * g) = pk;
                        *(f32x4 *)(rb + (2 * kTW + w) * kN + 16 * m + 4 * g) = pw;
                    }
                }
                dvj += __shfl_xor(dvj, 16, 64);
                dvj += __shfl_xor(dvj, 32, 64);
                if (g == 0)
                    d_v[cx.base(c0) + (size_t)tau * cx.tok_stride + j] =
                        (uint16_t)pack_bf16x2(fmaf(sBonus[tau], doj, dvj), 0.0f);
                }
                lds_barrier();
                if (tid < kN) {
                    float a = 0.0f, bsum = 0.0f, dw = 0.0f;
#pragma unroll
                    for (int q = 0; q < kTW; ++q) {
                        a += rb[(0 * kTW + q) * kN + tid];
                        bsum += rb[(1 * kTW + q) * kN + tid];
                        dw += rb[(2 * kTW + q) * kN + tid];
                    }
                    sDR[tau * kPF + tid] = a;
                    sDK[tau * kPF + tid] = bsum;
                    // dL/dg = dw w, dL/dx = dL/dg g with g = ln w = log2(w) ln 2
                    const float wt = tw[tau * kN + tid];
                    const float xg = PT ? x[cx.base(c0) + (size_t)tau * cx.tok_stride + tid]
                                        : x[(size_t)h * kN + tid];
                    const float gnat = -exp2_fast(xg * kLog2e);
                    const float dxv = dw * wt * gnat;
                    if (PT) d_x[cx.base(c0) + (size_t)tau * cx.tok_stride + tid] = dxv;
                    else fb_dx += dxv;
                }
            }
            // dS back to the block layout (after the last reads of w)
            lds_barrier();
            if (tbw)
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tw[(16 * m + 4 * g + e) * kN + 16 * w + c] = dSc[m][e];
            lds_barrier();
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) dS[t][e] = tw[(skey(t) + 4 * g + e) * kN + sval(t) + c];
        }
        // ---- products -----------------------------------------------------
        const Rsrc rdv = rsrc(d_v + cx.base(c0), cx.span(c0));
        // wave w: token tile P = w % 4, output columns of half hf = w / 4
        // (dA^T, dA and A are formed by both halves)
        const int hf = w >> 2;
        auto products = [&](auto tile) {
            constexpr int P = decltype(tile)::value;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            // dA^T[s][t] = v_s . do_t: s-tiles q <= P, t-tile P
            f32x4 dat[P + 1];
#pragma unroll
            for (int q = 0; q <= P; ++q) {
                dat[q] = zero;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    dat[q] = mfma(lds8(sm[B_V] + (16 * q + c) * kPC + 32 * kb + 8 * g),
                                  lds8(sm[B_DO] + (16 * P + c) * kPC + 32 * kb + 8 * g), dat[q]);
            }
            // diagonal: dbeta_t, then the strict causal mask (s < t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sl = 4 * g + e;
                if (sl == c && hf == 0) sDBeta[16 * P + c] = dat[P][e];
                dat[P][e] = sl < c ? dat[P][e] : 0.0f;
            }
            // dr~^T[i][t] (t = 16 P + c): K^^T dA^T + diag(e^{Lam_L}) S_c dO^T
            bf16x8 Bdo[2];  // (the dO operand is the same for every i)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Bdo[kb] = lds8(sm[B_DO] + (16 * P + c) * kPC + 32 * kb + 8 * g);
#pragma unroll 1
            for (int i2 = 0; i2 < 2; ++i2) {
                const int ii = 2 * hf + i2;
                f32x4 acc = zero, st = zero;
#pragma unroll
                for (int bk = 0; 2 * bk <= P; ++bk) {
                    bf16x8 Bh, Bl;
                    split8(dat[2 * bk], (2 * bk + 1 <= P) ? dat[(2 * bk + 1) % (P + 1)] : zero, Bh, Bl);
                    const bf16x8 Ah = lds_col4x2(sm[B_K], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g, 16 * ii, c);
                    const bf16x8 Al = lds_col4x2(sm[B_KL], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g, 16 * ii, c);
                    acc = mfma(Ah, Bh, acc);
                    acc = mfma(Ah, Bl, acc);
                    acc = mfma(Al, Bh, acc);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    st = mfma(lds8(sm[B_SC] + (16 * ii + c) * kPC + 32 * kb + 8 * g), Bdo[kb], st);
                    st = mfma(lds8(sm[B_SCL] + (16 * ii + c) * kPC + 32 * kb + 8 * g), Bdo[kb], st);
                }
                const f32x4 dd = *(const f32x4 *)&sDecay[16 * ii + 4 * g];
                acc += st * dd;
                *(f32x4 *)&sDR[(16 * P + c) * kPF + 16 * ii + 4 * g] = acc;
            }
            // dA[t][s]: t-tiles q >= P, s-tile P
            f32x4 da[4 - P];
#pragma unroll
            for (int q = P; q < 4; ++q) {
                da[q - P] = zero;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    da[q - P] = mfma(lds8(sm[B_DO] + (16 * q + c) * kPC + 32 * kb + 8 * g),
                                     lds8(sm[B_V] + (16 * P + c) * kPC + 32 * kb + 8 * g), da[q - P]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)  // diagonal tile: keep t > s
                da[0][e] = 4 * g + e > c ? da[0][e] : 0.0f;
            // dk^^T[i][s] (s = 16 P + c): R~^T dA + dS_end V^T
            bf16x8 Bv[2];  // (the V operand is the same for every i)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Bv[kb] = lds8(sm[B_V] + (16 * P + c) * kPC + 32 * kb + 8 * g);
#pragma unroll 1
            for (int i2 = 0; i2 < 2; ++i2) {
                const int ii = 2 * hf + i2;
                f32x4 acc = zero;
#pragma unroll
                for (int bk = P / 2; bk < 2; ++bk) {
                    const f32x4 t0 = (2 * bk >= P) ? da[2 * bk >= P ? 2 * bk - P : 0] : zero;
                    const f32x4 t1 = (2 * bk + 1 >= P) ? da[2 * bk + 1 >= P ? 2 * bk + 1 - P : 0] : zero;
                    bf16x8 Bh, Bl;
                    split8(t0, t1, Bh, Bl);
                    const bf16x8 Ah = lds_col4x2(sm[B_R], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g, 16 * ii, c);
                    const bf16x8 Al = lds_col4x2(sm[B_RL], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g, 16 * ii, c);
                    acc = mfma(Ah, Bh, acc);
                    acc = mfma(Ah, Bl, acc);
                    acc = mfma(Al, Bh, acc);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    acc = mfma(lds_col8(sm[B_DST], 32 * kb + 8 * g, 16 * ii, c), Bv[kb], acc);
                    acc = mfma(lds_col8(sm[B_DSTL], 32 * kb + 8 * g, 16 * ii, c), Bv[kb], acc);
                }
                *(f32x4 *)&sDK[(16 * P + c) * kPF + 16 * ii + 4 * g] = acc;
            }
            // A[t][s]: t-tiles q >= P, s-tile P
            f32x4 aa[4 - P];
#pragma unroll
            for (int q = P; q < 4; ++q) {
                aa[q - P] = zero;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    aa[q - P] = mfma(lds8(sm[B_R] + (16 * q + c) * kPC + 32 * kb + 8 * g),
                                     lds8(sm[B_K] + (16 * P + c) * kPC + 32 * kb + 8 * g), aa[q - P]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)  // diagonal tile: keep t > s
                aa[0][e] = 4 * g + e > c ? aa[0][e] : 0.0f;
            // dv^T[j][s] (s = 16 P + c): dO^T A + dS_end^T K^^T, plus beta_s do_s
            const float bon = sBonus[16 * P + c];
            bf16x8 Bk[2];  // (the K^ operand is the same for every j)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Bk[kb] = lds8(sm[B_K] + (16 * P + c) * kPC + 32 * kb + 8 * g);
#pragma unroll 1
            for (int j2 = 0; j2 < 2; ++j2) {
                const int jj = 2 * hf + j2;
                f32x4 acc = zero;
#pragma unroll
                for (int bk = P / 2; bk < 2; ++bk) {
                    const f32x4 t0 = (2 * bk >= P) ? aa[2 * bk >= P ? 2 * bk - P : 0] : zero;
                    const f32x4 t1 = (2 * bk + 1 >= P) ? aa[2 * bk + 1 >= P ? 2 * bk + 1 - P : 0] : zero;
                    acc = mfma(lds_col4x2(sm[B_DO], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g, 16 * jj, c),
                               pack8(t0, t1), acc);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    acc = mfma(lds8(sm[B_DST] + (16 * jj + c) * kPC + 32 * kb + 8 * g), Bk[kb], acc);
                const u32x2 dop = *(const u32x2 *)(sm[B_DO] + (16 * P + c) * kPC + 16 * jj + 4 * g);
                acc[0] = fmaf(bon, bf16_lo(dop.x), acc[0]);
                acc[1] = fmaf(bon, bf16_hi(dop.x), acc[1]);
                acc[2] = fmaf(bon, bf16_lo(dop.y), acc[2]);
                acc[3] = fmaf(bon, bf16_hi(dop.y), acc[3]);
                __builtin_amdgcn_raw_buffer_store_b64(
                    pack4(acc[0], acc[1], acc[2], acc[3]), rdv,
                    (uint32_t)(16 * P + c) * cx.tokb + 2 * (16 * jj + 4 * g), 0, 0);
            }
            // dS_c = diag(e^{Lam_L}) (dS_end + (R~_hi + R~_lo)^T dO)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int k0 = 32 * kb + 8 * g;
                bf16x8 Bd[2];
#pragma unroll
                for (int vj = 0; vj < 2; ++vj) Bd[vj] = lds_col8(sm[B_DO], k0, sval0 + 16 * vj, c);
                const bf16x8 Ah = lds_col8(sm[B_R], k0, skey0, c);
                const bf16x8 Al = lds_col8(sm[B_RL], k0, skey0, c);
#pragma unroll
                for (int vj = 0; vj < 2; ++vj) {
                    dS[vj] = mfma(Ah, Bd[vj], dS[vj]);
                    dS[vj] = mfma(Al, Bd[vj], dS[vj]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) dS[t] *= *(const f32x4 *)&sDecay[skey(t) + 4 * g];
        };
        if (!unsafe) {
            switch (w & 3) {  // wave-uniform
                case 0: products(std::integral_constant<int, 0>{}); break;
                case 1: products(std::integral_constant<int, 1>{}); break;
                case 2: products(std::integral_constant<int, 2>{}); break;
                default: products(std::integral_constant<int, 3>{}); break;
            }
        }
        lds_barrier();  // (3) dr~, dk^, dbeta in LDS

        // ---- dr, dk, du and the decay-gradient scan -------------------------
        f32x4 Dsum;       // this thread's D = r dr^a - k dk^a summed over its tokens
        float Dv[TP][4], rdr[TP][4];
        {
            const Rsrc rr_ = rsrc(d_r + cx.base(c0), cx.span(c0));
            const Rsrc rk_ = rsrc(d_k + cx.base(c0), cx.span(c0));
#pragma unroll
            for (int e = 0; e < TP; ++e) {
                const int tau = TP * cx.tq + e;
                const f32x4 dr4 = *(const f32x4 *)&sDR[tau * kPF + 4 * c];
                const f32x4 dk4 = *(const f32x4 *)&sDK[tau * kPF + 4 * c];
                const float db = sDBeta[tau];
                const float rr[4] = {bf16_lo(d.r[e].x), bf16_hi(d.r[e].x), bf16_lo(d.r[e].y),
                                     bf16_hi(d.r[e].y)};
                const float kk[4] = {bf16_lo(d.k[e].x), bf16_hi(d.k[e].x), bf16_lo(d.k[e].y),
                                     bf16_hi(d.k[e].y)};
                float drv[4], dkv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float dra = unsafe ? dr4[q] : dr4[q] * fr[e][q];
                    const float dka = unsafe ? dk4[q] : dk4[q] * fk[e][q];
                    drv[q] = fmaf(uq[q] * kk[q], db, dra);
                    dkv[q] = fmaf(uq[q] * rr[q], db, dka);
                    rdr[e][q] = rr[q] * dra;
                    Dv[e][q] = rdr[e][q] - kk[q] * dka;
                    du_acc[q] = fmaf(rr[q] * kk[q], db, du_acc[q]);
                }
                const uint32_t off = cx.off_rk + e * cx.tokb;
                __builtin_amdgcn_raw_buffer_store_b64(pack4(drv[0], drv[1], drv[2], drv[3]), rr_, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(pack4(dkv[0], dkv[1], dkv[2], dkv[3]), rk_, off, 0, 0);
            }
            // suffix sums: within the thread, then over the later token groups
            // of the wave (lanes 16 and 32 above), then over the later waves
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int e = TP - 2; e >= 0; --e) Dv[e][q] += Dv[e + 1][q];
                float s = Dv[0][q];
                const float s1 = __shfl_down(s, 16, 64);
                if (g <= 2) s += s1;
                const float s2 = __shfl_down(s, 32, 64);
                if (g <= 1) s += s2;
                Dsum[q] = s - Dv[0][q];  // exclusive: later groups of this wave
                if (g == 0) sScan[w][4 * c + q] = s;
            }
        }
        lds_barrier();  // (4) wave totals of the scan
        {
            f32x4 later = {0.f, 0.f, 0.f, 0.f}, total = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = NW - 1; j >= 0; --j) {
                const f32x4 t = *(const f32x4 *)&sScan[j][4 * c];
                if (j > w) later += t;
                total += t;
            }
            f32x4 dxv[TP];
#pragma unroll
            for (int e = 0; e < TP; ++e)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // suffix over the tokens from this one on, minus its own r dr^a
                    const float dg = carry[q] + later[q] + Dsum[q] + Dv[e][q] - rdr[e][q];
                    dxv[e][q] = dg * a2[e][q] * kLn2;
                    if (!unsafe) dx_acc[q] += dxv[e][q];
                }
            // (a fast-decay chunk wrote its decay gradient from dw directly)
            if (PT && !unsafe) {
                const Rsrc rx = rsrc(d_x + cx.base(c0), 2 * cx.span(c0));
#pragma unroll
                for (int e = 0; e < TP; ++e)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dxv[e]), rx,
                                                           2 * (cx.off_rk + e * cx.tokb), 0, 0);
            }
            carry += total;
        }
    }
    };

    // ---- gradient of the initial state, partial du (and Eagle dx) ----------
    auto finish = [&]() {
    if (d_s0 != nullptr) {
        const size_t sbase = (size_t)bh * kN * kN;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) d_s0[sbase + sidx(t, e)] = dS[t][e];
    }
    // sum over the 16 token groups: lanes 16 and 32 apart, then the waves
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        du_acc[q] += __shfl_xor(du_acc[q], 16, 64);
        du_acc[q] += __shfl_xor(du_acc[q], 32, 64);
        dx_acc[q] += __shfl_xor(dx_acc[q], 16, 64);
        dx_acc[q] += __shfl_xor(dx_acc[q], 32, 64);
    }
    lds_barrier();
    if (g == 0) {
        *(f32x4 *)&sScan[w][4 * c] = du_acc;
        *(f32x4 *)&sCF[w][4 * c] = dx_acc;
    }
    lds_barrier();
    if (tid < kN) {
        float su = 0.0f, sx = 0.0f;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            su += sScan[j][tid];
            sx += sCF[j][tid];
        }
        du_part[(size_t)bh * kN + tid] = su;
        if (!PT) dx_part[(size_t)bh * kN + tid] = sx + fb_dx;
    }
    };

    // ---- jobs ------------------------------------------------------------
    // With more than two heads per CU, workgroup i first sweeps the whole
    // heads i, i + grid, ... (sp.nfull of them), then its own head of the
    // split round.
    const int wg = blockIdx.x;
    const int own = wg + sp.nfull * (int)gridDim.x;
    int ext = 0, seg = 0;
    bool split = false;
    if (sp.extra != 0) {
        const int xcd = wg % sp.stride, local = wg / sp.stride;
        const int chain = local / sp.K;
        seg = local % sp.K;
        ext = xcd + sp.stride * chain;
        split = chain < sp.chains_per_xcd && ext < sp.extra;
    }
    const int e0 = nchunks - seg * nchunks / max(sp.K, 1);
    const int e1 = nchunks - (seg + 1) * nchunks / max(sp.K, 1);
    // Split: own head chunks [e0, n) (then parked), the extra head's chunks
    // [e1, e0), own head chunks [0, e0).  Slot flags and contents go through
    // agent-scope relaxed atomics, which act at the device's coherence point:
    // the producer's stores complete before its flag store (the launch's
    // tag), and the consumer reads the state only after it saw that tag.
    // Polls are bounded (about a second); the producer has a lower workgroup
    // index on the same XCD, so it is already running and the bound is never
    // reached.  If it were, the segment would go on from a NaN state (its
    // gradients read NaN) and the error word is set.  One loop, so that the
    // sweep is compiled once.
    const unsigned tag = (sp.extra != 0 && tid == 0) ? ws_tag(sp.ctrl) : 0u;
    __shared__ int s_late;
    auto receive = [&]() {
        const int slot = ext * (sp.K - 1) + seg - 1;
        if (tid == 0) {
            int polls = 0, late = 0;
            while (ld_agent(sp.flags + slot) != tag) {
                __builtin_amdgcn_s_sleep(8);
                if (++polls > (1 << 20)) {
                    ws_fail(sp.ctrl);
                    late = 1;
                    break;
                }
            }
            s_late = late;
        }
        lds_barrier();
        get_state(sp.slots + (size_t)slot * kThreads * kSF, true, s_late != 0);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the state has been read
        lds_barrier();
    };
    auto send = [&]() {
        const int slot = ext * (sp.K - 1) + seg;
        put_state(sp.slots + (size_t)slot * kThreads * kSF, true);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the state has landed
        lds_barrier();
        if (tid == 0) st_agent(sp.flags + slot, tag);
    };
    const int njobs = sp.nfull + (split ? 3 : 1);
#pragma clang loop unroll(disable)
    for (int j = 0; j < njobs; ++j) {
        const int job = j - sp.nfull;  // (< 0: a whole head before the split round)
        const bool extra = split && job == 1;
        set_head(job < 0 ? wg + j * (int)gridDim.x : extra ? sp.first_extra + ext : own);
        if (split && job == 2) {
            get_state(sp.park + (size_t)wg * kThreads * kSF, false);
            lds_barrier();  // (the previous job's last reads of sCF are done)
        } else if (extra && seg > 0) {
            receive();
        } else {
            init_state();
        }
        int hi = nchunks, lo = 0;
        if (split && job >= 0) {
            if (job == 0) lo = e0;
            else if (job == 1) hi = e0, lo = e1;
            else hi = e0;
        }
        run(hi, lo);
        if (split && job == 0) put_state(sp.park + (size_t)wg * kThreads * kSF, false);
        else if (extra && seg + 1 < sp.K) send();
        else finish();
    }
    if (sp.extra != 0 && tid == 0) ws_finish(sp.ctrl, tag);
}

// out[h][i] = sum over b of part[b][h][i], in sequence order
__global__ void sum_over_batch_kernel(int B, int HN, const float *part, float *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= HN) return;
    float s = 0.0f;
    for (int b = 0; b < B; ++b) s += part[(size_t)b * HN + i];
    out[i] = s;
}

// The balanced split of the reverse sweep (see the kernel), or none.
struct BwdPlan {
    int blocks;
    int64_t extra, nfull, K, chains_per_xcd;
    size_t slot_bytes, park_bytes;
};

// One workgroup per head while every head has a CU of its own.  Beyond that,
// one workgroup per CU: whole heads in rounds, and the last round's
// remainder, when it is at most half the CUs, as the balanced split (each
// workgroup sweeps its own head and one segment of an extra head).
// Otherwise the heads in rounds.
BwdPlan bwd_plan(int64_t heads, int T) {
    const int cus = device_cus(), xcds = device_xcds();
    BwdPlan p{};
    p.blocks = (int)heads;
    if (heads > cus && heads % cus != 0 && xcds > 0 && cus % xcds == 0 && T >= 4 * kL) {
        const int64_t extra = heads % cus, nfull = heads / cus - 1;
        const int64_t chains_per_xcd = (extra + xcds - 1) / xcds;
        // (at most kMaxSegs segments: each hand-off adds its latency to the
        // chain of an extra head's segments)
        const int64_t K = std::min<int64_t>((cus / xcds) / chains_per_xcd, kMaxSegs);
        if (K >= 2 && extra * (K - 1) <= kMaxSlots) {
            const size_t per = (size_t)kThreads * kSF * 4;  // one sweep state
            p.extra = extra;
            p.nfull = nfull;
            p.K = K;
            p.chains_per_xcd = chains_per_xcd;
            p.slot_bytes = (size_t)extra * (K - 1) * per;
            p.park_bytes = (size_t)cus * per;
            p.blocks = cus;
        }
    }
    return p;
}

constexpr size_t kFlagBytes = (size_t)kMaxSlots * 4;

size_t bwd_handoff_bytes(const BwdPlan &p) {
    return p.extra ? kWsCtrlBytes + kFlagBytes + p.slot_bytes + p.park_bytes : 0;
}

}  // namespace

// Layout of the backward's workspace: the hand-off area that both the
// state recomputation (a chunked forward) and the reverse sweep use, one
// after the other (at least the control block, so that the workspace's
// error word is always where rwkv_wkv_workspace_status reads it), then the
// chunk states, then the per-sequence partial sums of d_u and Eagle's d_x.
size_t bwd_states_offset(int B, int T, int H) {
    const size_t h = std::max({kWsCtrlBytes, chunk_workspace_bytes(B, T, H),
                               bwd_handoff_bytes(bwd_plan((int64_t)B * H, T))});
    return (h + 255) / 256 * 256;
}

size_t bwd_workspace_bytes(int B, int T, int H) {
    const size_t nchunks = (size_t)(T + kL - 1) / kL;
    return bwd_states_offset(B, T, H) + (size_t)B * H * (nchunks + 1) * kN * kN * 4 +
           2 * (size_t)B * H * kN * 4;
}

hipError_t launch_wkv_bwd(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                          const uint16_t *k, const uint16_t *v, const float *x, const float *u,
                          const float *state_in, const uint16_t *d_o, const float *d_sT,
                          uint16_t *d_r, uint16_t *d_k, uint16_t *d_v, float *d_x, float *d_u,
                          float *d_s0, void *ws, hipStream_t stream, bool states_saved) {
    const size_t nchunks = (size_t)(T + kL - 1) / kL;
    char *base = (char *)ws;
    float *chunk_states = (float *)(base + bwd_states_offset(B, T, H));
    float *du_part = chunk_states + (size_t)B * H * (nchunks + 1) * kN * kN;
    float *dx_part = du_part + (size_t)B * H * kN;
    hipError_t e = hipSuccess;
    if (!states_saved) {  // (else a forward stored them there)
        e = launch_wkv_chunked(per_token_decay, B, T, H, r, k, v, x, u, state_in, nullptr,
                               nullptr, ws, stream, chunk_states);
        if (e != hipSuccess) return e;
    }
    const BwdPlan p = bwd_plan((int64_t)B * H, T);
    BwdSplit sp{};
    if (p.extra != 0) {
        sp.extra = (int)p.extra;
        sp.nfull = (int)p.nfull;
        sp.first_extra = (int)((p.nfull + 1) * p.blocks);
        sp.K = (int)p.K;
        sp.stride = device_xcds();
        sp.chains_per_xcd = (int)p.chains_per_xcd;
        sp.ctrl = (WsCtrl *)base;
        sp.flags = (unsigned *)(base + kWsCtrlBytes);
        sp.slots = (float *)(base + kWsCtrlBytes + kFlagBytes);
        sp.park = (float *)(base + kWsCtrlBytes + kFlagBytes + p.slot_bytes);
    }
    const int blocks = p.blocks;
    if (per_token_decay)
        hipLaunchKernelGGL(wkv_bwd_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, T,
                           H, r, k, v, x, u, d_o, d_sT, chunk_states, d_r, d_k, d_v, d_x, du_part,
                           dx_part, d_s0, sp);
    else
        hipLaunchKernelGGL(wkv_bwd_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, T,
                           H, r, k, v, x, u, d_o, d_sT, chunk_states, d_r, d_k, d_v, d_x, du_part,
                           dx_part, d_s0, sp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int HN = H * kN;
    hipLaunchKernelGGL(sum_over_batch_kernel, dim3((unsigned)((HN + 255) / 256)), dim3(256), 0,
                       stream, B, HN, du_part, d_u);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!per_token_decay) {
        hipLaunchKernelGGL(sum_over_batch_kernel, dim3((unsigned)((HN + 255) / 256)), dim3(256), 0,
                           stream, B, HN, dx_part, d_x);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace wkv
