// wkv_chunk.hip -- Eagle (RWKV-5) / Finch (RWKV-6) WKV forward in
// time-parallel (chunked) mode on gfx950, bf16 MFMA with fp32 accumulation.
//
// Operation, per head (RWKV-5/6 summary, blob.wenxiaobai.com, section 4
// notation; 4.1.2 "Eagle time mixing"; 4.2.2 "Finch time mixing"):
//   o_t = r_t (S_{t-1} + diag(u) k_t^T v_t),  S_t = diag(w_t) S_{t-1} + k_t^T v_t,
//   w_t = exp(-exp(x_t)).
// Time-parallel evaluation (RWKV paper summary, section "Transformer-like
// parallelization"): the sequence is cut into chunks of L = 64 tokens.  With
// Lam_t = sum_{m<=t} log w_m (chunk-relative, fp32, kept in log2 units) and
// S the state entering the chunk, unrolling the recurrence gives
//   o_t = (r_t . e^{Lam_{t-1}}) S
//       + sum_{s<t} [sum_i r_t[i] k_s[i] e^{Lam_{t-1}[i] - Lam_s[i]}] v_s
//       + (sum_i r_t[i] u[i] k_t[i]) v_t
//   S'  = diag(e^{Lam_L}) S + sum_s (k_s . e^{Lam_L - Lam_s})^T v_s.
// The bracket factorises as r~_t . k~_s with r~ = r e^{Lam_{t-1} - c} and
// k~ = k e^{c - Lam_s} around the mid-chunk reference c = Lam_{L/2}, so each
// chunk is four 64x64x64 products on the matrix cores:
//   P1  A^T = K~ R~^T, masked causally, bonus on the diagonal
//   P2  O^T = V^T A^T + S^T Q^T            (Q = r . e^{Lam_{t-1}})
//   P3  S'  = diag(e^{Lam_L}) S + Kh^T V   (Kh = k . e^{Lam_L - Lam_s}, split
//       into bf16 hi + lo so the carried fp32 state loses no precision)
// Every factor except r~, k~ is at most 1.  r~ and k~ stay finite while the
// chunk's total log-decay stays above kSafeLog2 for every channel; a chunk
// that decays faster is applied token by token instead (exact at any decay).
//
// Work split: one workgroup of four wave64s per (sequence, head).  Wave p
// owns tokens [16p, 16p+16) of each chunk for P1 and P2, and value columns
// [16p, 16p+16) of the fp32 state for P3, which therefore never leaves its
// registers.  The chunk's operands are staged in LDS as bf16 tiles with a
// padded row pitch; the state is staged as a transposed bf16 tile, double
// buffered across chunks.  The next chunk's r, k, v, x are fetched into
// registers while the current chunk computes.  HBM traffic is the
// algorithmic minimum: r, k, v, o (and x for Finch) once, the state twice.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16): lane l = c + 16 g holds
// row c of the A operand and column c of the B operand, with eight k-slots
// indexed by (g, slot); both operands use the same (g, slot) -> k map, so
// any consistent map is valid.  The result lane l holds rows 4 g + e
// (e = 0..3) of column c.
#include "launchers.h"
#include "wkv_device.h"

namespace wkv {
namespace {

constexpr int kN = 64;     // head size
constexpr int kL = 64;     // chunk length
constexpr int kP = 72;     // LDS row pitch (bf16 elements) of the 64x64 tiles
constexpr int kTile = kN * kP;
// Smallest chunk log2-decay (per channel) handled by the factorised form:
// its factors stay below 2^110 and above 2^-110, far from fp32 / bf16 limits.
constexpr float kSafeLog2 = -110.0f;

enum { T_RT = 0, T_KT, T_Q, T_KHH, T_KHL, T_VT, T_ST0, T_ST1, T_COUNT };

struct Raw {       // one thread's share of a chunk: 4 tokens x 4 channels
    u32x2 r[4], k[4], v[4];  // bf16 pairs
    f32x4 x[4];              // Finch decay logits
};

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {
    return *(const bf16x8 *)p;
}
__device__ __forceinline__ bf16x8 lds4x2(const uint16_t *lo, const uint16_t *hi) {
    const u32x2 a = *(const u32x2 *)lo, b = *(const u32x2 *)hi;
    const u32x4 m = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, m);
}
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    const u32x2 r = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    return r;
}
__device__ __forceinline__ bf16x8 pack8(const f32x4 &lo, const f32x4 &hi) {
    const u32x4 m = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                     pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
    return __builtin_bit_cast(bf16x8, m);
}

template <bool PT>
__device__ __forceinline__ void load_raw(Raw &d, int c0, int tq, int cq, int T,
                                         size_t seq_base, size_t tok_stride,
                                         const uint16_t *r, const uint16_t *k,
                                         const uint16_t *v, const float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = c0 + 4 * tq + e;
        if (t < T) {
            const size_t off = seq_base + (size_t)t * tok_stride + 4 * cq;
            d.r[e] = *(const u32x2 *)(r + off);
            d.k[e] = *(const u32x2 *)(k + off);
            d.v[e] = *(const u32x2 *)(v + off);
            if (PT) d.x[e] = *(const f32x4 *)(x + off);
        } else {
            d.r[e] = u32x2{0u, 0u};
            d.k[e] = u32x2{0u, 0u};
            d.v[e] = u32x2{0u, 0u};
            if (PT) d.x[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// S_acc[m][e] = S[16 m + 4 g + e][16 w + c]  ->  st[j][i] (transposed bf16 tile)
__device__ __forceinline__ void stage_state(uint16_t *st, const f32x4 (&S)[4], int w, int g,
                                            int c) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
        *(u32x2 *)(st + (16 * w + c) * kP + 16 * m + 4 * g) =
            pack4(S[m][0], S[m][1], S[m][2], S[m][3]);
}

template <bool PT>
__global__ __launch_bounds__(256, 2) void wkv_chunk_kernel(
    int T, int H, const uint16_t *__restrict__ r, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ x,
    const float *__restrict__ u, const float *state_in, float *state_out,
    uint16_t *__restrict__ o) {
    __shared__ __align__(16) uint16_t sm[T_COUNT][kTile];
    __shared__ __align__(16) float sWave[4][kN];
    __shared__ __align__(16) float sBonus[kL];
    __shared__ __align__(16) float sDecay[kN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int cq = c;        // channel quad of the staging role
    const int tq = tid >> 4; // token quad of the staging role (= 4 w + g)

    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh % H;
    const size_t tok_stride = (size_t)H * kN;
    const size_t seq_base = (size_t)b * T * tok_stride + (size_t)h * kN;

    const f32x4 uq = *(const f32x4 *)(u + (size_t)h * kN + 4 * cq);
    f32x4 a2_static = {0.f, 0.f, 0.f, 0.f};
    if (!PT) {
        const f32x4 xs = *(const f32x4 *)(x + (size_t)h * kN + 4 * cq);
#pragma unroll
        for (int q = 0; q < 4; ++q) a2_static[q] = -exp2_fast(xs[q] * kLog2e) * kLog2e;
    }

    const size_t st_base = (size_t)bh * kN * kN;
    f32x4 S[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[m][e] = state_in ? state_in[st_base + (size_t)(16 * m + 4 * g + e) * kN + 16 * w + c]
                               : 0.0f;
    stage_state(sm[T_ST0], S, w, g, c);

    const int nchunks = (T + kL - 1) / kL;
    Raw cur, nxt;
    load_raw<PT>(cur, 0, tq, cq, T, seq_base, tok_stride, r, k, v, x);

    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = ch * kL;
        if (ch + 1 < nchunks)
            load_raw<PT>(nxt, c0 + kL, tq, cq, T, seq_base, tok_stride, r, k, v, x);

        // ---- log2 decays of my 4 tokens x 4 channels (0 on padding) --------
        float a2[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool valid = c0 + 4 * tq + e < T;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float val = PT ? -exp2_fast(cur.x[e][q] * kLog2e) * kLog2e : a2_static[q];
                a2[e][q] = valid ? val : 0.0f;
            }
        }
        // chunk-relative cumulative sums: thread, then wave (over g), then block
        float pre[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float tot = (a2[0][q] + a2[1][q]) + (a2[2][q] + a2[3][q]);
            float s = tot;
            const float s1 = __shfl_up(s, 16, 64);
            if (g >= 1) s += s1;
            const float s2 = __shfl_up(s, 32, 64);
            if (g >= 2) s += s2;
            const float ex = __shfl_up(s, 16, 64);
            pre[q] = (g == 0) ? 0.0f : ex;
            if (g == 3) sWave[w][4 * cq + q] = s;
        }
        __syncthreads();  // (1) wave totals visible; previous chunk fully consumed

        float LL[4], cmid[4];
        bool bad = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float t0 = sWave[0][4 * cq + q], t1 = sWave[1][4 * cq + q];
            const float t2 = sWave[2][4 * cq + q], t3 = sWave[3][4 * cq + q];
            const float before = (w == 0) ? 0.0f : (w == 1) ? t0 : (w == 2) ? (t0 + t1)
                                                                           : ((t0 + t1) + t2);
            pre[q] += before;
            cmid[q] = t0 + t1;
            LL[q] = ((t0 + t1) + t2) + t3;
            bad |= LL[q] < kSafeLog2;
        }

        // ---- stage the chunk's operands in LDS -------------------------------
        f32x4 er, ek;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            er[q] = exp2_fast(-cmid[q]);
            ek[q] = exp2_fast(cmid[q] - LL[q]);
        }
        float khh[4][4], khl[4][4], vv[4][4];
        f32x4 bsum;
        float run[4] = {pre[0], pre[1], pre[2], pre[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tau = 4 * tq + e;
            const float rr[4] = {bf16_lo(cur.r[e].x), bf16_hi(cur.r[e].x), bf16_lo(cur.r[e].y),
                                 bf16_hi(cur.r[e].y)};
            const float kk[4] = {bf16_lo(cur.k[e].x), bf16_hi(cur.k[e].x), bf16_lo(cur.k[e].y),
                                 bf16_hi(cur.k[e].y)};
            vv[e][0] = bf16_lo(cur.v[e].x);
            vv[e][1] = bf16_hi(cur.v[e].x);
            vv[e][2] = bf16_lo(cur.v[e].y);
            vv[e][3] = bf16_hi(cur.v[e].y);
            float qv[4], rt[4], kt[4];
            float bs = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lex = run[q];
                const float lin = run[q] + a2[e][q];
                run[q] = lin;
                const float fq = exp2_fast(lex);
                const float fk = exp2_fast(LL[q] - lin);
                qv[q] = rr[q] * fq;
                rt[q] = qv[q] * er[q];
                const float kh = kk[q] * fk;
                kt[q] = kh * ek[q];
                khh[e][q] = round_bf16(kh);
                khl[e][q] = kh - khh[e][q];
                bs = fmaf(rr[q] * uq[q], kk[q], bs);
            }
            bsum[e] = bs;
            *(u32x2 *)(sm[T_RT] + tau * kP + 4 * cq) = pack4(rt[0], rt[1], rt[2], rt[3]);
            *(u32x2 *)(sm[T_KT] + tau * kP + 4 * cq) = pack4(kt[0], kt[1], kt[2], kt[3]);
            *(u32x2 *)(sm[T_Q] + tau * kP + 4 * cq) = pack4(qv[0], qv[1], qv[2], qv[3]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = (4 * cq + q) * kP + 4 * tq;
            *(u32x2 *)(sm[T_KHH] + row) = pack4(khh[0][q], khh[1][q], khh[2][q], khh[3][q]);
            *(u32x2 *)(sm[T_KHL] + row) = pack4(khl[0][q], khl[1][q], khl[2][q], khl[3][q]);
            *(u32x2 *)(sm[T_VT] + row) = pack4(vv[0][q], vv[1][q], vv[2][q], vv[3][q]);
        }
        // bonus r_t diag(u) k_t^T: reduce over the 16 lanes sharing a token quad
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = bsum[e];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            s += __shfl_xor(s, 8, 64);
            bsum[e] = s;
        }
        if (c == 0) *(f32x4 *)(sBonus + 4 * tq) = bsum;
        if (tq == 0) {
            f32x4 d;
#pragma unroll
            for (int q = 0; q < 4; ++q) d[q] = exp2_fast(LL[q]);
            *(f32x4 *)(sDecay + 4 * cq) = d;
        }
        const bool unsafe = __syncthreads_or(bad);  // (2) operands staged

        uint16_t *st_cur = sm[T_ST0 + (ch & 1)];
        uint16_t *st_nxt = sm[T_ST0 + ((ch & 1) ^ 1)];
        if (!unsafe) {
            const int p = w;
            // P1: A^T tiles (sigma-tile q, tau-tile p), q <= p
            f32x4 at[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                at[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (q <= p) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const bf16x8 A = lds8(sm[T_KT] + (16 * q + c) * kP + 32 * kb + 8 * g);
                        const bf16x8 B = lds8(sm[T_RT] + (16 * p + c) * kP + 32 * kb + 8 * g);
                        at[q] = mfma(A, B, at[q]);
                    }
                }
                if (q == p) {  // causal mask, bonus on the diagonal
                    const float bon = sBonus[16 * p + c];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sl = 4 * g + e;
                        at[q][e] = sl < c ? at[q][e] : (sl == c ? bon : 0.0f);
                    }
                }
            }
            // P2: O^T = V^T A^T + S^T Q^T for tau-tile p, all value tiles n
            f32x4 ot[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) ot[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int bk = 0; bk < 2; ++bk) {
                if (2 * bk <= p) {
                    const bf16x8 Bop = pack8(at[2 * bk], at[2 * bk + 1]);
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        const uint16_t *row = sm[T_VT] + (16 * n + c) * kP + 32 * bk + 4 * g;
                        ot[n] = mfma(lds4x2(row, row + 16), Bop, ot[n]);
                    }
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 Bq = lds8(sm[T_Q] + (16 * p + c) * kP + 32 * kb + 8 * g);
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    ot[n] = mfma(lds8(st_cur + (16 * n + c) * kP + 32 * kb + 8 * g), Bq, ot[n]);
            }
            // P3: S' = diag(decay) S + (Kh_hi + Kh_lo)^T V for value tile w
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 d = *(const f32x4 *)(sDecay + 16 * m + 4 * g);
                S[m] *= d;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 Bv = lds8(sm[T_VT] + (16 * w + c) * kP + 32 * kb + 8 * g);
                    S[m] = mfma(lds8(sm[T_KHH] + (16 * m + c) * kP + 32 * kb + 8 * g), Bv, S[m]);
                    S[m] = mfma(lds8(sm[T_KHL] + (16 * m + c) * kP + 32 * kb + 8 * g), Bv, S[m]);
                }
            }
            stage_state(st_nxt, S, w, g, c);
            // outputs: lane holds O[tau = 16 p + c][16 n + 4 g + e]
            const int t = c0 + 16 * p + c;
            if (t < T) {
                uint16_t *op = o + seq_base + (size_t)t * tok_stride + 4 * g;
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    *(u32x2 *)(op + 16 * n) = pack4(ot[n][0], ot[n][1], ot[n][2], ot[n][3]);
            }
        } else {
            // Fast-decay chunk: apply its tokens one at a time.  Raw r, k
            // (bf16) replace the factorised tiles; w = 2^{a2} (fp32) spans
            // the Q and Kh_hi tiles.
            float *sw = (float *)sm[T_Q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * tq + e;
                *(u32x2 *)(sm[T_RT] + tau * kP + 4 * cq) = cur.r[e];
                *(u32x2 *)(sm[T_KT] + tau * kP + 4 * cq) = cur.k[e];
                f32x4 wv;
#pragma unroll
                for (int q = 0; q < 4; ++q) wv[q] = exp2_fast(a2[e][q]);
                *(f32x4 *)(sw + tau * kN + 4 * cq) = wv;
            }
            __syncthreads();  // (3) uniform: every thread took this branch
            const int nvalid = min(kL, T - c0);
            for (int tau = 0; tau < nvalid; ++tau) {
                const float vj = bf16_to_f32(sm[T_VT][(16 * w + c) * kP + tau]);
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x2 rp = *(const u32x2 *)(sm[T_RT] + tau * kP + 16 * m + 4 * g);
                    const u32x2 kp = *(const u32x2 *)(sm[T_KT] + tau * kP + 16 * m + 4 * g);
                    const f32x4 wv = *(const f32x4 *)(sw + tau * kN + 16 * m + 4 * g);
                    const float r4[4] = {bf16_lo(rp.x), bf16_hi(rp.x), bf16_lo(rp.y), bf16_hi(rp.y)};
                    const float k4[4] = {bf16_lo(kp.x), bf16_hi(kp.x), bf16_lo(kp.y), bf16_hi(kp.y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(r4[e], S[m][e], acc);
                        S[m][e] = fmaf(wv[e], S[m][e], k4[e] * vj);
                    }
                }
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                if (g == 0) {
                    const float ov = fmaf(sBonus[tau], vj, acc);
                    o[seq_base + (size_t)(c0 + tau) * tok_stride + 16 * w + c] =
                        (uint16_t)pack_bf16x2(ov, 0.0f);
                }
            }
            stage_state(st_nxt, S, w, g, c);
        }
        cur = nxt;
    }

    if (state_out != nullptr) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                state_out[st_base + (size_t)(16 * m + 4 * g + e) * kN + 16 * w + c] = S[m][e];
    }
}

}  // namespace

hipError_t launch_wkv_chunked(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                              const uint16_t *k, const uint16_t *v, const float *x,
                              const float *u, const float *state_in, float *state_out,
                              uint16_t *o, hipStream_t stream) {
    const unsigned blocks = (unsigned)((int64_t)B * H);
    if (per_token_decay)
        hipLaunchKernelGGL(wkv_chunk_kernel<true>, dim3(blocks), dim3(256), 0, stream, T, H, r,
                           k, v, x, u, state_in, state_out, o);
    else
        hipLaunchKernelGGL(wkv_chunk_kernel<false>, dim3(blocks), dim3(256), 0, stream, T, H, r,
                           k, v, x, u, state_in, state_out, o);
    return hipGetLastError();
}

}  // namespace wkv
