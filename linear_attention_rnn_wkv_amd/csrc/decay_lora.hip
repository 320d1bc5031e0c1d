// decay_lora.hip -- the Finch decay producer on gfx950 (RWKV-5/6 summary,
// 4.1.1 "Eagle token shift": a learned per-channel mix of x_t and x_{t-1};
// 4.2.1 "Finch token shift": the mix made data-dependent by a LoRA with
// A in R^{D x 32}, B in R^{32 x D} that takes the Eagle-style mixed value as
// its input, and LoRA_omega with A in R^{D x 64}, B in R^{64 x D}; 4.2.2
// "Finch time mixing": the decay logit of every token and channel).  Per
// token t of a sequence, x_{-1} being the caller's shift row (or zero):
//
//     dx = x_{t-1} - x_t,   y = x_t + dx * mu,   m = lam + act(y A1) B1,
//     z  = x_t + dx * m,    h = act(z A2),       d = omega + h B2.
//
// decay_lora_kernel writes h (rank 64, bf16) for every token; the chunked
// Finch kernel forms d from it per head, and lora_logits_kernel writes d
// for callers that want the logits themselves.
//
// Layout of the products: every product is taken transposed, weights as the
// A operand and tokens as the B operand columns (lane c of a 16-lane group
// = token c of the wave's 16), so the result of one product is already the
// B operand of the next:
//   pass 1:  (y A1)^T  [32 x 16]  += A1^T [32 x 64 ch] . y^T [64 ch x 16]
//   pass 2:  m^T       [64 x 16]   = B1^T [64 ch x 32] . act(y A1)^T
//            (z A2)^T  [64 x 16]  += A2^T [64 x 64 ch] . z^T
// with k-slots (g, e) of lane group g taken as {4g + e, 16 + 4g + e} of each
// 32-wide step: the accumulator rows a lane holds (4g + e of two 16-row
// tiles) are then exactly the k-slots of the next product's B operand.  A
// 64-channel block's weights and the workgroup's 128 token rows (and their
// previous-token rows) are staged through LDS with row-contiguous loads,
// shared by the eight waves; the weights are read down their columns with
// the transposing LDS load.  Two passes stream the channels: the mix of
// every channel needs act(y A1), a sum over all of them.
#include "launchers.h"
#include "wkv_tiles.h"

namespace wkv {
namespace {

using namespace tiles;

constexpr int kR1 = 32;               // rank of the mix's LoRA
constexpr int kR2 = 64;               // rank of LoRA_omega
constexpr int kKB = 64;               // channels per block
constexpr int kWaves = 8;
constexpr int kTokWG = 16 * kWaves;  // tokens per workgroup

template <bool TANH>
__device__ __forceinline__ float act(float s) {
    return TANH ? tanhf(s) : s;
}

// Pipeline over the channel blocks: the loads of block kb + kPD - 1 (its
// weights, the 128 token rows and each row's previous-token row, 128 bytes
// each, contiguous) go into register set (kb + kPD - 1) % kPD at step kb;
// block kb + 1 is written from its set to LDS buffer (kb + 1) % 2 at step
// kb, and block kb is computed from buffer kb % 2.  A buffer is rewritten
// one barrier after its last read.  Every step issues the same loads (past
// the last block they read it again and are not used) and every thread
// issues them all: the compiler waits for a load by counting the loads
// issued after it, and a count that differed between paths or lanes would
// make it wait for the newest ones too.
constexpr int kPD = 3;
constexpr int kXP = kN + 8;  // LDS pitch of the token tiles (bf16)

template <bool TANH>
__global__ __launch_bounds__(512, 1) void decay_lora_kernel(
    int rows, int T, int D, const uint16_t *__restrict__ x, const uint16_t *__restrict__ shift,
    const float *__restrict__ mu, const float *__restrict__ lam,
    const uint16_t *__restrict__ A1, const uint16_t *__restrict__ B1,
    const uint16_t *__restrict__ A2, uint16_t *__restrict__ h) {
    __shared__ __align__(16) uint16_t sA1[2][kKB * kPC];  // [channel][rank], 32 ranks
    __shared__ __align__(16) uint16_t sB1[2][kR1 * kPC];  // [rank][channel]
    __shared__ __align__(16) uint16_t sA2[2][kKB * kPC];  // [channel][rank]
    __shared__ __align__(16) float sMu[2][kKB], sLam[2][kKB];
    __shared__ __align__(16) uint16_t sX[2][kTokWG * kXP];  // [token][channel] x_t
    __shared__ __align__(16) uint16_t sP[2][kTokWG * kXP];  // [token][channel] x_{t-1}

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * kTokWG;
    // this lane's token in the products: column c of the wave's 16 (rows
    // past the end compute on clamped data and store nothing)
    const int row = row0 + 16 * w + c;
    const int nkb = D / kKB, last = nkb - 1;

    // Token staging: thread tid moves 16-byte piece q = tid & 7 of tile rows
    // i = tid / 8 and i + 64, for x_t and for x_{t-1} (the shift row, or
    // zero without one, at a sequence's first token).
    const int q = tid & 7;
    const uint16_t *src[4];
    bool zero[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = min(row0 + (tid >> 3) + 64 * j, rows - 1);
        const int t = r % T, b = r / T;
        src[j] = x + (size_t)r * D + 8 * q;
        src[2 + j] = (t > 0 ? x + (size_t)(r - 1) * D : (shift ? shift + (size_t)b * D : x)) + 8 * q;
        zero[j] = false;
        zero[2 + j] = t == 0 && shift == nullptr;
    }

    // Weights: threads (tid & 255) one 16-byte piece of the A1 block (64 rows
    // of 64 bytes) and of the B1 block (32 rows of 128 bytes), every thread
    // one of the A2 block (64 rows of 128 bytes), threads (tid & 15) four mu
    // and lam; only the first thread of each piece writes it to LDS.
    const int t8 = tid & 255, t4 = tid & 15;
    struct Stage {
        u32x4 tok[4];
        u32x4 a1, b1, a2;
        f32x4 m, l;
    };
    auto fetch = [&](int kb, Stage &st, bool pass2) {
        const int ch = kb * kKB;
        if (!pass2) {
            st.a1 = *(const u32x4 *)(A1 + (size_t)(ch + (t8 >> 2)) * kR1 + 8 * (t8 & 3));
            st.m = *(const f32x4 *)(mu + ch + 4 * t4);
        } else {
            st.a2 = *(const u32x4 *)(A2 + (size_t)(ch + (tid >> 3)) * kR2 + 8 * (tid & 7));
            st.b1 = *(const u32x4 *)(B1 + (size_t)(t8 >> 3) * D + ch + 8 * (t8 & 7));
            st.l = *(const f32x4 *)(lam + ch + 4 * t4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st.tok[j] = *(const u32x4 *)(src[j] + ch);
    };
    auto put = [&](int buf, const Stage &st, bool pass2) {
        if (!pass2) {
            if (tid < 256) *(u32x4 *)(sA1[buf] + (tid >> 2) * kPC + 8 * (tid & 3)) = st.a1;
            if (tid < 16) *(f32x4 *)&sMu[buf][4 * tid] = st.m;
        } else {
            *(u32x4 *)(sA2[buf] + (tid >> 3) * kPC + 8 * (tid & 7)) = st.a2;
            if (tid < 256) *(u32x4 *)(sB1[buf] + (tid >> 3) * kPC + 8 * (tid & 7)) = st.b1;
            if (tid < 16) *(f32x4 *)&sLam[buf][4 * tid] = st.l;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint16_t *dst = (j < 2 ? sX[buf] : sP[buf]) + ((tid >> 3) + 64 * (j & 1)) * kXP + 8 * q;
            *(u32x4 *)dst = zero[j] ? u32x4{0u, 0u, 0u, 0u} : st.tok[j];
        }
    };
    // x and dx of this lane's token, channel group M of the block in buffer
    auto xd = [&](int buf, int M, f32x4 &xf, f32x4 &df) {
        const int off = (16 * w + c) * kXP + 16 * M + 4 * g;
        const u32x2 xv = *(const u32x2 *)(sX[buf] + off), pv = *(const u32x2 *)(sP[buf] + off);
        xf = f32x4{bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
        df = f32x4{bf16_lo(pv.x), bf16_hi(pv.x), bf16_lo(pv.y), bf16_hi(pv.y)} - xf;
    };

    // one pass over the channel blocks
    Stage ring[kPD];
    auto pass = [&](bool pass2, auto compute) {
#pragma unroll
        for (int j = 0; j < kPD - 1; ++j) fetch(min(j, last), ring[j], pass2);
        put(0, ring[0], pass2);
        lds_barrier();
        for (int kb0 = 0; kb0 < nkb; kb0 += kPD) {
#pragma unroll
            for (int j = 0; j < kPD; ++j) {
                const int kb = kb0 + j;
                fetch(min(kb + kPD - 1, last), ring[(j + kPD - 1) % kPD], pass2);
                if (kb < nkb) {
                    compute(kb & 1);
                    if (kb + 1 < nkb) put((kb + 1) & 1, ring[(j + 1) % kPD], pass2);
                    lds_barrier();
                }
            }
        }
    };

    // ---- pass 1: (y A1)^T -------------------------------------------------
    f32x4 acc1[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    pass(false, [&](int cur) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            f32x4 y[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                f32x4 xf, df;
                xd(cur, 2 * s + i, xf, df);
                y[i] = xf + df * *(const f32x4 *)&sMu[cur][16 * (2 * s + i) + 4 * g];
            }
            const bf16x8 Bop = pack8(y[0], y[1]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
                acc1[m] = mfma(lds_col4x2(sA1[cur], 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * m, c),
                               Bop, acc1[m]);
        }
    });
    // act(y A1)^T as the B operand of the mix: k-slots {4g + e, 16 + 4g + e}
    f32x4 h1[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) h1[m][e] = act<TANH>(acc1[m][e]);
    const bf16x8 Bh1 = pack8(h1[0], h1[1]);

    // ---- pass 2: m, z and (z A2)^T ---------------------------------------
    f32x4 acc2[4];
#pragma unroll
    for (int M = 0; M < 4; ++M) acc2[M] = f32x4{0.f, 0.f, 0.f, 0.f};
    pass(true, [&](int cur) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // m^T of channel groups 2s, 2s+1 (rows 16 M + 4 g + e, token c)
            f32x4 z[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int M = 2 * s + i;
                const f32x4 mt = mfma(lds_col4x2(sB1[cur], 4 * g, 16 + 4 * g, 16 * M, c), Bh1,
                                      f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 xf, df;
                xd(cur, M, xf, df);
                z[i] = xf + df * (*(const f32x4 *)&sLam[cur][16 * M + 4 * g] + mt);
            }
            const bf16x8 Bz = pack8(z[0], z[1]);
#pragma unroll
            for (int M = 0; M < 4; ++M)
                acc2[M] = mfma(lds_col4x2(sA2[cur], 32 * s + 4 * g, 32 * s + 16 + 4 * g, 16 * M, c),
                               Bz, acc2[M]);
        }
    });
    // h = act(z A2): ranks 16 M + 4 g + e of token row
    if (row < rows) {
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = act<TANH>(acc2[M][e]);
            *(u32x2 *)(h + (size_t)row * kR2 + 16 * M + 4 * g) = pack4(v[0], v[1], v[2], v[3]);
        }
    }
}

// d = omega + h B2 for 64 tokens x one 64-channel head per workgroup (four
// waves, 16 tokens each): d^T [64 ch x 16 tok] = B2^T . h^T on bf16 MFMA,
// B2's head block staged in LDS.
__global__ __launch_bounds__(256) void lora_logits_kernel(int rows, int D,
                                                          const uint16_t *__restrict__ h,
                                                          const uint16_t *__restrict__ B2,
                                                          const float *__restrict__ omega,
                                                          float *__restrict__ d) {
    __shared__ __align__(16) uint16_t sB2[kR2 * kPC];  // [rank][channel]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int head = blockIdx.y, ch0 = head * kN;
    // 64 rows of 128 bytes: two 16-byte pieces per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i;
        *(u32x4 *)(sB2 + (p >> 3) * kPC + 8 * (p & 7)) =
            *(const u32x4 *)(B2 + (size_t)(p >> 3) * D + ch0 + 8 * (p & 7));
    }
    const int row = blockIdx.x * 64 + 16 * w + c;
    const bool valid = row < rows;
    const uint16_t *hr = h + (size_t)(valid ? row : rows - 1) * kR2;
    bf16x8 Bh[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) Bh[s] = *(const bf16x8 *)(hr + 32 * s + 8 * g);
    lds_barrier();
#pragma unroll
    for (int M = 0; M < 4; ++M) {
        f32x4 acc = *(const f32x4 *)(omega + ch0 + 16 * M + 4 * g);
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mfma(lds_col8(sB2, 32 * s + 8 * g, 16 * M, c), Bh[s], acc);
        if (valid) *(f32x4 *)(d + (size_t)row * D + ch0 + 16 * M + 4 * g) = acc;
    }
}

}  // namespace

hipError_t launch_decay_lora(int rows, int T, int D, bool tanh_act, const uint16_t *x,
                             const uint16_t *shift, const float *mu, const float *lam,
                             const uint16_t *A1, const uint16_t *B1, const uint16_t *A2,
                             uint16_t *h, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + kTokWG - 1) / kTokWG));
    if (tanh_act)
        hipLaunchKernelGGL(decay_lora_kernel<true>, grid, dim3(512), 0, stream, rows, T, D, x,
                           shift, mu, lam, A1, B1, A2, h);
    else
        hipLaunchKernelGGL(decay_lora_kernel<false>, grid, dim3(512), 0, stream, rows, T, D, x,
                           shift, mu, lam, A1, B1, A2, h);
    return hipGetLastError();
}

hipError_t launch_lora_logits(int rows, int D, const uint16_t *h, const uint16_t *B2,
                              const float *omega, float *d, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)(D / kN));
    hipLaunchKernelGGL(lora_logits_kernel, grid, dim3(256), 0, stream, rows, D, h, B2, omega, d);
    return hipGetLastError();
}

}  // namespace wkv
