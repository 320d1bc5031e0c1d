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
// The producer writes h (rank 64, bf16) for every token; the chunked Finch
// kernel forms d from it per head, and lora_logits_kernel writes d for
// callers that want the logits themselves.  Two producer kernels:
// decay_once_kernel (D up to 2560) reads the block input once and keeps it
// in registers between its two passes; decay_lora_kernel (any D) streams it
// through LDS twice.
//
// Layout of the products: every product is taken transposed, weights as the
// A operand and tokens as the B operand columns (lane c of a 16-lane group
// = one token of a 16-token tile), so the result of one product is already
// the B operand of the next:
//   pass 1:  (y A1)^T  [32 x 16]  += A1^T [32 x 64 ch] . y^T [64 ch x 16]
//   pass 2:  m^T       [64 x 16]   = B1^T [64 ch x 32] . act(y A1)^T
//            (z A2)^T  [64 x 16]  += A2^T [64 x 64 ch] . z^T
// The rank k-slots (g, e) of lane group g are {4g + e, 16 + 4g + e} of each
// 32-wide step: the accumulator rows a lane holds (4g + e of two 16-row
// tiles) are then exactly the k-slots of the next product's B operand.  Two
// passes over the channels are needed because the mix of every channel
// needs act(y A1), a sum over all of them.
//
// decay_lora_kernel: a 64-channel block's weights and the workgroup's 128
// token rows (and their previous-token rows) are staged through LDS with
// row-contiguous loads, shared by the eight waves; the weights are read
// down their columns with the transposing LDS load.
#include <type_traits>

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

// The same products with the block input read once, for D up to 8 x 5
// blocks of 64 channels.  A workgroup takes 32 consecutive token rows, lane c
// of a 16-lane group holding tokens 2c and 2c + 1 (product column c of the
// two token tiles n = 0, 1), and its eight waves split the channel blocks
// (wave w: blocks w, w + 8, ...).  Each wave keeps x_t of its blocks in
// registers from pass 1 to pass 2.  x_{t-1} is never loaded: for token
// 2c + 1 it is token 2c of the same lane, for token 2c it is token 2c - 1
// of lane c - 1, one DPP row shift; the tile's first token takes the row
// before the tile (or the shift row, or zero) from LDS, and a tile with a
// sequence start inside it loads those tokens' shift rows separately.  The
// sums over the channels, act(y A1) after pass 1 and act(z A2) after
// pass 2, are added over the waves through LDS in a fixed order.  The
// weights reach every wave as ready-made product operands: lora_pack_kernel
// lays A1, B1 and A2 out per block in the A operand's lane order once per
// call, 16 KB per block, which the workgroups read from L2 with one 16-byte
// load per lane and product.  Channel order inside a 32-channel half block
// s: lane group g holds channels 32 s + 8 g + j, j = 0..7, as the k-slots of
// the products that contract over channels, and as rows 4 g + e of the two
// 16-row tiles q of m^T (channel 32 s + 8 g + 4 q + e); the rank k-slots of
// m^T's product follow the accumulator rows of (y A1)^T, {4g + j, 16 + 4g +
// j - 4}.
constexpr int kFragsA1 = 4, kFragsB1 = 4, kFragsA2 = 8;  // per block: (s, m), (s, q), (s, M)
constexpr int kFrags = kFragsA1 + kFragsB1 + kFragsA2;
constexpr int kOnceWaves = 8, kOnceMaxKB = 5;  // blocks per wave held in registers
constexpr int kOnceMaxD = kOnceWaves * kOnceMaxKB * kKB;
constexpr int kOnceTok = 32;                   // tokens per workgroup
// operand register sets of the two passes (one step loaded ahead; deeper
// prefetch measured no faster)
constexpr int kP1 = 2, kP2 = 2;
// cache policy of the block input's loads: non-temporal (nt), so that the
// stream of rows, read once, does not evict the operand fragments from an
// XCD's L2, where every workgroup on it reads them again (measured: HBM
// reads 1.13x -> 1.04x of the input, 5 % less time)
constexpr int kStreamNT = 2;

// rank k-slot j of lane group g
__device__ __forceinline__ int kslot(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }
// b, or zeros when keep is false
__device__ __forceinline__ bf16x8 zero_unless(bool keep, const bf16x8 &b) {
    const u32x4 u = __builtin_bit_cast(u32x4, b);
    const u32x4 z = {keep ? u.x : 0u, keep ? u.y : 0u, keep ? u.z : 0u, keep ? u.w : 0u};
    return __builtin_bit_cast(bf16x8, z);
}

// One thread per (block, fragment, lane): the 8 bf16 of that lane's operand.
__global__ void lora_pack_kernel(int D, const uint16_t *__restrict__ A1,
                                 const uint16_t *__restrict__ B1,
                                 const uint16_t *__restrict__ A2, bf16x8 *__restrict__ packed) {
    const int nkb = D / kKB;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nkb * kFrags * 64) return;
    const int lane = idx & 63, f = (idx >> 6) % kFrags, kb = idx / (64 * kFrags);
    const int g = lane >> 4, c = lane & 15, ch0 = kb * kKB;
    uint16_t v[8];
    if (f < kFragsA1) {  // A1^T: row rank 16 m + c, k-slot j channel 32 s + 8 g + j
        const int s = f >> 1, m = f & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = A1[(size_t)(ch0 + 32 * s + 8 * g + j) * kR1 + 16 * m + c];
    } else if (f < kFragsA1 + kFragsB1) {  // B1^T: row channel of m^T row c, k-slot rank kslot
        const int s = (f - kFragsA1) >> 1, q = (f - kFragsA1) & 1;
        const int ch = ch0 + 32 * s + 8 * (c >> 2) + 4 * q + (c & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = B1[(size_t)kslot(g, j) * D + ch];
    } else {  // A2^T: row rank 16 M + c, k-slot j channel 32 s + 8 g + j
        const int s = (f - kFragsA1 - kFragsB1) >> 2, M = (f - kFragsA1 - kFragsB1) & 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = A2[(size_t)(ch0 + 32 * s + 8 * g + j) * kR2 + 16 * M + c];
    }
    const u32x4 m4 = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                      v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
    packed[idx] = __builtin_bit_cast(bf16x8, m4);
}

template <bool TANH, int KB, bool INNER>
__global__ __launch_bounds__(64 * kOnceWaves, 1) void decay_once_kernel(
    int rows, int T, int D, const uint16_t *__restrict__ x, const uint16_t *__restrict__ shift,
    const float *__restrict__ mu, const float *__restrict__ lam,
    const bf16x8 *__restrict__ packed, uint16_t *__restrict__ h) {
    constexpr int NW = kOnceWaves;
    // (mu, lam and the boundary row are staged by every thread, unconditionally:
    // 1024 x 4 floats and 512 x 8 bf16, zero past D)
    __shared__ __align__(16) float sMu[4 * 1024], sLam[4 * 1024];
    __shared__ __align__(16) uint16_t sBnd[8 * 512];  // x_{t-1} of the tile's first token
    __shared__ __align__(16) f32x4 sRed1[NW][4][64];    // partial (y A1)^T: [wave][2 m + n]
    __shared__ __align__(16) u32x2 sH1[2][2][64];       // act(y A1)^T, bf16: [n][m]
    __shared__ __align__(16) f32x4 sRed2[NW][8][64];    // partial (z A2)^T: [wave][2 M + n]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: block offsets in SGPRs)
    const int c = lane & 15, g = lane >> 4;
    const int nkb = D / kKB;
    const int r0 = blockIdx.x * kOnceTok, t0 = r0 % T;
    // a sequence starts inside the tile (its first token aside); only
    // possible, and only compiled in, when T is not a multiple of the tile
    const bool inner = INNER && T - t0 < kOnceTok && r0 + (T - t0) < rows;

    // mu, lam and the row before the tile go to LDS; every thread issues the
    // same five loads (past the end they read zero)
    const Rsrc rmu = rsrc(mu, (uint32_t)D * 4), rlam = rsrc(lam, (uint32_t)D * 4);
    const uint16_t *bnd = t0 > 0 ? x + (size_t)(r0 - 1) * D : shift ? shift + (size_t)(r0 / T) * D : x;
    const Rsrc rbnd = rsrc(bnd, t0 > 0 || shift ? (uint32_t)D * 2 : 0u);
    f32x4 smu[2], slam[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        smu[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rmu, (tid + 512 * j) * 16, 0, 0));
        slam[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rlam, (tid + 512 * j) * 16, 0, 0));
    }
    const u32x4 sb = __builtin_amdgcn_raw_buffer_load_b128(rbnd, tid * 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // (issued first: their LDS writes wait for them)

    // this lane's x_t: token 2c + n of the tile, channels 32 s + 8 g .. + 7
    // of each of its blocks (rows past the end read zero and store nothing)
    const Rsrc rx = rsrc(x + (size_t)r0 * D, (uint32_t)min(rows - r0, kOnceTok) * D * 2);
    const int vo0 = 2 * c * D * 2 + 16 * g, vo1 = vo0 + D * 2;
    auto blk = [&](int i) { return min(w + NW * i, nkb - 1); };  // (past the last: reread, unused)
    auto live = [&](int i) { return w + NW * i < nkb; };
    u32x4 xv[KB][2][2];
    auto load_x = [&](int i) {  // (issued with pass 1's operands of block i, so that
                                // pass 1 computes while later blocks arrive)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int so = blk(i) * kKB * 2 + 64 * s;
            xv[i][s][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, vo0, so, kStreamNT);
            xv[i][s][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, vo1, so, kStreamNT);
        }
    };
    const Rsrc rp = rsrc(packed, (uint32_t)nkb * kFrags * 64 * 16);
    auto frag = [&](int kb, int f) {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              rp, lane * 16, (kb * kFrags + f) * 1024, 0));
    };
    auto f4lo = [](const u32x4 &p) { return f32x4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)}; };
    auto f4hi = [](const u32x4 &p) { return f32x4{bf16_lo(p.z), bf16_hi(p.z), bf16_lo(p.w), bf16_hi(p.w)}; };
    // x_{t-1} of this lane's two tokens at channel ch (= 32 s + 8 g of block)
    auto prev = [&](const u32x4 &x0, const u32x4 &x1, int ch, u32x4 &p0, u32x4 &p1) {
        const u32x4 b = *(const u32x4 *)&sBnd[ch];
        p0.x = __builtin_amdgcn_update_dpp(b.x, x1.x, 0x111, 0xf, 0xf, false);  // row_shr:1
        p0.y = __builtin_amdgcn_update_dpp(b.y, x1.y, 0x111, 0xf, 0xf, false);
        p0.z = __builtin_amdgcn_update_dpp(b.z, x1.z, 0x111, 0xf, 0xf, false);
        p0.w = __builtin_amdgcn_update_dpp(b.w, x1.w, 0x111, 0xf, 0xf, false);
        p1 = x0;
        if (inner) {  // tokens that start a sequence inside the tile
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int r = r0 + 2 * c + n;
                if (2 * c + n > 0 && r < rows && r % T == 0) {
                    const u32x4 v = shift ? *(const u32x4 *)(shift + (size_t)(r / T) * D + ch)
                                          : u32x4{0u, 0u, 0u, 0u};
                    if (n == 0) p0 = v;
                    else p1 = v;
                }
            }
        }
    };

    // ---- pass 1: (y A1)^T, this wave's blocks, kP1 - 1 blocks of operands
    // ahead
    struct P1 {
        bf16x8 a[4];  // A1^T operands (s, m)
    };
    auto load1 = [&](P1 &p, int i) {
        load_x(i);
#pragma unroll
        for (int f = 0; f < kFragsA1; ++f) p.a[f] = frag(blk(i), f);
    };
    P1 r1[kP1];
    // the first block's rows and operands go out before the staging waits
#pragma unroll
    for (int j = 0; j < kP1 - 1; ++j)
        if (j < KB) load1(r1[j], j);
    __builtin_amdgcn_sched_barrier(0);
    // stage mu, lam and the boundary row
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = 4 * (tid + 512 * j);
        *(f32x4 *)&sMu[e] = smu[j];
        *(f32x4 *)&sLam[e] = slam[j];
    }
    *(u32x4 *)&sBnd[8 * tid] = sb;

    f32x4 acc1[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc1[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        if (i + kP1 - 1 < KB) load1(r1[(i + kP1 - 1) % kP1], i + kP1 - 1);
        __builtin_amdgcn_sched_barrier(0);  // (the loads stay ahead of the block's products)
        {
            // (no branch on a dead block, a repeat of the last one: its
            // operand is zeroed instead, so that the loads above stay where
            // they are rather than being moved into the branch)
            const bool lv = live(i);
            const P1 &cur = r1[i % kP1];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ch = blk(i) * kKB + 32 * s + 8 * g;
                const f32x4 m0 = *(const f32x4 *)&sMu[ch], m1 = *(const f32x4 *)&sMu[ch + 4];
                u32x4 p[2];
                prev(xv[i][s][0], xv[i][s][1], ch, p[0], p[1]);
                bf16x8 Bop[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const f32x4 xl = f4lo(xv[i][s][n]), xh = f4hi(xv[i][s][n]);
                    const f32x4 yl = xl + (f4lo(p[n]) - xl) * m0, yh = xh + (f4hi(p[n]) - xh) * m1;
                    Bop[n] = zero_unless(lv, pack8(yl, yh));
                }
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int n = 0; n < 2; ++n) acc1[m][n] = mfma(cur.a[2 * s + m], Bop[n], acc1[m][n]);
            }
        }
        // (keeps the scheduler from hoisting later blocks' loads: the kP1
        // register sets are the whole prefetch)
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) sRed1[w][2 * m + n][lane] = acc1[m][n];
    lds_barrier();
    if (w < 4) {  // tile (m, n) = (w / 2, w % 2): the sum over the waves, act
        f32x4 sum = sRed1[0][w][lane];
#pragma unroll
        for (int j = 1; j < NW; ++j) sum += sRed1[j][w][lane];
        sH1[w & 1][w >> 1][lane] = pack4(act<TANH>(sum[0]), act<TANH>(sum[1]),
                                          act<TANH>(sum[2]), act<TANH>(sum[3]));
    }
    lds_barrier();
    // act(y A1)^T of token tile n as the B operand of the mix: k-slots
    // {4g + e, 16 + 4g + e}
    bf16x8 Bh1[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const u32x2 lo = sH1[n][0][lane], hi = sH1[n][1][lane];
        Bh1[n] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    }

    // ---- pass 2: m, z and (z A2)^T, in half blocks (32 channels) ----------
    // (x_t taken as new values here: pass 1's conversions of it are
    // recomputed, not kept alive in registers through the reduction)
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int n = 0; n < 2; ++n) __asm__ volatile("" : "+v"(xv[i][s][n]));
    struct P2 {
        bf16x8 b[2];  // B1^T operands, m^T tiles q
        bf16x8 a[4];  // A2^T operands, rank tiles M
    };
    auto load2 = [&](P2 &p, int hs) {  // half step hs: block hs / 2, s = hs % 2
        const int kb = blk(hs >> 1), s = hs & 1;
#pragma unroll
        for (int q = 0; q < 2; ++q) p.b[q] = frag(kb, kFragsA1 + 2 * s + q);
#pragma unroll
        for (int M = 0; M < 4; ++M) p.a[M] = frag(kb, kFragsA1 + kFragsB1 + 4 * s + M);
    };
    f32x4 acc2[4][2];
#pragma unroll
    for (int M = 0; M < 4; ++M)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc2[M][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    P2 r2[kP2];
#pragma unroll
    for (int j = 0; j < kP2 - 1; ++j)
        if (j < 2 * KB) load2(r2[j], j);
#pragma unroll
    for (int hs = 0; hs < 2 * KB; ++hs) {
        const int i = hs >> 1, s = hs & 1;
        if (hs + kP2 - 1 < 2 * KB) load2(r2[(hs + kP2 - 1) % kP2], hs + kP2 - 1);
        {
            const bool lv = live(i);
            const P2 &cur = r2[hs % kP2];
            const int ch = blk(i) * kKB + 32 * s + 8 * g;
            const f32x4 l0 = *(const f32x4 *)&sLam[ch], l1 = *(const f32x4 *)&sLam[ch + 4];
            u32x4 p[2];
            prev(xv[i][s][0], xv[i][s][1], ch, p[0], p[1]);
            bf16x8 Bz[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                // m^T rows 4 g + e of tiles q: channels ch + 4 q + e
                const f32x4 mt0 = mfma(cur.b[0], Bh1[n], f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 mt1 = mfma(cur.b[1], Bh1[n], f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 xl = f4lo(xv[i][s][n]), xh = f4hi(xv[i][s][n]);
                const f32x4 zl = xl + (f4lo(p[n]) - xl) * (l0 + mt0);
                const f32x4 zh = xh + (f4hi(p[n]) - xh) * (l1 + mt1);
                Bz[n] = zero_unless(lv, pack8(zl, zh));
            }
#pragma unroll
            for (int M = 0; M < 4; ++M)
#pragma unroll
                for (int n = 0; n < 2; ++n) acc2[M][n] = mfma(cur.a[M], Bz[n], acc2[M][n]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int M = 0; M < 4; ++M)
#pragma unroll
        for (int n = 0; n < 2; ++n) sRed2[w][2 * M + n][lane] = acc2[M][n];
    lds_barrier();
    // h = act(z A2): wave w adds tile (M, n) = (w / 2, w % 2) over the waves
    // and stores ranks 16 M + 4 g + e of token 2c + n
    {
        f32x4 sum = sRed2[0][w][lane];
#pragma unroll
        for (int j = 1; j < NW; ++j) sum += sRed2[j][w][lane];
        const int row = r0 + 2 * c + (w & 1);
        if (row < rows)
            *(u32x2 *)(h + (size_t)row * kR2 + 16 * (w >> 1) + 4 * g) =
                pack4(act<TANH>(sum[0]), act<TANH>(sum[1]), act<TANH>(sum[2]), act<TANH>(sum[3]));
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

size_t lora_packed_bytes(int D) {
    return D / kKB <= kOnceWaves * kOnceMaxKB ? (size_t)(D / kKB) * kFrags * 64 * 16 : 0;
}

hipError_t launch_decay_lora(int rows, int T, int D, bool tanh_act, const uint16_t *x,
                             const uint16_t *shift, const float *mu, const float *lam,
                             const uint16_t *A1, const uint16_t *B1, const uint16_t *A2,
                             uint16_t *h, void *packed, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int nkb = D / kKB;
    if (lora_packed_bytes(D) != 0) {  // the block input read once
        if (packed == nullptr) return hipErrorInvalidValue;  // (the entry points size it)
        const int n = nkb * kFrags * 64;
        hipLaunchKernelGGL(lora_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, D, A1, B1, A2, (bf16x8 *)packed);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const dim3 grid((unsigned)((rows + kOnceTok - 1) / kOnceTok));
        const int kb_per_wave = (nkb + kOnceWaves - 1) / kOnceWaves;
        const bool aligned = T % kOnceTok == 0;  // no sequence starts inside a tile
        auto go = [&](auto tanh_tag, auto kb_tag) {
            constexpr bool TA = decltype(tanh_tag)::value;
            constexpr int K = decltype(kb_tag)::value;
            if (aligned)
                hipLaunchKernelGGL((decay_once_kernel<TA, K, false>), grid, dim3(64 * kOnceWaves),
                                   0, stream, rows, T, D, x, shift, mu, lam,
                                   (const bf16x8 *)packed, h);
            else
                hipLaunchKernelGGL((decay_once_kernel<TA, K, true>), grid, dim3(64 * kOnceWaves),
                                   0, stream, rows, T, D, x, shift, mu, lam,
                                   (const bf16x8 *)packed, h);
        };
        auto by_kb = [&](auto tanh_tag) {
            switch (kb_per_wave) {
                case 1: go(tanh_tag, std::integral_constant<int, 1>{}); break;
                case 2: go(tanh_tag, std::integral_constant<int, 2>{}); break;
                case 3: go(tanh_tag, std::integral_constant<int, 3>{}); break;
                case 4: go(tanh_tag, std::integral_constant<int, 4>{}); break;
                default: go(tanh_tag, std::integral_constant<int, 5>{}); break;
            }
        };
        if (tanh_act) by_kb(std::true_type{});
        else by_kb(std::false_type{});
        return hipGetLastError();
    }
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
