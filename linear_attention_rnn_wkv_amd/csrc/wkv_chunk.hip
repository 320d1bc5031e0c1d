// wkv_chunk.hip -- Eagle (RWKV-5) / Finch (RWKV-6) WKV forward in
// time-parallel (chunked) mode on gfx950, bf16 MFMA with fp32 accumulation.
//
// Operation, per head (RWKV-5/6 summary, blob.wenxiaobai.com, section 4
// notation; 4.1.2 "Eagle time mixing"; 4.2.2 "Finch time mixing"):
//   o_t = r_t (S_{t-1} + diag(u) k_t^T v_t),  S_t = diag(w_t) S_{t-1} + k_t^T v_t,
//   w_t = exp(-exp(x_t)).
// Time-parallel evaluation (RWKV paper summary, section "Transformer-like
// parallelization"): the sequence is cut into chunks of L = 64 tokens.  With
// Lam_t = sum_{m<=t} log w_m (chunk-relative, fp32, kept in log2 units),
// Lam_L its value at the chunk end and S the state entering the chunk,
// unrolling the recurrence gives
//   o_t = sum_{s<t} [sum_i r~_t[i] k^_s[i]] v_s + (sum_i r_t[i] u[i] k_t[i]) v_t
//         + r~_t (diag(e^{Lam_L}) S)
//   S'  = diag(e^{Lam_L}) S + K^^T V
// with r~_t = r_t e^{Lam_{t-1} - Lam_L} (>= |r|) and k^_s = k_s e^{Lam_L - Lam_s}
// (<= |k|): the factorisation is anchored at the chunk end, so the decayed
// state diag(e^{Lam_L}) S that the update needs is also the operand of the
// output term.  Each chunk is three products on the matrix cores:
//   P1  A^T = K^ R~^T, masked causally, bonus on the diagonal
//   P2  O^T = V^T A^T + (diag(e^{Lam_L}) S)^T R~^T
//   P3  S'  = diag(e^{Lam_L}) S + (K^_hi + K^_lo)^T V   (K^ split into bf16
//       hi + lo so the carried fp32 state loses no precision)
// r~ and k^ stay inside the fp32 / bf16 range while the chunk's total
// log2-decay of every channel is above kSafeLog2; a chunk that decays faster
// is applied token by token instead (exact at any decay).
//
// Work split: one workgroup of NW = 4 or 8 wave64s per (sequence, head);
// with NH = NW / 4 and TP = 16 / NW tokens per staging thread:
//   staging   thread t: channels 4 (t%16) + {0..3}, tokens TP (t/16) + {0..TP-1};
//             v: tokens t/8 + 8 NW j, channels 8 (t%8) + {0..7}
//   P1, P2    wave w: tokens [16 (w%4), +16), value columns [64/NH (w/4), +64/NH)
//   P3        wave w: key rows [(128/NW) (w/2), +128/NW), value columns
//             [32 (w%2), +32) -- a block, so each wave reads only its share
//             of K^ and V
// so the fp32 state never leaves registers (except in the fast-decay path).
// Eight waves give two waves per SIMD to one head; four waves let two heads
// share a CU.  The launcher picks eight while the heads fit on the CUs.
// Operands are staged in LDS as row-major ([token][channel]) bf16 64x64
// tiles with a padded pitch; operands that contract over tokens are read
// with the transposing LDS load (ds_read_b64_tr_b16), so no tile is ever
// written transposed.
//
// Pipeline: chunk c's operand reads and matrix products are issued before
// the barrier that publishes chunk c+1's decay totals, and their results are
// only consumed after it, so the matrix cores run while the VALU stages
// chunk c+1 (decay scan, factors, tiles).  Two barriers per chunk.  Chunk
// c+1's r, k, v are fetched while chunk c's products run; Finch's decay
// logits (the first operand a chunk's staging needs) one step ahead of that.  HBM traffic is the
// algorithmic minimum: r, k, v, o (and x for Finch) once, the state once
// each way.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16): lane l = c + 16 g holds
// row c of the A operand and column c of the B operand, with eight k-slots
// indexed by (g, slot); both operands use the same (g, slot) -> k map, so
// any consistent map is valid.  The result lane l holds rows 4 g + e
// (e = 0..3) of column c.  P1's accumulators are therefore P2's B operand
// without leaving registers.  The transposing load: in each group of 16
// lanes, lane j supplies the address of 4 consecutive elements of row j/4 of
// a 4 x 16 block and receives column j of that block (rows 0..3).
#include <algorithm>
#include <type_traits>

#include "launchers.h"
#include "wkv_device.h"
#include "wkv_tiles.h"

namespace wkv {
namespace {

using namespace tiles;

// LDS tiles, all row-major: r~, k^_hi, k^_lo, v as [token][channel]; the
// decayed state as [j][i].
enum { T_RS = 0, T_KRH, T_KRL, T_VR, T_ST, T_COUNT };
__device__ constexpr int pitch(int t) { return (t == T_RS || t == T_ST) ? kPR : kPC; }

// Balanced split of B*H = first_extra + extra heads over first_extra /
// (nfull + 1) workgroups, each of which first runs nfull whole heads (see the
// kernel); extra == 0: one head per workgroup.
struct Split {
    int extra, first_extra, K, stride, chains_per_xcd;
    int nfull;        // whole heads per workgroup before the split round
    WsCtrl *ctrl;     // control block of the hand-off workspace (epoch, error word)
    unsigned *flags;  // [extra * (K - 1)] slot flags: the launch's tag once a slot is full
    float *slots;     // [extra * (K - 1)][64][64] states between segments
    float *park;      // [workgroups][64][64] own heads' states during the extra segment
                      // (four-wave launches; eight waves keep them in registers)
};

// Finch decay logits from the decay producer: h [B T][64] bf16, the rank-64
// factor of LoRA_omega of every token; B2 [64][H N] bf16 (B_omega) and
// omega [H N] fp32.  A head's logits are d = omega + h B2[:, head].
struct Lora {
    const uint16_t *h, *B2;
    const float *omega;
};

// SAVE: instead of the outputs and the final state, store the state entering
// every chunk and the final state, [B H][nchunks + 1][64][64] fp32 key-major,
// for the backward pass.
// EPI: write, instead of o, the output after the time-mixing
// epilogue (RWKV-5/6 summary, 4.1.2: a LayerNorm on each head, i.e. a
// GroupNorm over the heads, and a SiLU gate):
//   y = ((o - mean) / sqrt(var + eps) * ln_w + ln_b) * g / (1 + e^-g),
// mean and (biased) variance over the 64 channels of one head and token,
// taken from the fp32 accumulators before any rounding.  With eight waves a
// token's channels are split over two waves: each forms the mean and the sum
// of squared deviations of its half, the halves are merged through LDS
// after the step's barrier, and the chunk's outputs are written at the start
// of the next step (before its products overwrite the accumulators).
template <bool PT, int NW, bool SAVE, bool EPI = false, bool LORA = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void wkv_chunk_kernel(
    int T, int H, const uint16_t *__restrict__ r, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ x,
    const float *__restrict__ u, const float *state_in, float *state_out,
    uint16_t *__restrict__ o, Split sp, float *chunk_states,
    const uint16_t *__restrict__ gate, const float *__restrict__ ln_w,
    const float *__restrict__ ln_b, float eps, Lora lr) {
    static_assert(!LORA || (PT && !SAVE && !EPI), "the decay producer feeds the plain Finch forward");
    constexpr int NH = NW / 4;        // value / key halves split across waves
    constexpr int NT = 4 / NH;        // 16-wide value (P2) or key (P3) tiles per wave
    constexpr int TP = Raw<NW>::TP;   // tokens per staging thread
    // Eight waves (one workgroup per CU) double-buffer the operand tiles, the
    // decay totals, the bonus and the range flags by chunk parity: chunk c
    // uses set c & 1, so one barrier per chunk suffices (see the step).
    constexpr bool DB = NW == 8;
    constexpr int NS = DB ? 2 : 1;
    __shared__ __align__(16) uint16_t sm[NS][T_COUNT][kTile];
    __shared__ __align__(16) float sWave[NS][NW][kN];  // per-wave log2-decay totals
    __shared__ __align__(16) float sDecay[NW][kN];     // e^{Lam_L}, one copy per wave
    __shared__ __align__(16) float sBonus[NS][kL];
    __shared__ int sBad[NS][NW];  // per wave: a channel of the next chunk decays too fast
    // EPI: outputs of a fast-decay chunk before the epilogue, [token][channel]
    __shared__ __align__(16) float sO[EPI ? kL * kN : 1];
    // EPI, eight waves: (mean, sum of squared deviations) of each half-token
    __shared__ __align__(16) f32x2 sStat[EPI ? NS : 1][NW][16];
    // EPI, eight waves: the chunk's gate, [token][channel] bf16, staged with
    // its operands (four waves, short of registers, load it per lane)
    constexpr bool GST = EPI && NW == 8;
    __shared__ __align__(16) uint16_t sG[GST ? NS : 1][GST ? kL * kPR : 1];
    // LORA: the head's block of B_omega, [rank][channel] bf16, and per wave
    // its tokens' decay logits on their way from the product's layout to
    // stage A's, [token][channel] fp32
    constexpr int kDP = kN + 4;
    __shared__ __align__(16) uint16_t sB2[LORA ? kN * kPC : 1];
    __shared__ __align__(16) float sD[LORA ? NW : 1][LORA ? 4 * TP : 1][LORA ? kDP : 1];

    // SAVE with no outputs (the backward's recomputation): the chunk states
    // need neither r nor the output products, so r is not read, the r~ and
    // decayed-state tiles are not staged, and only P3 runs (uniform)
    const bool states_only = SAVE && o == nullptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int g = lane >> 4;
    int c = lane & 15;
    // P1/P2 token tile and P2 value part.  The causal products grow with the
    // token tile, and after a barrier the waves' loads are taken in wave
    // order, so with eight waves the first four take the two heavy tiles
    // (both value halves) and the last four the light ones.  The wave holding
    // the other half of a token tile is then w ^ 1.
    const int hf = NW == 8 ? (w & 1) : 0;
    const int p = NW == 8 ? 3 - (w >> 1) : w;

    Ctx cx;
    cx.T = T;
    cx.cq = tid & 15;      // == c
    cx.tq = tid >> 4;      // token group (= 4 w + g)
    cx.vt = tid >> 3;
    cx.vo = tid & 7;
    cx.tok_stride = (size_t)H * kN;
    cx.tokb = (uint32_t)H * kN * 2;
    cx.off_rk = (uint32_t)(TP * cx.tq) * cx.tokb + 8 * cx.cq;
    cx.off_v = (uint32_t)cx.vt * cx.tokb + 16 * cx.vo;

    // State tiles of this wave (P3): a block of MI key tiles x 2 value tiles,
    // so a wave reads a half or a quarter of K^ and half of V per chunk.
    // S[t][e] = S[skey(t) + 4 g + e][sval(t) + c].
    constexpr int MI = 8 / NW;
    const int skey0 = 16 * MI * (w >> 1), sval0 = 32 * (w & 1);
    auto skey = [&](int t) { return skey0 + 16 * (t >> 1); };
    auto sval = [&](int t) { return sval0 + 16 * (t & 1); };
    static_assert(2 * MI == NT, "a wave holds NT state tiles");
    auto sidx = [&](int t, int e) { return (skey(t) + 4 * g + e) * kN + sval(t) + c; };
    f32x4 S[NT], SD[NT];

    const int nchunks = (T + kL - 1) / kL;

    // Per-head values, set by set_head.  Eagle: the log2-decay is a
    // per-channel constant, so the factors of a full chunk do not change
    // from chunk to chunk: their bases are computed once per head, and each
    // token's factor follows by one multiply.
    f32x4 uq, a2s, wq, eLL, eF1, eF2;
    f32x4 omq;         // LORA: omega of this thread's four channels
    size_t hrow0 = 0;  // LORA: the sequence's first row of h
    // LORA, eight waves: the head's B_omega operands of the logits product,
    // held in registers (four waves, short of registers, read them from sB2)
    constexpr bool B2REG = LORA && NW == 8;
    bf16x8 b2f[B2REG ? 8 : 1];
    // EPI on eight waves: this lane's norm weight and bias, held per head (on
    // four waves, where registers are short, read when they are used)
    constexpr bool LNREG = EPI && NW == 8;
    f32x4 lnw[LNREG ? NT : 1], lnb[LNREG ? NT : 1];
    int bh = 0;  // (sequence, head) of the current job
    auto ln_at = [&](int ni, const float *base) -> f32x4 {
        return *(const f32x4 *)(base + (size_t)(bh % H) * kN + 16 * (NT * hf + ni) + 4 * g);
    };
    auto set_head = [&](int head) {
        bh = head;
        const int b = head / H, h = head % H;
        cx.seq_base = (size_t)b * T * cx.tok_stride + (size_t)h * kN;
        uq = *(const f32x4 *)(u + (size_t)h * kN + 4 * cx.cq);
        if (LORA) {
            // the head's B_omega block: 64 rows of 128 bytes (no wave reads
            // sB2 between the previous job's last barrier and this one)
            omq = *(const f32x4 *)(lr.omega + (size_t)h * kN + 4 * cx.cq);
            hrow0 = (size_t)b * T;
            for (int q = tid; q < kN * 8; q += 64 * NW)
                *(u32x4 *)(sB2 + (q >> 3) * kPC + 8 * (q & 7)) =
                    *(const u32x4 *)(lr.B2 + (size_t)(q >> 3) * H * kN + (size_t)h * kN + 8 * (q & 7));
            lds_barrier();
            if constexpr (B2REG) {
#pragma unroll
                for (int f = 0; f < (B2REG ? 8 : 1); ++f)
                    b2f[f] = lds_col8(sB2, 32 * (f & 1) + 8 * g, 16 * (f >> 1), c);
            }
        }
        if (LNREG) {
#pragma unroll
            for (int ni = 0; ni < (LNREG ? NT : 1); ++ni) {
                lnw[ni] = ln_at(ni, ln_w);
                lnb[ni] = ln_at(ni, ln_b);
            }
        }
        a2s = f32x4{0.f, 0.f, 0.f, 0.f};
        wq = f32x4{1.f, 1.f, 1.f, 1.f};
        eLL = a2s;
        eF1 = wq;
        eF2 = wq;
        if (!PT) {
            const f32x4 xs = *(const f32x4 *)(x + (size_t)h * kN + 4 * cx.cq);
            const float t0 = (float)(TP * cx.tq);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a2s[q] = -exp2_fast(xs[q] * kLog2e) * kLog2e;
                wq[q] = exp2_fast(a2s[q]);
                eLL[q] = (float)kL * a2s[q];
                eF1[q] = exp2_fast(t0 * a2s[q] - eLL[q]);
                eF2[q] = exp2_fast(eLL[q] - (t0 + TP) * a2s[q]);
            }
        }
    };
    // the current head's state from state_in (zeros without one) / to state_out
    auto load_state = [&]() {
        const size_t base = (size_t)bh * kN * kN;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = state_in ? state_in[base + sidx(t, e)] : 0.0f;
    };
    // the state entering chunk ch of the current head (SAVE)
    // A lane holds rows 4 g + e (e = 0..3) of column c of each of its state
    // tiles; a 4 x 4 transpose inside each quad of lanes (two DPP exchanges,
    // lane bit 1 with register bit 1, then bit 0 with bit 0) gives lane c
    // row 4 g + (c & 3), columns 4 (c >> 2) .. + 3, stored as one 16-byte
    // write instead of four 4-byte ones (the memory pipeline the next
    // chunk's loads queue in is shared with these stores).
    auto save_chunk = [&](int ch) {
        const size_t base = ((size_t)bh * (nchunks + 1) + ch) * kN * kN;
        const int q = c & 3;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 x = S[t];
            f32x4 y = {dpp<0x4e>(x[0]), dpp<0x4e>(x[1]), dpp<0x4e>(x[2]), dpp<0x4e>(x[3])};
            if (q & 2) x[0] = y[2], x[1] = y[3];
            else x[2] = y[0], x[3] = y[1];
            y = f32x4{dpp<0xb1>(x[0]), dpp<0xb1>(x[1]), dpp<0xb1>(x[2]), dpp<0xb1>(x[3])};
            if (q & 1) x[0] = y[1], x[2] = y[3];
            else x[1] = y[0], x[3] = y[2];
            *(f32x4 *)(chunk_states + base + (size_t)(skey(t) + 4 * g + q) * kN + sval(t) +
                       4 * (c >> 2)) = x;
        }
    };
    auto save_state = [&]() {
        if (SAVE) save_chunk(nchunks);
        if (state_out == nullptr) return;
        const size_t base = (size_t)bh * kN * kN;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) state_out[base + sidx(t, e)] = S[t][e];
    };

    // a chunk's inputs in registers between their load and their staging
    // (EPI: the gate of the chunk, loaded in v's layout)
    Raw<NW> buf;
    u32x4 graw[GST ? Raw<NW>::NV : 1];
    int ch_end = nchunks;  // end of the current job's chunk range

    // ---- LORA: the decay logits of a chunk from h ---------------------
    // A wave forms d^T = B2^T h^T for a 16-token tile holding its own 4 TP
    // tokens (eight waves: the pair's tile, half of it kept): lane (c, g)
    // loads h of token c, ranks 32 s + 8 g .. + 7, as the B operand of k-step s.
    typedef u32x4 HOps[LORA ? 2 : 1];
    HOps hq;
    const int dlo = NW == 8 ? 8 * (w & 1) : 0;  // first own token in the tile
    auto load_h_to = [&](HOps &dst, int ch, bool ok) {
        const int c0 = ch * kL;
        const int tile = NW == 8 ? 16 * (w >> 1) : 16 * w;
        const uint16_t *base = lr.h + (hrow0 + (size_t)(ok ? c0 : 0)) * kN;
        const Rsrc rh = rsrc(base, ok ? (uint32_t)min(kL, T - c0) * kN * 2 : 0u);
#pragma unroll
        for (int s2 = 0; s2 < (LORA ? 2 : 1); ++s2)
            dst[s2] = __builtin_amdgcn_raw_buffer_load_b128(
                rh, (uint32_t)((tile + c) * kN + 32 * s2 + 8 * g) * 2, 0, 0);
    };
    auto load_h = [&](int ch, bool ok) { load_h_to(hq, ch, ok); };
    // the chunk's next decay operands: x, or h for the producer's logits
    auto load_dec = [&](int ch, bool ok) {
        if (LORA) load_h(ch, ok);
        else if (PT) load_x<NW>(buf, ch * kL, cx, x, ok);
    };
    // this thread's logits (tokens TP tq + e, channels 4 cq + q) from the h
    // operands hs of its tile: the product into the wave's sD rows, then
    // read back in stage A's layout
    auto lora_product = [&](const HOps &hs) {
#pragma unroll
        for (int M = 0; M < 4; ++M) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                bf16x8 a;
                if constexpr (B2REG) a = b2f[B2REG ? 2 * M + s2 : 0];
                else a = lds_col8(sB2, 32 * s2 + 8 * g, 16 * M, c);
                acc = mfma(a, __builtin_bit_cast(bf16x8, hs[LORA ? s2 : 0]), acc);
            }
            if (c >= dlo && c < dlo + 4 * TP)
                *(f32x4 *)&sD[LORA ? w : 0][LORA ? c - dlo : 0][16 * M + 4 * g] = acc;
        }
    };
    auto lora_read = [&](f32x4(&xv)[TP]) {
#pragma unroll
        for (int e = 0; e < TP; ++e)
            xv[e] = *(const f32x4 *)&sD[LORA ? w : 0][LORA ? TP * g + e : 0][4 * cx.cq] + omq;
    };
    auto lora_logits = [&](const HOps &hs, f32x4(&xv)[TP]) {
        lora_product(hs);
        lora_read(xv);
    };

    // ---- stage A (Finch): log2 decays and the in-wave part of their scan --
    float a2[TP][4], lower[4];
    // (LORA: with formed = true the product already ran, at the start of the
    // step, and its rows wait in sD)
    auto stageA = [&](int ch, const Raw<NW> &d, int set, bool formed = false) {
        if (!PT) return;
        const int c0 = ch * kL;
        f32x4 xv[TP];
        if constexpr (LORA) {
            if (formed) lora_read(xv);
            else lora_logits(hq, xv);
        } else {
#pragma unroll
            for (int e = 0; e < TP; ++e) xv[e] = d.x[e];
        }
#pragma unroll
        for (int e = 0; e < TP; ++e) {
            const bool valid = c0 + TP * cx.tq + e < T;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a2[e][q] = valid ? -exp2_fast(xv[e][q] * kLog2e) * kLog2e : 0.0f;
        }
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
        if (g == 3) *(f32x4 *)&sWave[set][w][4 * cx.cq] = wt;
    };

    // ---- stage B: prefix, factors and the operand tiles of a chunk --------
    // (Finch needs stage A of every wave, i.e. a barrier in between)
    auto stageB = [&](int ch, const Raw<NW> &d, int set) -> bool {
        const int c0 = ch * kL;
        f32x4 LL, F1, F2;     // chunk total; 2^{lex_first - LL}; 2^{LL - lin_last}
        float wv[TP][4];      // per-token decay factors 2^{a2}
        if (PT) {
            // partial sums over the waves in a fixed order: every thread of a
            // channel obtains the same bits for the chunk total
            f32x4 part = *(const f32x4 *)&sWave[set][0][4 * cx.cq];
            f32x4 before = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 1; j < NW; ++j) {
                if (j == w) before = part;
                part += *(const f32x4 *)&sWave[set][j][4 * cx.cq];
            }
            LL = part;
            f32x4 pre, lin;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                pre[q] = before[q] + lower[q];
                float run = pre[q];
#pragma unroll
                for (int e = 0; e < TP; ++e) {
                    run += a2[e][q];
                    wv[e][q] = exp2_fast(a2[e][q]);
                }
                lin[q] = run;
                F1[q] = exp2_fast(pre[q] - LL[q]);
                F2[q] = exp2_fast(LL[q] - lin[q]);
            }
        } else {
            const int nvalid = min(kL, T - c0);
            if (nvalid == kL) {
                LL = eLL;
                F1 = eF1;
                F2 = eF2;
            } else {  // ragged last chunk: tokens past T do not decay
                const float t0 = (float)min(TP * cx.tq, nvalid);
                const float t1 = (float)min(TP * cx.tq + TP, nvalid);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    LL[q] = (float)nvalid * a2s[q];
                    F1[q] = exp2_fast(t0 * a2s[q] - LL[q]);
                    F2[q] = exp2_fast(LL[q] - t1 * a2s[q]);
                }
            }
#pragma unroll
            for (int e = 0; e < TP; ++e) {
                const bool valid = c0 + TP * cx.tq + e < T;
#pragma unroll
                for (int q = 0; q < 4; ++q) wv[e][q] = valid ? wq[q] : 1.0f;
            }
        }
        bool bad = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) bad |= LL[q] < kSafeLog2;
        if (g == 0) {
            f32x4 dd;
#pragma unroll
            for (int q = 0; q < 4; ++q) dd[q] = exp2_fast(LL[q]);
            *(f32x4 *)&sDecay[w][4 * cx.cq] = dd;
        }
        // k^ factors run backwards from the last token, r~ factors forwards
        float f2[TP][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f2[TP - 1][q] = F2[q];
#pragma unroll
            for (int e = TP - 2; e >= 0; --e) f2[e][q] = f2[e + 1][q] * wv[e + 1][q];
        }
        f32x4 f1 = F1;
        float bs[TP];
#pragma unroll
        for (int e = 0; e < TP; ++e) {
            const int tau = TP * cx.tq + e;
            const float rr[4] = {bf16_lo(d.r[e].x), bf16_hi(d.r[e].x), bf16_lo(d.r[e].y),
                                 bf16_hi(d.r[e].y)};
            const float kk[4] = {bf16_lo(d.k[e].x), bf16_hi(d.k[e].x), bf16_lo(d.k[e].y),
                                 bf16_hi(d.k[e].y)};
            float rt[4], kh[4], khl[4];
            float sb = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                rt[q] = rr[q] * f1[q];
                f1[q] *= wv[e][q];
                kh[q] = kk[q] * f2[e][q];
                sb = fmaf(rr[q] * uq[q], kk[q], sb);
            }
            const u32x2 hi = pack4(kh[0], kh[1], kh[2], kh[3]);
            khl[0] = kh[0] - bf16_lo(hi.x);
            khl[1] = kh[1] - bf16_hi(hi.x);
            khl[2] = kh[2] - bf16_lo(hi.y);
            khl[3] = kh[3] - bf16_hi(hi.y);
            if (!states_only)
                *(u32x2 *)(sm[set][T_RS] + tau * pitch(T_RS) + 4 * cx.cq) = pack4(rt[0], rt[1], rt[2], rt[3]);
            *(u32x2 *)(sm[set][T_KRH] + tau * pitch(T_KRH) + 4 * cx.cq) = hi;
            *(u32x2 *)(sm[set][T_KRL] + tau * pitch(T_KRL) + 4 * cx.cq) = pack4(khl[0], khl[1], khl[2], khl[3]);
            bs[e] = row_sum16(sb);  // bonus r_t diag(u) k_t^T over the token's 64 channels
        }
#pragma unroll
        for (int j = 0; j < Raw<NW>::NV; ++j)
            *(u32x4 *)(sm[set][T_VR] + (cx.vt + 8 * NW * j) * pitch(T_VR) + 8 * cx.vo) = d.v[j];
        if (GST) {
#pragma unroll
            for (int j = 0; j < (GST ? Raw<NW>::NV : 1); ++j)
                *(u32x4 *)(sG[set] + (cx.vt + 8 * NW * j) * kPR + 8 * cx.vo) = graw[j];
        }
        if (c == 0) {
            if (TP == 4)
                *(f32x4 *)&sBonus[set][TP * cx.tq] = f32x4{bs[0], bs[1 % TP], bs[2 % TP], bs[3 % TP]};
            else
                *(f32x2 *)&sBonus[set][TP * cx.tq] = f32x2{bs[0], bs[1 % TP]};
        }
        return bad;
    };

    // decayed state of the next chunk, staged transposed as bf16
    auto stage_state = [&](int set) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 dd = *(const f32x4 *)&sDecay[w][skey(t) + 4 * g];
            SD[t] = S[t] * dd;
            if (!states_only)
                *(u32x2 *)(sm[set][T_ST] + (sval(t) + c) * pitch(T_ST) + skey(t) + 4 * g) =
                    pack4(SD[t][0], SD[t][1], SD[t][2], SD[t][3]);
        }
    };

    // ---- matrix phase of a chunk (fast path), specialised on the token tile
    f32x4 ot[NT];
    auto matrix_p = [&](auto tile, int set) {
        constexpr int P = decltype(tile)::value;
        f32x4 at[P + 1];
        if (!states_only) {
#pragma unroll
            for (int q = 0; q <= P; ++q) {  // P1: A^T tiles (sigma-tile q, tau-tile P)
                at[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 A = lds8(sm[set][T_KRH] + (16 * q + c) * pitch(T_KRH) + 32 * kb + 8 * g);
                    const bf16x8 B = lds8(sm[set][T_RS] + (16 * P + c) * pitch(T_RS) + 32 * kb + 8 * g);
                    at[q] = mfma(A, B, at[q]);
                }
            }
        }
        // P3: S' = diag(decay) S + (K^_hi + K^_lo)^T V (independent of P1)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int k0 = 32 * kb + 8 * g;
            bf16x8 Bv[2];
#pragma unroll
            for (int vj = 0; vj < 2; ++vj) Bv[vj] = lds_col8(sm[set][T_VR], k0, sval0 + 16 * vj, c);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const bf16x8 Ah = lds_col8(sm[set][T_KRH], k0, skey0 + 16 * mi, c);
                const bf16x8 Al = lds_col8(sm[set][T_KRL], k0, skey0 + 16 * mi, c);
#pragma unroll
                for (int vj = 0; vj < 2; ++vj) {
                    f32x4 &acc = SD[2 * mi + vj];  // becomes the new state
                    acc = mfma(Ah, Bv[vj], acc);
                    acc = mfma(Al, Bv[vj], acc);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) S[t] = SD[t];
        if (states_only) return;
        // P2 part 2: (decayed S)^T R~^T
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) ot[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 Br = lds8(sm[set][T_RS] + (16 * P + c) * pitch(T_RS) + 32 * kb + 8 * g);
#pragma unroll
            for (int ni = 0; ni < NT; ++ni)
                ot[ni] = mfma(lds8(sm[set][T_ST] + (16 * (NT * hf + ni) + c) * pitch(T_ST) + 32 * kb + 8 * g),
                              Br, ot[ni]);
        }
        // causal mask of the diagonal tile, bonus on its diagonal
        {
            const float bon = sBonus[set][16 * P + c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sl = 4 * g + e;
                at[P][e] = sl < c ? at[P][e] : (sl == c ? bon : 0.0f);
            }
        }
        // P2 part 1: V^T A^T over the causal sigma blocks
#pragma unroll
        for (int bk = 0; 2 * bk <= P; ++bk) {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const bf16x8 Bop = pack8(at[2 * bk], (2 * bk + 1 <= P) ? at[(2 * bk + 1) % (P + 1)]
                                                                   : zero);
#pragma unroll
            for (int ni = 0; ni < NT; ++ni)
                ot[ni] = mfma(lds_col4x2(sm[set][T_VR], 32 * bk + 4 * g, 32 * bk + 16 + 4 * g,
                                         16 * (NT * hf + ni), c),
                              Bop, ot[ni]);
        }
    };
    auto matrix = [&](int set) {
        switch (p) {  // wave-uniform
            case 0: matrix_p(std::integral_constant<int, 0>{}, set); break;
            case 1: matrix_p(std::integral_constant<int, 1>{}, set); break;
            case 2: matrix_p(std::integral_constant<int, 2>{}, set); break;
            default: matrix_p(std::integral_constant<int, 3>{}, set); break;
        }
    };

    // EPI: gq, this lane's gate values (token 16 p + c, channels 16 (NT hf +
    // ni) + 4 g + e) of a chunk.  Eight waves: the gate is loaded with the
    // chunk's r, k, v in v's coalesced layout (NV rows of 8 channels per
    // thread), written to sG by stage B and read from there after the
    // chunk's products.  Four waves: loaded into gq at the start of the step.
    u32x2 gq[EPI ? NT : 1];
    auto load_in = [&](int ch) {  // (past the job's chunks: issued, empty)
        const bool ok = ch < ch_end;
        load_rkv<NW>(buf, ch * kL, cx, r, k, v, ok, !states_only);
        if (GST) {
            const int c0 = ch * kL;
            const Rsrc rg = rsrc(gate + cx.base(ok ? c0 : 0), ok ? cx.span(c0) : 0u);
#pragma unroll
            for (int j = 0; j < (GST ? Raw<NW>::NV : 1); ++j)
                graw[j] = __builtin_amdgcn_raw_buffer_load_b128(rg, cx.off_v + j * 8 * NW * cx.tokb,
                                                                0, kReadOnce);
        }
    };
    auto gate_lds = [&](int set) {
#pragma unroll
        for (int ni = 0; ni < (GST ? NT : 1); ++ni)
            gq[ni] = *(const u32x2 *)(sG[set] + (16 * p + c) * kPR + 16 * (NT * hf + ni) + 4 * g);
    };
    auto load_gate = [&](int ch, bool ok) {  // (issued, empty, when not ok)
        const int c0 = ch * kL;
        const Rsrc rg = rsrc(gate + cx.base(c0), ok ? cx.span(c0) : 0u);
        const uint32_t off = (uint32_t)(16 * p + c) * cx.tokb + 2 * (16 * NT * hf + 4 * g);
#pragma unroll
        for (int ni = 0; ni < (EPI ? NT : 1); ++ni)
            gq[ni] = __builtin_amdgcn_raw_buffer_load_b64(rg, off + 32 * ni, 0, kReadOnce);
    };
    auto silu = [](float z) { return z * __builtin_amdgcn_rcpf(1.0f + exp_fast(-z)); };

    // EPI: y of this lane's outputs from the token's mean and 1 / sqrt(var +
    // eps), packed in yq; stored by epi_flush once the step's loads have been
    // consumed (stores share the in-order memory counter with loads, so a
    // store ahead of a load that is waited for is waited for too)
    u32x2 yq[EPI ? NT : 1];
    int yq_ch = -1;
    auto epi_compute = [&](float mean, float rstd) {
#pragma unroll
        for (int ni = 0; ni < (EPI ? NT : 1); ++ni) {
            const float gv[4] = {bf16_lo(gq[ni].x), bf16_hi(gq[ni].x), bf16_lo(gq[ni].y),
                                 bf16_hi(gq[ni].y)};
            f32x4 lw, lb;
            if constexpr (LNREG) {
                lw = lnw[ni];
                lb = lnb[ni];
            } else {
                lw = ln_at(ni, ln_w);
                lb = ln_at(ni, ln_b);
            }
            f32x4 yv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                yv[e] = fmaf((ot[ni][e] - mean) * rstd, lw[e], lb[e]) * silu(gv[e]);
            yq[ni] = pack4(yv[0], yv[1], yv[2], yv[3]);
        }
    };
    auto epi_flush = [&]() {  // (nothing pending: issued over an empty range)
        if (!EPI) return;
        const int c0 = max(yq_ch, 0) * kL;
        const Rsrc ro = rsrc(o + cx.base(c0), yq_ch >= 0 ? cx.span(c0) : 0u);
        const uint32_t off = (uint32_t)(16 * p + c) * cx.tokb + 2 * (16 * NT * hf + 4 * g);
#pragma unroll
        for (int ni = 0; ni < (EPI ? NT : 1); ++ni)
            __builtin_amdgcn_raw_buffer_store_b64(yq[ni], ro, off + 32 * ni, 0, 0);
        yq_ch = -1;
    };
    int epi_ch = -1, epi_set = 0;  // eight waves: a chunk whose outputs wait for the merge
    auto epi_finish = [&]() {
        if (!EPI || epi_ch < 0) return;
        const f32x2 a = sStat[epi_set][w][c], b = sStat[epi_set][w ^ 1][c];
        // two halves of 32 channels: n_a n_b / (n_a + n_b) = 16
        const float d = a[0] - b[0];
        const float mean = 0.5f * (a[0] + b[0]);
        const float m2 = a[1] + b[1] + 16.0f * d * d;
        epi_compute(mean, __builtin_amdgcn_rsqf(m2 * (1.0f / kN) + eps));
        yq_ch = epi_ch;
        epi_ch = -1;
    };

    // chunk ch's outputs (after a fast-decay chunk, ok is false: the stores
    // are issued over an empty range, token_by_token having written them)
    auto store_out = [&](int ch, int set, bool ok) {
        // (SAVE: the outputs too when the caller asked for them; the backward's
        // recomputation passes none, and the stores are then dropped)
        const int c0 = ch * kL;
        const Rsrc ro = rsrc(o + cx.base(c0), ok && (!SAVE || o != nullptr) ? cx.span(c0) : 0u);
        const uint32_t off = (uint32_t)(16 * p + c) * cx.tokb + 2 * (16 * NT * hf + 4 * g);
        if (EPI) {
            // this wave's channels of token 16 p + c: 4 NT in this lane, the
            // rest in lanes 16 and 32 apart; mean, then squared deviations
            constexpr float inv = 1.0f / (4 * NT * 4);
            float s = 0.0f;
#pragma unroll
            for (int ni = 0; ni < NT; ++ni)
#pragma unroll
                for (int e = 0; e < 4; ++e) s += ot[ni][e];
            s += __shfl_xor(s, 16, 64);
            s += __shfl_xor(s, 32, 64);
            const float mean = s * inv;
            float q = 0.0f;
#pragma unroll
            for (int ni = 0; ni < NT; ++ni)
#pragma unroll
                for (int e = 0; e < 4; ++e) q = fmaf(ot[ni][e] - mean, ot[ni][e] - mean, q);
            q += __shfl_xor(q, 16, 64);
            q += __shfl_xor(q, 32, 64);
            if (NH == 1) {  // the whole token is in this wave
                epi_compute(mean, __builtin_amdgcn_rsqf(q * (1.0f / kN) + eps));
                yq_ch = ok ? ch : -1;
                epi_flush();
            } else if (ok) {
                if (g == 0) sStat[set][w][c] = f32x2{mean, q};
                epi_ch = ch;
                epi_set = set;
            }
            return;
        }
#pragma unroll
        for (int ni = 0; ni < NT; ++ni)
            __builtin_amdgcn_raw_buffer_store_b64(pack4(ot[ni][0], ot[ni][1], ot[ni][2], ot[ni][3]),
                                                  ro, off + 32 * ni, 0, 0);
    };

    // ---- fast-decay chunk: its tokens one at a time with fp32 VALU ---------
    // Waves 0..3 take the state as 16-column slabs through LDS; r, k (bf16)
    // and w = 2^{a2} (fp32) are re-read and staged in the operand tiles.
    auto token_by_token = [&](int ch, int set) {
        const int c0 = ch * kL;
        float *sS = (float *)sm[set][T_RS];  // 64 x 64 fp32 spans the r~ and k^_hi tiles
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sS[(skey(t) + 4 * g + e) * kN + sval(t) + c] = S[t][e];
        lds_barrier();
        f32x4 Sc[4];
        if (w < 4) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Sc[m][e] = sS[(16 * m + 4 * g + e) * kN + 16 * w + c];
        }
        lds_barrier();
        // LORA: the chunk's logits formed again from its h on the VALU (hq and
        // sD hold a later chunk's), in the same thread layout as stage A
        f32x4 xl[LORA ? TP : 1];
        if constexpr (LORA) {
#pragma unroll
            for (int e = 0; e < (LORA ? TP : 1); ++e) {
                const int tau = TP * cx.tq + e;
                const uint16_t *hr = lr.h + (hrow0 + (size_t)min(c0 + tau, T - 1)) * kN;
                f32x4 acc = omq;
                for (int j = 0; j < kN; j += 2) {
                    const uint32_t hv = *(const uint32_t *)(hr + j);
                    const u32x2 b0 = *(const u32x2 *)(sB2 + j * kPC + 4 * cx.cq);
                    const u32x2 b1 = *(const u32x2 *)(sB2 + (j + 1) * kPC + 4 * cx.cq);
                    const float h0 = bf16_lo(hv), h1 = bf16_hi(hv);
                    acc[0] = fmaf(h0, bf16_lo(b0.x), fmaf(h1, bf16_lo(b1.x), acc[0]));
                    acc[1] = fmaf(h0, bf16_hi(b0.x), fmaf(h1, bf16_hi(b1.x), acc[1]));
                    acc[2] = fmaf(h0, bf16_lo(b0.y), fmaf(h1, bf16_lo(b1.y), acc[2]));
                    acc[3] = fmaf(h0, bf16_hi(b0.y), fmaf(h1, bf16_hi(b1.y), acc[3]));
                }
                xl[e] = acc;
            }
        }
        // re-read r, k, x of the chunk one token row at a time (few registers)
#pragma unroll 1
        for (int e = 0; e < TP; ++e) {
            const int tau = TP * cx.tq + e;
            const bool valid = c0 + tau < T;
            u32x2 rv = {0u, 0u}, kv = {0u, 0u};
            f32x4 xv = {0.f, 0.f, 0.f, 0.f};
            if (valid) {
                const size_t off = cx.seq_base + (size_t)(c0 + tau) * cx.tok_stride + 4 * cx.cq;
                rv = *(const u32x2 *)(r + off);
                kv = *(const u32x2 *)(k + off);
                if constexpr (LORA) {
#pragma unroll
                    for (int i = 0; i < (LORA ? TP : 1); ++i)
                        if (e == i) xv = xl[i];
                } else if (PT) {
                    xv = *(const f32x4 *)(x + off);
                }
            }
            f32x4 wv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = PT ? -exp2_fast(xv[q] * kLog2e) * kLog2e : a2s[q];
                wv[q] = valid ? exp2_fast(a) : 1.0f;
            }
            *(f32x4 *)(sS + tau * kN + 4 * cx.cq) = wv;
            *(u32x2 *)(sm[set][T_KRL] + tau * pitch(T_KRL) + 4 * cx.cq) = rv;
            *(u32x2 *)(sm[set][T_ST] + tau * pitch(T_ST) + 4 * cx.cq) = kv;
        }
        lds_barrier();
        if (w < 4) {
            const int nvalid = min(kL, T - c0);
            for (int tau = 0; tau < nvalid; ++tau) {
                const float vj = bf16_to_f32(sm[set][T_VR][tau * pitch(T_VR) + 16 * w + c]);
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x2 rp = *(const u32x2 *)(sm[set][T_KRL] + tau * pitch(T_KRL) + 16 * m + 4 * g);
                    const u32x2 kp = *(const u32x2 *)(sm[set][T_ST] + tau * pitch(T_ST) + 16 * m + 4 * g);
                    const f32x4 wv = *(const f32x4 *)(sS + tau * kN + 16 * m + 4 * g);
                    const float r4[4] = {bf16_lo(rp.x), bf16_hi(rp.x), bf16_lo(rp.y),
                                         bf16_hi(rp.y)};
                    const float k4[4] = {bf16_lo(kp.x), bf16_hi(kp.x), bf16_lo(kp.y),
                                         bf16_hi(kp.y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(r4[e], Sc[m][e], acc);
                        Sc[m][e] = fmaf(wv[e], Sc[m][e], k4[e] * vj);
                    }
                }
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                if (g == 0 && !SAVE) {
                    const float ov = fmaf(sBonus[set][tau], vj, acc);
                    if (EPI)
                        sO[tau * kN + 16 * w + c] = ov;
                    else
                        o[cx.seq_base + (size_t)(c0 + tau) * cx.tok_stride + 16 * w + c] =
                            (uint16_t)pack_bf16x2(ov, 0.0f);
                }
            }
        }
        lds_barrier();
        if (w < 4) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sS[(16 * m + 4 * g + e) * kN + 16 * w + c] = Sc[m][e];
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = sS[(skey(t) + 4 * g + e) * kN + sval(t) + c];
        if (EPI) {
            // the epilogue of the chunk from sO (written before the barrier
            // above): LPT threads per token, CPT channels each
            constexpr int CPT = kL * kN / (64 * NW), LPT = kN / CPT;
            const int tok = tid / LPT, qq = tid % LPT;
            float ov[CPT];
#pragma unroll
            for (int i = 0; i < CPT; ++i) ov[i] = sO[tok * kN + CPT * qq + i];
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) s += ov[i];
#pragma unroll
            for (int m = 1; m < LPT; m <<= 1) s += __shfl_xor(s, m, 64);
            const float mean = s * (1.0f / kN);
            float q = 0.0f;
#pragma unroll
            for (int i = 0; i < CPT; ++i) q = fmaf(ov[i] - mean, ov[i] - mean, q);
#pragma unroll
            for (int m = 1; m < LPT; m <<= 1) q += __shfl_xor(q, m, 64);
            const float rstd = __builtin_amdgcn_rsqf(q * (1.0f / kN) + eps);
            const int h = bh % H;
            const Rsrc rg = rsrc(gate + cx.base(c0), cx.span(c0));
            const Rsrc ro = rsrc(o + cx.base(c0), cx.span(c0));
            const uint32_t off = (uint32_t)tok * cx.tokb + 2 * (CPT * qq);
#pragma unroll
            for (int hh = 0; hh < CPT / 8; ++hh) {
                const u32x4 gv =
                    __builtin_amdgcn_raw_buffer_load_b128(rg, off + 16 * hh, 0, kReadOnce);
                const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
                u32x4 out;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int i0 = 8 * hh + 2 * m, ch0 = CPT * qq + i0;
                    const float y0 = fmaf((ov[i0] - mean) * rstd, ln_w[(size_t)h * kN + ch0],
                                          ln_b[(size_t)h * kN + ch0]) * silu(bf16_lo(gw[m]));
                    const float y1 = fmaf((ov[i0 + 1] - mean) * rstd, ln_w[(size_t)h * kN + ch0 + 1],
                                          ln_b[(size_t)h * kN + ch0 + 1]) * silu(bf16_hi(gw[m]));
                    const uint32_t pk = pack_bf16x2(y0, y1);
                    if (m == 0) out.x = pk;
                    else if (m == 1) out.y = pk;
                    else if (m == 2) out.z = pk;
                    else out.w = pk;
                }
                __builtin_amdgcn_raw_buffer_store_b128(out, ro, off + 16 * hh, 0, 0);
            }
        }
    };

    // ---- one pipelined step: matrix phase of chunk ch, staging of ch + 1 --
    // buf holds chunk ch + 1's inputs: staging of ch consumed it last step.
    // LDS barrier that also ORs a flag over the workgroup.  sBad[set][w] is
    // written again only after the next barrier (X), when every wave has
    // read it.
    auto barrier_or = [&](bool flag, int set) -> bool {
        const bool any = __builtin_amdgcn_ballot_w64(flag) != 0;
        if (lane == 0) sBad[set][w] = any ? 1 : 0;
        lds_barrier();
        int r = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) r |= sBad[set][j];
        return r != 0;
    };

    // Four waves, one tile set, two barriers per chunk.  buf holds chunk
    // ch + 1's inputs when step ch starts: its r, k, v were requested at the
    // start of the step, its x (Finch) right after the previous step's stage
    // A had read the registers, a whole step earlier.
    auto step2 = [&](int ch, bool unsafe) -> bool {
        // The lane indices, opaque to the compiler in each step: the LDS
        // addresses derived from them are formed where they are used instead
        // of being hoisted out of the loop into registers (four-wave kernels
        // have none to spare).
        asm volatile("" : "+v"(c), "+v"(g));
        const bool more = ch + 1 < ch_end;
        if (LORA && more) lora_product(hq);  // chunk ch + 1's logits, h loaded a step ago
        load_in(ch + 1);
        if (EPI) load_gate(ch, !unsafe);
        if (SAVE) save_chunk(ch);
        if (!unsafe) matrix(0);
        else token_by_token(ch, 0);
        if (more) stageA(ch + 1, buf, 0, LORA);
        load_dec(ch + 2, ch + 2 < ch_end);
        lds_barrier();  // (X) decay totals of ch + 1; chunk ch's tiles consumed
        bool bad = false;
        if (more) bad = stageB(ch + 1, buf, 0);
        store_out(ch, 0, !unsafe);
        if (more) stage_state(0);
        return barrier_or(bad, 0);  // (Y) operands of ch + 1 staged
    };
    // Eight waves, chunk c in set c & 1, one barrier per chunk.  When step
    // ch starts, chunk ch is staged in set ch & 1 and chunk ch + 1's decay
    // totals are in sWave[(ch + 1) & 1]; the step stages chunk ch + 1 in the
    // other set while chunk ch's products run, and scans chunk ch + 2's
    // decays, so nothing a wave writes is read by another before the barrier.
    auto step1 = [&](int ch, bool unsafe) -> bool {
        const int cur = ch & 1, nxt = cur ^ 1;
        const bool more = ch + 1 < ch_end;
        if (LORA && ch + 2 < ch_end) lora_product(hq);  // chunk ch + 2's, h loaded a step ago
        load_in(ch + 1);
        if (LORA) load_dec(ch + 3, ch + 3 < ch_end);
        else load_dec(ch + 2, ch + 2 < ch_end);
        epi_finish();  // the previous chunk's outputs, merged after its barrier
        if (EPI && !GST) load_gate(ch, !unsafe);
        if (SAVE) save_chunk(ch);
        // The two waves of a SIMD reach the products at different times;
        // the one in them issues first (measured: 1-2 % off the step), so
        // that both arrive at the barrier closer together.
        __builtin_amdgcn_s_setprio(1);
        if (!unsafe) matrix(cur);
        else token_by_token(ch, cur);
        __builtin_amdgcn_s_setprio(0);
        if (GST && !unsafe) gate_lds(cur);
        bool bad = false;
        if (more) bad = stageB(ch + 1, buf, nxt);
        if (more) stage_state(nxt);
        if (ch + 2 < ch_end) stageA(ch + 2, buf, cur, LORA);
        epi_flush();  // the previous chunk's y
        store_out(ch, cur, !unsafe);
        return barrier_or(bad, cur);  // chunk ch + 1 staged, ch + 2's totals out
    };
    // chunks [ch0, ch1) of the current head from the state in S
    auto run_job = [&](int ch0, int ch1) {
        if (ch0 >= ch1) return;
        ch_end = ch1;
        const int s0 = DB ? (ch0 & 1) : 0;
        load_dec(ch0, true);
        load_in(ch0);
        stageA(ch0, buf, s0);
        load_dec(ch0 + 1, ch0 + 1 < ch1);
        lds_barrier();
        const bool bad0 = stageB(ch0, buf, s0);
        stage_state(s0);
        // (DB: chunk ch0 + 1's scan after stage B of ch0 has used the scan
        // registers; the other parity's flags, next used two barriers later)
        if (DB && ch0 + 1 < ch1) stageA(ch0 + 1, buf, s0 ^ 1);
        if (DB && LORA) load_dec(ch0 + 2, ch0 + 2 < ch1);  // (the steps request ch + 3)
        bool unsafe = barrier_or(bad0, DB ? (s0 ^ 1) : 0);
        for (int ch = ch0; ch < ch1; ++ch) unsafe = DB ? step1(ch, unsafe) : step2(ch, unsafe);
        epi_finish();
        epi_flush();
    };

    // Balanced split (sp.extra > 0; eight waves and one workgroup per CU, or
    // four waves and two): workgroup i runs its own head i and one segment of
    // one of the sp.extra remaining heads.  The segments of an extra head run on workgroups i,
    // i + sp.stride, ... (the same XCD, dispatched in order), and segment s
    // starts after the workgroup's first s/K of its own head, by when segment
    // s-1 is done:
    //   own [0, a) -> extra segment s = [a, b) -> own [a, nchunks)
    // The state between segments goes through the handoff workspace.  Jobs
    // run in one loop, so that the chunk loop exists once in the code.
    // Past the split's range, workgroup i first runs the whole heads i,
    // i + grid, ... (sp.nfull of them), then its own head of the split round.
    const int wg = blockIdx.x;
    const int own = wg + sp.nfull * (int)gridDim.x;
    int ext = 0, seg = 0, a = nchunks, e1 = nchunks;
    bool split = false;
    if (sp.extra != 0) {
        const int xcd = wg % sp.stride, local = wg / sp.stride;
        const int chain = local / sp.K;
        seg = local % sp.K;
        ext = xcd + sp.stride * chain;  // extra head index among sp.extra
        split = chain < sp.chains_per_xcd && ext < sp.extra;
        a = seg * nchunks / sp.K;
        e1 = (seg + 1) * nchunks / sp.K;
    }
    auto ld = [](const void *ptr) { return ld_agent((const unsigned *)ptr); };
    auto st = [](void *ptr, unsigned val) { st_agent((unsigned *)ptr, val); };
    // the launch's tag (thread 0 alone polls and raises the flags)
    const unsigned tag = (sp.extra != 0 && tid == 0) ? ws_tag(sp.ctrl) : 0u;
    __shared__ int s_late;
    // the state entering segment seg, from the workgroup that ran seg - 1.
    // Slots and flags are touched only by agent-scope relaxed atomics: the
    // producer's state stores complete before its flag store, and the state
    // is read only after the flag shows this launch's tag.  Polls are
    // bounded (about a second); the producer has a lower workgroup index on
    // the same XCD, so it is already running and the bound is never reached.
    // If it were, the segment would go on from a NaN state (its outputs and
    // the head's final state read NaN) and the error word is set.
    auto receive = [&]() {
        const int slot = ext * (sp.K - 1) + seg - 1;
        const float *src = sp.slots + (size_t)slot * kN * kN;
        if (tid == 0) {
            int polls = 0, late = 0;
            while (ld(sp.flags + slot) != tag) {
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
        const bool late = s_late != 0;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = late ? __builtin_nanf("") : __uint_as_float(ld(src + sidx(t, e)));
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the state has been read
        lds_barrier();
    };
    auto send = [&]() {
        const int slot = ext * (sp.K - 1) + seg;
        float *dst = sp.slots + (size_t)slot * kN * kN;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) st(dst + sidx(t, e), __float_as_uint(S[t][e]));
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the state has landed
        lds_barrier();
        if (tid == 0) st(sp.flags + slot, tag);
    };
    f32x4 Sown[DB ? NT : 1];  // own head's state while the extra segment runs
    const int njobs = sp.nfull + (split ? 3 : 1);
#pragma clang loop unroll(disable)
    for (int j = 0; j < njobs; ++j) {
        const int job = j - sp.nfull;  // (< 0: a whole head before the split round)
        const bool extra = split && job == 1;
        set_head(job < 0 ? wg + j * (int)gridDim.x : extra ? sp.first_extra + ext : own);
        if (split && job == 2) {
            if (DB) {
#pragma unroll
                for (int t = 0; t < (DB ? NT : 1); ++t) S[t] = Sown[t];
            } else {  // (the same threads stored it)
                const float *park = sp.park + (size_t)wg * kN * kN;
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[t][e] = park[sidx(t, e)];
            }
        } else if (extra && seg > 0) {
            receive();
        } else {
            load_state();
        }
        const bool sj = split && job >= 0;
        run_job(sj && job > 0 ? a : 0, sj && job < 2 ? (job == 0 ? a : e1) : nchunks);
        if (split && job == 0) {
            if (DB) {
#pragma unroll
                for (int t = 0; t < (DB ? NT : 1); ++t) Sown[t] = S[t];
            } else {
                float *park = sp.park + (size_t)wg * kN * kN;
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) park[sidx(t, e)] = S[t][e];
            }
        } else if (extra && seg + 1 < sp.K) {
            send();
        } else {
            save_state();
        }
    }
    if (sp.extra != 0 && tid == 0) ws_finish(sp.ctrl, tag);
}

template <bool PT, int NW, bool SAVE = false, bool EPI = false, bool LORA = false>
void launch(int blocks, int T, int H, const uint16_t *r, const uint16_t *k, const uint16_t *v,
            const float *x, const float *u, const float *state_in, float *state_out,
            uint16_t *o, const Split &sp, hipStream_t stream, float *chunk_states = nullptr,
            const uint16_t *gate = nullptr, const float *ln_w = nullptr,
            const float *ln_b = nullptr, float eps = 0.0f, Lora lr = Lora{}) {
    hipLaunchKernelGGL((wkv_chunk_kernel<PT, NW, SAVE, EPI, LORA>), dim3((unsigned)blocks),
                       dim3(64 * NW), 0, stream, T, H, r, k, v, x, u, state_in, state_out, o,
                       sp, chunk_states, gate, ln_w, ln_b, eps, lr);
}

constexpr int kMaxSlots = 4096;  // hand-offs of one launch
constexpr int kMaxSegs = 16;     // segments per extra head

// How the heads of a launch are spread over workgroups (see the kernel).
struct Plan {
    bool wide;                  // eight waves per workgroup (else four)
    int blocks;                 // workgroups
    int64_t extra, nfull, first, K, chains_per_xcd;
    size_t slot_bytes, park_bytes;  // hand-off slots, parked own states
};

// Eight waves per head while every head has a CU of its own.  With up to half
// as many heads again, eight waves and the balanced split: one workgroup per
// CU, each running one head plus one K-th of an extra head.  Beyond that,
// four waves so that two heads share a CU, and past two heads per CU the same
// split over the 2 x CUs workgroups.  The segments of an extra head must sit
// on one XCD, so the split needs the CU count to be a multiple of the XCDs.
Plan plan(int64_t heads, int T) {
    const int cus = device_cus(), xcds = device_xcds();
    Plan p{};
    p.wide = heads <= cus;
    p.blocks = (int)heads;
    // (slots workgroups: whole heads in rounds, then the remainder split)
    auto split = [&](int64_t slots) {
        const int64_t nfull = heads / slots - 1, extra = heads % slots;
        if (extra == 0) return false;
        const int64_t chains_per_xcd = (extra + xcds - 1) / xcds;
        // (at most kMaxSegs segments: each hand-off adds its latency to the
        // chain of an extra head's segments)
        const int64_t K = std::min<int64_t>((slots / xcds) / chains_per_xcd, kMaxSegs);
        if (K < 2 || extra * (K - 1) > kMaxSlots) return false;
        p.extra = extra;
        p.nfull = nfull;
        p.first = (nfull + 1) * slots;
        p.K = K;
        p.chains_per_xcd = chains_per_xcd;
        p.slot_bytes = (size_t)extra * (K - 1) * kN * kN * 4;
        p.park_bytes = slots > cus ? (size_t)slots * kN * kN * 4 : 0;
        p.blocks = (int)slots;
        return true;
    };
    if (!p.wide && xcds > 0 && cus % xcds == 0 && T >= 4 * kL) {
        if (heads < 2 * (int64_t)cus && split(cus)) p.wide = true;
        else if (heads > 2 * (int64_t)cus) split(2 * (int64_t)cus);
    }
    return p;
}

constexpr size_t kFlagBytes = (size_t)kMaxSlots * 4;

size_t handoff_bytes(const Plan &p) {
    return p.extra ? kWsCtrlBytes + kFlagBytes + p.slot_bytes + p.park_bytes : 0;
}

}  // namespace

size_t chunk_workspace_bytes(int B, int T, int H) {
    return handoff_bytes(plan((int64_t)B * H, T));
}

hipError_t launch_wkv_chunked(bool per_token_decay, int B, int T, int H, const uint16_t *r,
                              const uint16_t *k, const uint16_t *v, const float *x,
                              const float *u, const float *state_in, float *state_out,
                              uint16_t *o, void *ws, hipStream_t stream, float *chunk_states,
                              const uint16_t *gate, const float *ln_w, const float *ln_b,
                              float eps, const uint16_t *lora_h, const uint16_t *lora_B2,
                              const float *lora_omega) {
    const Plan p = plan((int64_t)B * H, T);
    Split sp{};
    if (p.extra != 0) {
        if (ws == nullptr) return hipErrorInvalidValue;  // (the entry points check the size)
        char *base = (char *)ws;
        sp.extra = (int)p.extra;
        sp.nfull = (int)p.nfull;
        sp.first_extra = (int)p.first;
        sp.K = (int)p.K;
        sp.stride = device_xcds();
        sp.chains_per_xcd = (int)p.chains_per_xcd;
        sp.ctrl = (WsCtrl *)base;
        sp.flags = (unsigned *)(base + kWsCtrlBytes);
        sp.slots = (float *)(base + kWsCtrlBytes + kFlagBytes);
        sp.park = p.park_bytes ? (float *)(base + kWsCtrlBytes + kFlagBytes + p.slot_bytes)
                               : nullptr;
    }
    const bool wide = p.wide;
    const int blocks = p.blocks;
    // plain forward; the forward that also stores the state entering every
    // chunk (SAVE: the backward's recomputation, or a forward kept for the
    // backward); the forward with the output epilogue (EPI)
    auto go = [&](auto save_tag, auto epi_tag) {
        constexpr bool SV = decltype(save_tag)::value, EP = decltype(epi_tag)::value;
        float *so = state_out;
        uint16_t *out = o;
        if (per_token_decay) {
            if (wide) launch<true, 8, SV, EP>(blocks, T, H, r, k, v, x, u, state_in, so, out, sp, stream, chunk_states, gate, ln_w, ln_b, eps);
            else launch<true, 4, SV, EP>(blocks, T, H, r, k, v, x, u, state_in, so, out, sp, stream, chunk_states, gate, ln_w, ln_b, eps);
        } else {
            if (wide) launch<false, 8, SV, EP>(blocks, T, H, r, k, v, x, u, state_in, so, out, sp, stream, chunk_states, gate, ln_w, ln_b, eps);
            else launch<false, 4, SV, EP>(blocks, T, H, r, k, v, x, u, state_in, so, out, sp, stream, chunk_states, gate, ln_w, ln_b, eps);
        }
    };
    if (lora_h != nullptr) {  // Finch, the decay logits from the decay producer
        const Lora lr{lora_h, lora_B2, lora_omega};
        if (wide) launch<true, 8, false, false, true>(blocks, T, H, r, k, v, nullptr, u, state_in, state_out, o, sp, stream, nullptr, nullptr, nullptr, nullptr, 0.0f, lr);
        else launch<true, 4, false, false, true>(blocks, T, H, r, k, v, nullptr, u, state_in, state_out, o, sp, stream, nullptr, nullptr, nullptr, nullptr, 0.0f, lr);
    } else if (chunk_states != nullptr) {
        go(std::true_type{}, std::false_type{});
    } else if (gate != nullptr) {
        go(std::false_type{}, std::true_type{});
    } else {
        go(std::false_type{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_wkv_chunked_gated(bool per_token_decay, int B, int T, int H,
                                    const uint16_t *r, const uint16_t *k, const uint16_t *v,
                                    const float *x, const float *u, const float *state_in,
                                    float *state_out, const uint16_t *gate, const float *ln_w,
                                    const float *ln_b, float eps, uint16_t *y, void *ws,
                                    hipStream_t stream) {
    return launch_wkv_chunked(per_token_decay, B, T, H, r, k, v, x, u, state_in, state_out, y,
                              ws, stream, nullptr, gate, ln_w, ln_b, eps);
}

}  // namespace wkv
