// wkv_tiles.h -- tile helpers shared by the chunked Eagle / Finch kernels
// (forward and backward) on gfx950: sizes and LDS pitches of the 64 x 64
// operand tiles, the bf16 MFMA and LDS operand loads, barriers, DPP row sums,
// buffer resources and the per-thread operand loads of a chunk.
//
// MFMA operand convention (v_mfma_f32_16x16x32_bf16): lane l = c + 16 g holds
// row c of the A operand and column c of the B operand, with eight k-slots
// indexed by (g, slot); both operands use the same (g, slot) -> k map, so
// any consistent map is valid.  The result lane l holds rows 4 g + e
// (e = 0..3) of column c.  The transposing load: in each group of 16 lanes,
// lane j supplies the address of 4 consecutive elements of row j/4 of a
// 4 x 16 block and receives column j of that block (rows 0..3).
#pragma once

#include "wkv_device.h"

namespace wkv {
namespace tiles {

constexpr int kN = 64;     // head size
constexpr int kL = 64;     // chunk length
// LDS row pitches (bf16 elements) of the 64x64 tiles.  Rows read whole by
// 16-byte loads (r~, the decayed state) are 72 elements apart: 8 lanes reading
// rows c..c+7 hit 32 distinct banks.  Tiles read down their columns by the
// transposing load (k^_hi, k^_lo, v) are 80 apart: the 4 rows x 4 column
// groups that 16 lanes address then also cover 32 distinct banks.
constexpr int kPR = 72;
constexpr int kPC = 80;
constexpr int kTile = kN * kPC;
// Smallest chunk log2-decay (per channel) handled by the factorised form:
// r~ <= |r| 2^110 and k^ >= |k| 2^-110 stay far from fp32 / bf16 limits.
constexpr float kSafeLog2 = -110.0f;

template <int NW>
struct Raw {                           // one thread's share of a chunk
    static constexpr int TP = 16 / NW; // tokens per staging thread
    static constexpr int NV = 8 / NW;  // v rows per thread
    // 16 channel quads x (64 NW / 16) token groups x TP tokens cover the chunk
    static_assert(TP * (64 * NW / 16) == kL, "staging threads must cover the chunk");
    static_assert(NV * 8 * NW * 8 == kL * 8, "v loaders must cover the chunk");
    u32x2 r[TP], k[TP];                // TP tokens x 4 channels, bf16
    f32x4 x[TP];                       // Finch decay logits
    u32x4 v[NV];                       // NV tokens x 8 channels, bf16
};

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {
    return *(const bf16x8 *)p;
}
// transposing 8-byte LDS load (see the file comment)
__device__ __forceinline__ u32x2 lds_tr(const uint16_t *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 *lds_v4i16;
    const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16)p);
    return __builtin_bit_cast(u32x2, t);
}
// column (n0 + c) of rows k0..k0+7 of a row-major tile, for lane c of its
// 16-lane group: the operand of a product that contracts over rows
__device__ __forceinline__ bf16x8 lds_col8(const uint16_t *tile, int k0, int n0, int c) {
    const uint16_t *p = tile + (k0 + (c >> 2)) * kPC + n0 + 4 * (c & 3);
    const u32x2 a = lds_tr(p), b = lds_tr(p + 4 * kPC);
    const u32x4 m = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, m);
}
// rows k0..k0+3 and k1..k1+3 of column (n0 + c)
__device__ __forceinline__ bf16x8 lds_col4x2(const uint16_t *tile, int k0, int k1, int n0,
                                             int c) {
    const int off = (c >> 2) * kPC + n0 + 4 * (c & 3);
    const u32x2 a = lds_tr(tile + k0 * kPC + off), b = lds_tr(tile + k1 * kPC + off);
    const u32x4 m = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, m);
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations have
// completed (lgkmcnt(0)) before it arrives.  Unlike __syncthreads() it does
// not order global memory, which no thread here reads after another wrote
// it; the empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}
template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xf, 0xf, true));
}
// sum over the 16 lanes of a DPP row (every lane receives the total)
__device__ __forceinline__ float row_sum16(float s) {
    s += dpp<0x128>(s);  // row_ror:8
    s += dpp<0x124>(s);  // row_ror:4
    s += dpp<0x4e>(s);   // quad_perm [2,3,0,1]
    s += dpp<0xb1>(s);   // quad_perm [1,0,3,2]
    return s;
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

// Raw buffer resource over `bytes` bytes from `base` (gfx9 layout: no
// stride, no swizzle, 32-bit data format): a load past the end returns zero
// and a store past the end is dropped, which is how a ragged last chunk is
// masked without branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

// cache policy of the loads of r, k, v, the decay logits and the gate, each
// byte of which a kernel reads once: non-temporal (measured 1 % faster on the
// Finch forward, 3.5 % on the Eagle forward and 0.4 % on the forward with the
// epilogue, the same bytes read)
constexpr int kReadOnce = 2;

struct Ctx {
    int T, tq, cq, vt, vo;
    size_t seq_base, tok_stride;  // elements
    uint32_t tokb;                // bytes of one bf16 token row (H N 2)
    uint32_t off_rk, off_v;       // byte offsets of this thread's first r/k and v rows
    // bf16 bytes of chunk c0's rows up to its last valid token, and the
    // element offset of the chunk
    __device__ uint32_t span(int c0) const { return (uint32_t)(min(kL, T - c0) - 1) * tokb + 2 * kN; }
    __device__ size_t base(int c0) const { return seq_base + (size_t)c0 * tok_stride; }
};

// one thread's r, k, v of chunk c0 (rows past T read as zero).  With
// valid false the loads are still issued, over an empty range, and read
// zero: a load issued on every path keeps the count of outstanding memory
// operations the same on all of them, so that a later wait for an older
// load is not made to wait for this one too.  With_r false does the same
// for r alone (reads zero, no memory traffic).
template <int NW>
__device__ __forceinline__ void load_rkv(Raw<NW> &d, int c0, const Ctx &cx,
                                         const uint16_t *r, const uint16_t *k,
                                         const uint16_t *v, bool valid = true,
                                         bool with_r = true) {
    constexpr int TP = Raw<NW>::TP;
    const size_t cb = cx.base(valid ? c0 : 0);
    const uint32_t span = valid ? cx.span(c0) : 0u;
    const Rsrc rr = rsrc(r + cb, with_r ? span : 0u), rk = rsrc(k + cb, span),
               rv = rsrc(v + cb, span);
#pragma unroll
    for (int e = 0; e < TP; ++e) {
        const uint32_t off = cx.off_rk + e * cx.tokb;
        d.r[e] = __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, kReadOnce);
        d.k[e] = __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, kReadOnce);
    }
#pragma unroll
    for (int j = 0; j < Raw<NW>::NV; ++j)
        d.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, cx.off_v + j * 8 * NW * cx.tokb, 0,
                                                       kReadOnce);
}

// one thread's Finch decay logits of chunk c0 (rows past T read as zero;
// valid as for load_rkv)
template <int NW>
__device__ __forceinline__ void load_x(Raw<NW> &d, int c0, const Ctx &cx, const float *x,
                                       bool valid = true) {
    constexpr int TP = Raw<NW>::TP;
    const Rsrc rx = rsrc(x + cx.base(valid ? c0 : 0), valid ? 2 * cx.span(c0) : 0u);
#pragma unroll
    for (int e = 0; e < TP; ++e)
        d.x[e] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * (cx.off_rk + e * cx.tokb), 0,
                                                         kReadOnce));
}

}  // namespace tiles
}  // namespace wkv
