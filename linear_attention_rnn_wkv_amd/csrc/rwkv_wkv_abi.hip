// rwkv_wkv_abi.hip -- the C ABI: host-side validation and dispatch.
//
// Every entry point validates its arguments completely before the first HIP
// call, so a rejected call launches nothing and touches no output.
#include <stdint.h>

#include <algorithm>
#include <string.h>

#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "launchers.h"
#include "rwkv_wkv.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // per tensor; far above any HBM

struct Span {
    const void *p;
    int64_t bytes;
};

bool overlaps(Span a, Span b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// product of non-negative factors, or -1 when it exceeds kMaxElems
int64_t checked_mul(std::initializer_list<int64_t> f) {
    int64_t r = 1;
    for (int64_t x : f) {
        if (x < 0) return -1;
        if (x != 0 && r > kMaxElems / x) return -1;
        r *= x;
    }
    return r;
}

int hip_status(hipError_t e) { return e == hipSuccess ? RWKV_OK : RWKV_E_HIP; }

// An output must not overlap any input or other output.  `same_ok` marks the
// single permitted exact alias (state_out == state_in).
int check_outputs(std::initializer_list<Span> outs, std::initializer_list<Span> ins,
                  const void *same_a = nullptr, const void *same_b = nullptr) {
    for (const Span &o : outs) {
        for (const Span &i : ins) {
            if (o.p != nullptr && o.p == i.p && o.p == same_a && i.p == same_b &&
                same_a != nullptr)
                continue;
            if (overlaps(o, i)) return RWKV_E_ALIAS;
        }
    }
    for (auto a = outs.begin(); a != outs.end(); ++a)
        for (auto b = a + 1; b != outs.end(); ++b)
            if (overlaps(*a, *b)) return RWKV_E_ALIAS;
    return RWKV_OK;
}

// The caller's workspace: at least `need` bytes (then non-NULL and 16-byte
// aligned) and overlapping none of the call's other buffers.
int check_workspace(const void *ws, size_t ws_bytes, size_t need,
                    const std::vector<Span> &others) {
    if (need == 0) return RWKV_OK;
    if (ws == nullptr) return RWKV_E_NULL;
    if (ws_bytes < need) return RWKV_E_DIM;
    if (!aligned(ws, 16)) return RWKV_E_ALIGN;
    const Span sw{ws, (int64_t)need};
    for (const Span &o : others)
        if (overlaps(sw, o)) return RWKV_E_ALIAS;
    return RWKV_OK;
}

// Shared checks of the Eagle / Finch entry points.  x_elems: elements of x.
int check_matrix(int B, int T, int H, int N, const void *r, const void *k, const void *v,
                 const void *x, int64_t x_elems, const void *u, const void *s_in,
                 const void *s_out, bool s_in_required, const void *o) {
    if (B < 1 || H < 1 || N < 1 || T < 0) return RWKV_E_DIM;
    const int64_t tok = checked_mul({B, T, H, N});
    const int64_t st = checked_mul({B, H, N, N});
    if (tok < 0 || st < 0 || x_elems < 0) return RWKV_E_DIM;
    if (N != 64) return RWKV_E_UNSUPPORTED;
    if (s_in_required && s_in == nullptr) return RWKV_E_NULL;
    if (T > 0 && (r == nullptr || k == nullptr || v == nullptr || x == nullptr ||
                  u == nullptr || o == nullptr))
        return RWKV_E_NULL;
    for (const void *p : {r, k, v, x, u, s_in, s_out, o})
        if (p != nullptr && !aligned(p, 16)) return RWKV_E_ALIGN;
    const Span sr{r, tok * 2}, sk{k, tok * 2}, sv{v, tok * 2}, sx{x, x_elems * 4},
        su{u, (int64_t)H * N * 4}, ssi{s_in, st * 4}, sso{s_out, st * 4}, so{o, tok * 2};
    if (T == 0) return check_outputs({sso}, {ssi}, s_out, s_in);
    return check_outputs({so, sso}, {sr, sk, sv, sx, su, ssi}, s_out, s_in);
}

constexpr int kMaxChunkedHeads = 65536;

// Scratch of rwkv6_wkv_fwd_noalloc: the chunked forward's hand-off area in a
// fixed device array (one copy per GPU, zero at load as static storage is,
// kept until the process ends).  Host code never uses the array's name as a
// device address: the address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on its first use).
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
constexpr int64_t kMaxRwkv4Channels = 1 << 20;

int matrix_fwd(bool per_token, int B, int T, int H, int N, const rwkv_bf16 *r,
               const rwkv_bf16 *k, const rwkv_bf16 *v, const float *x, const float *u,
               const float *state_in, float *state_out, rwkv_bf16 *o, void *ws,
               size_t ws_bytes, hipStream_t s) {
    const int64_t x_elems = per_token ? checked_mul({B, T, H, N}) : checked_mul({H, N});
    int st = check_matrix(B, T, H, N, r, k, v, x, x_elems, u, state_in, state_out, false, o);
    if (st != RWKV_OK) return st;
    // a chunk's rows are addressed with 32-bit byte offsets
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    if (T == 0) {
        if (state_out == nullptr || state_out == state_in) return RWKV_OK;
        const int64_t n = (int64_t)B * H * N * N;
        if (state_in == nullptr) return hip_status(wkv::launch_fill(state_out, n, 0.0f, s));
        return hip_status(hipMemcpyAsync(state_out, state_in, n * 4,
                                         hipMemcpyDeviceToDevice, s));
    }
    const int64_t tok = checked_mul({B, T, H, N}), sts = checked_mul({B, H, N, N});
    st = check_workspace(ws, ws_bytes, wkv::chunk_workspace_bytes(B, T, H),
                         {Span{r, tok * 2}, Span{k, tok * 2}, Span{v, tok * 2},
                          Span{x, x_elems * 4}, Span{u, (int64_t)H * N * 4},
                          Span{state_in, sts * 4}, Span{state_out, sts * 4}, Span{o, tok * 2}});
    if (st != RWKV_OK) return st;
    return hip_status(wkv::launch_wkv_chunked(per_token, B, T, H, r, k, v, x, u,
                                              state_in, state_out, o, ws, s));
}

int matrix_fwd_gated(bool per_token, int B, int T, int H, int N, const rwkv_bf16 *r,
                     const rwkv_bf16 *k, const rwkv_bf16 *v, const float *x, const float *u,
                     const float *state_in, float *state_out, const rwkv_bf16 *gate,
                     const float *ln_w, const float *ln_b, float eps, rwkv_bf16 *y, void *ws,
                     size_t ws_bytes, hipStream_t s) {
    const int64_t x_elems = per_token ? checked_mul({B, T, H, N}) : checked_mul({H, N});
    int st = check_matrix(B, T, H, N, r, k, v, x, x_elems, u, state_in, state_out, false, y);
    if (st != RWKV_OK) return st;
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    if (!(eps >= 0.0f) || eps > 1e30f) return RWKV_E_DIM;  // also rejects NaN
    if (T > 0 && (gate == nullptr || ln_w == nullptr || ln_b == nullptr)) return RWKV_E_NULL;
    for (const void *p : {(const void *)gate, (const void *)ln_w, (const void *)ln_b})
        if (p != nullptr && !aligned(p, 16)) return RWKV_E_ALIGN;
    const int64_t tok = checked_mul({B, T, H, N}), st_el = checked_mul({B, H, N, N});
    const Span sy{y, tok * 2}, sso{state_out, st_el * 4}, sg{gate, tok * 2},
        sw{ln_w, (int64_t)H * N * 4}, sb{ln_b, (int64_t)H * N * 4};
    if (T > 0 && check_outputs({sy, sso}, {sg, sw, sb}) != RWKV_OK) return RWKV_E_ALIAS;
    if (T == 0) return matrix_fwd(per_token, B, T, H, N, r, k, v, x, u, state_in, state_out,
                                  y, ws, ws_bytes, s);
    st = check_workspace(ws, ws_bytes, wkv::chunk_workspace_bytes(B, T, H),
                         {Span{r, tok * 2}, Span{k, tok * 2}, Span{v, tok * 2},
                          Span{x, x_elems * 4}, Span{u, (int64_t)H * N * 4},
                          Span{state_in, st_el * 4}, sso, sy, sg, sw, sb});
    if (st != RWKV_OK) return st;
    return hip_status(wkv::launch_wkv_chunked_gated(per_token, B, T, H, r, k, v, x, u,
                                                    state_in, state_out, gate, ln_w, ln_b,
                                                    eps, y, ws, s));
}

// Checks of the decay producer's arguments (D = H N channels); `out` is the
// caller's output, which must not overlap them.
constexpr int kLoraR1 = 32, kLoraR2 = 64;

int check_lora(int B, int T, int D, int act, const void *x, const void *shift,
               const void *mu_x, const void *lam, const void *A1, const void *B1,
               const void *omega, const void *A2, const void *B2, Span out) {
    if (B < 1 || T < 0 || D < 1 || (act != 0 && act != 1)) return RWKV_E_DIM;
    const int64_t tok = checked_mul({B, T, D});
    if (tok < 0) return RWKV_E_DIM;
    // (rows are int-indexed; the logits kernel takes one 64-channel block per
    // grid row, at most 65535)
    if (D % 64 != 0 || D / 64 > 65535 || (int64_t)B * T >= ((int64_t)1 << 31))
        return RWKV_E_UNSUPPORTED;
    if (T == 0) return RWKV_OK;
    for (const void *p : {x, mu_x, lam, A1, B1, omega, A2, B2})
        if (p == nullptr) return RWKV_E_NULL;
    for (const void *p : {x, shift, mu_x, lam, A1, B1, omega, A2, B2})
        if (p != nullptr && !aligned(p, 16)) return RWKV_E_ALIGN;
    const int64_t vec = (int64_t)D * 4;
    const Span sx{x, tok * 2}, ss{shift, (int64_t)B * D * 2}, smu{mu_x, vec}, sl{lam, vec},
        sa1{A1, (int64_t)D * kLoraR1 * 2}, sb1{B1, (int64_t)D * kLoraR1 * 2}, so{omega, vec},
        sa2{A2, (int64_t)D * kLoraR2 * 2}, sb2{B2, (int64_t)D * kLoraR2 * 2};
    return check_outputs({out}, {sx, ss, smu, sl, sa1, sb1, so, sa2, sb2});
}

// The decay producer's inputs and `out`, as spans.
std::vector<Span> lora_spans(int B, int T, int D, const void *x, const void *shift,
                             const void *mu_x, const void *lam, const void *A1, const void *B1,
                             const void *omega, const void *A2, const void *B2, Span out) {
    const int64_t tok = (int64_t)B * T * D, vec = (int64_t)D * 4;
    return {Span{x, tok * 2},
            Span{shift, (int64_t)B * D * 2},
            Span{mu_x, vec},
            Span{lam, vec},
            Span{A1, (int64_t)D * kLoraR1 * 2},
            Span{B1, (int64_t)D * kLoraR1 * 2},
            Span{omega, vec},
            Span{A2, (int64_t)D * kLoraR2 * 2},
            Span{B2, (int64_t)D * kLoraR2 * 2},
            out};
}

int matrix_step(bool per_token, int B, int T, int H, int N, const rwkv_bf16 *r,
                const rwkv_bf16 *k, const rwkv_bf16 *v, const float *x, const float *u,
                float *state, rwkv_bf16 *o, hipStream_t stream) {
    const int64_t x_elems = per_token ? checked_mul({B, T, H, N}) : checked_mul({H, N});
    int st = check_matrix(B, T, H, N, r, k, v, x, x_elems, u, state, state, true, o);
    if (st != RWKV_OK) return st;
    if (T == 0) return RWKV_OK;
    return hip_status(wkv::launch_wkv_step(per_token, B, T, H, r, k, v, x, u, state, o,
                                           stream));
}

int matrix_bwd(bool per_token, int B, int T, int H, int N, const rwkv_bf16 *r,
               const rwkv_bf16 *k, const rwkv_bf16 *v, const float *x, const float *u,
               const float *state_in, const rwkv_bf16 *d_o, const float *d_state_out,
               rwkv_bf16 *d_r, rwkv_bf16 *d_k, rwkv_bf16 *d_v, float *d_x, float *d_u,
               float *d_state_in, void *workspace, size_t workspace_bytes, hipStream_t s,
               bool states_saved = false) {
    if (B < 1 || H < 1 || N < 1 || T < 0) return RWKV_E_DIM;
    const int64_t tok = checked_mul({B, T, H, N});
    const int64_t st = checked_mul({B, H, N, N});
    const int64_t hn = checked_mul({H, N});
    if (tok < 0 || st < 0 || hn < 0) return RWKV_E_DIM;
    if (N != 64) return RWKV_E_UNSUPPORTED;
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    const int64_t x_elems = per_token ? tok : hn;
    const int64_t dx_elems = per_token ? tok : hn;
    if (x == nullptr || u == nullptr || d_x == nullptr || d_u == nullptr) return RWKV_E_NULL;
    if (T > 0 && (r == nullptr || k == nullptr || v == nullptr || d_o == nullptr ||
                  d_r == nullptr || d_k == nullptr || d_v == nullptr || workspace == nullptr))
        return RWKV_E_NULL;
    for (const void *p : {(const void *)r, (const void *)k, (const void *)v, (const void *)x,
                          (const void *)u, (const void *)state_in, (const void *)d_o,
                          (const void *)d_state_out, (const void *)d_r, (const void *)d_k,
                          (const void *)d_v, (const void *)d_x, (const void *)d_u,
                          (const void *)d_state_in, (const void *)workspace})
        if (p != nullptr && !aligned(p, 16)) return RWKV_E_ALIGN;
    const size_t need = T > 0 ? wkv::bwd_workspace_bytes(B, T, H) : 0;
    if (T > 0 && workspace_bytes < need) return RWKV_E_DIM;
    const Span sr{r, tok * 2}, sk{k, tok * 2}, sv{v, tok * 2}, sx{x, x_elems * 4},
        su{u, hn * 4}, ssi{state_in, st * 4}, sdo{d_o, tok * 2}, sdso{d_state_out, st * 4},
        sdr{d_r, tok * 2}, sdk{d_k, tok * 2}, sdv{d_v, tok * 2}, sdx{d_x, dx_elems * 4},
        sdu{d_u, hn * 4}, sdsi{d_state_in, st * 4}, sws{workspace, (int64_t)need};
    const int chk = check_outputs({sdr, sdk, sdv, sdx, sdu, sdsi, sws},
                                  {sr, sk, sv, sx, su, ssi, sdo, sdso}, d_state_in, d_state_out);
    if (chk != RWKV_OK) return chk;
    if (T == 0) {  // no tokens: dS_0 = dS_T; the parameter gradients are zero
        hipError_t e = wkv::launch_fill(d_u, hn, 0.0f, s);
        if (e == hipSuccess && !per_token) e = wkv::launch_fill(d_x, hn, 0.0f, s);
        if (e == hipSuccess && d_state_in != nullptr)
            e = d_state_out ? hipMemcpyAsync(d_state_in, d_state_out, st * 4,
                                             hipMemcpyDeviceToDevice, s)
                            : wkv::launch_fill(d_state_in, st, 0.0f, s);
        return hip_status(e);
    }
    return hip_status(wkv::launch_wkv_bwd(per_token, B, T, H, r, k, v, x, u, state_in, d_o,
                                          d_state_out, d_r, d_k, d_v, d_x, d_u, d_state_in,
                                          workspace, s, states_saved));
}

// The forward that also stores, in a backward workspace, the state entering
// every chunk (and the final state), as the backward's recomputation would.
int matrix_fwd_save(bool per_token, int B, int T, int H, int N, const rwkv_bf16 *r,
                    const rwkv_bf16 *k, const rwkv_bf16 *v, const float *x, const float *u,
                    const float *state_in, float *state_out, rwkv_bf16 *o, void *workspace,
                    size_t workspace_bytes, hipStream_t s) {
    const int64_t x_elems = per_token ? checked_mul({B, T, H, N}) : checked_mul({H, N});
    int st = check_matrix(B, T, H, N, r, k, v, x, x_elems, u, state_in, state_out, false, o);
    if (st != RWKV_OK) return st;
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    if (T == 0) return matrix_fwd(per_token, B, T, H, N, r, k, v, x, u, state_in, state_out, o,
                                  nullptr, 0, s);
    if (workspace == nullptr) return RWKV_E_NULL;
    if (!aligned(workspace, 16)) return RWKV_E_ALIGN;
    const size_t need = wkv::bwd_workspace_bytes(B, T, H);
    if (workspace_bytes < need) return RWKV_E_DIM;
    const int64_t tok = checked_mul({B, T, H, N}), sts = checked_mul({B, H, N, N});
    const Span sws{workspace, (int64_t)need};
    st = check_outputs({sws, Span{o, tok * 2}, Span{state_out, sts * 4}},
                       {Span{r, tok * 2}, Span{k, tok * 2}, Span{v, tok * 2},
                        Span{x, x_elems * 4}, Span{u, (int64_t)H * N * 4},
                        Span{state_in, sts * 4}},
                       state_out, state_in);
    if (st != RWKV_OK) return st;
    float *states = (float *)((char *)workspace + wkv::bwd_states_offset(B, T, H));
    return hip_status(wkv::launch_wkv_chunked(per_token, B, T, H, r, k, v, x, u, state_in,
                                              state_out, o, workspace, s, states));
}

}  // namespace

extern "C" {

const char *rwkv_wkv_strerror(int status) {
    switch (status) {
        case RWKV_OK: return "ok";
        case RWKV_E_NULL: return "a required pointer is NULL";
        case RWKV_E_DIM: return "invalid dimension (B, H, N < 1, T < 0, or size overflow)";
        case RWKV_E_UNSUPPORTED:
            return "unsupported shape (Eagle/Finch head size must be 64; RWKV-4 sequence too long)";
        case RWKV_E_ALIGN: return "pointer not aligned as required";
        case RWKV_E_ALIAS: return "an output overlaps an input or another output";
        case RWKV_E_HIP: return "the HIP runtime rejected a launch or copy";
        case RWKV_E_TIMEOUT:
            return "a workgroup gave up waiting for another's hand-off; outputs are invalid";
        default: return "unknown status";
    }
}

int rwkv_wkv_workspace_status(void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace == nullptr) return RWKV_E_NULL;
    if (workspace_bytes < wkv::kWsCtrlBytes) return RWKV_E_DIM;
    if (!aligned(workspace, 16)) return RWKV_E_ALIGN;
    unsigned *word = (unsigned *)((char *)workspace + wkv::kWsErrOffset);
    unsigned v = 0;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return RWKV_E_HIP;
    if (v == 0) return RWKV_OK;
    static const unsigned zero = 0;
    e = hipMemcpyAsync(word, &zero, 4, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return e == hipSuccess ? RWKV_E_TIMEOUT : RWKV_E_HIP;
}

size_t rwkv4_wkv_fwd_workspace_bytes(int B, int T, int H, int N) {
    if (B < 1 || T < 1 || H < 1 || N < 1) return 0;
    const int64_t C = checked_mul({H, N});
    if (C < 0 || C > kMaxRwkv4Channels || (int64_t)B * ((C + 31) / 32) > INT32_MAX) return 0;
    return wkv::rwkv4_workspace_bytes(B, T, (int)C);
}

int rwkv4_wkv_fwd(int B, int T, int H, int N, const float *k, const float *v,
                  const float *w, const float *u, const float *state_in,
                  float *state_out, float *y, void *workspace, size_t workspace_bytes,
                  hipStream_t s) {
    if (B < 1 || H < 1 || N < 1 || T < 0) return RWKV_E_DIM;
    const int64_t C = checked_mul({H, N});
    const int64_t tok = checked_mul({B, T, H, N});
    const int64_t st = checked_mul({B, 3, H, N});
    if (C < 0 || tok < 0 || st < 0 || C > INT32_MAX / 2) return RWKV_E_DIM;
    // a pass of the scan addresses its rows with 32-bit byte offsets
    if (C > kMaxRwkv4Channels) return RWKV_E_UNSUPPORTED;
    // one workgroup per batch entry and block of 32 channels
    if ((int64_t)B * ((C + 31) / 32) > INT32_MAX) return RWKV_E_UNSUPPORTED;
    if (T > 0 && (k == nullptr || v == nullptr || w == nullptr || u == nullptr ||
                  y == nullptr))
        return RWKV_E_NULL;
    for (const void *p : {(const void *)k, (const void *)v, (const void *)w,
                          (const void *)u, (const void *)state_in,
                          (const void *)state_out, (const void *)y})
        if (p != nullptr && !aligned(p, 4)) return RWKV_E_ALIGN;
    const Span sk{k, tok * 4}, sv{v, tok * 4}, sw{w, C * 4}, su{u, C * 4},
        ssi{state_in, st * 4}, sso{state_out, st * 4}, sy{y, tok * 4};
    int chk = (T == 0) ? check_outputs({sso}, {ssi}, state_out, state_in)
                       : check_outputs({sy, sso}, {sk, sv, sw, su, ssi}, state_out, state_in);
    if (chk != RWKV_OK) return chk;
    if (T == 0) {
        if (state_out == nullptr || state_out == state_in) return RWKV_OK;
        if (state_in == nullptr)
            return hip_status(wkv::launch_rwkv4_empty_state(B, (int)C, state_out, s));
        return hip_status(hipMemcpyAsync(state_out, state_in, st * 4,
                                         hipMemcpyDeviceToDevice, s));
    }
    chk = check_workspace(workspace, workspace_bytes, wkv::rwkv4_workspace_bytes(B, T, (int)C),
                          {sk, sv, sw, su, ssi, sso, sy});
    if (chk != RWKV_OK) return chk;
    return hip_status(
        wkv::launch_rwkv4(B, T, (int)C, k, v, w, u, state_in, state_out, y, workspace, s));
}

int rwkv4_wkv_step(int B, int T, int H, int N, const float *k, const float *v,
                   const float *w, const float *u, float *state, float *y, hipStream_t stream) {
    if (B < 1 || H < 1 || N < 1 || T < 0) return RWKV_E_DIM;
    const int64_t C = checked_mul({H, N});
    const int64_t tok = checked_mul({B, T, H, N});
    const int64_t st = checked_mul({B, 3, H, N});
    if (C < 0 || tok < 0 || st < 0 || C > INT32_MAX / 2) return RWKV_E_DIM;
    // one thread per (sequence, channel)
    if ((int64_t)B * C > ((int64_t)1 << 38)) return RWKV_E_UNSUPPORTED;
    if (state == nullptr) return RWKV_E_NULL;
    if (T > 0 && (k == nullptr || v == nullptr || w == nullptr || u == nullptr ||
                  y == nullptr))
        return RWKV_E_NULL;
    for (const void *p : {(const void *)k, (const void *)v, (const void *)w,
                          (const void *)u, (const void *)state, (const void *)y})
        if (p != nullptr && !aligned(p, 4)) return RWKV_E_ALIGN;
    const Span sk{k, tok * 4}, sv{v, tok * 4}, sw{w, C * 4}, su{u, C * 4}, ss{state, st * 4},
        sy{y, tok * 4};
    if (T == 0) return RWKV_OK;
    // state is read and written in place: it must not overlap the inputs or y
    const int chk = check_outputs({sy, ss}, {sk, sv, sw, su});
    if (chk != RWKV_OK) return chk;
    return hip_status(wkv::launch_rwkv4_step(B, T, (int)C, k, v, w, u, state, y, stream));
}

size_t rwkv_wkv_fwd_workspace_bytes(int B, int T, int H, int N) {
    if (B < 1 || T < 1 || H < 1 || N != 64 || H > kMaxChunkedHeads ||
        (int64_t)B * H > INT32_MAX)
        return 0;
    return wkv::chunk_workspace_bytes(B, T, H);
}

int rwkv5_wkv_fwd(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                  const rwkv_bf16 *v, const float *x, const float *u,
                  const float *state_in, float *state_out, rwkv_bf16 *o, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd(false, B, T, H, N, r, k, v, x, u, state_in, state_out, o, workspace,
                      workspace_bytes, stream);
}

int rwkv6_wkv_fwd(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                  const rwkv_bf16 *v, const float *x, const float *u,
                  const float *state_in, float *state_out, rwkv_bf16 *o, void *workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd(true, B, T, H, N, r, k, v, x, u, state_in, state_out, o, workspace,
                      workspace_bytes, stream);
}

int rwkv5_wkv_fwd_gated(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                        const rwkv_bf16 *v, const float *x, const float *u,
                        const float *state_in, float *state_out, const rwkv_bf16 *gate,
                        const float *ln_w, const float *ln_b, float eps, rwkv_bf16 *y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd_gated(false, B, T, H, N, r, k, v, x, u, state_in, state_out, gate, ln_w,
                            ln_b, eps, y, workspace, workspace_bytes, stream);
}

int rwkv6_wkv_fwd_gated(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                        const rwkv_bf16 *v, const float *x, const float *u,
                        const float *state_in, float *state_out, const rwkv_bf16 *gate,
                        const float *ln_w, const float *ln_b, float eps, rwkv_bf16 *y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd_gated(true, B, T, H, N, r, k, v, x, u, state_in, state_out, gate, ln_w,
                            ln_b, eps, y, workspace, workspace_bytes, stream);
}

size_t rwkv_wkv_bwd_workspace_bytes(int B, int T, int H, int N) {
    if (B < 1 || T < 1 || H < 1 || N != 64 || H > kMaxChunkedHeads ||
        (int64_t)B * H > INT32_MAX)
        return 0;
    return wkv::bwd_workspace_bytes(B, T, H);
}

int rwkv5_wkv_bwd(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                  const rwkv_bf16 *v, const float *x, const float *u, const float *state_in,
                  const rwkv_bf16 *d_o, const float *d_state_out, rwkv_bf16 *d_r,
                  rwkv_bf16 *d_k, rwkv_bf16 *d_v, float *d_x, float *d_u, float *d_state_in,
                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return matrix_bwd(false, B, T, H, N, r, k, v, x, u, state_in, d_o, d_state_out, d_r, d_k,
                      d_v, d_x, d_u, d_state_in, workspace, workspace_bytes, stream);
}

int rwkv6_wkv_bwd(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                  const rwkv_bf16 *v, const float *x, const float *u, const float *state_in,
                  const rwkv_bf16 *d_o, const float *d_state_out, rwkv_bf16 *d_r,
                  rwkv_bf16 *d_k, rwkv_bf16 *d_v, float *d_x, float *d_u, float *d_state_in,
                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return matrix_bwd(true, B, T, H, N, r, k, v, x, u, state_in, d_o, d_state_out, d_r, d_k,
                      d_v, d_x, d_u, d_state_in, workspace, workspace_bytes, stream);
}

int rwkv5_wkv_fwd_save(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                       const rwkv_bf16 *v, const float *x, const float *u,
                       const float *state_in, float *state_out, rwkv_bf16 *o, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd_save(false, B, T, H, N, r, k, v, x, u, state_in, state_out, o, workspace,
                           workspace_bytes, stream);
}

int rwkv6_wkv_fwd_save(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                       const rwkv_bf16 *v, const float *x, const float *u,
                       const float *state_in, float *state_out, rwkv_bf16 *o, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    return matrix_fwd_save(true, B, T, H, N, r, k, v, x, u, state_in, state_out, o, workspace,
                           workspace_bytes, stream);
}

int rwkv5_wkv_bwd_saved(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                        const rwkv_bf16 *v, const float *x, const float *u,
                        const rwkv_bf16 *d_o, const float *d_state_out, rwkv_bf16 *d_r,
                        rwkv_bf16 *d_k, rwkv_bf16 *d_v, float *d_x, float *d_u,
                        float *d_state_in, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return matrix_bwd(false, B, T, H, N, r, k, v, x, u, nullptr, d_o, d_state_out, d_r, d_k,
                      d_v, d_x, d_u, d_state_in, workspace, workspace_bytes, stream, true);
}

int rwkv6_wkv_bwd_saved(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                        const rwkv_bf16 *v, const float *x, const float *u,
                        const rwkv_bf16 *d_o, const float *d_state_out, rwkv_bf16 *d_r,
                        rwkv_bf16 *d_k, rwkv_bf16 *d_v, float *d_x, float *d_u,
                        float *d_state_in, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return matrix_bwd(true, B, T, H, N, r, k, v, x, u, nullptr, d_o, d_state_out, d_r, d_k,
                      d_v, d_x, d_u, d_state_in, workspace, workspace_bytes, stream, true);
}

int rwkv5_wkv_step(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                   const rwkv_bf16 *v, const float *x, const float *u, float *state,
                   rwkv_bf16 *o, hipStream_t stream) {
    return matrix_step(false, B, T, H, N, r, k, v, x, u, state, o, stream);
}

int rwkv6_wkv_step(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                   const rwkv_bf16 *v, const float *x, const float *u, float *state,
                   rwkv_bf16 *o, hipStream_t stream) {
    return matrix_step(true, B, T, H, N, r, k, v, x, u, state, o, stream);
}

int rwkv6_wkv_fwd_noalloc(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                          const rwkv_bf16 *v, const float *x, const float *u,
                          const float *state_in, float *state_out, rwkv_bf16 *o,
                          hipStream_t stream) {
    const int64_t x_elems = checked_mul({B, T, H, N});
    const int st = check_matrix(B, T, H, N, r, k, v, x, x_elems, u, state_in, state_out, false, o);
    if (st != RWKV_OK) return st;
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    const size_t need = T > 0 ? wkv::chunk_workspace_bytes(B, T, H) : 0;
    if (need > kStaticScratchBytes) return RWKV_E_UNSUPPORTED;
    void *ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return RWKV_E_HIP;
    return matrix_fwd(true, B, T, H, N, r, k, v, x, u, state_in, state_out, o, ws, need, stream);
}

size_t rwkv6_decay_lora_workspace_bytes(int B, int T, int D) {
    if (B < 1 || T < 1 || D < 64 || D % 64 != 0 || D / 64 > 65535 ||
        (int64_t)B * T >= ((int64_t)1 << 31))
        return 0;
    return wkv::lora_workspace_bytes(B, T, D);
}

int rwkv6_decay_lora(int B, int T, int D, int act, const rwkv_bf16 *x, const rwkv_bf16 *shift,
                     const float *mu_x, const float *lam, const rwkv_bf16 *A1,
                     const rwkv_bf16 *B1, const float *omega, const rwkv_bf16 *A2,
                     const rwkv_bf16 *B2, float *d, void *workspace, size_t workspace_bytes,
                     hipStream_t s) {
    const int64_t tok = checked_mul({B, T, D});
    if (T > 0 && d == nullptr) return RWKV_E_NULL;
    if (d != nullptr && !aligned(d, 16)) return RWKV_E_ALIGN;
    int st = check_lora(B, T, D, act, x, shift, mu_x, lam, A1, B1, omega, A2, B2,
                        Span{d, tok * 4});
    if (st != RWKV_OK || T == 0) return st;
    st = check_workspace(workspace, workspace_bytes, wkv::lora_workspace_bytes(B, T, D),
                         lora_spans(B, T, D, x, shift, mu_x, lam, A1, B1, omega, A2, B2,
                                    Span{d, tok * 4}));
    if (st != RWKV_OK) return st;
    const int rows = B * T;
    uint16_t *h = (uint16_t *)workspace;
    void *packed = (char *)workspace + wkv::lora_packed_offset(B, T);
    hipError_t e = wkv::launch_decay_lora(rows, T, D, act == 1, x, shift, mu_x, lam, A1, B1, A2,
                                          h, packed, s);
    if (e != hipSuccess) return RWKV_E_HIP;
    return hip_status(wkv::launch_lora_logits(rows, D, h, B2, omega, d, s));
}

size_t rwkv6_wkv_fwd_lora_workspace_bytes(int B, int T, int H, int N) {
    if (B < 1 || T < 1 || H < 1 || N != 64 || H > kMaxChunkedHeads ||
        (int64_t)B * H > INT32_MAX || (int64_t)H * N / 64 > 65535 ||
        (int64_t)B * T >= ((int64_t)1 << 31))
        return 0;
    return wkv::lora_fwd_workspace_bytes(B, T, H);
}

int rwkv6_wkv_fwd_lora(int B, int T, int H, int N, const rwkv_bf16 *r, const rwkv_bf16 *k,
                       const rwkv_bf16 *v, const rwkv_bf16 *x, const rwkv_bf16 *shift,
                       const float *mu_x, const float *lam, const rwkv_bf16 *A1,
                       const rwkv_bf16 *B1, const float *omega, const rwkv_bf16 *A2,
                       const rwkv_bf16 *B2, int act, const float *u, const float *state_in,
                       float *state_out, rwkv_bf16 *o, void *workspace, size_t workspace_bytes,
                       hipStream_t s) {
    // the WKV's own arguments (u stands in for the logits, which are formed
    // on the device), then the producer's against both outputs
    int st = check_matrix(B, T, H, N, r, k, v, u, checked_mul({H, N}), u, state_in, state_out,
                          false, o);
    if (st != RWKV_OK) return st;
    if (H > kMaxChunkedHeads || (int64_t)B * H > INT32_MAX) return RWKV_E_UNSUPPORTED;
    const int64_t D = (int64_t)H * N, tok = checked_mul({B, T, H, N});
    const int64_t sts = checked_mul({B, H, N, N});
    const Span so{o, tok * 2}, sso{state_out, sts * 4};
    st = check_lora(B, T, (int)D, act, x, shift, mu_x, lam, A1, B1, omega, A2, B2, so);
    if (st != RWKV_OK) return st;
    if (T > 0) {
        st = check_lora(B, T, (int)D, act, x, shift, mu_x, lam, A1, B1, omega, A2, B2, sso);
        if (st != RWKV_OK) return st;
    }
    if (T == 0)
        return matrix_fwd(true, B, T, H, N, r, k, v, u, u, state_in, state_out, o, nullptr, 0, s);
    std::vector<Span> spans =
        lora_spans(B, T, (int)D, x, shift, mu_x, lam, A1, B1, omega, A2, B2, so);
    spans.insert(spans.end(), {sso, Span{r, tok * 2}, Span{k, tok * 2}, Span{v, tok * 2},
                               Span{u, (int64_t)H * N * 4}, Span{state_in, sts * 4}});
    st = check_workspace(workspace, workspace_bytes, wkv::lora_fwd_workspace_bytes(B, T, H),
                         spans);
    if (st != RWKV_OK) return st;
    const int rows = B * T;
    char *part = (char *)workspace + wkv::lora_fwd_factor_offset(B, T, H);
    uint16_t *h = (uint16_t *)part;
    void *packed = part + wkv::lora_packed_offset(B, T);
    hipError_t e = wkv::launch_decay_lora(rows, T, (int)D, act == 1, x, shift, mu_x, lam, A1, B1,
                                          A2, h, packed, s);
    if (e != hipSuccess) return RWKV_E_HIP;
    return hip_status(wkv::launch_wkv_chunked(true, B, T, H, r, k, v, nullptr, u, state_in,
                                              state_out, o, workspace, s, nullptr, nullptr,
                                              nullptr, nullptr, 0.0f, h, B2, omega));
}

}  // extern "C"

namespace wkv {

namespace {
// Per-device attribute cache (the library's only state).
int device_attr(hipDeviceAttribute_t attr, int fallback, int (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
    int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, attr, dev) != hipSuccess || n <= 0) n = fallback;
        __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    }
    return n;
}
int g_cus[64], g_xcds[64];
}  // namespace

int device_cus() { return device_attr(hipDeviceAttributeMultiprocessorCount, 256, g_cus); }

// (1 when the runtime cannot say: the segments of a split then need no
// particular placement to stay on one die)
int device_xcds() { return device_attr(hipDeviceAttributeNumberOfXccs, 1, g_xcds); }

// the decay producer's scratch: act(z A2) of every token (128 bytes each),
// then the weights laid out as product operands
size_t lora_packed_offset(int B, int T) { return ((size_t)B * T * 64 * 2 + 255) / 256 * 256; }

size_t lora_workspace_bytes(int B, int T, int D) {
    return lora_packed_offset(B, T) + lora_packed_bytes(D);
}

// (after the chunked forward's hand-off area, and at least its control block)
size_t lora_fwd_factor_offset(int B, int T, int H) {
    return (std::max(kWsCtrlBytes, chunk_workspace_bytes(B, T, H)) + 255) / 256 * 256;
}

size_t lora_fwd_workspace_bytes(int B, int T, int H) {
    return lora_fwd_factor_offset(B, T, H) + lora_workspace_bytes(B, T, 64 * H);
}

}  // namespace wkv
