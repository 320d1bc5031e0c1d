// stream_probe.hip -- plain streaming kernels that measure the HBM bandwidth
// one MI355X actually reaches (read only, copy, write only), the reference
// the bench sets each operator's bytes against.  Not part of the operator
// library: bench.py loads it on its own.
//
// Each thread moves 16-byte vectors; a workgroup covers a contiguous span of
// the buffer in steps of blockDim vectors, with `kUnroll` loads in flight per
// thread, and the grid strides over the rest.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

// NT: non-temporal loads / stores (cache policy nt) instead of plain ones
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p) {
    return NT ? __builtin_nontemporal_load(p) : *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4 *p, const u32x4 &v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NT>
__global__ void read_kernel(const u32x4 *__restrict__ src, size_t n, u32x4 *sink) {
    const size_t step = (size_t)gridDim.x * blockDim.x * kUnroll;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t base = (size_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n;
         base += step) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = base + (size_t)j * blockDim.x;
            v[j] = i < n ? ld<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= v[j];
    }
    // (never true for the bench's buffers of ones; keeps the loads alive)
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

template <bool NTL, bool NTS>
__global__ void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
    const size_t step = (size_t)gridDim.x * blockDim.x * kUnroll;
    for (size_t base = (size_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n;
         base += step) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = base + (size_t)j * blockDim.x;
            if (i < n) v[j] = ld<NTL>(src + i);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = base + (size_t)j * blockDim.x;
            if (i < n) st<NTS>(dst + i, v[j]);
        }
    }
}

template <bool NT>
__global__ void write_kernel(u32x4 *__restrict__ dst, size_t n, unsigned val) {
    const size_t step = (size_t)gridDim.x * blockDim.x * kUnroll;
    const u32x4 v = {val, val, val, val};
    for (size_t base = (size_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n;
         base += step) {
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t i = base + (size_t)j * blockDim.x;
            if (i < n) st<NT>(dst + i, v);
        }
    }
}

}  // namespace

extern "C" {

// kind 0: read `bytes` of src (dst: a sink of blockDim 16-byte words, never
// written in practice); 1: copy src to dst; 2: write dst; 3, 4, 5: the same
// with non-temporal loads and stores; 6: copy with non-temporal loads and
// plain stores.  bytes a multiple of
// 16, pointers 16-byte aligned, blocks and threads (a multiple of 64, at most
// 1024) positive.  Returns 0, or -1 for invalid arguments, -2 for a launch
// error.
int stream_probe(int kind, const void *src, void *dst, size_t bytes, int blocks, int threads,
                 hipStream_t stream) {
    if (bytes % 16 != 0 || blocks < 1 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
        return -1;
    const size_t n = bytes / 16;
    const u32x4 *s = (const u32x4 *)src;
    u32x4 *d = (u32x4 *)dst;
    if (d == nullptr || (kind != 2 && kind != 5 && s == nullptr)) return -1;
    const dim3 g(blocks), b(threads);
    switch (kind) {
        case 0: hipLaunchKernelGGL(read_kernel<false>, g, b, 0, stream, s, n, d); break;
        case 3: hipLaunchKernelGGL(read_kernel<true>, g, b, 0, stream, s, n, d); break;
        case 1: hipLaunchKernelGGL((copy_kernel<false, false>), g, b, 0, stream, s, d, n); break;
        case 4: hipLaunchKernelGGL((copy_kernel<true, true>), g, b, 0, stream, s, d, n); break;
        case 6: hipLaunchKernelGGL((copy_kernel<true, false>), g, b, 0, stream, s, d, n); break;
        case 2: hipLaunchKernelGGL(write_kernel<false>, g, b, 0, stream, d, n, 0x3f800000u); break;
        case 5: hipLaunchKernelGGL(write_kernel<true>, g, b, 0, stream, d, n, 0x3f800000u); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
