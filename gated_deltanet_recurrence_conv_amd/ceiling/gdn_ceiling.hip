// gdn_ceiling.hip -- hand-written HBM stream and matrix-core loops for gfx950
// that measure the sustained ceilings the Gated DeltaNet kernels are priced
// against (read-only, write-only, copy and mixed read:write streams over
// buffers far larger than the 256 MiB Infinity Cache; back-to-back bf16 MFMA).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_ceiling.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct StreamArgs {
    const u4* src[2];
    u4* dst[3];
    u4* sink;
    size_t n;
};

template <bool NT>
__device__ __forceinline__ u4 ld(const u4* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u4* p, u4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// R read buffers, W write buffers, U vectors per thread per pass.  Grid
// stride (BLK = 0): a pass of the grid covers nthr * U consecutive vectors.
// Blocked (BLK > 0): workgroup g streams the contiguous blocks g, g + grid,
// ... of BLK vectors, U vectors per thread per pass inside a block.
template <int R, int W, int U, bool NT, int BLK>
__global__ __launch_bounds__(256) void stream_kernel(StreamArgs a)
{
    const size_t tid = BLK ? threadIdx.x : static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    const size_t nthr = BLK ? 256 : static_cast<size_t>(gridDim.x) * 256;
    u4 acc = {0u, 0u, 0u, 0u};
    const size_t nblk = BLK ? (a.n + BLK - 1) / BLK : 1;
    for (size_t blk = BLK ? blockIdx.x : 0; blk < nblk; blk += BLK ? gridDim.x : 1) {
    const size_t lo = BLK ? blk * BLK : 0;
    const size_t hi = BLK ? (lo + BLK < a.n ? lo + BLK : a.n) : a.n;
    for (size_t base = lo + tid; base < hi; base += nthr * U) {
        u4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = u4{static_cast<uint32_t>(base), 1u, 2u, 3u};
        u4 in[R > 0 ? R : 1][U];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t i = base + u * nthr;
                in[r][u] = i < hi ? ld<NT>(a.src[r] + i) : u4{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (R > 0) {
                v[u] = in[0][u];
#pragma unroll
                for (int r = 1; r < R; ++r) v[u] += in[r][u];
            }
            acc ^= v[u];
        }
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t i = base + u * nthr;
                if (i < hi) st<NT>(a.dst[w] + i, v[u]);
            }
    }
    }
    if constexpr (W == 0) {
        // fold the workgroup's reads so that none of them is dead
        __shared__ u4 red[256];
        red[threadIdx.x] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            u4 s = red[0];
            for (int i = 1; i < 256; ++i) s ^= red[i];
            a.sink[blockIdx.x] = s;
        }
    }
}

constexpr int kBlockVectors = 4096;   // 64 KiB per block in the blocked layout

template <int R, int W, int U>
hipError_t launch_stream_u(const StreamArgs& a, int grid, bool nt, bool blocked, hipStream_t s)
{
    if (blocked) {
        if (nt) hipLaunchKernelGGL((stream_kernel<R, W, U, true, kBlockVectors>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((stream_kernel<R, W, U, false, kBlockVectors>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (nt) hipLaunchKernelGGL((stream_kernel<R, W, U, true, 0>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((stream_kernel<R, W, U, false, 0>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <int R, int W>
hipError_t launch_stream_rw(const StreamArgs& a, int grid, int unroll, bool nt, bool blk, hipStream_t s)
{
    switch (unroll) {
    case 1: return launch_stream_u<R, W, 1>(a, grid, nt, blk, s);
    case 2: return launch_stream_u<R, W, 2>(a, grid, nt, blk, s);
    case 4: return launch_stream_u<R, W, 4>(a, grid, nt, blk, s);
    case 8: return launch_stream_u<R, W, 8>(a, grid, nt, blk, s);
    default: return hipErrorInvalidValue;
    }
}

template <int R>
hipError_t launch_stream_r(const StreamArgs& a, int W, int grid, int unroll, bool nt, bool blk, hipStream_t s)
{
    switch (W) {
    case 0: return launch_stream_rw<R, 0>(a, grid, unroll, nt, blk, s);
    case 1: return launch_stream_rw<R, 1>(a, grid, unroll, nt, blk, s);
    case 2: return launch_stream_rw<R, 2>(a, grid, unroll, nt, blk, s);
    case 3: return launch_stream_rw<R, 3>(a, grid, unroll, nt, blk, s);
    default: return hipErrorInvalidValue;
    }
}

__device__ __forceinline__ f32x4 mfma(const u4& a, const u4& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__global__ __launch_bounds__(256) void mfma_kernel(float* out, int iters)
{
    const uint32_t lane = threadIdx.x & 63;
    // small finite bf16 operands that differ per lane (0x3c00..: ~0.0078)
    const uint32_t e = 0x3c003c00u + (lane & 7) * 0x00010001u;
    u4 a = {e, e + 0x00010001u, e, e}, b = {e, e, e + 0x00020002u, e};
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mfma(a, b, acc[i]);
    }
    float* o = out + (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[4 * i + j] = acc[i][j];
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int gdn_ceiling_stream(const void* const* src, int n_read, void* const* dst, int n_write, size_t n_vec16,
                       void* sink, int grid, int unroll, int mode, void* stream)
{
    if (n_read < 0 || n_read > 2 || n_write < 0 || n_write > 3 || grid <= 0 || n_vec16 == 0) return -1;
    if ((n_read > 0 && !src) || (n_write > 0 && !dst) || (n_write == 0 && !sink)) return -1;
    StreamArgs a{};
    for (int r = 0; r < n_read; ++r) {
        if (!src[r] || !al16(src[r])) return -1;
        a.src[r] = static_cast<const u4*>(src[r]);
    }
    for (int w = 0; w < n_write; ++w) {
        if (!dst[w] || !al16(dst[w])) return -1;
        a.dst[w] = static_cast<u4*>(dst[w]);
    }
    if (sink && !al16(sink)) return -1;
    a.sink = static_cast<u4*>(sink);
    a.n = n_vec16;
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool nt = (mode & 1) != 0;
    const bool blk = (mode & 2) != 0;
    hipError_t e;
    switch (n_read) {
    case 0: e = launch_stream_r<0>(a, n_write, grid, unroll, nt, blk, s); break;
    case 1: e = launch_stream_r<1>(a, n_write, grid, unroll, nt, blk, s); break;
    default: e = launch_stream_r<2>(a, n_write, grid, unroll, nt, blk, s); break;
    }
    return e == hipSuccess ? 0 : static_cast<int>(e);
}

int gdn_ceiling_mfma_bf16(float* out, int grid, int iters, void* stream)
{
    if (!out || !al16(out) || grid <= 0 || iters <= 0) return -1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : static_cast<int>(e);
}

}  // extern "C"
