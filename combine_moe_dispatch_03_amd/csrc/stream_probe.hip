// Reference streaming kernels for gfx950: plain reads, copies and writes over
// device buffers, with and without the non-temporal cache policy.  They are no
// part of the dispatch/combine path; they measure what HBM streaming reaches on
// this GPU for access patterns like the path's own (grid-stride streams, and
// whole rows written by one workgroup), so the path's kernels can be compared
// with a ceiling measured on the same device.  Built as libmoe_stream_probe.so.
//
// C ABI (one entry point):
//
//   int moe_probe_stream(int kind, int nt, void *dst, const void *src,
//                        int64_t bytes, int grid, int64_t row_bytes,
//                        int rows_per_block, hipStream_t stream);
//
//   kind MOE_PROBE_READ    reads src[0, bytes) grid-stride over `grid`
//                          workgroups; dst receives at most one 4-byte word
//                          per workgroup (so needs grid * 4 bytes).
//   kind MOE_PROBE_COPY    copies src[0, bytes) to dst[0, bytes), grid-stride.
//   kind MOE_PROBE_WRITE   fills dst[0, bytes) grid-stride (src unused).
//   kind MOE_PROBE_ROWS    fills dst with rows of `row_bytes`: workgroup b
//                          writes rows b*R ... b*R + R - 1 (R =
//                          rows_per_block), floor(bytes / (row_bytes * R))
//                          workgroups (`grid` unused, src unused).
//   kind MOE_PROBE_ONESHOT_WRITE / MOE_PROBE_ONESHOT_COPY
//                          no loop: workgroup b covers the 256 * V vectors
//                          from b * 256 * V on (V = rows_per_block, 1 ... 8),
//                          lane i the vectors at i, i + 256, ...;
//                          floor(bytes / (4096 * V)) workgroups (`grid` and
//                          `row_bytes` unused).
//   kind MOE_PROBE_EMPTY   `grid` workgroups of 256 lanes, each of whose lane 0
//                          stores one 4-byte word to dst (dst needs grid * 4
//                          bytes): the floor of a launch of that many
//                          workgroups.
//   nt != 0 marks the loads and stores non-temporal.
//   bytes, row_bytes and both pointers must be multiples of 16; grid in
//   [1, 1 << 20].  Returns 0, -1 for bad arguments (nothing launched), or the
//   hipError_t of a failed launch.  Asynchronous on `stream`; every access
//   stays inside [0, bytes) of its buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p) {
    return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4 *p, const u32x4 &v) {
    if (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Four independent 16-byte accesses in flight per lane and loop turn.
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4 *src, int64_t n,
                                                              uint32_t *sink, uint32_t magic) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = ld<NT>(src + i), b = ld<NT>(src + i + stride);
        const u32x4 c = ld<NT>(src + i + 2 * stride), d = ld<NT>(src + i + 3 * stride);
        const u32x4 x = a ^ b ^ c ^ d;
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    for (; i < n; i += stride) {
        const u32x4 a = ld<NT>(src + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    // keeps the loads live; the host passes a value no lane reaches in practice
    if (acc == magic) sink[blockIdx.x] = acc;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(u32x4 *dst, const u32x4 *src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = ld<NT>(src + i), b = ld<NT>(src + i + stride);
        const u32x4 c = ld<NT>(src + i + 2 * stride), d = ld<NT>(src + i + 3 * stride);
        st<NT>(dst + i, a);
        st<NT>(dst + i + stride, b);
        st<NT>(dst + i + 2 * stride, c);
        st<NT>(dst + i + 3 * stride, d);
    }
    for (; i < n; i += stride) st<NT>(dst + i, ld<NT>(src + i));
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_write_kernel(u32x4 *dst, int64_t n, uint32_t value) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const u32x4 v = {value, value, value, value};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) st<NT>(dst + i, v);
}

// Workgroup b writes rows b*rpb ... b*rpb + rpb - 1, each `vpr` vectors long,
// the 256 lanes striding over a row (the shape of one token's row written to
// its destinations by one workgroup).
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_rows_kernel(u32x4 *dst, int64_t vpr, int rpb,
                                                              uint32_t value) {
    const u32x4 v = {value, value, value, value};
    for (int j = 0; j < rpb; ++j) {
        u32x4 *row = dst + ((int64_t)blockIdx.x * rpb + j) * vpr;
        for (int64_t c = threadIdx.x; c < vpr; c += kThreads) st<NT>(row + c, v);
    }
}

// One pass, no loop: each lane moves V vectors (block-contiguous stripes).
template <bool NT, int V, bool COPY>
__global__ __launch_bounds__(kThreads) void probe_oneshot_kernel(u32x4 *dst, const u32x4 *src,
                                                                 uint32_t value) {
    const int64_t base = (int64_t)blockIdx.x * kThreads * V + threadIdx.x;
    u32x4 v[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        if (COPY)
            v[q] = ld<NT>(src + base + q * kThreads);
        else
            v[q] = u32x4{value, value, value, value};
    }
#pragma unroll
    for (int q = 0; q < V; ++q) st<NT>(dst + base + q * kThreads, v[q]);
}

template <bool NT, bool COPY>
void launch_oneshot(int v, unsigned blocks, u32x4 *d, const u32x4 *s, uint32_t value, hipStream_t stream) {
    switch (v) {
    case 1: hipLaunchKernelGGL((probe_oneshot_kernel<NT, 1, COPY>), dim3(blocks), dim3(kThreads), 0, stream, d, s, value); break;
    case 2: hipLaunchKernelGGL((probe_oneshot_kernel<NT, 2, COPY>), dim3(blocks), dim3(kThreads), 0, stream, d, s, value); break;
    case 4: hipLaunchKernelGGL((probe_oneshot_kernel<NT, 4, COPY>), dim3(blocks), dim3(kThreads), 0, stream, d, s, value); break;
    default: hipLaunchKernelGGL((probe_oneshot_kernel<NT, 8, COPY>), dim3(blocks), dim3(kThreads), 0, stream, d, s, value); break;
    }
}

__global__ __launch_bounds__(kThreads) void probe_empty_kernel(uint32_t *dst) {
    if (threadIdx.x == 0) dst[blockIdx.x] = blockIdx.x;
}

}  // namespace

extern "C" {

enum {
    MOE_PROBE_READ = 0,
    MOE_PROBE_COPY = 1,
    MOE_PROBE_WRITE = 2,
    MOE_PROBE_ROWS = 3,
    MOE_PROBE_ONESHOT_WRITE = 4,
    MOE_PROBE_ONESHOT_COPY = 5,
    MOE_PROBE_EMPTY = 6,
};

int moe_probe_stream(int kind, int nt, void *dst, const void *src, int64_t bytes, int grid,
                     int64_t row_bytes, int rows_per_block, hipStream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0 || dst == nullptr || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return -1;
    const int64_t n = bytes / 16;
    const bool uses_src = kind == MOE_PROBE_READ || kind == MOE_PROBE_COPY || kind == MOE_PROBE_ONESHOT_COPY;
    if (uses_src && (src == nullptr || reinterpret_cast<uintptr_t>(src) % 16 != 0)) return -1;
    const bool uses_grid = kind == MOE_PROBE_READ || kind == MOE_PROBE_COPY || kind == MOE_PROBE_WRITE ||
                           kind == MOE_PROBE_EMPTY;
    if (uses_grid && (grid < 1 || grid > (1 << 20))) return -1;
    const uint32_t value = 0x3F803F80u;     // bf16 pairs of 1.0
    u32x4 *d = static_cast<u32x4 *>(dst);
    const u32x4 *s = static_cast<const u32x4 *>(src);
    switch (kind) {
    case MOE_PROBE_READ:
        if ((int64_t)grid * 4 > bytes) return -1;   // one sink word per workgroup in dst
        if (nt)
            hipLaunchKernelGGL(probe_read_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, s, n,
                               static_cast<uint32_t *>(dst), 0x9E3779B9u);
        else
            hipLaunchKernelGGL(probe_read_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, s, n,
                               static_cast<uint32_t *>(dst), 0x9E3779B9u);
        break;
    case MOE_PROBE_COPY:
        if (nt)
            hipLaunchKernelGGL(probe_copy_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, d, s, n);
        else
            hipLaunchKernelGGL(probe_copy_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, d, s, n);
        break;
    case MOE_PROBE_WRITE:
        if (nt)
            hipLaunchKernelGGL(probe_write_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, d, n, value);
        else
            hipLaunchKernelGGL(probe_write_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, d, n, value);
        break;
    case MOE_PROBE_ROWS: {
        if (row_bytes <= 0 || row_bytes % 16 != 0 || rows_per_block < 1) return -1;
        const int64_t blocks = bytes / (row_bytes * rows_per_block);
        if (blocks < 1 || blocks > (int64_t(1) << 31) - 1) return -1;
        const int64_t vpr = row_bytes / 16;
        if (nt)
            hipLaunchKernelGGL(probe_rows_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, d,
                               vpr, rows_per_block, value);
        else
            hipLaunchKernelGGL(probe_rows_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, d,
                               vpr, rows_per_block, value);
        break;
    }
    case MOE_PROBE_ONESHOT_WRITE:
    case MOE_PROBE_ONESHOT_COPY: {
        const int v = rows_per_block;
        if (v != 1 && v != 2 && v != 4 && v != 8) return -1;
        const int64_t blocks = n / ((int64_t)kThreads * v);
        if (blocks < 1 || blocks > (int64_t(1) << 31) - 1) return -1;
        if (kind == MOE_PROBE_ONESHOT_COPY) {
            if (nt)
                launch_oneshot<true, true>(v, (unsigned)blocks, d, s, value, stream);
            else
                launch_oneshot<false, true>(v, (unsigned)blocks, d, s, value, stream);
        } else {
            if (nt)
                launch_oneshot<true, false>(v, (unsigned)blocks, d, s, value, stream);
            else
                launch_oneshot<false, false>(v, (unsigned)blocks, d, s, value, stream);
        }
        break;
    }
    case MOE_PROBE_EMPTY:
        if ((int64_t)grid * 4 > bytes) return -1;
        hipLaunchKernelGGL(probe_empty_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<uint32_t *>(dst));
        break;
    default:
        return -1;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
