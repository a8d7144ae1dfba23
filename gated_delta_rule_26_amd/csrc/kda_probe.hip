// Measurement probes: the device's practical peaks, against which the KDA kernels' roofline
// fractions are also reported (next to the published ones).
//
// * copy: dst = src over `bytes`, 16-byte vectors, non-temporal loads (the state stream of the
//   decode step reads the same way): the practical HBM bandwidth of a kernel that reads each
//   byte once and writes each byte once.
// * read: a read-only stream (non-temporal 16-byte loads, 64 KB per workgroup), the practical
//   read bandwidth: the bound of a read-mostly kernel such as the prefill.
// * rmw: an in-place read-modify-write stream (x *= factor, non-temporal loads and stores,
//   16 KB per workgroup): the access pattern of the decode step's state, and its practical
//   bound.
// * fp16 / bf16 matrix cores: every wave runs a loop of independent matrix-core products on
//   several accumulators (16x16x32 or 32x32x16 instructions, the same flops per iteration),
//   the operands held in registers; the accumulators are written out at the end so nothing is
//   optimised away.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Eight 16-byte loads per thread are issued before any store (the decode step's pattern: a
// thread reads its whole slice, then writes it), so enough bytes are in flight per CU.
constexpr int kCopyVec = 8;

__global__ __launch_bounds__(256) void probe_copy_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst,
                                                         int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * 256 * kCopyVec + threadIdx.x;
    f32x4 v[kCopyVec];
#pragma unroll
    for (int u = 0; u < kCopyVec; ++u) {
        const int64_t i = base + (int64_t)u * 256;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyVec; ++u) {
        const int64_t i = base + (int64_t)u * 256;
        if (i < n) dst[i] = v[u];
    }
}

// Read and in-place read-modify-write streams: each workgroup of 256 threads owns one slab of
// NV * 4 KB, issues all its 16-byte non-temporal loads, then (RMW) writes the slab back with
// non-temporal stores. Buffer resources bound every slab by the array's end (loads past it
// read zero, stores past it are dropped). Measured on this part: reads peak with 64 KB slabs,
// in-place read-modify-write with 16 KB slabs (more workgroups in flight per CU).
template <int NV> __device__ __forceinline__ rsrc_t slab_rsrc(const void *base, int64_t bytes) {
    const int64_t start = (int64_t)blockIdx.x * NV * 4096;
    const int64_t left = bytes - start;
    return make_rsrc(static_cast<const char *>(base) + start, (uint32_t)(left < NV * 4096 ? left : NV * 4096));
}

template <int NV> __global__ __launch_bounds__(256) void probe_read_kernel(const void *src, int64_t bytes) {
    const rsrc_t r = slab_rsrc<NV>(src, bytes);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NV; ++p)
        acc += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (p * 256 + threadIdx.x) * 16, 0, 2));
    // the sum is consumed by an empty statement the compiler must keep, so every load is
    // issued and waited for, and nothing is written
    __asm__ volatile("" : : "v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
}

template <int NV> __global__ __launch_bounds__(256) void probe_rmw_kernel(void *buf, int64_t bytes, float factor) {
    const rsrc_t r = slab_rsrc<NV>(buf, bytes);
    f32x4 v[NV];
#pragma unroll
    for (int p = 0; p < NV; ++p)
        v[p] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (p * 256 + threadIdx.x) * 16, 0, 2));
#pragma unroll
    for (int p = 0; p < NV; ++p)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[p] * factor), r, (p * 256 + threadIdx.x) * 16, 0, 2);
}

constexpr int kReadSlab = 16;  // 64 KB per workgroup
constexpr int kRmwSlab = 4;    // 16 KB per workgroup

constexpr int kProbeAcc = 8;

// SHAPE 0: v_mfma_f32_16x16x32_{f16,bf16} (eight 4-float accumulators per lane);
// SHAPE 1: v_mfma_f32_32x32x16_{f16,bf16} (four 16-float accumulators per lane).
// H: the operand type, _Float16 or __bf16.
template <typename H> struct ProbeOps;
template <> struct ProbeOps<_Float16> {
    typedef f16x8 V;
    static __device__ f32x4 m16(V a, V b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
    template <typename A> static __device__ A m32(V a, V b, A c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
template <> struct ProbeOps<__bf16> {
    typedef bf16x8 V;
    static __device__ f32x4 m16(V a, V b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
    template <typename A> static __device__ A m32(V a, V b, A c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};

template <int SHAPE, typename H> __global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *sink) {
    using Ops = ProbeOps<H>;
    typename Ops::V a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<H>(1e-3f * (threadIdx.x + e));
        b[e] = static_cast<H>(1e-3f * (blockIdx.x + e));
    }
    float out = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 acc[kProbeAcc];
#pragma unroll
        for (int j = 0; j < kProbeAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kProbeAcc; ++j) acc[j] = Ops::m16(a, b, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < kProbeAcc; ++j) out += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
        typedef float f32x16 __attribute__((ext_vector_type(16)));
        f32x16 acc[kProbeAcc / 2];
#pragma unroll
        for (int j = 0; j < kProbeAcc / 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kProbeAcc / 2; ++j)
                acc[j] = Ops::m32(a, b, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < kProbeAcc / 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) out += acc[j][e];
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = out;
}

}  // namespace

hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    const int64_t n = bytes / 16, blocks = (n + 256 * kCopyVec - 1) / (256 * kCopyVec);
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst), n);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void *src, int64_t bytes, hipStream_t stream) {
    const int64_t blocks = (bytes + kReadSlab * 4096 - 1) / (kReadSlab * 4096);
    hipLaunchKernelGGL((probe_read_kernel<kReadSlab>), dim3((unsigned)blocks), dim3(256), 0, stream, src, bytes);
    return hipGetLastError();
}

hipError_t launch_probe_rmw(void *buf, int64_t bytes, float factor, hipStream_t stream) {
    const int64_t blocks = (bytes + kRmwSlab * 4096 - 1) / (kRmwSlab * 4096);
    hipLaunchKernelGGL((probe_rmw_kernel<kRmwSlab>), dim3((unsigned)blocks), dim3(256), 0, stream, buf, bytes, factor);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int32_t bf16, int32_t shape, int32_t iters, int32_t blocks, float *sink,
                             hipStream_t stream) {
    const dim3 g((unsigned)blocks), t(256);
    if (bf16) {
        if (shape == 0) hipLaunchKernelGGL((probe_mfma_kernel<0, __bf16>), g, t, 0, stream, iters, sink);
        else hipLaunchKernelGGL((probe_mfma_kernel<1, __bf16>), g, t, 0, stream, iters, sink);
    } else {
        if (shape == 0) hipLaunchKernelGGL((probe_mfma_kernel<0, _Float16>), g, t, 0, stream, iters, sink);
        else hipLaunchKernelGGL((probe_mfma_kernel<1, _Float16>), g, t, 0, stream, iters, sink);
    }
    return hipGetLastError();
}

int64_t probe_mfma_flops_per_iter_and_thread() {
    // per wave and iteration: eight 16x16x32 products, or four 32x32x16 ones (the same
    // 2 * 8 * 16 * 16 * 32 flops), shared by the wave's 64 lanes
    return (int64_t)kProbeAcc * 2 * 16 * 16 * 32 / 64;
}

}  // namespace kda
