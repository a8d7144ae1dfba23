// The KDA layer's short causal convolution (kernel size 4, [loading page] section 3) with its
// conv state (the decode cache's conv_states, [loading page] section 6).
//
// Per channel c of a [tokens, C] tensor and per sequence, with W = 4 taps:
//   y_t[c] = act(bias[c] + sum_{j < W} w[c][j] * x_{t - (W-1) + j}[c])
// where inputs before the sequence's first token come from its conv state (the W - 1 previous
// inputs, oldest first; zeros without one), and act is the identity or SiLU. The final conv
// state is the sequence's last W - 1 inputs (shifted in from the initial state when the
// sequence is shorter than W - 1).
//
// The work is elementwise along channels and a 4-tap window along tokens: HBM-bound (one read
// and one write per element, plus a 3-row halo per token strip). Each thread owns 8
// consecutive channels (one 16-byte bf16 vector, two for float32) of a strip of tokens and
// slides the window through registers; consecutive threads cover consecutive channels, so
// every row access is coalesced. The strip's rows are loaded a batch at a time, all of a
// batch's loads issued before the first is used, so that each thread keeps several rows in
// flight rather than one (the bytes in flight per compute unit set a stream's rate); the
// outputs go out as non-temporal stores. Measured on the long-context shape (3 x [131072,
// 4096] bf16): one row in flight and 32-token strips 1.46 ms; 8-row batches 1.38 ms; 64-token
// strips (half the halo reloads) and non-temporal outputs 1.28 ms, about the rate of a device
// copy. 16-row batches, 128- and 256-token strips and non-temporal input loads were no faster.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kConvW = 4;      // taps
constexpr int kConvVec = 8;    // channels per thread
constexpr int kConvStrip = 64; // tokens per thread (prefill)
constexpr int kConvBatch = 8;  // rows of a strip loaded together
static_assert(kConvStrip % kConvBatch == 0, "whole batches per full strip");
constexpr int kConvThreads = 256;

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float (&v)[8]) {
        const u32x4 r = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(r[e] << 16);
            v[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ u32x4 pack(const float (&v)[8]) {
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (uint32_t)bf16_bits(v[2 * e]) | ((uint32_t)bf16_bits(v[2 * e + 1]) << 16);
        return r;
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float (&v)[8]) {
        *reinterpret_cast<u32x4 *>(p) = pack(v);
    }
    // a streamed output, not read again here: non-temporal
    static __device__ __forceinline__ void store_stream(bf16_t *p, const float (&v)[8]) {
        __builtin_nontemporal_store(pack(v), reinterpret_cast<u32x4 *>(p));
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    static __device__ __forceinline__ void store_stream(float *p, const float (&v)[8]) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p + 4));
    }
};

__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// Sequence n and its token range [start, end) for packed token index t (cu_seqlens: the last
// n with cu[n] <= t, skipping empty sequences), or the fixed-length layout.
__device__ __forceinline__ void seq_of(const ConvArgs &a, int64_t t, int &n, int64_t &start, int64_t &end) {
    if (a.cu_seqlens) {
        int lo = 0, hi = a.n_seqs - 1;  // invariant: cu[lo] <= t < cu[hi + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_seqlens[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        packed_range(a.cu_seqlens, n, a.tokens, start, end);
    } else {
        n = (int)(t / a.seq_len);
        start = (int64_t)n * a.seq_len;
        end = start + a.seq_len;
    }
}

// Input p of sequence n relative to its start (p < 0: row W - 1 + p of its conv state).
template <typename T>
__device__ __forceinline__ void hist_row(const ConvArgs &a, int n, int64_t start, int64_t p, int c0, float (&v)[8]) {
    if (p >= 0) {
        Vec8<T>::load(static_cast<const T *>(a.x) + (start + p) * a.C + c0, v);
    } else if (a.s0 && p >= -(kConvW - 1)) {  // (p is below that only for invalid offsets)
        Vec8<T>::load(static_cast<const T *>(a.s0) + ((int64_t)n * (kConvW - 1) + (kConvW - 1) + p) * a.C + c0, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_fwd_kernel(ConvArgs a) {
    const int c0 = kConvVec * (blockIdx.y * kConvThreads + threadIdx.x);
    if (c0 >= a.C) return;
    const int64_t t0 = (int64_t)blockIdx.x * kConvStrip;
    if (t0 >= a.tokens) return;
    const int64_t t1 = t0 + kConvStrip < a.tokens ? t0 + kConvStrip : a.tokens;

    float w[kConvW][8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const f32x4 wc = *reinterpret_cast<const f32x4 *>(a.w + (int64_t)(c0 + e) * kConvW);
#pragma unroll
        for (int j = 0; j < kConvW; ++j) w[j][e] = wc[j];
        b[e] = a.bias ? a.bias[c0 + e] : 0.f;
    }

    int n;
    int64_t start, end;
    seq_of(a, t0, n, start, end);
    float win[kConvW - 1][8];  // the W - 1 inputs before token t, oldest first
#pragma unroll
    for (int j = 0; j < kConvW - 1; ++j) hist_row<T>(a, n, start, t0 - start - (kConvW - 1) + j, c0, win[j]);

    const T *const xc = static_cast<const T *>(a.x) + c0;
    T *const yc = static_cast<T *>(a.y) + c0;
    for (int64_t tb = t0; tb < t1; tb += kConvBatch) {
        // the batch's rows (past the strip's end: its last row again, loaded but not used)
        float xr[kConvBatch][8];
#pragma unroll
        for (int i = 0; i < kConvBatch; ++i) Vec8<T>::load(xc + (tb + i < t1 ? tb + i : t1 - 1) * a.C, xr[i]);
#pragma unroll
        for (int i = 0; i < kConvBatch; ++i) {
            const int64_t t = tb + i;
            if (t >= t1) break;
            if (t == end) {  // the next (non-empty) sequence starts here
                seq_of(a, t, n, start, end);
#pragma unroll
                for (int j = 0; j < kConvW - 1; ++j) hist_row<T>(a, n, start, -(kConvW - 1) + j, c0, win[j]);
            }
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = b[e];
#pragma unroll
                for (int j = 0; j < kConvW - 1; ++j) acc += w[j][e] * win[j][e];
                acc += w[kConvW - 1][e] * xr[i][e];
                y[e] = a.silu ? silu_f(acc) : acc;
            }
            Vec8<T>::store_stream(yc + t * a.C, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
#pragma unroll
                for (int j = 0; j < kConvW - 2; ++j) win[j][e] = win[j + 1][e];
                win[kConvW - 2][e] = xr[i][e];
            }
        }
    }
}

// Final conv states: the last W - 1 inputs of every sequence (read before written, so the
// output may alias the initial state). Launched after conv_fwd_kernel, which reads s0.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_state_kernel(ConvArgs a) {
    const int c0 = kConvVec * (blockIdx.y * kConvThreads + threadIdx.x);
    const int n = blockIdx.x;
    if (c0 >= a.C) return;
    int64_t start, end;
    if (a.cu_seqlens) {
        packed_range(a.cu_seqlens, n, a.tokens, start, end);
    } else {
        start = (int64_t)n * a.seq_len;
        end = start + a.seq_len;
    }
    float v[kConvW - 1][8];
#pragma unroll
    for (int j = 0; j < kConvW - 1; ++j) hist_row<T>(a, n, start, end - start - (kConvW - 1) + j, c0, v[j]);
#pragma unroll
    for (int j = 0; j < kConvW - 1; ++j)
        Vec8<T>::store(static_cast<T *>(a.s_out) + ((int64_t)n * (kConvW - 1) + j) * a.C + c0, v[j]);
}

// Decode: one token per sequence; the state [N, W-1, C] is read and shifted in place.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_update_kernel(ConvArgs a) {
    const int c0 = kConvVec * (blockIdx.y * kConvThreads + threadIdx.x);
    const int n = blockIdx.x;
    if (c0 >= a.C) return;
    T *st = static_cast<T *>(a.s_out) + (int64_t)n * (kConvW - 1) * a.C + c0;
    float win[kConvW - 1][8], xt[8], y[8];
#pragma unroll
    for (int j = 0; j < kConvW - 1; ++j) Vec8<T>::load(st + (int64_t)j * a.C, win[j]);
    Vec8<T>::load(static_cast<const T *>(a.x) + (int64_t)n * a.C + c0, xt);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const f32x4 wc = *reinterpret_cast<const f32x4 *>(a.w + (int64_t)(c0 + e) * kConvW);
        float acc = a.bias ? a.bias[c0 + e] : 0.f;
#pragma unroll
        for (int j = 0; j < kConvW - 1; ++j) acc += wc[j] * win[j][e];
        acc += wc[kConvW - 1] * xt[e];
        y[e] = a.silu ? silu_f(acc) : acc;
    }
    Vec8<T>::store(static_cast<T *>(a.y) + (int64_t)n * a.C + c0, y);
#pragma unroll
    for (int j = 0; j < kConvW - 2; ++j) Vec8<T>::store(st + (int64_t)j * a.C, win[j + 1]);
    Vec8<T>::store(st + (int64_t)(kConvW - 2) * a.C, xt);
}

template <typename T>
hipError_t launch_conv_t(const ConvArgs &a, bool update, hipStream_t stream) {
    const unsigned cblocks = (unsigned)((a.C / kConvVec + kConvThreads - 1) / kConvThreads);
    if (update) {
        hipLaunchKernelGGL(conv_update_kernel<T>, dim3((unsigned)a.n_seqs, cblocks), dim3(kConvThreads), 0,
                           stream, a);
        return hipGetLastError();
    }
    const int64_t strips = (a.tokens + kConvStrip - 1) / kConvStrip;
    if (strips > 0) {
        hipLaunchKernelGGL(conv_fwd_kernel<T>, dim3((unsigned)strips, cblocks), dim3(kConvThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.s_out) {
        hipLaunchKernelGGL(conv_state_kernel<T>, dim3((unsigned)a.n_seqs, cblocks), dim3(kConvThreads), 0,
                           stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

bool conv_supported(int32_t dtype, int32_t C, int32_t W) {
    return (dtype == 0 || dtype == 1) && W == kConvW && C > 0 && C % kConvVec == 0;
}

hipError_t launch_conv(int32_t dtype, const ConvArgs &a, bool update, hipStream_t stream) {
    if (!conv_supported(dtype, a.C, kConvW)) return hipErrorInvalidValue;
    if (a.n_seqs == 0) return hipSuccess;
    return dtype == 1 ? launch_conv_t<bf16_t>(a, update, stream) : launch_conv_t<float>(a, update, stream);
}

}  // namespace kda
