// KDA decode step: one token per (sequence, head) on a persistent float32 state.
//
// Per (sequence, head), with the state S (Dk x Dv, rows = key channels) in HBM:
//   S' = Diag(exp(g)) S;  p = S'^T k;  r = S'^T (scale q);  u = beta (v - p)
//   o  = r + (scale q . k) u;  S <- S' + k u^T
// which is one step of S_t = (I - beta k k^T) Diag(exp g) S_{t-1} + beta k v^T followed by
// o_t = S_t^T (scale q): the token-by-token recurrent mode used for incremental decoding
// ([loading page] sections 5 and 6: the recurrent state carried by the decode cache).
//
// The state is read once and written once: the step is HBM-bound (7 flops per 8 bytes).
// One workgroup owns one (sequence, head) state. Threads tile the state as rows x float4
// columns, so every wave reads and writes whole contiguous 512-byte rows; each thread keeps
// its Dk*Dv/NT values in registers between the read and the write. Both column reductions
// (p and r) are finished in the same sweep with cross-lane shuffles and one LDS exchange
// between waves, then the rank-1 update is applied to the values still in registers.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int DK, int DV> struct DecodeShape {
    static constexpr int TPR = DV / 4;                               // threads per row
    static constexpr int RPP = (256 / TPR) < DK ? (256 / TPR) : DK;  // rows per pass
    static constexpr int NT = TPR * RPP;                             // threads
    static constexpr int NPASS = DK / RPP;                           // row passes per thread
    static constexpr int NWAVE = (NT + 63) / 64;
    static_assert(DV % 4 == 0 && 64 % TPR == 0, "Dv must be 4..256, a power of two");
    static_assert(DK % RPP == 0 && NT >= 64 && NT <= 256, "unsupported decode shape");
};

__device__ __forceinline__ f32x4 shfl_xor4(f32x4 x, int m) {
    f32x4 r;
    r.x = __shfl_xor(x.x, m);
    r.y = __shfl_xor(x.y, m);
    r.z = __shfl_xor(x.z, m);
    r.w = __shfl_xor(x.w, m);
    return r;
}

template <typename Tin, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int TPR = Sh::TPR, RPP = Sh::RPP, NT = Sh::NT, NPASS = Sh::NPASS;

    __shared__ float sk[DK], sq[DK], sa[DK], sv[DV];
    __shared__ f32x4 red[Sh::NWAVE][2][TPR];
    __shared__ float sqk;

    const int tid = threadIdx.x;
    const int64_t item = blockIdx.x;  // n * H + h
    const Tin *q = static_cast<const Tin *>(a.q) + item * DK;
    const Tin *k = static_cast<const Tin *>(a.k) + item * DK;
    const Tin *v = static_cast<const Tin *>(a.v) + item * DV;
    const float *g = a.g + item * DK;
    float *S = a.state + item * (int64_t)(DK * DV);

    for (int c = tid; c < DK; c += NT) {
        sk[c] = to_f32(k[c]);
        sq[c] = a.scale * to_f32(q[c]);
        sa[c] = __expf(g[c]);
    }
    for (int j = tid; j < DV; j += NT) sv[j] = to_f32(v[j]);
    __syncthreads();

    const int cg = tid % TPR, rr = tid / TPR;
    const int lane = tid & 63, wave = tid >> 6;

    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
        s[p] = *reinterpret_cast<const f32x4 *>(S + (p * RPP + rr) * DV + 4 * cg);

    if (wave == 0) {  // scale * (q . k), off the critical path of the state sweep
        float acc = 0.f;
        for (int c = lane; c < DK; c += 64) acc += sq[c] * sk[c];
        for (int m = 32; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
        if (lane == 0) sqk = acc;
    }

    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int r = p * RPP + rr;
        s[p] *= sa[r];
        pk += s[p] * sk[r];
        pq += s[p] * sq[r];
    }
#pragma unroll
    for (int m = TPR; m < 64; m <<= 1) {
        pk += shfl_xor4(pk, m);
        pq += shfl_xor4(pq, m);
    }
    if (lane < TPR) {
        red[wave][0][cg] = pk;
        red[wave][1][cg] = pq;
    }
    __syncthreads();

    f32x4 P = red[0][0][cg], R = red[0][1][cg];
#pragma unroll
    for (int w = 1; w < Sh::NWAVE; ++w) {
        P += red[w][0][cg];
        R += red[w][1][cg];
    }
    const float b = a.beta[item];
    f32x4 vv = {sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]};
    const f32x4 u = b * (vv - P);
    if (rr == 0) *reinterpret_cast<f32x4 *>(a.o + item * DV + 4 * cg) = R + sqk * u;

#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int r = p * RPP + rr;
        *reinterpret_cast<f32x4 *>(S + r * DV + 4 * cg) = s[p] + sk[r] * u;
    }
}

template <typename Tin, int D>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    using Sh = DecodeShape<D, D>;
    const int64_t items = (int64_t)a.N * a.H;
    hipLaunchKernelGGL((decode_kernel<Tin, D, D>), dim3((unsigned)items), dim3(Sh::NT), 0, stream, a);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_decode_d(int32_t D, const DecodeArgs &a, hipStream_t stream) {
    switch (D) {
    case 16: return launch_decode_t<Tin, 16>(a, stream);
    case 32: return launch_decode_t<Tin, 32>(a, stream);
    case 64: return launch_decode_t<Tin, 64>(a, stream);
    case 128: return launch_decode_t<Tin, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int32_t in_dtype, int32_t Dk, int32_t Dv) {
    return (in_dtype == 0 || in_dtype == 1) && Dk == Dv &&
           (Dk == 16 || Dk == 32 || Dk == 64 || Dk == 128);
}

hipError_t launch_decode(int32_t in_dtype, int32_t Dk, int32_t Dv, const DecodeArgs &a,
                         hipStream_t stream) {
    if (!decode_supported(in_dtype, Dk, Dv)) return hipErrorInvalidValue;
    if (a.N == 0) return hipSuccess;
    return in_dtype == 1 ? launch_decode_d<bf16_t>(Dk, a, stream)
                         : launch_decode_d<float>(Dk, a, stream);
}

}  // namespace kda
