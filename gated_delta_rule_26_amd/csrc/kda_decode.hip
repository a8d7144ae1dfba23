// KDA decode step and short recurrent prefill: L tokens per (sequence, head) on a persistent
// float32 state (L = 1: the decode step).
//
// Per (sequence, head), with the state S (Dk x Dv, rows = key channels) in HBM:
//   S' = Diag(exp(g)) S;  p = S'^T k;  r = S'^T (scale q);  u = beta (v - p)
//   o  = r + (scale q . k) u;  S <- S' + k u^T
// which is one step of S_t = (I - beta k k^T) Diag(exp g) S_{t-1} + beta k v^T followed by
// o_t = S_t^T (scale q): the token-by-token recurrent mode used for incremental decoding
// ([loading page] sections 5 and 6: the recurrent state carried by the decode cache).
//
// The state is read once and written once per call, however many tokens L the call carries
// (the token-by-token "fused_recurrent" mode for short queries, [loading page] section 5):
// one token is HBM-bound (7 flops per 8 bytes); L tokens divide the state traffic by L.
// One workgroup owns one (sequence, head) state. Threads tile the state as rows x float4
// columns, so every wave reads and writes whole contiguous 512-byte rows; each thread keeps
// its Dk*Dv/NT values in registers between the read and the write. The read is non-temporal
// and so is the write: with 1000 steps back to back (each step reads the state the previous
// one has just written) both hints together reach the device's in-place read-modify-write
// rate for 64 KB per workgroup, about 5.6-5.7 TB/s, against about 5.3 TB/s with plain stores.
// (Splitting a state's value columns over four workgroups, exact since column j of the update
// needs only column j of S, measured slower: 128-byte row pieces 512 bytes apart instead of
// contiguous rows.) Both column reductions (p and r) are finished in the same sweep with
// cross-lane shuffles and one LDS exchange between waves, then the rank-1 update is applied
// to the values still in registers.
//
// Fused layer steps (kda_decode_step_fused): the gate from its pre-activation,
// g = -exp(A_log[h]) softplus(x + dt_bias[h, c]); q and k normalised, which only rescales the
// two reductions (p by 1/||k||, r by 1/||q||), q.k, and the rank-1 update; and the output's
// gated RMSNorm over its Dv values, done by the threads that hold them.
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

// MULTI: L = a.L tokens per sequence; otherwise one (the decode step: a compile-time single
// iteration keeps the state out of loop-carried registers). FUSED: the layer steps of a.f
// (otherwise compiled out: the core step carries no branches or registers for them).
template <typename Tin, int DK, int DV, bool MULTI, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int TPR = Sh::TPR, RPP = Sh::RPP, NT = Sh::NT, NPASS = Sh::NPASS;
    static_assert(NT >= DK && NT >= DV, "one staged channel per thread");

    // a token's inputs, double-buffered so that staging token t + 1 never waits for readers of t
    __shared__ float sk[2][DK], sq[2][DK], sa[2][DK];
    __shared__ __attribute__((aligned(16))) float sv[2][DV];
    __shared__ __attribute__((aligned(16))) float sz[2][DV];  // fused output norm: gate pre-activation
    __shared__ __attribute__((aligned(16))) float sw[DV];     // ... and gain
    __shared__ f32x4 red[Sh::NWAVE][2][TPR];
    __shared__ float sqk[2][3];  // scale q.k (normalised when fused), 1/||k||, 1/||q|| (or 1, 1)

    const int tid = threadIdx.x;
    const int64_t item = blockIdx.x;  // n * H + h
    // the sequence and head are needed only for several tokens per call (their rows) and for
    // the fused gate's per-head parameters: one token's row is the item itself
    const int64_t n = MULTI ? item / a.H : 0;
    const int h = MULTI || FUSED ? (int)(item % a.H) : 0;
    float *S = a.state + item * (int64_t)(DK * DV);
    const int cg = tid % TPR, rr = tid / TPR;
    const int lane = tid & 63, wave = tid >> 6;
    const bool fgate = FUSED && a.f.gx, fnorm = FUSED && a.f.og, fqk = FUSED && a.f.norm_qk;
    const float rate = fgate ? expf(a.f.A_log[h]) : 0.f;
    const float gbias = (fgate && tid < DK) ? a.f.dt_bias[h * DK + tid] : 0.f;
    if (fnorm && tid < DV) sw[tid] = a.f.ow[tid];

    // token t of this sequence is row (n * L + t) * H + h of the [N, L, H, D] inputs; the
    // next token's values are loaded into registers while the current one computes
    const int L = MULTI ? a.L : 1;
    auto row = [&](int t) { return MULTI ? (n * L + t) * a.H + h : item; };
    // raw token values, converted when staged: every thread loads (lanes past Dk or Dv repeat a
    // channel), so no branch holds a wait for them
    Tin nk{}, nq{}, nv{}, nz{}, ngx{};
    float ng = 0.f, nb = 0.f, bcur = 0.f;
    auto fetch = [&](int t) {
        const int64_t r = row(t);
        const int ck = tid % DK, cv = tid % DV;
        nb = a.beta[r];
        nk = static_cast<const Tin *>(a.k)[r * DK + ck];
        nq = static_cast<const Tin *>(a.q)[r * DK + ck];
        if (fgate)
            ngx = static_cast<const Tin *>(a.f.gx)[r * DK + ck];
        else
            ng = a.g[r * DK + ck];
        nv = static_cast<const Tin *>(a.v)[r * DV + cv];
        if (fnorm) nz = static_cast<const Tin *>(a.f.og)[r * DV + cv];
    };
    auto stage = [&](int b) {
        bcur = nb;
        if (tid < DK) {
            sk[b][tid] = to_f32(nk);
            sq[b][tid] = a.scale * to_f32(nq);
            sa[b][tid] = __expf(fgate ? -rate * softplus_f(to_f32(ngx) + gbias) : ng);
        }
        if (tid < DV) {
            sv[b][tid] = to_f32(nv);
            if (fnorm) sz[b][tid] = to_f32(nz);
        }
    };

    // the token's few loads go out first and the state's after them: loads complete in issue
    // order, so staging the token (and its barrier) then waits for its own loads only and
    // overlaps the state's, which the sweep waits for
    fetch(0);
    f32x4 s[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
        s[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (p * RPP + rr) * DV + 4 * cg));
    __builtin_amdgcn_sched_barrier(0);  // nothing that waits for the token moves above the state's loads
    for (int t = 0; t < L; ++t) {
        const int b = t & 1;
        stage(b);
        if (t + 1 < L) fetch(t + 1);
        __syncthreads();

        if (wave == 0) {  // scale * (q . k) and the norms, off the critical path of the state sweep
            float acc = 0.f, kk = 0.f, qq = 0.f;
            for (int c = lane; c < DK; c += 64) {
                acc += sq[b][c] * sk[b][c];
                kk += sk[b][c] * sk[b][c];
                qq += sq[b][c] * sq[b][c];
            }
            for (int m = 32; m > 0; m >>= 1) {
                acc += __shfl_xor(acc, m);
                kk += __shfl_xor(kk, m);
                qq += __shfl_xor(qq, m);
            }
            if (lane == 0) {
                // sq holds scale * q, so 1/||q|| = |scale| / ||sq|| (any scale, zero included)
                const float rk = fqk ? rsqrt_or_zero(kk) : 1.f;
                const float rq = fqk ? fabsf(a.scale) * rsqrt_or_zero(qq) : 1.f;
                sqk[b][0] = acc * rk * rq;
                sqk[b][1] = rk;
                sqk[b][2] = rq;
            }
        }

        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int r = p * RPP + rr;
            s[p] *= sa[b][r];
            pk += s[p] * sk[b][r];
            pq += s[p] * sq[b][r];
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
        const float bt = bcur;
        const float rk = FUSED ? sqk[b][1] : 1.f, rq = FUSED ? sqk[b][2] : 1.f;
        const f32x4 vv = *reinterpret_cast<const f32x4 *>(&sv[b][4 * cg]);
        const f32x4 u = bt * (vv - rk * P);
        if (rr == 0) {
            const f32x4 ov = rq * R + sqk[b][0] * u;
            const int64_t oo = row(t) * DV + 4 * cg;
            if (fnorm) {  // gated RMSNorm over the Dv outputs, held by the TPR lanes of row 0
                float ss = ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w;
#pragma unroll
                for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m);
                const float r = rsqrt_or_zero(ss * (1.f / DV) + a.f.oeps);
                const f32x4 z = *reinterpret_cast<const f32x4 *>(&sz[b][4 * cg]);
                const f32x4 w = *reinterpret_cast<const f32x4 *>(sw + 4 * cg);
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = ov[e] * r * w[e] * sigmoid_f(z[e]);
                if (a.f.o_bf16) {
                    const u32x2 packed = {(uint32_t)bf16_bits(y.x) | ((uint32_t)bf16_bits(y.y) << 16),
                                          (uint32_t)bf16_bits(y.z) | ((uint32_t)bf16_bits(y.w) << 16)};
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.o) + oo) = packed;
                } else {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.o) + oo) = y;
                }
            } else {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(a.o) + oo) = ov;
            }
        }

        const f32x4 uk = rk * u;  // the update writes the normalised key: k_raw (u / ||k||)^T
#pragma unroll
        for (int p = 0; p < NPASS; ++p) s[p] += sk[b][p * RPP + rr] * uk;
    }

#pragma unroll
    for (int p = 0; p < NPASS; ++p)
        __builtin_nontemporal_store(s[p], reinterpret_cast<f32x4 *>(S + (p * RPP + rr) * DV + 4 * cg));
}

template <typename Tin, int D>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    using Sh = DecodeShape<D, D>;
    const int64_t items = (int64_t)a.N * a.H;
    // the core step and the core recurrent mode share one arithmetic (no fused steps compiled
    // in), so L tokens in one call give the bits of L successive decode steps
    const bool fused = a.f.gx || a.f.og || a.f.norm_qk;
    if (a.L > 1 && fused)
        hipLaunchKernelGGL((decode_kernel<Tin, D, D, true, true>), dim3((unsigned)items), dim3(Sh::NT), 0, stream, a);
    else if (a.L > 1)
        hipLaunchKernelGGL((decode_kernel<Tin, D, D, true, false>), dim3((unsigned)items), dim3(Sh::NT), 0, stream, a);
    else if (fused)
        hipLaunchKernelGGL((decode_kernel<Tin, D, D, false, true>), dim3((unsigned)items), dim3(Sh::NT), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<Tin, D, D, false, false>), dim3((unsigned)items), dim3(Sh::NT), 0, stream, a);
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
    if (a.N == 0 || a.L == 0) return hipSuccess;
    return in_dtype == 1 ? launch_decode_d<bf16_t>(Dk, a, stream)
                         : launch_decode_d<float>(Dk, a, stream);
}

}  // namespace kda
