// KDA chunked backward pass (gfx950): the gradients of a loss through the chunked prefill,
// i.e. dq, dk, dv, dg, dbeta and dS_init from dL/do and dL/dS_final. Training runs the layer in
// chunk mode only ([loading page] section 5, the mode switch); the forward it differentiates is
// the chunkwise form of [KV-cache page] section 6.
//
// Per chunk of C tokens, with G_i the running sum of g inside the chunk, gC = G_{C-1}, S the
// state entering the chunk and dS' = dL/d(state leaving it), the forward computes
//   A~_ij = sum_c k_i k_j e^{G_i - G_j} (j < i),  M_ij = scale sum_c q_i k_j e^{G_i - G_j} (j <= i)
//   T = (I + Diag(beta) A~)^-1,  W = T Diag(beta) (k e^G),  U~ = T Diag(beta) V
//   U = U~ - W S,  O = (scale q e^G) S + M U,  S' = Diag(e^{gC}) S + (k e^{gC - G})^T U
// and its reverse-mode derivative is, with Qg = scale q e^G, Kd = k e^{gC - G}, Kg = k e^G,
//   dU  = M^T dO + Kd dS'                        dS = Diag(e^{gC}) dS' + Qg^T dO - W^T dU
//   dQg = dO S^T,  dKd = U dS'^T,  dW = -dU S^T,  dM = tril(dO U^T),  d e^{gC} = rowsum(S * dS')
//   dT  = dU (Diag(beta) V)^T + dW (Diag(beta) Kg)^T
//   dv  = Diag(beta) T^T dU,  dKg = Diag(beta) T^T dW,  dA = -strictly_lower(T^T dT T^T)
// plus the pairwise terms of A~ and M (per channel, e^{G_i - G_j} <= 1 for j <= i) and, for g,
// the reverse running sum of dL/dG inside the chunk.
//
// Mapping to the MI355X. Everything is float32 (fp32 matrix cores, v_mfma_f32_16x16x4f32).
// Three launches, each a plain pass over a per-(chunk, head) record in the workspace:
//  1. prep    (one workgroup per chunk and head): G, Qg, Kd, e^{gC}, A~ and M as 16x16 block
//             pairs on the matrix cores (decay split at block boundaries; pair by pair for a
//             block decaying below e^-60), T by column substitution in one wave, W and U~.
//  2. state   the forward state pass (chunks in order: the state entering each chunk, and U)
//             and the reverse one (chunks in reverse: dS' and dU, then dS_init) side by side,
//             per chain and 16 value columns; the reverse pass needs only prep's records.
//  3. grad    (per chunk and head): the products with S, dS', U and dU, then T^T dW, T^T dU
//             and T^T dT T^T (dv, dbeta), then the pair terms of A~ and M on the matrix cores
//             (pair by pair for channels of extremely decaying blocks), then dq, dk and the
//             reverse running sum of dG; the partial gradients never leave the registers.
// Chunks of a packed batch are numbered by slot n + floor(start_n / C) + j (sequence n, chunk j),
// which is unique and below N + ceil(tokens / C), so the records need no host-side lengths.
#include <atomic>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// The records of kda_chunk_bwd_noalloc, for callers that cannot allocate (code under graph
// capture, tight training loops): one copy of this array per device the library runs on,
// held until the process ends. In host code the name stands for a host-side shadow, not for
// device memory: host code uses only the address bwd_scratch() looks up. Calls that overlap
// on one device share it and race.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

namespace {

// Per-(chunk, head) record in the workspace (float offsets; rows are tokens of the chunk).
template <int C, int DK, int DV> struct BRec {
    static constexpr int64_t oG = 0;                  // [C][DK] G (running sum of g)
    static constexpr int64_t oQg = oG + C * DK;       // [C][DK] scale q e^G
    static constexpr int64_t oKd = oQg + C * DK;      // [C][DK] k e^{gC - G}
    static constexpr int64_t oW = oKd + C * DK;       // [C][DK] W
    static constexpr int64_t oU = oW + C * DK;        // [C][DV] U~, then U
    static constexpr int64_t odU = oU + C * DV;       // [C][DV] dU
    static constexpr int64_t oEg = odU + C * DV;      // [DK]    e^{gC}
    static constexpr int64_t oA = oEg + DK;           // [C][C]  A~ (strictly lower), then dA~
    static constexpr int64_t oM = oA + C * C;         // [C][C]  M^T (upper), then dM (lower)
    static constexpr int64_t oT = oM + C * C;         // [C][C]  T
    static constexpr int64_t oKdT = oT + C * C;       // [DK][C] Kd^T
    static constexpr int64_t oWT = oKdT + DK * C;     // [DK][C] W^T
    static constexpr int64_t oQgT = oWT + DK * C;     // [DK][C] Qg^T
    static constexpr int64_t oH = oQgT + DK * C;      // [DK][DV] state entering the chunk
    static constexpr int64_t odH = oH + DK * DV;      // [DK][DV] dL/d(state leaving the chunk)
    static constexpr int64_t FLOATS = (odH + DK * DV + 63) & ~int64_t(63);
};

// Token range [start, end) of sequence n (packed offsets clamped to [0, T]).
__device__ __forceinline__ void seq_range(const BwdArgs &a, int n, int64_t &start, int64_t &end) {
    if (a.cu_seqlens) {
        packed_range(a.cu_seqlens, n, a.seq_len, start, end);
    } else {
        start = (int64_t)n * a.seq_len;
        end = start + a.seq_len;
    }
}

__device__ __forceinline__ int64_t seq_start(const BwdArgs &a, int n) {
    int64_t s, e;
    seq_range(a, n, s, e);
    return s;
}

template <int C> __device__ __forceinline__ int64_t slot_base(const BwdArgs &a, int n) {
    return n + seq_start(a, n) / C;
}

// The chunk of record slot s: its sequence n, first token t0 and valid rows L (false: unused).
template <int C> __device__ bool locate(const BwdArgs &a, int64_t s, int &n, int64_t &t0, int &L) {
    int lo = 0, hi = a.n_seqs - 1;  // the last n with slot_base(n) <= s (strictly increasing)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_base<C>(a, mid) <= s) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    int64_t st, en;
    seq_range(a, n, st, en);
    const int64_t len = en - st;
    const int64_t j = s - slot_base<C>(a, n);
    if (j < 0 || j * C >= len) return false;
    t0 = st + j * C;
    L = (int)(len - j * C < C ? len - j * C : C);
    return true;
}

__device__ __forceinline__ float sum16(float x) {  // over the 16 lanes of a row
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

__device__ __forceinline__ void mma(f32x4 &acc, f32x4 a, f32x4 b) { Mma<float>::mma(acc, a, b); }

// A 16-token block whose decay falls below e^-60 in some channel has diagonal-block factors
// beyond float32's comfortable range; such blocks are summed pair by pair.
constexpr float kExtremeLogDecay = 60.f;
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------------------------------------
// 1. prep
// ------------------------------------------------------------------------------------------
template <typename Tin, int C, int DK, int DV>
__global__ __launch_bounds__(512) void bwd_prep_kernel(BwdArgs a) {
    using R = BRec<C, DK, DV>;
    constexpr int NT = 512;
    constexpr int DX = DK > DV ? DK : DV;
    constexpr int LDK = DK + 4, LDX = DX + 4, LDA = C + 4;
    __shared__ __align__(16) float sK[C * LDK];
    __shared__ __align__(16) float sQ[C * LDX];   // q, then beta k e^G
    __shared__ __align__(16) float sG[C * LDX];   // G, then beta v
    __shared__ __align__(16) float sA[C * LDA];   // A~
    __shared__ __align__(16) float sT[C * LDA];   // T
    __shared__ float sB[C];
    __shared__ int sExt[C / 16];                   // 16-token blocks decaying below e^-60

    const int64_t s = blockIdx.x;
    const int h = blockIdx.y;
    int n, L;
    int64_t t0;
    if (!locate<C>(a, s, n, t0, L)) return;
    float *rec = a.ws + (s * a.H + h) * R::FLOATS;
    const int tid = threadIdx.x;
    const int64_t rsk = (int64_t)a.H * DK, rsv = (int64_t)a.H * DV;

    for (int idx = tid; idx < C * DK / 4; idx += NT) {
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        f32x4 kv = zero4(), qv = zero4(), gv = zero4();
        if (i < L) {
            const int64_t off = (t0 + i) * rsk + (int64_t)h * DK + c;
            kv = load4(static_cast<const Tin *>(a.k) + off);
            qv = load4(static_cast<const Tin *>(a.q) + off);
            gv = load4(a.g + off);
        }
        *reinterpret_cast<f32x4 *>(sK + i * LDK + c) = kv;
        *reinterpret_cast<f32x4 *>(sQ + i * LDX + c) = qv;
        *reinterpret_cast<f32x4 *>(sG + i * LDX + c) = gv;
    }
    if (tid < C) sB[tid] = tid < L ? a.beta[(t0 + tid) * a.H + h] : 0.f;
    if (tid < C / 16) sExt[tid] = 0;
    __syncthreads();
    if (tid < DK) {  // running sum along the chunk, one thread per channel
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            acc += sG[i * LDX + tid];
            sG[i * LDX + tid] = acc;
        }
        rec[R::oEg + tid] = __expf(acc);
#pragma unroll
        for (int b = 0; b < C / 16; ++b)
            if (sG[16 * b * LDX + tid] - sG[(16 * b + 15) * LDX + tid] > kExtremeLogDecay) sExt[b] = 1;
    }
    __syncthreads();
    for (int idx = tid; idx < C * DK / 4; idx += NT) {
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        const f32x4 G = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
        const f32x4 gC = *reinterpret_cast<const f32x4 *>(sG + (C - 1) * LDX + c);
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(sQ + i * LDX + c);
        f32x4 qg, kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qg[e] = a.scale * qv[e] * __expf(G[e]);
            kd[e] = kv[e] * __expf(gC[e] - G[e]);
        }
        *reinterpret_cast<f32x4 *>(rec + R::oG + i * DK + c) = G;
        *reinterpret_cast<f32x4 *>(rec + R::oQg + i * DK + c) = qg;
        *reinterpret_cast<f32x4 *>(rec + R::oKd + i * DK + c) = kd;
    }
    for (int idx = tid; idx < DK * C / 4; idx += NT) {  // the same, transposed ([channel][row])
        const int c = idx / (C / 4), i0 = 4 * (idx % (C / 4));
        f32x4 qg, kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float G = sG[(i0 + e) * LDX + c], gC = sG[(C - 1) * LDX + c];
            qg[e] = a.scale * sQ[(i0 + e) * LDX + c] * __expf(G);
            kd[e] = sK[(i0 + e) * LDK + c] * __expf(gC - G);
        }
        *reinterpret_cast<f32x4 *>(rec + R::oQgT + c * C + i0) = qg;
        *reinterpret_cast<f32x4 *>(rec + R::oKdT + c * C + i0) = kd;
    }
    // A~ and M as 16x16 block pairs (I, J <= I) on the matrix cores, one pair per wave at a time:
    // e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j} with r the last row of block J (both factors
    // <= 1) or, on the diagonal, the block's first row (the second factor at most the block's
    // inverse decay). A diagonal block decaying below e^-60 in some channel is summed pair by
    // pair instead (one exp per pair and channel, exact for any decay).
    {
        const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
        constexpr int IT = C / 16, NPB = IT * (IT + 1) / 2;
        for (int pb = wave; pb < NPB; pb += NT / 64) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= pb) ++I;
            const int J = pb - I * (I + 1) / 2;
            const bool diag = I == J;
            if (diag && sExt[I]) {
                for (int pp = lane; pp < 136; pp += 64) {   // pairs (i, j <= i) of the block
                    int ri = 0;
                    while ((ri + 1) * (ri + 2) / 2 <= pp) ++ri;
                    const int i = 16 * I + ri, j = 16 * I + pp - ri * (ri + 1) / 2;
                    float sa = 0.f, sm = 0.f;
                    for (int c = 0; c < DK; c += 4) {
                        const f32x4 ki = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
                        const f32x4 kj = *reinterpret_cast<const f32x4 *>(sK + j * LDK + c);
                        const f32x4 qi = *reinterpret_cast<const f32x4 *>(sQ + i * LDX + c);
                        const f32x4 Gi = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
                        const f32x4 Gj = *reinterpret_cast<const f32x4 *>(sG + j * LDX + c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float kjE = kj[e] * __expf(Gi[e] - Gj[e]);
                            sa += ki[e] * kjE;
                            sm += qi[e] * kjE;
                        }
                    }
                    const float av = j < i ? sa : 0.f;
                    sA[i * LDA + j] = av;
                    rec[R::oA + i * C + j] = av;
                    rec[R::oM + j * C + i] = a.scale * sm;   // M^T
                }
                for (int pp = lane; pp < 256; pp += 64) {   // the block above its diagonal
                    const int i = 16 * I + (pp >> 4), j = 16 * I + (pp & 15);
                    if (j > i) {
                        sA[i * LDA + j] = 0.f;
                        rec[R::oA + i * C + j] = 0.f;
                        rec[R::oM + j * C + i] = 0.f;
                    }
                }
                continue;
            }
            const int r = diag ? 16 * I : 16 * J + 15;
            f32x4 accA = zero4(), accM = zero4();
#pragma unroll 2
            for (int cs = 0; cs < DK / 16; ++cs) {
                const int c0 = 16 * cs + 4 * q4;
                const f32x4 Gr = *reinterpret_cast<const f32x4 *>(sG + r * LDX + c0);
                const f32x4 ki = *reinterpret_cast<const f32x4 *>(sK + (16 * I + lr) * LDK + c0);
                const f32x4 qi = *reinterpret_cast<const f32x4 *>(sQ + (16 * I + lr) * LDX + c0);
                const f32x4 Gi = *reinterpret_cast<const f32x4 *>(sG + (16 * I + lr) * LDX + c0);
                const f32x4 kj = *reinterpret_cast<const f32x4 *>(sK + (16 * J + lr) * LDK + c0);
                const f32x4 Gj = *reinterpret_cast<const f32x4 *>(sG + (16 * J + lr) * LDX + c0);
                f32x4 Ka, Qa, Kb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float EI = __expf(Gi[e] - Gr[e]);
                    Ka[e] = ki[e] * EI;
                    Qa[e] = qi[e] * EI;
                    Kb[e] = kj[e] * __expf(Gr[e] - Gj[e]);
                }
                mma(accA, Ka, Kb);
                mma(accM, Qa, Kb);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * q4 + e, j = 16 * J + lr;
                const float av = j < i ? accA[e] : 0.f;
                sA[i * LDA + j] = av;
                rec[R::oA + i * C + j] = av;
                rec[R::oM + j * C + i] = j <= i ? a.scale * accM[e] : 0.f;   // M^T
            }
        }
    }
    for (int p = tid; p < C * C; p += NT) {   // blocks above the diagonal
        const int i = p / C, j = p % C;
        if ((j >> 4) > (i >> 4)) {
            sA[i * LDA + j] = 0.f;
            rec[R::oA + p] = 0.f;
            rec[R::oM + j * C + i] = 0.f;
        }
    }
    __syncthreads();
    if (tid < 64) {
        // T = (I + Diag(beta) A~)^-1 by forward substitution, lane = column
        const int col = tid;
        float x[C];
#pragma unroll
        for (int i = 0; i < C; ++i) x[i] = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < (i + 3) / 4 * 4; m += 4) {
                const f32x4 ar = *reinterpret_cast<const f32x4 *>(sA + i * LDA + m);
                acc += ar[0] * x[m] + ar[1] * x[m + 1] + ar[2] * x[m + 2] + ar[3] * x[m + 3];
            }
            x[i] = (i == col ? 1.f : 0.f) - sB[i] * acc;
        }
        if (col < C) {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                sT[i * LDA + col] = x[i];
                rec[R::oT + i * C + col] = x[i];
            }
        }
    } else {
        for (int idx = tid - 64; idx < C * DK / 4; idx += NT - 64) {  // beta k e^G over q
            const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
            const f32x4 G = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = sB[i] * kv[e] * __expf(G[e]);
            *reinterpret_cast<f32x4 *>(sQ + i * LDX + c) = r;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * DV / 4; idx += NT) {  // beta v over G
        const int i = idx / (DV / 4), c = 4 * (idx % (DV / 4));
        f32x4 vv = zero4();
        if (i < L) vv = load4(static_cast<const Tin *>(a.v) + (t0 + i) * rsv + (int64_t)h * DV + c);
        *reinterpret_cast<f32x4 *>(sG + i * LDX + c) = vv * sB[i];
    }
    __syncthreads();
    // W = T (beta k e^G), U~ = T (beta v): 16 x 16 tiles over the waves
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
    constexpr int TW = (C / 16) * (DK / 16), TU = (C / 16) * (DV / 16);
    for (int t = wave; t < TW + TU; t += NT / 64) {
        const bool isW = t < TW;
        const int tt = isW ? t : t - TW;
        const int nct = isW ? DK / 16 : DV / 16;
        const int it = tt / nct, nt = tt % nct;
        const float *X = isW ? sQ : sG;
        f32x4 acc = zero4();
        for (int ms = 0; ms <= it; ++ms) {
            const int m0 = 16 * ms + 4 * q4;
            const f32x4 A = *reinterpret_cast<const f32x4 *>(sT + (16 * it + lr) * LDA + m0);
            f32x4 B;
#pragma unroll
            for (int e = 0; e < 4; ++e) B[e] = X[(m0 + e) * LDX + 16 * nt + lr];
            mma(acc, A, B);
        }
        float *dst = rec + (isW ? R::oW : R::oU);
        const int ld = isW ? DK : DV;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(16 * it + 4 * q4 + e) * ld + 16 * nt + lr] = acc[e];
        if (isW) *reinterpret_cast<f32x4 *>(rec + R::oWT + (16 * nt + lr) * C + 16 * it + 4 * q4) = acc;
    }
}

// ------------------------------------------------------------------------------------------
// 2. forward state pass: one workgroup per (chain, 16 value columns); wave w holds the 16x16
//    state tiles of its key-channel tiles in accumulator registers. Every operand is one
//    16-byte load per lane, and the next chunk's operands are loaded while this one computes.
// ------------------------------------------------------------------------------------------
template <int C, int DK, int DV> struct StatePass {
    static constexpr int KT = DK / 16;
    static constexpr int NW = KT < 4 ? KT : 4;
    static constexpr int KTW = KT / NW;
    static constexpr int IT = C / 16;
    static constexpr int NOWN = IT >= NW ? IT / NW : 1;   // row tiles whose U a wave owns
    static_assert(KT % NW == 0, "key tiles spread evenly");
    static_assert(IT % NW == 0 || IT == 1, "row tiles spread evenly");
};

template <int C, int DK, int DV> struct FwdOps {
    using P = StatePass<C, DK, DV>;
    f32x4 W[P::IT][P::KTW];     // W rows 16 it + lr, channels 16 kt + 4 q4 ..
    f32x4 KdT[P::KTW][P::IT];   // Kd^T rows 16 kt + lr, tokens 16 it + 4 q4 ..
    f32x4 eg[P::KTW];           // e^{gC} of channels 16 kt + 4 q4 ..
    f32x4 Ut[P::NOWN];          // U~ of the owned row tiles, accumulator layout
};

template <int C, int DK, int DV>
__device__ __forceinline__ void fwd_state_pass(const BwdArgs &a, int chain, int vb) {
    using R = BRec<C, DK, DV>;
    using P = StatePass<C, DK, DV>;
    constexpr int IT = P::IT, KTW = P::KTW, NW = P::NW, NOWN = P::NOWN;
    __shared__ f32x4 sPart[NW][IT][64];
    const int n = chain / a.H, h = chain % a.H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, q4 = lane >> 4;
    int64_t st, en;
    seq_range(a, n, st, en);
    const int64_t len = en - st;
    const int nch = (int)((len + C - 1) / C);
    const int64_t base = slot_base<C>(a, n);
    const int col = 16 * vb + lr;
    auto rec_of = [&](int j) { return a.ws + ((base + j) * a.H + h) * R::FLOATS; };
    auto own = [&](int o) { return wave + NW * o; };
    auto load = [&](const float *rec, FwdOps<C, DK, DV> &o) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                o.W[it][kk] = *reinterpret_cast<const f32x4 *>(rec + R::oW + (16 * it + lr) * DK + 16 * kt + 4 * q4);
                o.KdT[kk][it] = *reinterpret_cast<const f32x4 *>(rec + R::oKdT + (16 * kt + lr) * C + 16 * it + 4 * q4);
            }
            o.eg[kk] = *reinterpret_cast<const f32x4 *>(rec + R::oEg + 16 * kt + 4 * q4);
        }
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o.Ut[ow][e] = own(ow) < IT ? rec[R::oU + (16 * own(ow) + 4 * q4 + e) * DV + col] : 0.f;
    };

    f32x4 S[KTW];
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
        const int kt = wave * KTW + kk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[kk][e] = a.s0 ? a.s0[(((int64_t)n * a.H + h) * DK + 16 * kt + 4 * q4 + e) * DV + col] : 0.f;
    }
    // one chunk with operands `cur`, loading the next chunk's into `nxt`; the loop below
    // alternates two operand sets, so the loads stay in flight across the chunk
    auto step = [&](int j, FwdOps<C, DK, DV> &cur, FwdOps<C, DK, DV> &nxt) {
        float *rec = rec_of(j);
        if (j + 1 < nch) load(rec_of(j + 1), nxt);
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[R::oH + (16 * kt + 4 * q4 + e) * DV + col] = S[kk][e];
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) mma(acc, cur.W[it][kk], S[kk]);
            f32x4 part = -acc;
#pragma unroll
            for (int ow = 0; ow < NOWN; ++ow)
                if (own(ow) == it) part += cur.Ut[ow];   // the owner of row tile it adds U~
            sPart[wave][it][lane] = part;
        }
        __syncthreads();
        f32x4 U[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            U[it] = sPart[0][it][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) U[it] += sPart[w][it][lane];
        }
        __syncthreads();
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow)
#pragma unroll
            for (int it = 0; it < IT; ++it)
                if (own(ow) == it) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rec[R::oU + (16 * it + 4 * q4 + e) * DV + col] = U[it][e];
                }
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            S[kk] *= cur.eg[kk];
#pragma unroll
            for (int it = 0; it < IT; ++it) mma(S[kk], cur.KdT[kk][it], U[it]);
        }
    };
    FwdOps<C, DK, DV> o0, o1;
    if (nch > 0) load(rec_of(0), o0);
    int j = 0;
    for (; j + 1 < nch; j += 2) {
        step(j, o0, o1);
        step(j + 1, o1, o0);
    }
    if (j < nch) step(j, o0, o1);
}

// ------------------------------------------------------------------------------------------
// 3. reverse state pass: dS held like S above, chunks in reverse order; the next chunk's Kd,
//    M^T, e^{gC} and dO are loaded while this one computes.
// ------------------------------------------------------------------------------------------
template <int C, int DK, int DV> struct RevOps {
    using P = StatePass<C, DK, DV>;
    f32x4 Kd[P::IT][P::KTW];    // Kd rows 16 it + lr, channels 16 kt + 4 q4 ..
    f32x4 MT[P::NOWN][P::IT];   // M^T rows of the owned tiles, tokens 16 ms + 4 q4 ..
    f32x4 eg[P::KTW];
    f32x4 dO[P::IT];            // dO rows 16 ms + 4 q4 + e, column col (zero past the end)
};

template <int C, int DK, int DV>
__device__ __forceinline__ void rev_state_pass(const BwdArgs &a, int chain, int vb) {
    using R = BRec<C, DK, DV>;
    using P = StatePass<C, DK, DV>;
    constexpr int IT = P::IT, KTW = P::KTW, NW = P::NW, NOWN = P::NOWN;
    __shared__ f32x4 sPart[NW][IT][64];
    const int n = chain / a.H, h = chain % a.H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, q4 = lane >> 4;
    int64_t st, en;
    seq_range(a, n, st, en);
    const int64_t len = en - st;
    const int nch = (int)((len + C - 1) / C);
    const int64_t base = slot_base<C>(a, n);
    const int col = 16 * vb + lr;
    const int64_t sbase = ((int64_t)n * a.H + h) * DK;
    const int64_t rsv = (int64_t)a.H * DV;
    auto rec_of = [&](int j) { return a.ws + ((base + j) * a.H + h) * R::FLOATS; };
    auto own = [&](int o) { return wave + NW * o; };
    auto load = [&](int j, RevOps<C, DK, DV> &o) {
        const float *rec = rec_of(j);
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int it = 0; it < IT; ++it)
                o.Kd[it][kk] = *reinterpret_cast<const f32x4 *>(rec + R::oKd + (16 * it + lr) * DK + 16 * kt + 4 * q4);
            o.eg[kk] = *reinterpret_cast<const f32x4 *>(rec + R::oEg + 16 * kt + 4 * q4);
        }
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow)
#pragma unroll
            for (int ms = 0; ms < IT; ++ms)
                o.MT[ow][ms] = own(ow) < IT && ms >= own(ow)   // M[m][i] = 0 for m < i
                    ? *reinterpret_cast<const f32x4 *>(rec + R::oM + (16 * own(ow) + lr) * C + 16 * ms + 4 * q4)
                    : zero4();
        const int64_t t0 = st + (int64_t)j * C;
        const int L = (int)(len - (int64_t)j * C < C ? len - (int64_t)j * C : C);
        const float *dorow = a.dout + (t0 + 4 * q4) * rsv + (int64_t)h * DV + col;
#pragma unroll
        for (int ms = 0; ms < IT; ++ms)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o.dO[ms][e] = 16 * ms + 4 * q4 + e < L ? dorow[(int64_t)(16 * ms + e) * rsv] : 0.f;
    };

    f32x4 dS[KTW];
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
        const int kt = wave * KTW + kk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[kk][e] = a.dsT ? a.dsT[(sbase + 16 * kt + 4 * q4 + e) * DV + col] : 0.f;
    }
    auto step = [&](int j, RevOps<C, DK, DV> &cur, RevOps<C, DK, DV> &nxt) {
        float *rec = rec_of(j);
        if (j > 0) load(j - 1, nxt);
        // Qg^T and W^T are needed only after the exchange below: loaded here, not a chunk ahead
        // (a third prefetched set costs more in register moves than it saves)
        f32x4 QgT[KTW][IT], WT[KTW][IT];
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                QgT[kk][it] = *reinterpret_cast<const f32x4 *>(rec + R::oQgT + (16 * kt + lr) * C + 16 * it + 4 * q4);
                WT[kk][it] = -*reinterpret_cast<const f32x4 *>(rec + R::oWT + (16 * kt + lr) * C + 16 * it + 4 * q4);
            }
        }
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[R::odH + (16 * kt + 4 * q4 + e) * DV + col] = dS[kk][e];
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) mma(acc, cur.Kd[it][kk], dS[kk]);
#pragma unroll
            for (int ow = 0; ow < NOWN; ++ow)
                if (own(ow) == it) {   // M^T dO for the owned row tile
#pragma unroll
                    for (int ms = 0; ms < IT; ++ms)
                        if (ms >= it) mma(acc, cur.MT[ow][ms], cur.dO[ms]);
                }
            sPart[wave][it][lane] = acc;
        }
        __syncthreads();
        f32x4 dU[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            dU[it] = sPart[0][it][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) dU[it] += sPart[w][it][lane];
        }
        __syncthreads();
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow)
#pragma unroll
            for (int it = 0; it < IT; ++it)
                if (own(ow) == it) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rec[R::odU + (16 * it + 4 * q4 + e) * DV + col] = dU[it][e];
                }
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            dS[kk] *= cur.eg[kk];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                mma(dS[kk], QgT[kk][it], cur.dO[it]);
                mma(dS[kk], WT[kk][it], dU[it]);
            }
        }
    };
    RevOps<C, DK, DV> o0, o1;
    if (nch > 0) load(nch - 1, o0);
    int j = nch - 1;
    for (; j >= 1; j -= 2) {
        step(j, o0, o1);
        step(j - 1, o1, o0);
    }
    if (j == 0) step(0, o0, o1);
    if (a.ds0) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
#pragma unroll
            for (int e = 0; e < 4; ++e) a.ds0[(sbase + 16 * kt + 4 * q4 + e) * DV + col] = dS[kk][e];
        }
    }
}

// The two state passes depend only on prep's records (and dL/do), not on each other: one
// launch runs both, the forward chains in grid layer z = 0 and the reverse ones in z = 1.
template <int C, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_state_kernel(BwdArgs a) {
    if (blockIdx.z == 0) fwd_state_pass<C, DK, DV>(a, blockIdx.x, blockIdx.y);
    else rev_state_pass<C, DK, DV>(a, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------------------------------
// 4. grad: one workgroup of 8 waves per (chunk, head). First the products with S, dS', U and
//    dU, then T^T dW, T^T dU and T^T dT T^T (dv, dbeta, partial dq, dk, dG, and dA~, dM kept in
//    LDS), then the pair terms of A~ and M (below), then dq, dk and the reverse running sum of
//    dG. Wave w holds key channels 16 w .. 16 w + 15; lane (lr, q4) holds rows 16 X + 4 q4 + e
//    of channel 16 w + lr throughout, so the partial gradients stay in registers.
// ------------------------------------------------------------------------------------------
template <typename Tin, int C, int DK, int DV>
__global__ __launch_bounds__(512) void bwd_grad_kernel(BwdArgs a) {
    using R = BRec<C, DK, DV>;
    constexpr int NT = 512, NWV = 8, IT = C / 16, KT = DK / 16, VT = DV / 16;
    constexpr int NLT = IT * (IT + 1) / 2;  // lower-triangle 16x16 tiles (it >= mt)
    constexpr int LDK = DK + 4, LDA = C + 4, LDV = DV + 4;
    constexpr int NSRC = KT + VT + IT;      // dbeta partial sums, one row per source
    static_assert(KT <= NWV && VT <= NWV, "one key / value column tile per wave");
    constexpr int LDG = DK + 1;
    // the pair-term phase's arrays, over dO / U / T / dT / X once those are done
    constexpr int NG2 = 2 * IT * DK + KT * 768 + C * LDG;
    constexpr int NOU0 = 2 * C * LDV > 3 * C * LDA ? 2 * C * LDV : 3 * C * LDA;
    constexpr int NOU = NOU0 > NG2 ? NOU0 : NG2;
    // dU, and dO then U, staged once for all waves; T, dT and T^T dT later take dO's and U's space
    __shared__ __align__(16) float sdU[C * LDV];
    __shared__ __align__(16) float sOU[NOU];
    __shared__ __align__(16) float sW[C * LDK];   // dW, then dA~ ([C][LDA])
    __shared__ __align__(16) float sdM[C * LDA];  // dM (lower, with the diagonal)
    __shared__ float sDb[NSRC][C];
    float *sdO = sOU, *sU = sOU + C * LDV;
    float *sT = sOU, *sdT = sOU + C * LDA, *sX = sOU + 2 * C * LDA;
    float *sdA = sW;
    float *sGs = sOU, *sGe = sOU + IT * DK, *sBlk = sOU + 2 * IT * DK, *sDG = sBlk + KT * 768;
    static_assert(C * LDA <= C * LDK, "dA~ fits over dW");

    const int64_t s = blockIdx.x;
    const int h = blockIdx.y;
    int n, L;
    int64_t t0;
    if (!locate<C>(a, s, n, t0, L)) return;
    float *rec = a.ws + (s * a.H + h) * R::FLOATS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
    const int64_t rsk = (int64_t)a.H * DK, rsv = (int64_t)a.H * DV;
    const Tin *kin = static_cast<const Tin *>(a.k);
    const Tin *vin = static_cast<const Tin *>(a.v);
    auto tile_of = [](int p, int &it, int &mt) {  // p-th lower tile, row-major
        it = 0;
        while ((it + 1) * (it + 2) / 2 <= p) ++it;
        mt = p - it * (it + 1) / 2;
    };
    auto beta_of = [&](int i) { return i < L ? a.beta[(t0 + i) * a.H + h] : 0.f; };

    for (int idx = tid; idx < C * DV / 4; idx += NT) {
        const int i = idx / (DV / 4), j = 4 * (idx % (DV / 4));
        f32x4 dOv = zero4();
        if (i < L) dOv = *reinterpret_cast<const f32x4 *>(a.dout + (t0 + i) * rsv + (int64_t)h * DV + j);
        *reinterpret_cast<f32x4 *>(sdO + i * LDV + j) = dOv;
        *reinterpret_cast<f32x4 *>(sU + i * LDV + j) = *reinterpret_cast<const f32x4 *>(rec + R::oU + i * DV + j);
        *reinterpret_cast<f32x4 *>(sdU + i * LDV + j) = *reinterpret_cast<const f32x4 *>(rec + R::odU + i * DV + j);
    }
    for (int idx = tid; idx < NSRC * C; idx += NT) (&sDb[0][0])[idx] = 0.f;
    // this wave's rows of S and dS' (key tile ct = wave): the B fragments below
    const int ct = wave;
    f32x4 hB[VT], dhB[VT];
    if (ct < KT) {
#pragma unroll
        for (int js = 0; js < VT; ++js) {
            hB[js] = *reinterpret_cast<const f32x4 *>(rec + R::oH + (16 * ct + lr) * DV + 16 * js + 4 * q4);
            dhB[js] = *reinterpret_cast<const f32x4 *>(rec + R::odH + (16 * ct + lr) * DV + 16 * js + 4 * q4);
        }
    }
    __syncthreads();

    // dQg = dO S^T, dKd = U dS'^T, dW = -dU S^T for key tile ct; d e^{gC} = rowsum(S * dS')
    f32x4 dq_p[IT], dk_p[IT], dG_p[IT];
    if (ct < KT) {
        f32x4 aQ[IT], aK[IT], aW[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) aQ[it] = aK[it] = aW[it] = zero4();
        float dgc = 0.f;
#pragma unroll
        for (int js = 0; js < VT; ++js) {
            const int j0 = 16 * js + 4 * q4;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int i = 16 * it + lr;
                mma(aQ[it], *reinterpret_cast<const f32x4 *>(sdO + i * LDV + j0), hB[js]);
                mma(aK[it], *reinterpret_cast<const f32x4 *>(sU + i * LDV + j0), dhB[js]);
                mma(aW[it], *reinterpret_cast<const f32x4 *>(sdU + i * LDV + j0), hB[js]);
            }
            dgc += hB[js][0] * dhB[js][0] + hB[js][1] * dhB[js][1] + hB[js][2] * dhB[js][2] + hB[js][3] * dhB[js][3];
        }
        const int c = 16 * ct + lr;
        const float gC = rec[R::oG + (C - 1) * DK + c];
        float cs = 0.f;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * q4 + e;
                const float G = rec[R::oG + i * DK + c], Qg = rec[R::oQg + i * DK + c];
                const float Kd = rec[R::oKd + i * DK + c];
                sW[i * LDK + c] = -aW[it][e];
                dq_p[it][e] = a.scale * __expf(G) * aQ[it][e];
                dk_p[it][e] = __expf(gC - G) * aK[it][e];
                dG_p[it][e] = Qg * aQ[it][e] - Kd * aK[it][e];
                cs += Kd * aK[it][e];
            }
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        dgc += __shfl_xor(dgc, 16);
        dgc += __shfl_xor(dgc, 32);
        // gC is G of the last valid row (g is zero past it): its gradient goes to row L - 1
        const float term = rec[R::oEg + c] * dgc + cs;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (16 * it + 4 * q4 + e == L - 1) dG_p[it][e] += term;
    }
    // dM = tril(dO U^T), written over M
    for (int p = wave; p < NLT; p += NWV) {
        int it, mt;
        tile_of(p, it, mt);
        f32x4 acc = zero4();
#pragma unroll
        for (int js = 0; js < VT; ++js) {
            const int j0 = 16 * js + 4 * q4;
            mma(acc, *reinterpret_cast<const f32x4 *>(sdO + (16 * it + lr) * LDV + j0),
                *reinterpret_cast<const f32x4 *>(sU + (16 * mt + lr) * LDV + j0));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * it + 4 * q4 + e, m = 16 * mt + lr;
            sdM[r * LDA + m] = m <= r ? acc[e] : 0.f;
        }
    }
    __syncthreads();  // dO and U no longer read: T, dT, X take their space; sW complete
    for (int idx = tid; idx < C * C / 4; idx += NT) {
        const int i = idx / (C / 4), m = 4 * (idx % (C / 4));
        *reinterpret_cast<f32x4 *>(sT + i * LDA + m) = *reinterpret_cast<const f32x4 *>(rec + R::oT + i * C + m);
    }
    for (int p = tid; p < C * C; p += NT) {  // dT above the diagonal tiles is never formed
        const int i = p / C, m = p % C;
        if ((m >> 4) > (i >> 4)) sdT[i * LDA + m] = 0.f;
    }
    __syncthreads();

    // dT = dU (beta v)^T + dW (beta k e^G)^T, lower tiles
    for (int p = wave; p < NLT; p += NWV) {
        int it, mt;
        tile_of(p, it, mt);
        const int m = 16 * mt + lr;
        const float bm = beta_of(m);
        f32x4 acc = zero4();
        for (int js = 0; js < VT; ++js) {
            const int j0 = 16 * js + 4 * q4;
            f32x4 vb = zero4();
            if (m < L) vb = load4(vin + (t0 + m) * rsv + (int64_t)h * DV + j0) * bm;
            mma(acc, *reinterpret_cast<const f32x4 *>(sdU + (16 * it + lr) * LDV + j0), vb);
        }
        for (int cs = 0; cs < KT; ++cs) {
            const int c0 = 16 * cs + 4 * q4;
            f32x4 kb = zero4();
            if (m < L) {
                const f32x4 kv = load4(kin + (t0 + m) * rsk + (int64_t)h * DK + c0);
                const f32x4 G = *reinterpret_cast<const f32x4 *>(rec + R::oG + m * DK + c0);
#pragma unroll
                for (int e = 0; e < 4; ++e) kb[e] = bm * kv[e] * __expf(G[e]);
            }
            mma(acc, *reinterpret_cast<const f32x4 *>(sW + (16 * it + lr) * LDK + c0), kb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sdT[(16 * it + 4 * q4 + e) * LDA + m] = acc[e];
    }
    // dKg = Diag(beta) T^T dW for key tile ct (T[m][i] = 0 for m < i)
    if (ct < KT) {
        const int c = 16 * ct + lr;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 acc = zero4();
            for (int ms = it; ms < IT; ++ms) {
                f32x4 A, B;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 16 * ms + 4 * q4 + e;
                    A[e] = sT[m * LDA + 16 * it + lr];
                    B[e] = sW[m * LDK + c];
                }
                mma(acc, A, B);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * q4 + e;
                const float bi = beta_of(i);
                const float G = rec[R::oG + i * DK + c];
                const float eG = __expf(G);
                const float kv = i < L ? to_f32(kin[(t0 + i) * rsk + (int64_t)h * DK + c]) : 0.f;
                const float dKg = bi * acc[e];
                dk_p[it][e] += eG * dKg;
                dG_p[it][e] += kv * eG * dKg;
                const float rs = sum16(acc[e] * kv * eG);
                if (lr == 0) sDb[ct][i] = rs;
            }
        }
    }
    // dv = Diag(beta) T^T dU for value tile vt = wave
    if (wave < VT) {
        const int vt = wave, j = 16 * vt + lr;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 acc = zero4();
            for (int ms = it; ms < IT; ++ms) {
                f32x4 A, B;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 16 * ms + 4 * q4 + e;
                    A[e] = sT[m * LDA + 16 * it + lr];
                    B[e] = sdU[m * LDV + j];
                }
                mma(acc, A, B);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * q4 + e;
                const float vv = i < L ? to_f32(vin[(t0 + i) * rsv + (int64_t)h * DV + j]) : 0.f;
                const float rs = sum16(acc[e] * vv);
                if (lr == 0) sDb[KT + vt][i] = rs;
                if (i < L) a.dv[(t0 + i) * rsv + (int64_t)h * DV + j] = beta_of(i) * acc[e];
            }
        }
    }
    __syncthreads();  // sdT complete
    // X = T^T dT (lower tiles suffice)
    for (int p = wave; p < NLT; p += NWV) {
        int it, lt;
        tile_of(p, it, lt);
        f32x4 acc = zero4();
        for (int ms = it; ms < IT; ++ms) {
            f32x4 A, B;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * ms + 4 * q4 + e;
                A[e] = sT[m * LDA + 16 * it + lr];
                B[e] = sdT[m * LDA + 16 * lt + lr];
            }
            mma(acc, A, B);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sX[(16 * it + 4 * q4 + e) * LDA + 16 * lt + lr] = acc[e];
    }
    __syncthreads();
    // dA = -strictly_lower(X T^T); dbeta += rowsum(dA A~); dA~ = Diag(beta) dA over A~
    for (int p = wave; p < NLT; p += NWV) {
        int it, jt;
        tile_of(p, it, jt);
        f32x4 acc = zero4();
        for (int ls = 0; ls <= jt; ++ls) {
            const f32x4 A = *reinterpret_cast<const f32x4 *>(sX + (16 * it + lr) * LDA + 16 * ls + 4 * q4);
            const f32x4 B = *reinterpret_cast<const f32x4 *>(sT + (16 * jt + lr) * LDA + 16 * ls + 4 * q4);
            mma(acc, A, B);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * q4 + e, j = 16 * jt + lr;
            const float dA = j < i ? -acc[e] : 0.f;
            const float At = rec[R::oA + i * C + j];
            const float rs = sum16(dA * At);
            if (lr == 0) sDb[KT + VT + jt][i] = rs;
            sdA[i * LDA + j] = beta_of(i) * dA;
        }
    }
    // the tiles above the diagonal of dA~ (in dW's space) are read by no block pair below
    __syncthreads();  // dA~ complete; T, dT and X no longer read
    if (tid < L) {
        float db = 0.f;
#pragma unroll
        for (int r = 0; r < NSRC; ++r) db += sDb[r][tid];
        a.dbeta[(t0 + tid) * a.H + h] = db;
    }

    // ---- the pair terms of A~ and M on the matrix cores. For the block pair (I, J), J <= I,
    // e^{G_i - G_j} = e^{G_i - G_r} e^{G_r - G_j} with r the last row of block J (J < I: both
    // factors <= 1) or the first row of block I (diagonal: the second factor is at most the
    // block's inverse decay). A channel whose diagonal block decays below e^-60 takes that
    // block pair by pair instead (exact for any decay).
    //   dKa = dA~ Kb,  dQa = scale dM Kb,  dKb = dA~^T Ka + scale dM^T Qa
    //   dk += dKa e^{G_i - G_r} + dKb e^{G_r - G_j},  dq += dQa e^{G_i - G_r}
    //   dG_i += Ka dKa + Qa dQa,  dG_j -= Kb dKb
    for (int idx = tid; idx < IT * DK; idx += NT) {
        const int b = idx / DK, cc = idx % DK;
        sGs[b * DK + cc] = rec[R::oG + (16 * b) * DK + cc];
        sGe[b * DK + cc] = rec[R::oG + (16 * b + 15) * DK + cc];
    }
    __syncthreads();
    const float scale = a.scale;
    if (ct < KT) {
        const int c = 16 * ct + lr;
        // this lane's rows of k, q, G (zero past the sequence end; G is constant there). Row
        // 16 X + 4 q4 + e of the token arrays is at lane_off + (16 X + e) * rsk: one per-lane
        // offset plus a uniform one, so no per-row address stays live.
        const int64_t lane_off = (t0 + 4 * q4) * rsk + (int64_t)h * DK + c;
        const Tin *kl = kin + lane_off;
        const Tin *ql = static_cast<const Tin *>(a.q) + lane_off;
        float kr[IT][4], qr[IT][4], Gr[IT][4];
#pragma unroll
        for (int X = 0; X < IT; ++X)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * X + 4 * q4 + e;
                const int64_t ro = (int64_t)(16 * X + e) * rsk;
                kr[X][e] = i < L ? to_f32(kl[ro]) : 0.f;
                qr[X][e] = i < L ? to_f32(ql[ro]) : 0.f;
                Gr[X][e] = rec[R::oG + i * DK + c];
            }
        float dq[IT][4], dk[IT][4], dG[IT][4];
#pragma unroll
        for (int X = 0; X < IT; ++X)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dq[X][e] = dq_p[X][e];
                dk[X][e] = dk_p[X][e];
                dG[X][e] = dG_p[X][e];
            }
#pragma unroll
        for (int I = 0; I < IT; ++I) {
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const bool diag = J == I;
                const float Gref = diag ? sGs[I * DK + c] : sGe[J * DK + c];
                // a channel whose diagonal block decays below e^-60 is done pair by pair below;
                // zero factors drop its block-pair terms (and keep its MFMA columns finite)
                const bool ext = diag && (sGs[I * DK + c] - sGe[I * DK + c] > kExtremeLogDecay);
                f32x4 Ka, Qa, Kb, EI, EJ;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    EI[e] = ext ? 0.f : __expf(Gr[I][e] - Gref);          // <= 1
                    EJ[e] = ext ? 0.f : __expf(Gref - Gr[J][e]);          // <= 1 off the diagonal
                    Ka[e] = kr[I][e] * EI[e];
                    Qa[e] = qr[I][e] * EI[e];
                    Kb[e] = kr[J][e] * EJ[e];
                }
                f32x4 aKa = zero4(), aQa = zero4(), aKb = zero4();
                {
                    const f32x4 Ar = *reinterpret_cast<const f32x4 *>(sdA + (16 * I + lr) * LDA + 16 * J + 4 * q4);
                    const f32x4 Mr = *reinterpret_cast<const f32x4 *>(sdM + (16 * I + lr) * LDA + 16 * J + 4 * q4);
                    mma(aKa, Ar, Kb);
                    mma(aQa, Mr * scale, Kb);
                    f32x4 Ac, Mc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Ac[e] = sdA[(16 * I + 4 * q4 + e) * LDA + 16 * J + lr];
                        Mc[e] = sdM[(16 * I + 4 * q4 + e) * LDA + 16 * J + lr] * scale;
                    }
                    mma(aKb, Ac, Ka);
                    mma(aKb, Mc, Qa);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dk[I][e] += aKa[e] * EI[e];
                    dq[I][e] += aQa[e] * EI[e];
                    dk[J][e] += aKb[e] * EJ[e];
                    dG[I][e] += Ka[e] * aKa[e] + Qa[e] * aQa[e];
                    dG[J][e] -= Kb[e] * aKb[e];
                }
                if (diag && __any(ext)) {
                    // pair by pair for the channels of an extreme block: the block's rows of this
                    // wave's channels go through LDS ([k, q, G][row][channel])
                    float *blk = sBlk + ct * 768;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * q4 + e;
                        blk[(0 * 16 + r) * 16 + lr] = kr[I][e];
                        blk[(1 * 16 + r) * 16 + lr] = qr[I][e];
                        blk[(2 * 16 + r) * 16 + lr] = Gr[I][e];
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    if (ext) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int ri = 4 * q4 + e, i = 16 * I + ri;
                            const float ki = kr[I][e], qi = qr[I][e], Gi = Gr[I][e];
                            float pq = 0.f, pk = 0.f, pg = 0.f;
#pragma unroll 1
                            for (int r = 0; r < 16; ++r) {
                                const int j = 16 * I + r;
                                const float kj = blk[r * 16 + lr], qj = blk[(16 + r) * 16 + lr];
                                const float Gj = blk[(32 + r) * 16 + lr];
                                if (r <= ri) {   // as the row: pairs (i, j <= i)
                                    const float E = __expf(Gi - Gj);
                                    const float dAij = sdA[i * LDA + j], dMij = scale * sdM[i * LDA + j];
                                    pq += dMij * kj * E;
                                    pk += dAij * kj * E;
                                    pg += (dAij * ki + dMij * qi) * kj * E;
                                }
                                if (r >= ri) {   // as the column: pairs (j >= i, i)
                                    const float E = __expf(Gj - Gi);
                                    const float z = (sdA[j * LDA + i] * kj + scale * sdM[j * LDA + i] * qj) * E;
                                    pk += z;
                                    pg -= z * ki;
                                }
                            }
                            dq[I][e] += pq;
                            dk[I][e] += pk;
                            dG[I][e] += pg;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // one block pair at a time (register pressure)
            }
        }
        // dq and dk are complete; dG goes to LDS for the running sum
#pragma unroll
        for (int X = 0; X < IT; ++X)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * X + 4 * q4 + e;
                if (i < L) {
                    const int64_t o = lane_off + (int64_t)(16 * X + e) * rsk;
                    a.dq[o] = dq[X][e];
                    a.dk[o] = dk[X][e];
                }
                sDG[i * LDG + c] = dG[X][e];
            }
    }
    __syncthreads();
    if (tid < DK) {
        float cum = 0.f;
        for (int i = L - 1; i >= 0; --i) {
            cum += sDG[i * LDG + tid];
            a.dg[(t0 + i) * rsk + (int64_t)h * DK + tid] = cum;
        }
    }
}

template <typename Tin, int C, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
    using P = StatePass<C, DK, DV>;
    const dim3 gs((unsigned)a.nslots, (unsigned)a.H);
    hipLaunchKernelGGL((bwd_prep_kernel<Tin, C, DK, DV>), gs, dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gc((unsigned)(a.n_seqs * a.H), (unsigned)(DV / 16), 2);
    hipLaunchKernelGGL((bwd_state_kernel<C, DK, DV>), gc, dim3(64 * P::NW), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grad_kernel<Tin, C, DK, DV>), gs, dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int C, int DK, int DV> constexpr int64_t rec_floats() { return BRec<C, DK, DV>::FLOATS; }

}  // namespace

hipError_t bwd_scratch(void **ptr) {
    static std::atomic<void *> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {  // first use on this device, with the device current: its copy's address
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

bool chunk_bwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv) {
    if (chunk == 64 && Dk == 128 && Dv == 128) return in_dtype == 0 || in_dtype == 1;
    if (chunk == 16 && Dk == 16 && Dv == 16) return in_dtype == 0;
    return false;
}

size_t chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                                 int32_t in_dtype, int32_t num_seqs) {
    if (!chunk_bwd_supported(in_dtype, chunk, Dk, Dv) || B < 1 || T < 0 || H < 1 || num_seqs < 0) return 0;
    const int64_t tokens = (int64_t)B * T;
    const int64_t slots = num_seqs + (tokens + chunk - 1) / chunk;
    const int64_t rec = chunk == 64 ? rec_floats<64, 128, 128>() : rec_floats<16, 16, 16>();
    return (size_t)(slots * H * rec * (int64_t)sizeof(float));
}

hipError_t launch_chunk_bwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv, const BwdArgs &a,
                            hipStream_t stream) {
    if (!chunk_bwd_supported(in_dtype, chunk, Dk, Dv)) return hipErrorInvalidValue;
    if (a.n_seqs == 0) return hipSuccess;
    if (chunk == 64) {
        return in_dtype == 1 ? launch_bwd_t<bf16_t, 64, 128, 128>(a, stream)
                             : launch_bwd_t<float, 64, 128, 128>(a, stream);
    }
    return launch_bwd_t<float, 16, 16, 16>(a, stream);
}

}  // namespace kda
