// KDA chunked prefill (gfx950): the chunkwise-parallel form of the gated delta rule with
// per-channel decay ([KV-cache page] section 3: chunk_size 64; section 6: chunked parallel
// form and WY representation).
//
// Per chunk of C tokens with state S (Dk x Dv, rows = key channels) entering it, and
// G_i = sum_{t<=i} g_t per key channel counted from the chunk start:
//   A_ij = beta_i sum_c k_i[c] k_j[c] e^{G_i[c]-G_j[c]}   (j < i)        [C x C]
//   M_ij = scale sum_c q_i[c] k_j[c] e^{G_i[c]-G_j[c]}    (j <= i)       [C x C]
//   T    = (I + A)^{-1}                                   (UT / WY transform)
//   W    = T (beta k * e^G),   U~ = T Diag(beta) V
//   U    = U~ - W S
//   O    = (scale q * e^G) S + M U
//   S   <- Diag(e^{G_C}) S + (k * e^{G_C - G})^T U
// which equals the token-by-token recurrence S_t = (I - beta k k^T) Diag(e^g) S + beta k v^T,
// o_t = S_t^T (scale q) exactly up to rounding (unroll the recurrence inside the chunk).
//
// Mapping to the MI355X:
// * One workgroup (4 waves) runs one chain: a (sequence, head, V-block of VB columns). The
//   chunks of a chain are sequential; columns of S evolve independently (column j of U, O
//   and S' only depends on column j of S), so V-blocks multiply the parallelism. Workgroups
//   of one (sequence, head) get the same blockIdx % 8, i.e. the same XCD and L2, which then
//   serves the q/k/g tiles they all read.
// * The state stays on chip for the whole sequence: each wave owns a fixed set of 16x16
//   tiles of S in float32 accumulator registers, and a transposed bf16 copy sits in LDS as
//   the matrix-core operand.
// * All C x C and C x D products are 16x16 matrix-core tiles (bf16 inputs, float32
//   accumulation; a float32 instantiation uses the float32 matrix cores).
// * Decay factors never overflow: inside a chunk every e^{G_i - G_j} is split at a 16-token
//   block boundary, so each operand carries a factor <= 1 (or, inside one diagonal 16x16
//   block, at most the inverse decay of 16 tokens). Only one exp per (token, channel).
// * T is built in float32: forward substitution on the four diagonal 16x16 blocks, then
//   block merges T_IJ = -T_II sum_K A_IK T_KJ on the matrix cores with each float32 factor
//   split into a bf16 head and tail (about float32 accuracy).
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int align16(int x) { return (x + 15) & ~15; }

template <typename OP, int C, int DK, int DV, int VB> struct ChunkShape {
    static constexpr int NT = 256;
    static constexpr int NB = C / 16;                       // 16-token blocks per chunk
    static constexpr int NFAR = (NB - 1) * (NB - 2) / 2;    // block pairs (J, I), I >= J + 2
    static constexpr int PAD = 16 / (int)sizeof(OP);         // 16-byte row padding
    static constexpr int LDK = DK + PAD;                     // [token][channel] operand rows
    static constexpr int LDC = C + PAD;                      // [channel or column][token] rows
    static constexpr int LCF = C + 4;                        // float32 [token][token] rows
    static constexpr int NVB = DV / VB;
    static constexpr int VT = VB / 16;                       // 16-wide column tiles per V-block
    static constexpr int KT = DK / 16;
    static constexpr int NUT = NB * VT;                      // U / O tiles
    static constexpr int NST = KT * VT;                      // state tiles
    static constexpr int UPW = (NUT + 3) / 4;
    static constexpr int SPW = (NST + 3) / 4;
    static constexpr int NBLK = NB * (NB + 1) / 2;           // lower 16x16 blocks of a C x C
    static constexpr int AMPW = (2 * NBLK + 3) / 4;
    static constexpr int NPAIR = NB * DK / 2;                // (block, channel pair) jobs
    static constexpr int WPW = (NB * KT + 3) / 4;
    static constexpr int SZ = (int)sizeof(OP);

    // --- LDS map (bytes). Region P first holds the A/M operands, then (after A and M have
    // been formed) the float32 A and T, M and W.
    static constexpr int oLk = 0;
    static constexpr int oLq = oLk + align16(C * LDK * SZ);
    static constexpr int oR = oLq + align16(C * LDK * SZ);
    static constexpr int oRd = oR + align16(C * LDK * SZ);
    static constexpr int oRfar = oRd + align16(C * LDK * SZ);
    static constexpr int P_OPS = oRfar + align16(NFAR * 16 * LDK * SZ);
    static constexpr int oAf = 0;
    static constexpr int oTf = oAf + align16(C * LCF * 4);
    static constexpr int oTtf = oTf + align16(C * LCF * 4);
    static constexpr int oMb = oTtf + align16(C * LCF * 4);
    static constexpr int oWb = oMb + align16(C * LDC * SZ);
    static constexpr int P_REUSE = oWb + align16(C * LDK * SZ);
    static constexpr int P_END = P_OPS > P_REUSE ? P_OPS : P_REUSE;
    // region Q: operands of the state pass
    static constexpr int oXt = P_END;
    static constexpr int oQg = oXt + align16(DK * LDC * SZ);
    static constexpr int oKdT = oQg + align16(C * LDK * SZ);
    // small buffers
    static constexpr int oYt = oKdT + align16(DK * LDC * SZ);
    static constexpr int oUt = oYt + align16(VB * LDC * SZ);
    static constexpr int oSt = oUt + align16(VB * LDC * SZ);
    static constexpr int oDd = oSt + align16(VB * LDK * SZ);
    static constexpr int oGc = oDd + align16(NB * DK * 4);
    static constexpr int oBeta = oGc + align16(DK * 4);
    static constexpr int oMdiag = oBeta + align16(C * 4);
    static constexpr int BYTES = oMdiag + align16(C * 4);

    static_assert(C % 16 == 0 && C >= 16 && C <= 64, "chunk must be 16, 32, 48 or 64");
    static_assert(DK % 16 == 0 && DV % VB == 0 && VB % 16 == 0, "bad tile sizes");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one CU exceeded");
};

// Index of the off-diagonal block pair (J, I), I >= J + 2, in the far-operand table.
__device__ __forceinline__ int far_index(int NB, int J, int I) {
    int idx = 0;
    for (int j = 0; j < J; ++j) idx += NB - 2 - j;
    return idx + (I - J - 2);
}

template <typename T> struct Tag {
    typedef T type;
};

// A 16-token block whose decay reaches this (per channel) is "extreme": its balanced
// fp16 decay factors (up to 2^(-log2(D)/2)) would leave fp16's range.
constexpr float kExtremeBlockDecay = 2.0611536e-9f;  // e^-20

template <typename OP> __device__ __forceinline__ float exp_gate(float x);
template <> __device__ __forceinline__ float exp_gate<_Float16>(float x) { return __expf(x); }
template <> __device__ __forceinline__ float exp_gate<float>(float x) { return expf(x); }

template <typename Tin, typename OP, int C, int DK, int DV, int VB>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(ChunkArgs a) {
    using Sh = ChunkShape<OP, C, DK, DV, VB>;
    using MM = Mma<OP>;
    typedef typename MM::frag frag;
    constexpr int NB = Sh::NB, LDK = Sh::LDK, LDC = Sh::LDC, LCF = Sh::LCF, VT = Sh::VT,
                  KT = Sh::KT;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::BYTES];
    OP *const Lk = reinterpret_cast<OP *>(smem + Sh::oLk);
    OP *const Lq = reinterpret_cast<OP *>(smem + Sh::oLq);
    OP *const Rk = reinterpret_cast<OP *>(smem + Sh::oR);
    OP *const Rd = reinterpret_cast<OP *>(smem + Sh::oRd);
    OP *const Rfar = reinterpret_cast<OP *>(smem + Sh::oRfar);
    float *const Af = reinterpret_cast<float *>(smem + Sh::oAf);
    float *const Tf = reinterpret_cast<float *>(smem + Sh::oTf);
    float *const Ttf = reinterpret_cast<float *>(smem + Sh::oTtf);
    OP *const Mb = reinterpret_cast<OP *>(smem + Sh::oMb);
    OP *const Wb = reinterpret_cast<OP *>(smem + Sh::oWb);
    OP *const Xt = reinterpret_cast<OP *>(smem + Sh::oXt);
    OP *const Qg = reinterpret_cast<OP *>(smem + Sh::oQg);
    OP *const KdT = reinterpret_cast<OP *>(smem + Sh::oKdT);
    OP *const Yt = reinterpret_cast<OP *>(smem + Sh::oYt);
    OP *const Ut = reinterpret_cast<OP *>(smem + Sh::oUt);
    OP *const St = reinterpret_cast<OP *>(smem + Sh::oSt);
    float *const Dd = reinterpret_cast<float *>(smem + Sh::oDd);
    float *const gC = reinterpret_cast<float *>(smem + Sh::oGc);
    float *const sbeta = reinterpret_cast<float *>(smem + Sh::oBeta);
    float *const mdiag = reinterpret_cast<float *>(smem + Sh::oMdiag);
    // fp16 operands: A and M may switch to bf16 for one chunk if its decay is extreme
    constexpr bool kDual = std::is_same<OP, _Float16>::value;
    static_assert(!kDual || DK == 128, "the fp16 path maps one wave to one 16-token block");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // ---- work item: blockIdx -> (sequence, head, V-block); same XCD for one (seq, head)
    const int G = a.n_seqs * a.H;
    const int x8 = blockIdx.x & 7, s8 = blockIdx.x >> 3;
    const int vb = s8 % Sh::NVB;
    const int gi = (s8 / Sh::NVB) * 8 + x8;
    if (gi >= G) return;
    const int n = gi / a.H, h = gi % a.H;
    const int H = a.H;
    int64_t tok0, L;
    if (a.cu_seqlens) {
        tok0 = a.cu_seqlens[n];
        L = (int64_t)a.cu_seqlens[n + 1] - tok0;
    } else {
        tok0 = (int64_t)n * a.seq_len;
        L = a.seq_len;
    }
    const Tin *const qg = static_cast<const Tin *>(a.q);
    const Tin *const kg = static_cast<const Tin *>(a.k);
    const Tin *const vg = static_cast<const Tin *>(a.v);
    const int64_t state_base = ((int64_t)n * H + h) * DK * DV + (int64_t)vb * VB;

    // ---- the state: wave-owned 16x16 tiles, float32, accumulator layout
    f32x4 S[Sh::SPW];
#pragma unroll
    for (int j = 0; j < Sh::SPW; ++j) {
        const int s = wave + 4 * j;
        S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s < Sh::NST) {
            const int rK = s / VT, cv = s % VT;
            if (a.s0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[j][e] = a.s0[state_base + (int64_t)(16 * rK + 4 * lq + e) * DV + 16 * cv + lr];
            }
            MM::store4(St + (16 * cv + lr) * LDK + 16 * rK + 4 * lq, S[j]);
        }
    }

    const int64_t nchunks = (L + C - 1) / C;
    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t t0 = tok0 + ci * C;
        const int Lc = (int)((L - ci * C) < C ? (L - ci * C) : C);
        __syncthreads();

        // ---- phase 0: stage beta and the V-block; per-(block, channel) decay factors
        if (tid < C) sbeta[tid] = tid < Lc ? a.beta[(t0 + tid) * H + h] : 0.f;
        for (int idx = tid; idx < C * (VB / 4); idx += Sh::NT) {
            const int i = idx / (VB / 4), n4 = (idx % (VB / 4)) * 4;
            f32x4 vv = {0.f, 0.f, 0.f, 0.f};
            if (i < Lc) vv = load4(vg + ((t0 + i) * H + h) * DV + vb * VB + n4);
#pragma unroll
            for (int e = 0; e < 4; ++e) Yt[(n4 + e) * LDC + i] = static_cast<OP>(vv[e]);
        }

        const bool pj = tid < Sh::NPAIR;
        const int b = tid / (DK / 2), c0 = 2 * (tid % (DK / 2));
        float al0[16], al1[16], sf0[16], sf1[16], k0[16], k1[16], q0[16], q1[16];
        float dblk0 = 1.f, dblk1 = 1.f;
        if (pj) {
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                const int i = 16 * b + ii;
                if (i < Lc) {
                    const int64_t base = ((t0 + i) * H + h) * DK + c0;
                    const f32x2 gg = load2(a.g + base);
                    const f32x2 kk = load2(kg + base);
                    const f32x2 qq = load2(qg + base);
                    al0[ii] = exp_gate<OP>(gg.x);
                    al1[ii] = exp_gate<OP>(gg.y);
                    k0[ii] = kk.x;
                    k1[ii] = kk.y;
                    q0[ii] = qq.x * a.scale;
                    q1[ii] = qq.y * a.scale;
                } else {
                    al0[ii] = al1[ii] = 1.f;
                    k0[ii] = k1[ii] = q0[ii] = q1[ii] = 0.f;
                }
            }
            // exclusive suffix products (decay from token i+1 to the block end) ...
            float r0 = 1.f, r1 = 1.f;
#pragma unroll
            for (int ii = 15; ii >= 0; --ii) {
                sf0[ii] = r0;
                sf1[ii] = r1;
                r0 *= al0[ii];
                r1 *= al1[ii];
            }
            // ... and inclusive prefix products (decay from the block start to token i)
            r0 = r1 = 1.f;
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                r0 *= al0[ii];
                r1 *= al1[ii];
                al0[ii] = r0;
                al1[ii] = r1;
            }
            Dd[b * DK + c0] = r0;  // whole-block decay
            Dd[b * DK + c0 + 1] = r1;
            dblk0 = r0;
            dblk1 = r1;
        }
        bool extreme = false;
        if constexpr (kDual) {
            extreme = __syncthreads_or(pj && (dblk0 < kExtremeBlockDecay || dblk1 < kExtremeBlockDecay));
            if (extreme) {
                // exact scale * q_i . k_i for the diagonal of M (one wave = one block)
#pragma unroll
                for (int ii = 0; ii < 16; ++ii) {
                    float d = q0[ii] * k0[ii] + q1[ii] * k1[ii];
#pragma unroll
                    for (int m = 32; m > 0; m >>= 1) d += __shfl_xor(d, m);
                    if (lane == 0) mdiag[16 * b + ii] = d;
                }
            }
        } else {
            __syncthreads();
        }

        if (pj) {
            float pre0 = 1.f, pre1 = 1.f, post0 = 1.f, post1 = 1.f;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                if (bb < b) {
                    pre0 *= Dd[bb * DK + c0];
                    pre1 *= Dd[bb * DK + c0 + 1];
                } else if (bb > b) {
                    post0 *= Dd[bb * DK + c0];
                    post1 *= Dd[bb * DK + c0 + 1];
                }
            }
            const float d0 = Dd[b * DK + c0], d1 = Dd[b * DK + c0 + 1];
            if (b == 0) {
                gC[c0] = d0 * post0;
                gC[c0 + 1] = d1 * post1;
            }
            const float inv0 = 1.f / d0, inv1 = 1.f / d1;
            // fp16 A/M operands: rows of block I are multiplied by a per-channel power of two
            // near D_I^(-1/2), the right operands paired with block I by its inverse. Products
            // are unchanged (exact scaling); the diagonal blocks' factors then stay within
            // [D^(1/2), D^(-1/2)] instead of [D, 1/D].
            const bool bal = kDual && !extreme;
            auto balance = [&](float d) {
                return bal ? ldexpf(1.f, (int)floorf(-0.5f * __log2f(d))) : 1.f;
            };
            auto st_am = [&](OP *p, float x, float y) {
                if constexpr (kDual) {
                    if (extreme) {
                        Mma<__bf16>::store_pair(reinterpret_cast<__bf16 *>(p), x, y);
                        return;
                    }
                }
                MM::store_pair(p, x, y);
            };
            const float sb0 = balance(d0), sb1 = balance(d1);
            const float nx0 = b + 1 < NB ? 1.f / balance(Dd[(b + 1) * DK + c0]) : 1.f;
            const float nx1 = b + 1 < NB ? 1.f / balance(Dd[(b + 1) * DK + c0 + 1]) : 1.f;
            OP xt0[16], xt1[16], kd0[16], kd1[16];
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                const int i = 16 * b + ii;
                const float bt = sbeta[i];
                const float ks0 = k0[ii] * sf0[ii], ks1 = k1[ii] * sf1[ii];
                st_am(Lk + i * LDK + c0, bt * k0[ii] * al0[ii] * sb0, bt * k1[ii] * al1[ii] * sb1);
                st_am(Lq + i * LDK + c0, q0[ii] * al0[ii] * sb0, q1[ii] * al1[ii] * sb1);
                st_am(Rk + i * LDK + c0, ks0 * nx0, ks1 * nx1);
                st_am(Rd + i * LDK + c0, ks0 * inv0 / sb0, ks1 * inv1 / sb1);
                MM::store_pair(Qg + i * LDK + c0, q0[ii] * al0[ii] * pre0, q1[ii] * al1[ii] * pre1);
                xt0[ii] = static_cast<OP>(bt * k0[ii] * al0[ii] * pre0);
                xt1[ii] = static_cast<OP>(bt * k1[ii] * al1[ii] * pre1);
                kd0[ii] = static_cast<OP>(ks0 * post0);
                kd1[ii] = static_cast<OP>(ks1 * post1);
            }
            // right operands of blocks (I, b) with I >= b + 2 carry the decay of the blocks
            // strictly between them
            float m0 = 1.f, m1 = 1.f;
#pragma unroll
            for (int I = 2; I < NB; ++I) {
                if (I >= b + 2) {
                    m0 *= Dd[(I - 1) * DK + c0];
                    m1 *= Dd[(I - 1) * DK + c0 + 1];
                    const float f0 = m0 / balance(Dd[I * DK + c0]);
                    const float f1 = m1 / balance(Dd[I * DK + c0 + 1]);
                    OP *dst = Rfar + far_index(NB, b, I) * 16 * LDK + c0;
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii)
                        st_am(dst + ii * LDK, k0[ii] * sf0[ii] * f0, k1[ii] * sf1[ii] * f1);
                }
            }
#pragma unroll
            for (int ii = 0; ii < 16; ii += 4) {
                typedef typename MM::frag f4;
                f4 x0, x1, y0, y1;
                x0 = f4{xt0[ii], xt0[ii + 1], xt0[ii + 2], xt0[ii + 3]};
                x1 = f4{xt1[ii], xt1[ii + 1], xt1[ii + 2], xt1[ii + 3]};
                y0 = f4{kd0[ii], kd0[ii + 1], kd0[ii + 2], kd0[ii + 3]};
                y1 = f4{kd1[ii], kd1[ii + 1], kd1[ii + 2], kd1[ii + 3]};
                *reinterpret_cast<f4 *>(Xt + c0 * LDC + 16 * b + ii) = x0;
                *reinterpret_cast<f4 *>(Xt + (c0 + 1) * LDC + 16 * b + ii) = x1;
                *reinterpret_cast<f4 *>(KdT + c0 * LDC + 16 * b + ii) = y0;
                *reinterpret_cast<f4 *>(KdT + (c0 + 1) * LDC + 16 * b + ii) = y1;
            }
        }
        __syncthreads();

        // ---- phase A: lower 16x16 blocks of A (strictly lower) and M (lower) on the MFMAs
        f32x4 am[Sh::AMPW];
        auto am_phase = [&](auto tag) {
            using AM = typename decltype(tag)::type;
            typedef typename AM::elem E;
#pragma unroll
            for (int j = 0; j < Sh::AMPW; ++j) {
                const int x = wave + 4 * j;
                am[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (x < 2 * Sh::NBLK) {
                    const bool isM = x >= Sh::NBLK;
                    int y = isM ? x - Sh::NBLK : x, I = 0;
                    while (y > I) { y -= I + 1; ++I; }
                    const int J = y;
                    const OP *left = (isM ? Lq : Lk) + (16 * I + lr) * LDK + 4 * lq;
                    const OP *right;
                    if (I == J) right = Rd + (16 * J + lr) * LDK;
                    else if (I == J + 1) right = Rk + (16 * J + lr) * LDK;
                    else right = Rfar + (far_index(NB, J, I) * 16 + lr) * LDK;
                    right += 4 * lq;
                    const E *le = reinterpret_cast<const E *>(left);
                    const E *ri = reinterpret_cast<const E *>(right);
#pragma unroll
                    for (int kk = 0; kk < KT; ++kk)
                        AM::mma(am[j], AM::load(le + 16 * kk), AM::load(ri + 16 * kk));
                    if (I == J) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = 4 * lq + e;
                            if (isM ? (row < lr) : (row <= lr)) am[j][e] = 0.f;
                            if (kDual && extreme && isM && row == lr) am[j][e] = mdiag[16 * I + lr];
                        }
                    }
                }
            }
        };
        if constexpr (kDual) {
            if (extreme) am_phase(Tag<Mma<__bf16>>{});
            else am_phase(Tag<MM>{});
        } else {
            am_phase(Tag<MM>{});
        }
        __syncthreads();  // operands of phase A are dead from here on
#pragma unroll
        for (int j = 0; j < Sh::AMPW; ++j) {
            const int x = wave + 4 * j;
            if (x < 2 * Sh::NBLK) {
                const bool isM = x >= Sh::NBLK;
                int y = isM ? x - Sh::NBLK : x, I = 0;
                while (y > I) { y -= I + 1; ++I; }
                const int J = y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * I + 4 * lq + e, col = 16 * J + lr;
                    if (isM) Mb[row * LDC + col] = static_cast<OP>(am[j][e]);
                    else Af[row * LCF + col] = am[j][e];
                }
            }
        }
        __syncthreads();

        // ---- phase T: T = (I + A)^{-1}; diagonal blocks by forward substitution
        if (wave < NB && lane < 16) {
            const int o = 16 * wave, c = lane;
            float xv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s -= Af[(o + i) * LCF + o + j] * xv[j];
                xv[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Tf[(o + i) * LCF + o + c] = xv[i];
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<f32x4 *>(Ttf + (o + c) * LCF + o + i) =
                    f32x4{xv[i], xv[i + 1], xv[i + 2], xv[i + 3]};
        }
        __syncthreads();
        // off-diagonal blocks by distance: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
#pragma unroll
        for (int d = 1; d < NB; ++d) {
            for (int J = wave; J < NB - d; J += 4) {
                const int I = J + d;
                f32x4 P = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K) {
                    const f32x4 av = *reinterpret_cast<const f32x4 *>(Af + (16 * I + lr) * LCF + 16 * K + 4 * lq);
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(Ttf + (16 * J + lr) * LCF + 16 * K + 4 * lq);
                    MM::mma_split(P, av, bv);
                }
                const f32x4 tii = *reinterpret_cast<const f32x4 *>(Tf + (16 * I + lr) * LCF + 16 * I + 4 * lq);
                f32x4 Tij = {0.f, 0.f, 0.f, 0.f};
                MM::mma_split(Tij, tii, P);
                Tij = -Tij;
#pragma unroll
                for (int e = 0; e < 4; ++e) Tf[(16 * I + 4 * lq + e) * LCF + 16 * J + lr] = Tij[e];
                *reinterpret_cast<f32x4 *>(Ttf + (16 * J + lr) * LCF + 16 * I + 4 * lq) = Tij;
            }
            __syncthreads();
        }

        // ---- phase W: W = T X (X = beta k e^G), and U~ = T Diag(beta) V
#pragma unroll
        for (int j = 0; j < Sh::WPW; ++j) {
            const int x = wave + 4 * j;
            if (x < NB * KT) {
                const int I = x / KT, cK = x % KT;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int J = 0; J <= I; ++J) {
                    const f32x4 tv = *reinterpret_cast<const f32x4 *>(Tf + (16 * I + lr) * LCF + 16 * J + 4 * lq);
                    MM::mma(acc, MM::from_f32(tv), MM::load(Xt + (16 * cK + lr) * LDC + 16 * J + 4 * lq));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Wb[(16 * I + 4 * lq + e) * LDK + 16 * cK + lr] = static_cast<OP>(acc[e]);
            }
        }
        f32x4 Ur[Sh::UPW];
#pragma unroll
        for (int j = 0; j < Sh::UPW; ++j) {
            const int u = wave + 4 * j;
            Ur[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (u < Sh::NUT) {
                const int I = u / VT, cv = u % VT;
                for (int J = 0; J <= I; ++J) {
                    f32x4 tv = *reinterpret_cast<const f32x4 *>(Tf + (16 * I + lr) * LCF + 16 * J + 4 * lq);
                    const f32x4 bt = *reinterpret_cast<const f32x4 *>(sbeta + 16 * J + 4 * lq);
                    tv *= bt;
                    const frag th = MM::from_f32(tv);
                    const frag tl = MM::from_f32(tv - MM::to_f32(th));
                    const frag yv = MM::load(Yt + (16 * cv + lr) * LDC + 16 * J + 4 * lq);
                    MM::mma(Ur[j], tl, yv);
                    MM::mma(Ur[j], th, yv);
                }
            }
        }
        __syncthreads();

        // ---- state pass (a): U = U~ - W S
#pragma unroll
        for (int j = 0; j < Sh::UPW; ++j) {
            const int u = wave + 4 * j;
            if (u < Sh::NUT) {
                const int I = u / VT, cv = u % VT;
                f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KT; ++kk)
                    MM::mma(ws, MM::load(Wb + (16 * I + lr) * LDK + 16 * kk + 4 * lq),
                            MM::load(St + (16 * cv + lr) * LDK + 16 * kk + 4 * lq));
                MM::store4(Ut + (16 * cv + lr) * LDC + 16 * I + 4 * lq, Ur[j] - ws);
            }
        }
        __syncthreads();

        // ---- (b): O = (scale q e^G) S + M U, written straight to HBM
#pragma unroll
        for (int j = 0; j < Sh::UPW; ++j) {
            const int u = wave + 4 * j;
            if (u < Sh::NUT) {
                const int I = u / VT, cv = u % VT;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KT; ++kk)
                    MM::mma(acc, MM::load(Qg + (16 * I + lr) * LDK + 16 * kk + 4 * lq),
                            MM::load(St + (16 * cv + lr) * LDK + 16 * kk + 4 * lq));
                for (int J = 0; J <= I; ++J)
                    MM::mma(acc, MM::load(Mb + (16 * I + lr) * LDC + 16 * J + 4 * lq),
                            MM::load(Ut + (16 * cv + lr) * LDC + 16 * J + 4 * lq));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * I + 4 * lq + e;
                    if (row < Lc) a.o[((t0 + row) * H + h) * DV + vb * VB + 16 * cv + lr] = acc[e];
                }
            }
        }

        // ---- (c): S <- Diag(e^{G_C}) S + (k e^{G_C - G})^T U
#pragma unroll
        for (int j = 0; j < Sh::SPW; ++j) {
            const int s = wave + 4 * j;
            if (s < Sh::NST) {
                const int rK = s / VT, cv = s % VT;
                const f32x4 dec = *reinterpret_cast<const f32x4 *>(gC + 16 * rK + 4 * lq);
                f32x4 acc = S[j] * dec;
#pragma unroll
                for (int J = 0; J < NB; ++J)
                    MM::mma(acc, MM::load(KdT + (16 * rK + lr) * LDC + 16 * J + 4 * lq),
                            MM::load(Ut + (16 * cv + lr) * LDC + 16 * J + 4 * lq));
                S[j] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < Sh::SPW; ++j) {
            const int s = wave + 4 * j;
            if (s < Sh::NST) {
                const int rK = s / VT, cv = s % VT;
                MM::store4(St + (16 * cv + lr) * LDK + 16 * rK + 4 * lq, S[j]);
            }
        }
    }

    if (a.s_out) {
#pragma unroll
        for (int j = 0; j < Sh::SPW; ++j) {
            const int s = wave + 4 * j;
            if (s < Sh::NST) {
                const int rK = s / VT, cv = s % VT;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.s_out[state_base + (int64_t)(16 * rK + 4 * lq + e) * DV + 16 * cv + lr] = S[j][e];
            }
        }
    }
}

template <typename Tin, typename OP, int C, int DK, int DV, int VB>
hipError_t launch_t(const ChunkArgs &a, hipStream_t stream) {
    using Sh = ChunkShape<OP, C, DK, DV, VB>;
    const int64_t G = (int64_t)a.n_seqs * a.H;
    const int64_t blocks = ((G + 7) / 8) * 8 * Sh::NVB;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((chunk_fwd_kernel<Tin, OP, C, DK, DV, VB>), dim3((unsigned)blocks),
                       dim3(Sh::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool chunk_fwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv) {
    if (Dk != Dv) return false;
    if (in_dtype == 1) return chunk == 64 && Dk == 128;
    if (in_dtype == 0)
        return (chunk == 16 && Dk == 16) || (chunk == 64 && (Dk == 32 || Dk == 64));
    return false;
}

hipError_t launch_chunk_fwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv,
                            const ChunkArgs &a, hipStream_t stream) {
    if (!chunk_fwd_supported(in_dtype, chunk, Dk, Dv)) return hipErrorInvalidValue;
    if (a.n_seqs == 0) return hipSuccess;
    if (in_dtype == 1) return launch_t<bf16_t, _Float16, 64, 128, 128, 32>(a, stream);
    if (chunk == 16) return launch_t<float, float, 16, 16, 16, 16>(a, stream);
    if (Dk == 32) return launch_t<float, float, 64, 32, 32, 32>(a, stream);
    return launch_t<float, float, 64, 64, 64, 16>(a, stream);
}

}  // namespace kda
