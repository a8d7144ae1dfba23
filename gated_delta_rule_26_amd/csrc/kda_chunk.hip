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
// Mapping to the MI355X (one workgroup of NW waves per (sequence, head) chain):
// * The chunks of a chain run in order; everything inside a chunk is parallel. Each wave
//   owns DV/(16 NW) 16-column tiles of the state for the whole sequence, in float32
//   accumulator registers. The state pass (U, O, S update) runs entirely from registers:
//   an accumulator tile is directly a matrix-core B fragment, so the only shared operands
//   are the per-chunk A-side matrices in LDS and the state pass has no barrier.
// * The next chunk's q, k, v, g and beta are loaded into registers while the current chunk
//   computes: v, g and beta once P0 has consumed the current ones, k and q after P1. Rows
//   past the sequence end fall outside the buffer bounds and read as zero.
// * Decay factors never overflow: inside a chunk every e^{G_i - G_j} is split at a
//   16-token block boundary, so each operand carries a factor <= 1 or, inside a diagonal
//   16x16 block, at most the inverse decay D^-1 of the block's 16 tokens. One exp per
//   (token, channel). With fp16 operands each channel of a block is balanced by a power of
//   two near D^(-1/2), keeping every factor within fp16's range. A chunk in which some
//   block decays below e^-12 (float32 operands: e^-60) is "extreme": its diagonal blocks of
//   A and M are summed pair by pair in float32 from the cumulative log-decay (one exp per
//   pair and channel, exact for any decay), and its off-diagonal blocks, whose factors are
//   all <= 1, use unbalanced operands.
// * T is never formed beyond its 16x16 diagonal blocks: those are inverted in registers as
//   (I - L)(I + L^2)(I + L^4)(I + L^8) on the matrix cores (transposes by products with the
//   identity), and W and U~ come from block forward substitution (I + A) W = beta k e^G,
//   (I + A) U~ = Diag(beta) V.
#include <atomic>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int align16(int x) { return (x + 15) & ~15; }

// A 16-token block whose decay D falls below this (in some channel) is "extreme": its
// diagonal-block factors span D^-1, which float32 cannot hold beyond e^-60 and which fp16,
// even balanced to D^(+-1/2), holds only with subnormal (imprecise) small factors beyond
// about e^-12. Such a chunk computes its diagonal blocks pair by pair.
template <typename OP> constexpr float extreme_block_decay() {
    return std::is_same<OP, float>::value ? 8.7565108e-27f   // e^-60
                                          : 6.1442124e-6f;   // e^-12
}

template <typename OP, int TSZ, int C, int DK, int DV, int NW> struct ChunkShape {
    static constexpr int NT = 64 * NW;
    static constexpr int NB = C / 16;                       // 16-token blocks per chunk
    static constexpr int NFAR = (NB - 1) * (NB - 2) / 2;    // block pairs (J, I), I >= J + 2
    static constexpr int PAD = 16 / (int)sizeof(OP);        // 16-byte row padding
    static constexpr int LDK = DK + PAD;                    // [token][channel] operand rows
    static constexpr int LDC = C + PAD;                     // [channel][token] operand rows
    static constexpr int KT = DK / 16;
    static constexpr int VT = DV / 16;
    // state column tiles: the value columns of S, or (transition pass) the Dk columns of X
    static constexpr int NCT = VT;
    static constexpr int CPW = NCT >= NW ? NCT / NW : 1;    // state column tiles per wave
    static constexpr int WPW = KT >= NW ? KT / NW : 1;      // W column tiles per wave
    static constexpr int NOFFA = NB * (NB - 1) / 2;         // off-diagonal blocks of A
    static constexpr int NOFF = 2 * NOFFA;                  // ... and of M
    static constexpr int OFFW = NW;                         // waves doing off-diagonal jobs
    static constexpr int OPW = NOFF > 0 ? (NOFF + OFFW - 1) / OFFW : 1;
    static constexpr int NVJ = (C / 4) * (DV / 4);          // 4x4 value-tile jobs per chunk
    static constexpr int VPT = (NVJ + NT - 1) / NT;           // value-tile jobs per thread
    static constexpr int NEJ = NB * (DK / 2);                 // (block, channel pair) jobs
    static constexpr int JPT = (NEJ + 32 * NW - 1) / (32 * NW);  // per 32-lane half-wave slot
    static constexpr int SZ = (int)sizeof(OP);

    // LDS map (bytes). Region P first holds the A/M operands, then -A, the diagonal blocks
    // of T and M ([token][token], columns in perm order) and W.
    static constexpr int oLk = 0;
    static constexpr int oLq = oLk + align16(C * LDK * SZ);
    static constexpr int oRk = oLq + align16(C * LDK * SZ);
    static constexpr int oRd = oRk + align16(C * LDK * SZ);
    static constexpr int oRfar = oRd + align16(C * LDK * SZ);
    static constexpr int P_OPS = oRfar + align16(NFAR * 16 * LDK * SZ);
    static constexpr int oAn = 0;
    static constexpr int oTd = oAn + align16(C * LDC * SZ);
    static constexpr int oMb = oTd + align16(C * LDC * SZ);
    static constexpr int oWb = oMb + align16(C * LDC * SZ);
    static constexpr int P_REUSE = oWb + align16(C * LDK * SZ);
    static constexpr int P_END = P_OPS > P_REUSE ? P_OPS : P_REUSE;
    // Extreme chunks, before the operands are built (so over region P and the Xt, Qg, KdT
    // arrays): float64 cumulative log-decay and raw k, q (input type, TSZ bytes), all
    // [channel][token], and the partial sums of the channel-split waves.
    static constexpr int SPL = (NW / NB < DK / 32 ? NW / NB : DK / 32) > 1
                                   ? (NW / NB < DK / 32 ? NW / NB : DK / 32) : 1;
    static constexpr int LDG = C + 2;
    static constexpr int LDT = C + 16 / TSZ;
    static constexpr int oXG = 0;
    static constexpr int oXK = oXG + align16(DK * LDG * 8);
    static constexpr int oXQ = oXK + align16(DK * LDT * TSZ);
    static constexpr int oXP = oXQ + align16(DK * LDT * TSZ);
    static constexpr int X_END = oXP + align16((SPL - 1) * NB * 8 * 64 * 4);
    static constexpr int oXt = P_END;                        // (beta k e^G)^T  [channel][token]
    static constexpr int oQg = oXt + align16(DK * LDC * SZ); // scale q e^G     [token][channel]
    static constexpr int oKdT = oQg + align16(C * LDK * SZ); // (k e^{G_C-G})^T [channel][token]
    static constexpr int oYt = oKdT + align16(DK * LDC * SZ); // V^T        [column][token]
    static constexpr int oDd = oYt + align16(DV * LDC * SZ);
    static constexpr int oGc = oDd + align16(NB * DK * 4);
    static constexpr int oBeta = oGc + align16(DK * 4);
    // fused q/k normalisation: per-token partial sums of squares [k, q][channel half][token]
    static constexpr int oNrm = oBeta + align16(C * 4);
    static constexpr int oGain = oNrm + align16(4 * C * 4);  // fused output norm gain [DV]
    static constexpr int oFlag = oGain + align16(DV * 4);   // per-wave extreme-chunk votes [NW]
    static constexpr int BYTES = oFlag + align16(NW * 4);

    static_assert(C % 16 == 0 && C >= 16 && C <= 64, "chunk must be 16, 32, 48 or 64");
    static_assert(DK % 16 == 0 && DV % 16 == 0, "head dims must be multiples of 16");
    static_assert(NCT < NW || NCT % NW == 0, "state tiles must spread evenly over waves");
    static_assert(KT < NW || KT % NW == 0, "W tiles must spread evenly over waves");
    static_assert(NB <= NW, "one wave per diagonal block");
    static_assert(C % Step<OP>::KS == 0 && DK % Step<OP>::KS == 0, "step size");
    static_assert(BYTES <= 160 * 1024, "LDS budget of one CU exceeded");
    static_assert(X_END <= oYt, "extreme-chunk staging must fit before the V^T array");
    static_assert(DK % (4 * SPL) == 0, "channel split");
};

// The part of M [C][C] (columns in step order) that the product M U reads: the 16-row band I
// reads its first KS (I / TPS + 1) columns, i.e. the 16x16 blocks on and below the diagonal
// plus, with two-tile steps, the zero block right of the diagonal for even I. The record
// keeps only those columns, band after band, each row contiguous (fp16 operands, C = 64:
// 6 KB instead of 8).
template <typename OP, int C> struct MBands {
    static constexpr int KS = Step<OP>::KS, TPS = Step<OP>::TPS, SZ = (int)sizeof(OP), NB = C / 16;
    static_assert(C % KS == 0 && KS * ((NB - 1) / TPS + 1) <= C, "bands within the chunk");
    // 16-byte pieces per row of band I, and the first piece of band I
    static constexpr int ppr(int I) { return KS * (I / TPS + 1) * SZ / 16; }
    static constexpr int base(int I) {
        int b = 0;
        for (int i = 0; i < I; ++i) b += 16 * ppr(i);
        return b;
    }
    static constexpr int NP = base(NB);  // pieces in all
    // Every band is a whole number of 64-piece groups (16 rows of KS * SZ = 64 bytes or a
    // multiple), so the 64 pieces y = 64 g .. 64 g + 63 that one wave copies lie in one band.
    static_assert(KS * SZ % 64 == 0, "bands of whole 64-piece groups");
    // piece y (0 <= y < NP) -> row and first column (elements) of its 16 bytes; the lanes of
    // a wave must pass y of one 64-piece group (the band is then worked out once per wave)
    static __device__ __forceinline__ void piece(int y, int &row, int &col) {
        const int g = __builtin_amdgcn_readfirstlane(y & ~63);
        int I = 0;
#pragma unroll
        for (int k = 1; k < NB; ++k) I += g >= base(k) ? 1 : 0;
        row = 0;
        col = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (I == k) {
                const int yy = y - base(k);
                row = 16 * k + yy / ppr(k);
                col = (yy % ppr(k)) * (16 / SZ);
            }
    }
};

// Per-chunk record of a split segment (global memory, written by the chunked forward and read
// by the replay passes). Dense copies of the LDS operands in the same element order:
// W [C][Dk] and Qg [C][Dk] (columns in step order), Kd^T [Dk][C], the bands of M read by
// M U (MBands), then gC [Dk] float32 and U~ (operand type) in accumulator order
// [Dv/16][C/16][64 lanes][4].
template <typename OP, int C, int DK, int DV> struct Record {
    static constexpr int SZ = (int)sizeof(OP);
    static constexpr int oW = 0;
    static constexpr int oQ = oW + C * DK * SZ;
    static constexpr int oK = oQ + C * DK * SZ;
    static constexpr int oM = oK + DK * C * SZ;
    static constexpr int OPS = oM + 16 * MBands<OP, C>::NP;  // the LDS-staged part
    static constexpr int oG = OPS;
    static constexpr int oU = oG + DK * 4;
    static constexpr int BYTES = (oU + C * DV * SZ + 255) & ~255;
};

// Index of the off-diagonal block pair (J, I), I >= J + 2, in the far-operand table.
__device__ __forceinline__ int far_index(int NB, int J, int I) {
    int idx = 0;
    for (int j = 0; j < J; ++j) idx += NB - 2 - j;
    return idx + (I - J - 2);
}

// (I, J) of the x-th strictly-lower 16x16 block, row-major order.
__device__ __forceinline__ void lower_block(int x, int &I, int &J) {
    I = 1;
    while (x >= I) {
        x -= I;
        ++I;
    }
    J = x;
}

template <typename OP> __device__ __forceinline__ float exp_gate(float x) { return __expf(x); }
template <> __device__ __forceinline__ float exp_gate<float>(float x) { return expf(x); }

// Raw pair of consecutive inputs as loaded (bf16 pair in 32 bits, or two floats).
template <typename Tin> struct Raw2;
template <> struct Raw2<bf16_t> {
    typedef uint32_t type;
    static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    static __device__ __forceinline__ f32x2 f32(type u) {
        return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
    }
};
template <> struct Raw2<float> {
    typedef f32x2 type;
    static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
        return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    static __device__ __forceinline__ f32x2 f32(type u) { return u; }
};

// Raw four consecutive inputs as loaded.
template <typename Tin> struct Raw4;
template <> struct Raw4<bf16_t> {
    typedef uint2 type;
    static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    }
    static __device__ __forceinline__ f32x4 f32(type u) {
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
    }
};
template <> struct Raw4<float> {
    typedef f32x4 type;
    static __device__ __forceinline__ type load(rsrc_t r, int voff, int soff) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    static __device__ __forceinline__ f32x4 f32(type u) { return u; }
};

// Raw inputs staged in LDS (exact: bf16 values keep their 16 bits).
template <typename Tin> struct Stage;
template <> struct Stage<bf16_t> {
    static __device__ __forceinline__ void store8(bf16_t *p, const float *v) {
        uint4 u;
        u.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
        u.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
        u.z = (__float_as_uint(v[4]) >> 16) | (__float_as_uint(v[5]) & 0xffff0000u);
        u.w = (__float_as_uint(v[6]) >> 16) | (__float_as_uint(v[7]) & 0xffff0000u);
        *reinterpret_cast<uint4 *>(p) = u;
    }
    static __device__ __forceinline__ f32x4 load4(const bf16_t *p) {
        return Raw4<bf16_t>::f32(*reinterpret_cast<const uint2 *>(p));
    }
    static __device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(p->bits); }
};
template <> struct Stage<float> {
    static __device__ __forceinline__ void store8(float *p, const float *v) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    static __device__ __forceinline__ f32x4 load4(const float *p) {
        return *reinterpret_cast<const f32x4 *>(p);
    }
    static __device__ __forceinline__ float load1(const float *p) { return *p; }
};

// Product of two 16x16 accumulator tiles, X^T Y, on the matrix cores of operand type OP.
// An accumulator tile used as the A fragment is read transposed (lane holds X[4q+e][l%16],
// which the A operand takes as A[l%16][4q+e]).
template <typename OP> __device__ __forceinline__ f32x4 mm_tn(f32x4 x, f32x4 y) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    Mma<OP>::mma(acc, Mma<OP>::from_f32(x), Mma<OP>::from_f32(y));
    return acc;
}

// The chunked forward, one workgroup per chain (STORE = false), or, for a sequence split,
// one per (chain, segment) (STORE = true): segment 0 starts from the initial state and every
// later segment from zero; no outputs are written; each chunk's record (W, the read-out and
// state-update operands, U~) is stored for the replay passes, and the segment's final state
// R_p goes to ws_r[p] (p < nseg-1).
// ---- the output norm (the layer's o_norm: a gated RMSNorm with a sigmoid gate), fused into
// the output store of a chunk. The waves stage their 16-column output tiles in LDS
// (ostage_tile); after a barrier, 8 threads per row normalise and store whole rows
// (onorm_rows), with 16-byte loads of the output gate and 16-byte stores.
template <int C, int DV, int NW> struct ONorm {
    static constexpr int LD = DV + 4;                 // staged row stride (floats), 16-byte rows
    static constexpr int BYTES = C * LD * 4;
    static constexpr int TPRW = 64 * NW / C;          // threads per row
    static constexpr int CPT = DV / TPRW;             // columns per thread
    static constexpr bool OK = CPT == 16 && (TPRW & (TPRW - 1)) == 0 && TPRW <= 64;
};

// Lane (lr, q) of a wave holds rows 16I + 4q + e of column 16 * wave + lr of the chunk's outputs.
template <int C, int DV, int NW>
__device__ __forceinline__ void ostage_tile(float *Ob, int I, f32x4 o) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ob[(16 * I + 4 * q4 + e) * ONorm<C, DV, NW>::LD + 16 * wave + lr] = o[e];
}

// This thread's 16 output-gate pre-activations (bf16): row tid / TPRW, columns from
// CPT * (tid % TPRW); zero past the chunk end.
template <int C, int DV, int NW>
__device__ __forceinline__ void load_ogate(const ChunkArgs &a, int64_t t0, int Lc, int h, u32x4 (&zr)[2]) {
    using ON = ONorm<C, DV, NW>;
    const int row = threadIdx.x / ON::TPRW, c0 = ON::CPT * (threadIdx.x % ON::TPRW);
    zr[0] = zr[1] = u32x4{0u, 0u, 0u, 0u};
    if (row < Lc) {
        const uint16_t *p = static_cast<const uint16_t *>(a.f.og) + (t0 + row) * (int64_t)(a.H * DV) + h * DV + c0;
        zr[0] = *reinterpret_cast<const u32x4 *>(p);
        zr[1] = *reinterpret_cast<const u32x4 *>(p + 8);
    }
}

// y = o / sqrt(mean of the row's Dv squares + eps) * gain * sigmoid(z), stored as float32 or
// bf16 for rows < Lc. Ob: the staged outputs (complete: call after a barrier); gain: [DV]
// in LDS.
template <int C, int DV, int NW>
__device__ __forceinline__ void onorm_rows(const ChunkArgs &a, const float *Ob, const float *gain,
                                           const u32x4 (&zr)[2], int64_t t0, int Lc, int h) {
    using ON = ONorm<C, DV, NW>;
    static_assert(ON::OK, "row epilogue shape");
    const int row = threadIdx.x / ON::TPRW, c0 = ON::CPT * (threadIdx.x % ON::TPRW);
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(Ob + row * ON::LD + c0 + 4 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * i + e] = v[e];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += x[i] * x[i];
    static_assert(ON::TPRW == 8, "row sums over 8 lanes");
    ss += lane_xor<1>(ss);
    ss += lane_xor<2>(ss);
    ss += lane_xor<4>(ss);
    const float rs = rsqrt_or_zero(ss * (1.f / DV) + a.f.oeps);
    float y[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 w = *reinterpret_cast<const f32x4 *>(gain + c0 + 4 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * i + e;
            const uint32_t zb = zr[j >> 3][(j >> 1) & 3];
            const float z = bf16_to_f32((uint16_t)((j & 1) ? zb >> 16 : zb & 0xffffu));
            y[j] = x[j] * rs * w[e] * sigmoid_f(z);
        }
    }
    if (row >= Lc) return;
    const int64_t off = (t0 + row) * (int64_t)(a.H * DV) + h * DV + c0;
    if (a.f.o_bf16) {
        uint16_t *p = static_cast<uint16_t *>(a.o) + off;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pk[e] = (uint32_t)bf16_bits(y[8 * hf + 2 * e]) | ((uint32_t)bf16_bits(y[8 * hf + 2 * e + 1]) << 16);
            *reinterpret_cast<u32x4 *>(p + 8 * hf) = pk;
        }
    } else {
        float *p = static_cast<float *>(a.o) + off;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4 *>(p + 4 * i) = f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
    }
}

// FUSE bit 0 (FIN): the gate comes from its pre-activation (a.f.gx) and q, k are normalised
// in-kernel when a.f.norm_qk; bit 1 (FOUT): the outputs pass the gated RMSNorm (a.f.og).
template <typename Tin, typename OP, int C, int DK, int DV, int NW, bool STORE, int FUSE>
__global__ __launch_bounds__(64 * NW, 1) void chunk_fwd_kernel(ChunkArgs a) {
    using Sh = ChunkShape<OP, (int)sizeof(Tin), C, DK, DV, NW>;
    using MM = Mma<OP>;
    using ST = Step<OP>;
    using RW = Raw2<Tin>;
    using R4 = Raw4<Tin>;
    constexpr int NB = Sh::NB, LDK = Sh::LDK, LDC = Sh::LDC, KT = Sh::KT,
                  CPW = Sh::CPW, KS = ST::KS, TPS = ST::TPS;
    constexpr bool kBalance = std::is_same<OP, _Float16>::value;  // fp16 range balancing
    constexpr bool FIN = (FUSE & 1) != 0, FOUT = (FUSE & 2) != 0;
    // the fused steps assume one (block, channel pair) job per thread, the two 64-channel
    // halves of a token in a pair of waves, and one value column tile per wave
    static_assert(!FIN || (Sh::JPT == 1 && DK == 128 && 32 * NW == Sh::NEJ), "fused input shape");
    static_assert(!FOUT || (Sh::NCT == NW && Sh::CPW == 1), "fused output shape");
    // fused output norm: the outputs are staged over the A/M operands, dead from P4 on
    static_assert(!FOUT || Sh::P_REUSE + ONorm<C, DV, NW>::BYTES <= Sh::P_END, "output staging");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Sh::BYTES];
    OP *const Lk = reinterpret_cast<OP *>(smem + Sh::oLk);
    OP *const Lq = reinterpret_cast<OP *>(smem + Sh::oLq);
    OP *const Rk = reinterpret_cast<OP *>(smem + Sh::oRk);
    OP *const Rd = reinterpret_cast<OP *>(smem + Sh::oRd);
    OP *const Rfar = reinterpret_cast<OP *>(smem + Sh::oRfar);
    OP *const An = reinterpret_cast<OP *>(smem + Sh::oAn);  // -A (strictly lower blocks)
    OP *const Td = reinterpret_cast<OP *>(smem + Sh::oTd);  // diagonal blocks of T
    OP *const Mb = reinterpret_cast<OP *>(smem + Sh::oMb);
    OP *const Wb = reinterpret_cast<OP *>(smem + Sh::oWb);
    OP *const Xt = reinterpret_cast<OP *>(smem + Sh::oXt);
    OP *const Qg = reinterpret_cast<OP *>(smem + Sh::oQg);
    OP *const KdT = reinterpret_cast<OP *>(smem + Sh::oKdT);
    OP *const Yt = reinterpret_cast<OP *>(smem + Sh::oYt);
    // V^T row r holds 4-token groups in XOR-swizzled order (group tg at tg ^ ((r >> 3) & m)):
    // the staging stores of 16 lanes, rows 4 apart, then fall in distinct LDS banks, and so
    // do the 16 rows that one lane group of the reader spans
    auto yt_col = [](int r, int tg) {
        constexpr int m = C / 4 - 1 < 7 ? C / 4 - 1 : 7;
        return 4 * (tg ^ ((r >> 3) & m));
    };
    float *const Dd = reinterpret_cast<float *>(smem + Sh::oDd);
    float *const gC = reinterpret_cast<float *>(smem + Sh::oGc);
    float *const sbeta = reinterpret_cast<float *>(smem + Sh::oBeta);
    double *const xG = reinterpret_cast<double *>(smem + Sh::oXG);
    Tin *const xK = reinterpret_cast<Tin *>(smem + Sh::oXK);
    Tin *const xQ = reinterpret_cast<Tin *>(smem + Sh::oXQ);
    float *const xP = reinterpret_cast<float *>(smem + Sh::oXP);
    float *const nrm = reinterpret_cast<float *>(smem + Sh::oNrm);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, q4 = lane >> 4;
    f32x4 Id;  // 16x16 identity in accumulator layout (transposes by products)
#pragma unroll
    for (int e = 0; e < 4; ++e) Id[e] = (4 * q4 + e == lr) ? 1.f : 0.f;
    typedef typename MM::frag frag4;

    // ---- blockIdx -> (chain = (sequence, head), segment)
    const int H = a.H;
    const int chains = a.n_seqs * H;
    const int segs = STORE ? a.nseg : 1;
    if ((int)blockIdx.x >= chains * segs) return;
    const int chain = blockIdx.x / segs, seg = blockIdx.x % segs;
    // split: the segments whose outputs come from the output replay (seg >= a.out_from)
    // record their chunks' operands; segment 0 starts from the true initial state and, with
    // out_from = 1, writes its outputs itself
    const bool store = STORE && seg >= a.out_from;
    // packed batches run their sequences longest first when an order is given
    const int n = a.order ? a.order[chain / H] : chain / H, h = chain % H;
    int64_t tok0, L;
    if (a.cu_seqlens) {
        int64_t end;
        packed_range(a.cu_seqlens, n, a.seq_len, tok0, end);
        L = end - tok0;
    } else {
        tok0 = (int64_t)n * a.seq_len;
        L = a.seq_len;
    }
    if (a.seg_len) {
        tok0 += (int64_t)seg * a.seg_len;
        L = L - (int64_t)seg * a.seg_len < a.seg_len ? L - (int64_t)seg * a.seg_len : a.seg_len;
    }
    const Tin *const qg = static_cast<const Tin *>(a.q);
    const Tin *const kg = static_cast<const Tin *>(a.k);
    const Tin *const vg = static_cast<const Tin *>(a.v);
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;

    // ---- per-thread element jobs: (16-token block b, channel pair, half hh of the block);
    // the two halves of a block sit in lanes l and l^32 of one wave
    const int hh = lane >> 5;
    int jb[Sh::JPT], jc[Sh::JPT];
    bool jok[Sh::JPT];
#pragma unroll
    for (int jj = 0; jj < Sh::JPT; ++jj) {
        const int lidx = wave * 32 + (lane & 31) + jj * 32 * NW;
        jb[jj] = lidx / (DK / 2);
        jc[jj] = 2 * (lidx % (DK / 2));
        jok[jj] = jb[jj] < NB;
    }
    // fused gate: the head's rate exp(A_log[h]) and the biases of this thread's two channels
    float grate = 0.f, gb0 = 0.f, gb1 = 0.f;
    if constexpr (FIN) {
        grate = expf(a.f.A_log[h]);
        gb0 = a.f.dt_bias[h * DK + jc[0]];
        gb1 = a.f.dt_bias[h * DK + jc[0] + 1];
    }

    // ---- state: this wave's column tiles (ct = wave + NW*j) of S (or X), float32
    // accumulator layout
    const bool owns = wave < Sh::NCT;
    const float *sinit = a.s0 ? a.s0 + sbase : nullptr;
    if (STORE && seg > 0) sinit = nullptr;
    float *const Ob = reinterpret_cast<float *>(smem + Sh::P_REUSE);  // fused output staging
    float *const sgain = reinterpret_cast<float *>(smem + Sh::oGain);
    int *const sflag = reinterpret_cast<int *>(smem + Sh::oFlag);
    if (FOUT && tid < DV) sgain[tid] = a.f.ow[tid];  // read after the loop's first barrier
    f32x4 S[CPW][KT];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int ct = wave + NW * j;
#pragma unroll
        for (int r = 0; r < KT; ++r) {
            S[j][r] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (owns && sinit) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[j][r][e] = sinit[(int64_t)(16 * r + 4 * q4 + e) * DV + 16 * ct + lr];
            }
        }
    }

    // ---- register prefetch of one chunk's q, k, g (this thread's 8 tokens x 2 channels),
    // beta, and a 4-token x 4-column tile of v
    typename RW::type pk[Sh::JPT][8], pq[Sh::JPT][8];
    typename R4::type pv[Sh::VPT][4];
    // gate input: float32 log-decay, or (fused) its pre-activation in the input type
    typename std::conditional<FIN, typename RW::type, f32x2>::type pg[Sh::JPT][8];
    float pbeta = 0.f;
    auto vjob = [&](int vv, int &tg, int &cg) {
        const int x = tid + vv * Sh::NT;
        tg = x / (DV / 4);
        cg = x % (DV / 4);
        return x < Sh::NVJ;
    };
    // Per-lane byte offsets from a chunk's first token (rows past the chunk end, or lanes
    // without a job, land beyond the buffer bound and read as zero: alpha = e^0 = 1, k = q =
    // v = beta = 0, i.e. padding tokens that change nothing).
    constexpr int ESZ = (int)sizeof(Tin);
    const int krow = H * DK, vrow = H * DV;  // elements per token row
    int ko[Sh::JPT], vo[Sh::VPT];
#pragma unroll
    for (int jj = 0; jj < Sh::JPT; ++jj)
        ko[jj] = jok[jj] ? (16 * jb[jj] + 8 * hh) * krow + h * DK + jc[jj] : C * krow;
#pragma unroll
    for (int vv = 0; vv < Sh::VPT; ++vv) {
        int tg, cg;
        vo[vv] = vjob(vv, tg, cg) ? 4 * tg * vrow + h * DV + 4 * cg : C * vrow;
    }
    // part 1: v, g and beta (consumed by P0 and the extreme-chunk path); part 2: k and q
    // (consumed up to P1); 0: both
    auto prefetch = [&](int64_t t0, int Lc, int part) {
        const rsrc_t rq = make_rsrc(qg + t0 * krow, (uint32_t)(Lc * krow * ESZ));
        const rsrc_t rk = make_rsrc(kg + t0 * krow, (uint32_t)(Lc * krow * ESZ));
        const rsrc_t rg = FIN ? make_rsrc(static_cast<const Tin *>(a.f.gx) + t0 * krow, (uint32_t)(Lc * krow * ESZ))
                              : make_rsrc(a.g + t0 * krow, (uint32_t)(Lc * krow * 4));
        const rsrc_t rv = make_rsrc(vg + t0 * vrow, (uint32_t)(Lc * vrow * ESZ));
        const rsrc_t rb = make_rsrc(a.beta + t0 * H, (uint32_t)(Lc * H * 4));
        auto part1 = [&]() {
#pragma unroll
            for (int vv = 0; vv < Sh::VPT; ++vv)
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[vv][r] = R4::load(rv, vo[vv] * ESZ, r * vrow * ESZ);
#pragma unroll
            for (int jj = 0; jj < Sh::JPT; ++jj) {
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    if constexpr (FIN)
                        pg[jj][ii] = RW::load(rg, ko[jj] * ESZ, ii * krow * ESZ);
                    else
                        pg[jj][ii] = Raw2<float>::load(rg, ko[jj] * 4, ii * krow * 4);
                }
            }
            pbeta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rb, (tid < C ? tid * H + h : C * H) * 4, 0, 0));
        };
        auto part2 = [&]() {
#pragma unroll
            for (int jj = 0; jj < Sh::JPT; ++jj) {
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    pk[jj][ii] = RW::load(rk, ko[jj] * ESZ, ii * krow * ESZ);
                    pq[jj][ii] = RW::load(rq, ko[jj] * ESZ, ii * krow * ESZ);
                }
            }
        };
        // with the fused input steps P0 reads k and q first (their norms), so they go first
        if (FIN && part == 0) {
            part2();
            part1();
        } else {
            if (part != 2) part1();
            if (part != 1) part2();
        }
    };

    const int64_t nchunks = (L + C - 1) / C;
    // Without the fused input steps, the next chunk's v, g and beta loads go out before P1 and
    // each chunk's operands are recorded after its own state pass; with them (a heavier P0),
    // all loads go out after P1 and the records are copied at the top of the next chunk, which
    // measured faster there.
    constexpr bool kEarlyLoads = !FIN, kLateRecords = !FIN;
    // record the LDS operands (W, Qg, Kd^T, M, gC) of chunk cr of a split segment
    // (each thread copies 16-byte pieces tid, tid + NT, ...: one base offset per row width)
    // M's banded pieces at LDS offsets worked out once (with the fused input steps, where
    // the records are copied at the top of the next chunk, at the copy: fewer registers held)
    using MB = MBands<OP, C>;
    constexpr int MPT = (MB::NP + Sh::NT - 1) / Sh::NT;
    auto m_offset = [&](int m) {
        int r = 0, c = 0;
        if (tid + m * Sh::NT < MB::NP) MB::piece(tid + m * Sh::NT, r, c);
        return r * LDC + c;
    };
    int moff[MPT];
#pragma unroll
    for (int m = 0; m < MPT; ++m) moff[m] = kLateRecords ? m_offset(m) : 0;
    auto record_ops = [&](int64_t cr) {
        using Rc = Record<OP, C, DK, DV>;
        uint8_t *const rp = a.rec + (((int64_t)seg * chains + chain) * a.rec_chunks + cr) * Rc::BYTES;
        constexpr int NT = Sh::NT;
        // the copy offsets are recomputed from the thread index at each copy (a few integer
        // operations) rather than kept across the chunk loop, where they would be spilled
        int tid_ = tid;
        if (!kLateRecords) asm volatile("" : "+v"(tid_));
        auto copy_rows = [&](const OP *src, int ld, auto rows_c, auto per_c, uint8_t *dst) {
            constexpr int rows = decltype(rows_c)::value, per = decltype(per_c)::value;  // per: pieces per row
            const int tid = tid_;
            const int r0 = tid / per, c0 = tid % per;
            const uint8_t *s0 = reinterpret_cast<const uint8_t *>(src + r0 * ld) + c0 * 16;
#pragma unroll
            for (int m = 0; m < (rows * per + NT - 1) / NT; ++m) {
                if ((rows * per) % NT == 0 || tid + m * NT < rows * per)
                    *reinterpret_cast<u32x4 *>(dst + (tid + m * NT) * 16) =
                        *reinterpret_cast<const u32x4 *>(s0 + (m * NT / per) * ld * (int)sizeof(OP));
            }
        };
        using IC = std::integral_constant<int, 0>;
        (void)IC{};
        copy_rows(Wb, LDK, std::integral_constant<int, C>{}, std::integral_constant<int, DK * Rc::SZ / 16>{}, rp + Rc::oW);
        copy_rows(Qg, LDK, std::integral_constant<int, C>{}, std::integral_constant<int, DK * Rc::SZ / 16>{}, rp + Rc::oQ);
        copy_rows(KdT, LDC, std::integral_constant<int, DK>{}, std::integral_constant<int, C * Rc::SZ / 16>{}, rp + Rc::oK);
#pragma unroll
        for (int m = 0; m < MPT; ++m) {
            const int y = tid + m * NT;
            if (MB::NP % NT == 0 || y < MB::NP)
                *reinterpret_cast<u32x4 *>(rp + Rc::oM + 16 * y) =
                    *reinterpret_cast<const u32x4 *>(Mb + (kLateRecords ? moff[m] : m_offset(m)));
        }
        if (tid < DK / 4)
            *reinterpret_cast<f32x4 *>(rp + Rc::oG + 16 * tid) = *reinterpret_cast<const f32x4 *>(gC + 4 * tid);
    };
    if (nchunks > 0) prefetch(tok0, (int)(L < C ? L : C), 0);

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t t0 = tok0 + ci * C;
        const int Lc = (int)((L - ci * C) < C ? (L - ci * C) : C);
        __syncthreads();  // the previous chunk's readers of LDS are done
        if (!kLateRecords && store && ci > 0) record_ops(ci - 1);

        // ---- P0: gates -> within-block decay products (prefix incl., suffix excl.)
        float al0[Sh::JPT][8], al1[Sh::JPT][8], sf0[Sh::JPT][8], sf1[Sh::JPT][8];
        float dk0[Sh::JPT], dk1[Sh::JPT];  // decay of the job's whole 16-token block
        // per-token factors of this thread's 8 tokens: 1/||k|| and scale/||q|| (fused
        // normalisation; otherwise 1 and scale), set after P0
        float rk[8], rq[8];
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
            rk[ii] = 1.f;
            rq[ii] = a.scale;
        }
        // k and q of token ii of job jj (zero past the sequence end), from the prefetch registers
        auto kq = [&](int jj, int ii, float &k0, float &k1, float &q0, float &q1) {
            const f32x2 kk = RW::f32(pk[jj][ii]);
            const f32x2 qq = RW::f32(pq[jj][ii]);
            k0 = kk.x * rk[ii];
            k1 = kk.y * rk[ii];
            q0 = qq.x * rq[ii];
            q1 = qq.y * rq[ii];
        };
        // log-decay of token ii of job jj; fused: from the pre-activation, and g = 0 (no
        // decay) for tokens past the sequence end
        auto gval = [&](int jj, int ii) -> f32x2 {
            if constexpr (FIN) {
                if (16 * jb[jj] + 8 * hh + ii >= Lc) return f32x2{0.f, 0.f};
                const f32x2 x = RW::f32(pg[jj][ii]);
                return f32x2{-grate * softplus_f(x.x + gb0), -grate * softplus_f(x.y + gb1)};
            } else {
                return pg[jj][ii];
            }
        };
        if constexpr (FIN) {
            if (a.f.norm_qk) {
                // per-token sums of squares of k and q over this wave's 64 channels: a butterfly
                // over the 16 lanes of each lane group leaves value bitrev4(lane & 15) in each
                // lane, then the two 16-lane groups of the half-wave are added
                float sq[16];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const f32x2 kk = RW::f32(pk[0][ii]), qq = RW::f32(pq[0][ii]);
                    sq[ii] = kk.x * kk.x + kk.y * kk.y;
                    sq[8 + ii] = qq.x * qq.x + qq.y * qq.y;
                }
                row_transpose_sum16(sq);
                sq[0] += __shfl_xor(sq[0], 16);
                if (!(lane & 16)) {
                    const int l = lane & 15;
                    const int vi = ((l & 1) << 3) | ((l & 2) << 1) | ((l & 4) >> 1) | ((l & 8) >> 3);
                    const int kind = vi >> 3, chalf = jc[0] >> 6;
                    nrm[(2 * kind + chalf) * C + 16 * jb[0] + 8 * hh + (vi & 7)] = sq[0];
                }
            }
        }
        bool ext_local = false;
#pragma unroll
        for (int jj = 0; jj < Sh::JPT; ++jj) {
            float h0 = 1.f, h1 = 1.f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                const f32x2 gg = gval(jj, ii);
                al0[jj][ii] = exp_gate<OP>(gg.x);
                al1[jj][ii] = exp_gate<OP>(gg.y);
            }
#pragma unroll
            for (int ii = 7; ii >= 0; --ii) {  // exclusive suffix within this half
                sf0[jj][ii] = h0;
                sf1[jj][ii] = h1;
                h0 *= al0[jj][ii];
                h1 *= al1[jj][ii];
            }
            const float o0 = __shfl_xor(h0, 32), o1 = __shfl_xor(h1, 32);  // the other half
            float r0 = hh ? o0 : 1.f, r1 = hh ? o1 : 1.f;
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {  // inclusive prefix from the block start
                r0 *= al0[jj][ii];
                r1 *= al1[jj][ii];
                al0[jj][ii] = r0;
                al1[jj][ii] = r1;
                if (!hh) {
                    sf0[jj][ii] *= o0;
                    sf1[jj][ii] *= o1;
                }
            }
            dk0[jj] = h0 * o0;
            dk1[jj] = h1 * o1;
            if (jok[jj] && !hh) {
                Dd[jb[jj] * DK + jc[jj]] = dk0[jj];
                Dd[jb[jj] * DK + jc[jj] + 1] = dk1[jj];
            }
            ext_local |= jok[jj] && (dk0[jj] < extreme_block_decay<OP>() ||
                                     dk1[jj] < extreme_block_decay<OP>());
        }
        if (tid < C) sbeta[tid] = pbeta;
#pragma unroll
        for (int vv = 0; vv < Sh::VPT; ++vv) {  // v^T: 4 columns x 4 consecutive tokens per store
            int tg, cg;
            if (vjob(vv, tg, cg)) {
                f32x4 vr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vr[r] = R4::f32(pv[vv][r]);
                typedef typename MM::frag f4;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f4 *>(Yt + (4 * cg + c) * LDC + yt_col(4 * cg + c, tg)) =
                        MM::from_f32(f32x4{vr[0][c], vr[1][c], vr[2][c], vr[3][c]});
            }
        }
        // work-group OR of the votes with one barrier: a ballot per wave into its own slot
        // (rewritten every chunk; the previous chunk's reads are behind the loop's first
        // barrier), then every thread ORs the slots
        const bool wave_ext = __ballot(ext_local) != 0ull;  // every lane's vote (all lanes active)
        if (lane == 0) sflag[wave] = wave_ext;
        __syncthreads();
        int any_ext = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any_ext |= sflag[w];
        const bool extreme = any_ext != 0;
        // fused normalisation: 1/||.|| of token t from the two channel halves' sums
        auto tok_rnorm = [&](int kind, int t) { return rsqrt_or_zero(nrm[2 * kind * C + t] + nrm[(2 * kind + 1) * C + t]); };
        // this thread's 8 tokens' factors, read where P1 consumes them (short live range)
        auto load_rnorm = [&]() {
            if constexpr (FIN) {
                if (a.f.norm_qk) {
                    const int t = 16 * jb[0] + 8 * hh;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const f32x4 k0 = *reinterpret_cast<const f32x4 *>(nrm + t + 4 * hf);
                        const f32x4 k1 = *reinterpret_cast<const f32x4 *>(nrm + C + t + 4 * hf);
                        const f32x4 q0 = *reinterpret_cast<const f32x4 *>(nrm + 2 * C + t + 4 * hf);
                        const f32x4 q1 = *reinterpret_cast<const f32x4 *>(nrm + 3 * C + t + 4 * hf);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            rk[4 * hf + e] = rsqrt_or_zero(k0[e] + k1[e]);
                            rq[4 * hf + e] = a.scale * rsqrt_or_zero(q0[e] + q1[e]);
                        }
                    }
                }
            }
        };

        // ---- extreme chunks: the diagonal 16x16 blocks of A and M pair by pair in float32
        // (as transposed tiles: lane (lr, q) holds row lr, columns 4q..4q+3),
        // A_ij = beta_i sum_c k_i[c] k_j[c] e^{G_i[c]-G_j[c]}, M_ij likewise with scale q_i,
        // from the cumulative log-decay G summed in float64 (G_i - G_j keeps float32 accuracy
        // however large G grows; no factor leaves the float range for any decay)
        f32x4 dAt = {0.f, 0.f, 0.f, 0.f}, dMt = {0.f, 0.f, 0.f, 0.f};
        if (extreme) {
#pragma unroll
            for (int jj = 0; jj < Sh::JPT; ++jj) {
                double G0[8], G1[8];
                float kk0[8], kk1[8], qq0[8], qq1[8];
                double c0s = 0.0, c1s = 0.0;
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const f32x2 gg = gval(jj, ii);
                    c0s += (double)gg.x;
                    c1s += (double)gg.y;
                    G0[ii] = c0s;
                    G1[ii] = c1s;
                    const f32x2 kk = RW::f32(pk[jj][ii]);
                    const f32x2 qq = RW::f32(pq[jj][ii]);
                    kk0[ii] = kk.x;
                    kk1[ii] = kk.y;
                    qq0[ii] = qq.x;
                    qq1[ii] = qq.y;
                }
                const double f0 = __shfl_xor(c0s, 32), f1 = __shfl_xor(c1s, 32);  // first half
                if (jok[jj]) {
#pragma unroll
                    for (int ii = 0; ii < 8; ++ii) {
                        G0[ii] += hh ? f0 : 0.0;
                        G1[ii] += hh ? f1 : 0.0;
                    }
                    const int c0 = jc[jj], tc = 16 * jb[jj] + 8 * hh;
#pragma unroll
                    for (int ii = 0; ii < 8; ii += 2) {
                        *reinterpret_cast<f64x2 *>(xG + c0 * Sh::LDG + tc + ii) = f64x2{G0[ii], G0[ii + 1]};
                        *reinterpret_cast<f64x2 *>(xG + (c0 + 1) * Sh::LDG + tc + ii) = f64x2{G1[ii], G1[ii + 1]};
                    }
                    Stage<Tin>::store8(xK + c0 * Sh::LDT + tc, kk0);
                    Stage<Tin>::store8(xK + (c0 + 1) * Sh::LDT + tc, kk1);
                    Stage<Tin>::store8(xQ + c0 * Sh::LDT + tc, qq0);
                    Stage<Tin>::store8(xQ + (c0 + 1) * Sh::LDT + tc, qq1);
                }
            }
            __syncthreads();
            const int I = wave % NB, sp = wave / NB;
            f32x4 a4 = {0.f, 0.f, 0.f, 0.f}, m4 = {0.f, 0.f, 0.f, 0.f};
            if (sp < Sh::SPL) {
                constexpr int CH = DK / Sh::SPL;
                const int ti = 16 * I + lr, tj = 16 * I + 4 * q4;  // row token i, column tokens j
#pragma unroll 4
                for (int c = sp * CH; c < (sp + 1) * CH; ++c) {
                    const double gi = xG[c * Sh::LDG + ti];
                    const f64x2 gj01 = *reinterpret_cast<const f64x2 *>(xG + c * Sh::LDG + tj);
                    const f64x2 gj23 = *reinterpret_cast<const f64x2 *>(xG + c * Sh::LDG + tj + 2);
                    const float gd[4] = {(float)(gi - gj01.x), (float)(gi - gj01.y),
                                         (float)(gi - gj23.x), (float)(gi - gj23.y)};
                    const float ki = Stage<Tin>::load1(xK + c * Sh::LDT + ti);
                    const float qi = Stage<Tin>::load1(xQ + c * Sh::LDT + ti);
                    const f32x4 kj = Stage<Tin>::load4(xK + c * Sh::LDT + tj);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ex = kj[e] * exp_gate<OP>(fminf(gd[e], 0.f));
                        a4[e] += ki * ex;
                        m4[e] += qi * ex;
                    }
                }
                if (sp > 0) {
                    float *dst = xP + ((sp - 1) * NB + I) * 512 + lane;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dst[e * 64] = a4[e];
                        dst[(4 + e) * 64] = m4[e];
                    }
                }
            }
            __syncthreads();
            if (sp == 0) {
#pragma unroll
                for (int r = 1; r < Sh::SPL; ++r) {
                    const float *src = xP + ((r - 1) * NB + I) * 512 + lane;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a4[e] += src[e * 64];
                        m4[e] += src[(4 + e) * 64];
                    }
                }
                const float bi = sbeta[16 * I + lr];
                // raw k and q were staged: the fused normalisation scales row i and column j
                const bool nq = FIN && a.f.norm_qk;
                const float rki = nq ? tok_rnorm(0, 16 * I + lr) : 1.f;
                const float rqi = nq ? tok_rnorm(1, 16 * I + lr) : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = 4 * q4 + e;
                    const float rkj = nq ? tok_rnorm(0, 16 * I + col) : 1.f;
                    dAt[e] = lr > col ? bi * a4[e] * rki * rkj : 0.f;
                    dMt[e] = lr >= col ? a.scale * m4[e] * rqi * rkj : 0.f;
                }
            }
            __syncthreads();  // the staging area is overwritten by the operands below
        }

        // the next chunk's v, g and beta (without the fused input steps): their registers are
        // free from here on, and the loads overlap P1
        if (kEarlyLoads && ci + 1 < nchunks) {
            const int64_t rem = L - (ci + 1) * C;
            prefetch(t0 + C, (int)(rem < C ? rem : C), 1);
        }

        // ---- P1: matrix-core operands
        // fp16, ordinary chunks: rows of block I carry a per-channel power of two 2^e_I near
        // D_I^(-1/2) and the right operands paired with block I carry 2^-e_I (exact: products
        // are unchanged). Extreme chunks need no Rd and no balancing: every factor left is
        // <= 1, so fp16 underflow costs at most 2^-25 absolutely.
        {
            const bool bal = kBalance && !extreme;
            auto bexp = [&](float d) { return bal ? (int)floorf(-0.5f * __log2f(d)) : 0; };
            auto st = [&](OP *p, float x, float y) { MM::store_pair(p, x, y); };
#pragma unroll
            for (int jj = 0; jj < Sh::JPT; ++jj) {
                if (!jok[jj]) continue;
                // with Dk >= 64 a wave's jobs share one block: keep b in a scalar register
                const int b = DK >= 64 ? __builtin_amdgcn_readfirstlane(jb[jj]) : jb[jj];
                const int c0 = jc[jj];
                float k0[8], k1[8], q0[8], q1[8];
                load_rnorm();
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) kq(jj, ii, k0[ii], k1[ii], q0[ii], q1[ii]);
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
                const float d0 = dk0[jj], d1 = dk1[jj];
                if (b == 0 && !hh) {
                    gC[c0] = d0 * post0;
                    gC[c0 + 1] = d1 * post1;
                }
                const int e0 = bexp(d0), e1 = bexp(d1);
                const int n0 = b + 1 < NB ? bexp(Dd[(b + 1) * DK + c0]) : 0;
                const int n1 = b + 1 < NB ? bexp(Dd[(b + 1) * DK + c0 + 1]) : 0;
                const float sb0 = ldexpf(1.f, e0), sb1 = ldexpf(1.f, e1);      // left scale
                const float nx0 = ldexpf(1.f, -n0), nx1 = ldexpf(1.f, -n1);    // right, block b+1
                // Rd = Rk * rd (unused, and possibly not finite, in extreme chunks)
                const float rd0 = __builtin_amdgcn_rcpf(d0) * ldexpf(1.f, n0 - e0);
                const float rd1 = __builtin_amdgcn_rcpf(d1) * ldexpf(1.f, n1 - e1);
                const float pq0 = pre0 * ldexpf(1.f, -e0), pq1 = pre1 * ldexpf(1.f, -e1);
                const float po0 = post0 * ldexpf(1.f, n0), po1 = post1 * ldexpf(1.f, n1);
                const int cp = ST::perm(c0);  // c0 even: c0, c0+1 stay adjacent in perm order
                OP xt0[8], xt1[8], kd0[8], kd1[8];
                float btv[8];
                *reinterpret_cast<f32x4 *>(btv) = *reinterpret_cast<const f32x4 *>(sbeta + 16 * b + 8 * hh);
                *reinterpret_cast<f32x4 *>(btv + 4) = *reinterpret_cast<const f32x4 *>(sbeta + 16 * b + 8 * hh + 4);
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const int i = 16 * b + 8 * hh + ii;
                    const float bt = btv[ii];
                    const float lk0 = bt * k0[ii] * al0[jj][ii] * sb0, lk1 = bt * k1[ii] * al1[jj][ii] * sb1;
                    const float lq0 = q0[ii] * al0[jj][ii] * sb0, lq1 = q1[ii] * al1[jj][ii] * sb1;
                    const float rk0 = k0[ii] * sf0[jj][ii] * nx0, rk1 = k1[ii] * sf1[jj][ii] * nx1;
                    st(Lk + i * LDK + c0, lk0, lk1);
                    st(Lq + i * LDK + c0, lq0, lq1);
                    st(Rk + i * LDK + c0, rk0, rk1);
                    st(Rd + i * LDK + c0, rk0 * rd0, rk1 * rd1);
                    MM::store_pair(Qg + i * LDK + cp, lq0 * pq0, lq1 * pq1);
                    xt0[ii] = static_cast<OP>(lk0 * pq0);
                    xt1[ii] = static_cast<OP>(lk1 * pq1);
                    kd0[ii] = static_cast<OP>(rk0 * po0);
                    kd1[ii] = static_cast<OP>(rk1 * po1);
                }
                // right operands of blocks (I, b), I >= b + 2: decay of the blocks in between
                float m0 = ldexpf(1.f, n0), m1 = ldexpf(1.f, n1);  // undo the block b+1 scale
#pragma unroll
                for (int I = 2; I < NB; ++I) {
                    if (I >= b + 2) {
                        m0 *= Dd[(I - 1) * DK + c0];
                        m1 *= Dd[(I - 1) * DK + c0 + 1];
                        const float f0 = m0 * ldexpf(1.f, -bexp(Dd[I * DK + c0]));
                        const float f1 = m1 * ldexpf(1.f, -bexp(Dd[I * DK + c0 + 1]));
                        OP *dst = Rfar + (far_index(NB, b, I) * 16 + 8 * hh) * LDK + c0;
#pragma unroll
                        for (int ii = 0; ii < 8; ++ii) {
                            const float rk0 = k0[ii] * sf0[jj][ii] * nx0, rk1 = k1[ii] * sf1[jj][ii] * nx1;
                            st(dst + ii * LDK, rk0 * f0, rk1 * f1);
                        }
                    }
                }
                typedef typename MM::frag f4;
                const int tcol = 16 * b + 8 * hh;
#pragma unroll
                for (int ii = 0; ii < 8; ii += 4) {
                    const int tp = ST::perm(tcol + ii);  // groups of 4 tokens stay contiguous
                    *reinterpret_cast<f4 *>(Xt + c0 * LDC + tcol + ii) = f4{xt0[ii], xt0[ii + 1], xt0[ii + 2], xt0[ii + 3]};
                    *reinterpret_cast<f4 *>(Xt + (c0 + 1) * LDC + tcol + ii) = f4{xt1[ii], xt1[ii + 1], xt1[ii + 2], xt1[ii + 3]};
                    *reinterpret_cast<f4 *>(KdT + c0 * LDC + tp) = f4{kd0[ii], kd0[ii + 1], kd0[ii + 2], kd0[ii + 3]};
                    *reinterpret_cast<f4 *>(KdT + (c0 + 1) * LDC + tp) = f4{kd1[ii], kd1[ii + 1], kd1[ii + 2], kd1[ii + 3]};
                }
            }
        }

        // the next chunk's k and q (read by P1 up to here): all its inputs are in flight
        if (ci + 1 < nchunks) {
            const int64_t rem = L - (ci + 1) * C;
            prefetch(t0 + C, (int)(rem < C ? rem : C), kEarlyLoads ? 2 : 0);
        }
        __syncthreads();

        // ---- P2: A and M 16x16 blocks, as transposed tiles (lane (lr, q) holds row 16I+lr,
        // columns 16J+4q..+3, which the write-out stores as one vector); the diagonal blocks'
        // waves also invert I + A_II
        auto am_t = [&](bool isM, int I, int J) {
            const OP *left = (isM ? Lq : Lk) + (16 * I + lr) * LDK;
            const OP *right = I == J       ? Rd + (16 * J + lr) * LDK
                              : I == J + 1 ? Rk + (16 * J + lr) * LDK
                                           : Rfar + (far_index(NB, J, I) * 16 + lr) * LDK;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS)
                ST::mma(acc, ST::contig(right, kk, q4), ST::contig(left, kk, q4));
            return acc;
        };
        f32x4 tdiag_t = {0.f, 0.f, 0.f, 0.f}, mdiag_t = {0.f, 0.f, 0.f, 0.f};
        const bool dj = wave < NB;
        if (dj) {
            const int I = wave;
            f32x4 Lt = extreme ? dAt : am_t(false, I, I);  // L^T in accumulator layout
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (lr <= 4 * q4 + e) Lt[e] = 0.f;  // L strictly lower
            // (I + L)^{-1} = (I - L)(I + L^2)(I + L^4)(I + L^8), L strictly lower 16x16
            const f32x4 Lm = mm_tn<OP>(Lt, Id);
            const f32x4 L2 = mm_tn<OP>(Lt, Lm), L2t = mm_tn<OP>(Lm, Lt);
            const f32x4 L4 = mm_tn<OP>(L2t, L2), L4t = mm_tn<OP>(L2, L2t);
            const f32x4 L8 = mm_tn<OP>(L4t, L4);
            const f32x4 P1 = Id - Lm, P1t = Id - Lt;
            const f32x4 P2 = P1 + mm_tn<OP>(P1t, L2), P2t = P1t + mm_tn<OP>(L2, P1t);
            const f32x4 P3 = P2 + mm_tn<OP>(P2t, L4), P3t = P2t + mm_tn<OP>(L4, P2t);
            (void)P3;
            tdiag_t = P3t + mm_tn<OP>(L8, P3t);  // T^T = P3^T + L8^T P3^T
            if (extreme) {
                mdiag_t = dMt;
            } else {
                mdiag_t = am_t(true, I, I);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lr < 4 * q4 + e) mdiag_t[e] = 0.f;  // M lower, diagonal included
            }
        }
        f32x4 offv[Sh::OPW];
        // off-diagonal jobs x = ow + OFFW j, dealt from the last wave down: the waves that also
        // invert a diagonal block (wave < NB) get the fewest
        const int ow = NW - 1 - wave;
#pragma unroll
        for (int j = 0; j < Sh::OPW; ++j) {
            offv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (Sh::NOFF > 0) {
                const int x = ow + Sh::OFFW * j;
                if (ow >= 0 && x < Sh::NOFF) {
                    int I, J;
                    lower_block(x % Sh::NOFFA, I, J);
                    offv[j] = am_t(x >= Sh::NOFFA, I, J);
                }
            }
        }
        __syncthreads();  // A/M operands are dead from here on
        if (dj) {
            const int I = wave, off = (16 * I + lr) * LDC + ST::perm(16 * I + 4 * q4);
            *reinterpret_cast<frag4 *>(Td + off) = MM::from_f32(tdiag_t);
            *reinterpret_cast<frag4 *>(An + off) = MM::from_f32(f32x4{0.f, 0.f, 0.f, 0.f});
            *reinterpret_cast<frag4 *>(Mb + off) = MM::from_f32(mdiag_t);
        }
#pragma unroll
        for (int j = 0; j < Sh::OPW; ++j) {
            const int x = ow + Sh::OFFW * j;
            if (Sh::NOFF > 0 && ow >= 0 && x < Sh::NOFF) {
                int I, J;
                lower_block(x % (Sh::NOFFA > 0 ? Sh::NOFFA : 1), I, J);
                const int off = (16 * I + lr) * LDC + ST::perm(16 * J + 4 * q4);
                if (x >= Sh::NOFFA) *reinterpret_cast<frag4 *>(Mb + off) = MM::from_f32(offv[j]);
                else *reinterpret_cast<frag4 *>(An + off) = MM::from_f32(-offv[j]);
            }
        }
        // zero the upper blocks (I, I+1), I even, of M: the paired-tile steps of M U read them
        if constexpr (TPS == 2) {
            constexpr int NZB = NB / 2;  // even I with I + 1 < NB
            for (int idx = tid; idx < NZB * 64; idx += Sh::NT) {
                const int z = idx / 64, r = (idx / 4) % 16, gq = idx % 4;
                const int I = 2 * z;
                *reinterpret_cast<typename MM::frag *>(Mb + (16 * I + r) * LDC + ST::perm(16 * (I + 1) + 4 * gq)) =
                    MM::from_f32(f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
        __syncthreads();

        // ---- P4: block forward substitution for W (fp16 result, to LDS) and U~ (registers):
        // X_I <- T_II (X_I - sum_{J<I} A_IJ X_J), the sum in paired-tile steps over -A
        auto subst_row = [&](f32x4 *Xs, int I, f32x4 r) {
#pragma unroll
            for (int p = 0; p < (I + TPS - 1) / TPS; ++p)
                ST::mma(r, ST::permuted(An + (16 * I + lr) * LDC, p * KS, q4), ST::regs(&Xs[p * TPS]));
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            MM::mma(x, *reinterpret_cast<const frag4 *>(Td + (16 * I + lr) * LDC + ST::perm(16 * I + 4 * q4)),
                    MM::from_f32(r));
            return x;
        };
#pragma unroll
        for (int j = 0; j < Sh::WPW; ++j) {
            const int cK = wave + NW * j;
            if (cK < KT) {
                f32x4 Wt[NB];
#pragma unroll
                for (int I = 0; I < NB; ++I) Wt[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    const f32x4 w = subst_row(Wt, I, MM::to_f32(MM::load(Xt + (16 * cK + lr) * LDC + 16 * I + 4 * q4)));
                    Wt[I] = w;
                    // row-major store of the tile through its transpose: 4 channels per lane
                    *reinterpret_cast<frag4 *>(Wb + (16 * I + lr) * LDK + ST::perm(16 * cK + 4 * q4)) =
                        MM::from_f32(mm_tn<OP>(w, Id));
                }
            }
        }
        f32x4 Ur[CPW][NB];
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int cv = wave + NW * j;
#pragma unroll
            for (int I = 0; I < NB; ++I) Ur[j][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 0; I < NB; ++I)
                Ur[j][I] = subst_row(Ur[j], I, MM::to_f32(MM::load(Yt + (16 * cv + lr) * LDC + yt_col(16 * cv + lr, 4 * I + q4))) *
                                                   *reinterpret_cast<const f32x4 *>(sbeta + 16 * I + 4 * q4));
        }
        __syncthreads();

        // ---- split segments after the first: record U~ of this chunk (the LDS operands are
        // recorded after P5, where fewer registers are live and waves done with P5 copy while
        // the others finish; with the fused input steps, at the top of the next chunk)
        if (store && owns) {
            using Rc = Record<OP, C, DK, DV>;
            uint8_t *const rp = a.rec + (((int64_t)seg * chains + chain) * a.rec_chunks + ci) * Rc::BYTES;
#pragma unroll
            for (int j = 0; j < CPW; ++j)
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    *reinterpret_cast<frag4 *>(rp + Rc::oU + (((wave + NW * j) * NB + I) * 64 + lane) * 4 * Rc::SZ) =
                        MM::from_f32(Ur[j][I]);
        }

        // ---- P5: state pass, registers only: U = U~ - W S; O = Qg S + M U; S' = gC S + Kd^T U
        if (owns) {
            const rsrc_t ro = make_rsrc(static_cast<float *>(a.o) + t0 * vrow, (uint32_t)(Lc * vrow * 4));
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int cv = wave + NW * j;
                const int oo = (4 * q4 * vrow + h * DV + 16 * cv + lr) * 4;
                typename ST::frag sfr[DK / KS];
#pragma unroll
                for (int p = 0; p < DK / KS; ++p) sfr[p] = ST::regs(&S[j][p * TPS]);
                f32x4 U[NB];
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < DK / KS; ++p)
                        ST::mma(ws, ST::permuted(Wb + (16 * I + lr) * LDK, p * KS, q4), sfr[p]);
                    U[I] = Ur[j][I] - ws;
                }
                typename ST::frag ufr[C / KS];
#pragma unroll
                for (int p = 0; p < C / KS; ++p) ufr[p] = ST::regs(&U[p * TPS]);
                auto o_tile = [&](int I) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < DK / KS; ++p)
                        ST::mma(o, ST::permuted(Qg + (16 * I + lr) * LDK, p * KS, q4), sfr[p]);
#pragma unroll
                    for (int p = 0; p <= I / TPS; ++p)
                        ST::mma(o, ST::permuted(Mb + (16 * I + lr) * LDC, p * KS, q4), ufr[p]);
                    return o;
                };
                if constexpr (FOUT) {
                    if (!store) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) ostage_tile<C, DV, NW>(Ob, I, o_tile(I));
                    }
                }
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    if (store || FOUT) break;  // recording segments: the outputs come from the replay
                    const f32x4 o = o_tile(I);
                    // rows past the chunk end are dropped by the buffer bound
                    const int so = 16 * I * vrow * 4;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.x), ro, oo, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.y), ro, oo, so + vrow * 4, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.z), ro, oo, so + 2 * vrow * 4, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.w), ro, oo, so + 3 * vrow * 4, 0);
                }
#pragma unroll
                for (int r = 0; r < KT; ++r) {
                    f32x4 acc = S[j][r] * *reinterpret_cast<const f32x4 *>(gC + 16 * r + 4 * q4);
#pragma unroll
                    for (int p = 0; p < C / KS; ++p)
                        ST::mma(acc, ST::permuted(KdT + (16 * r + lr) * LDC, p * KS, q4), ufr[p]);
                    S[j][r] = acc;
                }
            }
        }
        if constexpr (FOUT) {
            if (!store) {  // uniform per workgroup
                u32x4 zr[2];
                load_ogate<C, DV, NW>(a, t0, Lc, h, zr);
                __syncthreads();  // every wave's output tile is staged
                onorm_rows<C, DV, NW>(a, Ob, sgain, zr, t0, Lc, h);
            }
        }
        if (kLateRecords && store) record_ops(ci);
    }

    if (!kLateRecords && store && nchunks > 0) {
        __syncthreads();
        record_ops(nchunks - 1);
    }


    float *dst = nullptr;
    if (STORE)  // split: segment p's final state (from the initial state for p = 0, else zero)
        dst = seg < segs - 1 ? a.ws_r + ((int64_t)seg * chains + chain) * DK * DV : nullptr;
    else if (a.s_out)
        dst = a.s_out + sbase;
    if (owns && dst) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            const int ct = wave + NW * j;
            constexpr int ld = DV;
            const int col = 16 * ct + lr;
#pragma unroll
            for (int r = 0; r < KT; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(int64_t)(16 * r + 4 * q4 + e) * ld + col] = S[j][r][e];
        }
    }
}


// Replay of split segments from their records (no inputs are read again).
// XMODE: segment p's linear part X_p (state X = I, U~ = 0, no outputs) -> ws_x[p], for
//        p = 1 .. nseg-2.
// else:  segment p from its true start state S_p = ws_s[p]: outputs, and the final state of
//        the last segment, for p = out_from .. nseg-1 (with out_from = 1 segment 0 wrote its
//        outputs in the forward).
// The state pass is the forward kernel's: U = U~ - W S; O = Qg S + M U; S' = gC S + Kd^T U.
// Each chunk's staged operands are loaded into registers one chunk ahead.
template <typename OP, int C, int DK, int DV, int NW, bool XMODE, bool FOUT = false>
__global__ __launch_bounds__(64 * NW, 1) void replay_kernel(ChunkArgs a) {
    using Sh = ChunkShape<OP, 2, C, DK, DV, NW>;
    using Rc = Record<OP, C, DK, DV>;
    using MM = Mma<OP>;
    using ST = Step<OP>;
    constexpr int NB = Sh::NB, LDK = Sh::LDK, LDC = Sh::LDC, KT = Sh::KT, CPW = Sh::CPW,
                  KS = ST::KS, TPS = ST::TPS, NT = 64 * NW, SZ = Rc::SZ;
    static_assert(DK == DV || !XMODE, "X lives in the state's column tiles");
    static_assert(!FOUT || (!XMODE && Sh::NCT == NW && CPW == 1), "fused output shape");
    constexpr int WROW = DK * SZ, KROW = C * SZ;  // record row bytes
    // 16-byte pieces to stage: W, Qg, Kd^T, M (XMODE: W and Kd^T)
    constexpr int N16 = (XMODE ? Rc::oQ + (Rc::oM - Rc::oK) : Rc::OPS) / 16;
    static_assert(Rc::oM % (16 * 64) == 0, "a wave's staged pieces of M lie in one band");
    constexpr int PPT = (N16 + NT - 1) / NT;                      // pieces per thread

    __shared__ __attribute__((aligned(16))) OP Wl[C * LDK];
    __shared__ __attribute__((aligned(16))) OP Ql[XMODE ? 8 : C * LDK];
    __shared__ __attribute__((aligned(16))) OP Kl[DK * LDC];
    __shared__ __attribute__((aligned(16))) OP Ml[XMODE ? 8 : C * LDC];
    __shared__ __attribute__((aligned(16))) float gl[DK];
    __shared__ __attribute__((aligned(16))) float Ob[FOUT ? C * ONorm<C, DV, NW>::LD : 4];  // output staging
    __shared__ __attribute__((aligned(16))) float sgain[FOUT ? DV : 4];
    __shared__ __attribute__((aligned(16))) float Xs[XMODE ? DK * DV : 4];  // X_p, reordered

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, q4 = lane >> 4;
    const int H = a.H, chains = a.n_seqs * H;
    // segments 1 .. nseg-2 (X) or out_from .. nseg-1 (outputs)
    const int first = XMODE ? 1 : a.out_from;
    const int segs = XMODE ? a.nseg - 2 : a.nseg - a.out_from;
    if (segs <= 0 || (int)blockIdx.x >= chains * segs) return;
    const int chain = blockIdx.x / segs, p = first + (int)blockIdx.x % segs;
    const int n = chain / H, h = chain % H;
    const int64_t tok0 = (int64_t)n * a.seq_len + (int64_t)p * a.seg_len;
    const int64_t rem = (int64_t)a.seq_len - (int64_t)p * a.seg_len;
    const int64_t L = rem < a.seg_len ? rem : a.seg_len;
    const int nch = (int)((L + C - 1) / C);
    const uint8_t *const rbase = a.rec + ((int64_t)p * chains + chain) * a.rec_chunks * Rc::BYTES;
    const int vrow = H * DV;

    const bool owns = wave < Sh::NCT;
    if (FOUT && tid < DV) sgain[tid] = a.f.ow[tid];  // read after the loop's first barrier
    f32x4 S[CPW][KT];
    const float *sinit = XMODE ? nullptr : a.ws_s + ((int64_t)p * chains + chain) * DK * DV;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int ct = wave + NW * j;
#pragma unroll
        for (int r = 0; r < KT; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * r + 4 * q4 + e;
                S[j][r][e] = !owns ? 0.f
                             : XMODE ? (row == 16 * ct + lr ? 1.f : 0.f)
                                     : sinit[(int64_t)row * DV + 16 * ct + lr];
            }
    }

    // staged piece x -> its byte offset in the record and its LDS address
    auto rec_off = [](int x) {
        const int b = 16 * x;
        return (XMODE && b >= Rc::oQ) ? b - Rc::oQ + Rc::oK : b;
    };
    // LDS offsets of the pieces of M this thread stages, worked out once (M's pieces start at
    // a multiple of 64, so each wave's pieces are all of M or all before it)
    int mlo[PPT];
#pragma unroll
    for (int m = 0; m < PPT; ++m) {
        const int x = tid + m * NT;
        int r = 0, c = 0;
        if (!XMODE && x >= Rc::oM / 16 && x < N16) MBands<OP, C>::piece(x - Rc::oM / 16, r, c);
        mlo[m] = r * LDC + c;
    }
    auto lds_of = [&](int b, int m) -> OP * {
        if (b < Rc::oQ) return Wl + (b / WROW) * LDK + (b % WROW) / SZ;
        if (b < Rc::oK) return Ql + ((b - Rc::oQ) / WROW) * LDK + ((b - Rc::oQ) % WROW) / SZ;
        if (b < Rc::oM) return Kl + ((b - Rc::oK) / KROW) * LDC + ((b - Rc::oK) % KROW) / SZ;
        return Ml + mlo[m];
    };
    u32x4 pre[PPT];
    f32x4 preg = {0.f, 0.f, 0.f, 0.f};
    typename MM::frag preu[CPW][NB];
    if (nch > 0)
        {
            const uint8_t *rp_ = rbase + (int64_t)(0) * Rc::BYTES;
#pragma unroll
            for (int m = 0; m < PPT; ++m) {
                const int x = tid + m * NT;
                pre[m] = *reinterpret_cast<const u32x4 *>(rp_ + rec_off(x < N16 ? x : 0));
            }
            if (tid < DK / 4) preg = *reinterpret_cast<const f32x4 *>(rp_ + Rc::oG + 16 * tid);
            if (!XMODE && owns) {
#pragma unroll
                for (int j = 0; j < CPW; ++j)
#pragma unroll
                    for (int I = 0; I < NB; ++I)
                        preu[j][I] = *reinterpret_cast<const typename MM::frag *>(
                            rp_ + Rc::oU + (((wave + NW * j) * NB + I) * 64 + lane) * 4 * SZ);
            }
        }


    for (int ci = 0; ci < nch; ++ci) {
        __syncthreads();  // the previous chunk's readers of LDS are done
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
            const int x = tid + m * NT;
            if (x < N16) *reinterpret_cast<u32x4 *>(lds_of(rec_off(x), m)) = pre[m];
        }
        if (tid < DK / 4) *reinterpret_cast<f32x4 *>(gl + 4 * tid) = preg;
        f32x4 Ur[CPW][NB];
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int I = 0; I < NB; ++I) Ur[j][I] = XMODE ? f32x4{0.f, 0.f, 0.f, 0.f} : MM::to_f32(preu[j][I]);
        __syncthreads();
        if (ci + 1 < nch)  // in flight during the state pass
            {
                const uint8_t *rp_ = rbase + (int64_t)(ci + 1) * Rc::BYTES;
#pragma unroll
                for (int m = 0; m < PPT; ++m) {
                    const int x = tid + m * NT;
                    pre[m] = *reinterpret_cast<const u32x4 *>(rp_ + rec_off(x < N16 ? x : 0));
                }
                if (tid < DK / 4) preg = *reinterpret_cast<const f32x4 *>(rp_ + Rc::oG + 16 * tid);
                if (!XMODE && owns) {
#pragma unroll
                    for (int j = 0; j < CPW; ++j)
#pragma unroll
                        for (int I = 0; I < NB; ++I)
                            preu[j][I] = *reinterpret_cast<const typename MM::frag *>(
                                rp_ + Rc::oU + (((wave + NW * j) * NB + I) * 64 + lane) * 4 * SZ);
                }
            }


        const int64_t t0 = tok0 + (int64_t)ci * C;
        const int Lc = (int)((L - (int64_t)ci * C) < C ? (L - (int64_t)ci * C) : C);
        if (owns) {
            const rsrc_t ro = make_rsrc(static_cast<float *>(a.o) + t0 * vrow, XMODE ? 0u : (uint32_t)(Lc * vrow * 4));
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int cv = wave + NW * j;
                const int oo = (4 * q4 * vrow + h * DV + 16 * cv + lr) * 4;
                typename ST::frag sfr[DK / KS];
#pragma unroll
                for (int pp = 0; pp < DK / KS; ++pp) sfr[pp] = ST::regs(&S[j][pp * TPS]);
                f32x4 U[NB];
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pp = 0; pp < DK / KS; ++pp)
                        ST::mma(ws, ST::permuted(Wl + (16 * I + lr) * LDK, pp * KS, q4), sfr[pp]);
                    U[I] = Ur[j][I] - ws;
                }
                typename ST::frag ufr[C / KS];
#pragma unroll
                for (int pp = 0; pp < C / KS; ++pp) ufr[pp] = ST::regs(&U[pp * TPS]);
                if constexpr (!XMODE) {
                    auto o_tile = [&](int I) {
                        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int pp = 0; pp < DK / KS; ++pp)
                            ST::mma(o, ST::permuted(Ql + (16 * I + lr) * LDK, pp * KS, q4), sfr[pp]);
#pragma unroll
                        for (int pp = 0; pp <= I / TPS; ++pp)
                            ST::mma(o, ST::permuted(Ml + (16 * I + lr) * LDC, pp * KS, q4), ufr[pp]);
                        return o;
                    };
                    if constexpr (FOUT) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) ostage_tile<C, DV, NW>(Ob, I, o_tile(I));
                    }
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        if (FOUT) break;
                        const f32x4 o = o_tile(I);
                        const int so = 16 * I * vrow * 4;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.x), ro, oo, so, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.y), ro, oo, so + vrow * 4, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.z), ro, oo, so + 2 * vrow * 4, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o.w), ro, oo, so + 3 * vrow * 4, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < KT; ++r) {
                    f32x4 acc = S[j][r] * *reinterpret_cast<const f32x4 *>(gl + 16 * r + 4 * q4);
#pragma unroll
                    for (int pp = 0; pp < C / KS; ++pp)
                        ST::mma(acc, ST::permuted(Kl + (16 * r + lr) * LDC, pp * KS, q4), ufr[pp]);
                    S[j][r] = acc;
                }
            }
        }
        if constexpr (FOUT) {
            u32x4 zr[2];
            load_ogate<C, DV, NW>(a, t0, Lc, h, zr);
            __syncthreads();  // every wave's output tile is staged
            onorm_rows<C, DV, NW>(a, Ob, sgain, zr, t0, Lc, h);
        }
    }

    if constexpr (XMODE) {
        // X_p as the combine reads it, built in LDS and then copied out in 16-byte pieces.
        // Float32 path: element (row 16 i + m, column 16 s + 4 g + j) at float
        // ((i * KT + s) * 64 + m + 16 g) * 4 + j. Otherwise split into bf16 head and tail:
        // element (row 16 i + m, column 32 s + 8 g + j) at bf16 (((i * KT/2 + s) * 2 + h) * 64
        // + m + 16 g) * 8 + j, h = 0 for the head and 1 for the tail.
        if (owns) {
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int ct = wave + NW * j;
#pragma unroll
                for (int r = 0; r < KT; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = S[j][r][e];
                        if constexpr (std::is_same<OP, float>::value) {
                            Xs[((r * KT + ct) * 64 + 4 * q4 + e + 16 * (lr >> 2)) * 4 + (lr & 3)] = v;
                        } else {
                            const int o = (((r * (KT / 2) + (ct >> 1)) * 2) * 64 + 4 * q4 + e +
                                           16 * (2 * (ct & 1) + (lr >> 3))) * 8 + (lr & 7);
                            const __bf16 hd = f32_to_bf16(v);
                            const __bf16 tl = f32_to_bf16(v - static_cast<float>(hd));
                            reinterpret_cast<__bf16 *>(Xs)[o] = hd;
                            reinterpret_cast<__bf16 *>(Xs)[o + 64 * 8] = tl;
                        }
                    }
            }
        }
        __syncthreads();
        u32x4 *const xd = reinterpret_cast<u32x4 *>(a.ws_x + ((int64_t)p * chains + chain) * DK * DV);
        for (int x = tid; x < DK * DV / 4; x += NT) xd[x] = reinterpret_cast<const u32x4 *>(Xs)[x];
        return;
    }
    float *dst = nullptr;
    if (a.s_out && p == a.nseg - 1) dst = a.s_out + (int64_t)chain * DK * DV;
    if (owns && dst) {
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int r = 0; r < KT; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(int64_t)(16 * r + 4 * q4 + e) * DV + 16 * (wave + NW * j) + lr] = S[j][r][e];
    }
}

// Split combine: S_0 = the initial state (or zero), S_1 = R_0 (segment 0 ran from the
// initial state), then S_{p+1} = X_p S_p + R_p. One workgroup per (chain, 16-column block).
// Each step is a [Dk x Dk] x [Dk x 16] product on the matrix cores, float32-accurate: with
// SPLIT, each factor is a bf16 head plus a bf16 tail and the three leading cross products
// are summed (16x16x32 bf16 instructions); otherwise float32 instructions. Every wave owns
// 16-row tiles of the result and keeps them in its accumulators. The X replay stores X_p in
// this product's A-operand order (with SPLIT already split, heads and tails in separate
// 16-byte pieces), so a wave loads its own fragments straight into registers with
// contiguous 16-byte loads, two steps ahead, into the registers the previous step has
// finished with (X and R do not depend on S); the loads go out group by group between the
// products, so that the memory pipeline's queue does not hold up the matrix cores. The
// running block S_p reaches the other waves through LDS, transposed so that a B fragment is
// contiguous (with SPLIT already split by its writer), in two buffers by step parity: one
// barrier per step. Writes ws_s[p], p < nseg.
template <int DK, int DV, bool SPLIT>
__global__ __launch_bounds__(256) void split_combine_kernel(ChunkArgs a) {
    constexpr int RT = DK / 16;           // 16-row tiles of the result
    constexpr int TPW = (RT + 3) / 4;     // tiles per wave: wave w owns tiles w, w + 4, ...
    constexpr int KW = SPLIT ? 32 : 16;   // reduction indices per instruction group
    constexpr int NK = DK / KW;           // ... groups per product
    constexpr int NP = SPLIT ? 2 : 1;     // 16-byte pieces per lane and group (head, tail)
    constexpr int LDT = DK + 4;           // padded row of the transposed running block (floats)
    constexpr int LDH = DK + 8;           // ... of its bf16 head and tail
    static_assert(DK % KW == 0, "split maps need Dk a multiple of 32");
    __shared__ __attribute__((aligned(16))) float curT[SPLIT ? 1 : 2][16 * LDT];
    __shared__ __attribute__((aligned(16))) __bf16 curH[SPLIT ? 2 : 1][2][16 * LDH];
    const int chains = a.n_seqs * a.H;
    // Workgroup b runs on XCD b % 8: a chain's DV / 16 column blocks all take the same
    // residue, so they share one XCD's L2 and each X_p comes from HBM once per chain, not once
    // per column block (the grid is rounded up to whole groups of 8 chains)
    constexpr int NCB = DV / 16;
    const int kb = (int)blockIdx.x >> 3;
    const int chain = (kb / NCB) * 8 + (int)(blockIdx.x & 7), cb = kb % NCB;
    if (chain >= chains) return;
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // tile t of this wave exists (always, once there are at least four tiles)
    auto has = [&](int t) { return RT % 4 == 0 || wave + 4 * t < RT; };
    const int nseg = a.nseg;
    const int64_t cstride = (int64_t)chains * DK * DV;
    // this lane's elements of a state-shaped [DK x DV] block: rows 16 i + 4 q4 + e of the
    // wave's tiles i, column 16 cb + lr
    const int64_t lane_off = (int64_t)chain * DK * DV + (int64_t)(4 * q4) * DV + 16 * cb + lr;
    u32x4 x[3][TPW][NK][NP];  // A fragments of X_{p-1}, X_p, X_{p+1}, by p mod 3
    f32x4 r[3][TPW];          // this lane's values of R_{p-1}, R_p, R_{p+1}
    // Loads of X_p's group k (and with k = 0, R_p). Every step issues the same loads (p is
    // clamped into the maps that exist, 0 .. nseg-2, and a clamped load is never used), so
    // the wait before each use counts exactly the loads issued after it.
    auto fetch = [&](u32x4 (&xb)[TPW][NK][NP], f32x4 (&rb)[TPW], int p, int k) {
        p = p < nseg - 2 ? p : nseg - 2;
        const u32x4 *X = reinterpret_cast<const u32x4 *>(a.ws_x + ((int64_t)p * chains + chain) * DK * DK);
        const float *R = a.ws_r + (int64_t)p * cstride + lane_off;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int i = wave + 4 * t;
            if (has(t)) {
#pragma unroll
                for (int h = 0; h < NP; ++h) xb[t][k][h] = X[((i * NK + k) * NP + h) * 64 + lane];
                if (k == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rb[t][e] = R[(int64_t)(16 * i + e) * DV];
                }
            }
        }
    };
    f32x4 acc[TPW];  // this wave's tiles of S_p
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int i = wave + 4 * t;
        if (has(t)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t o = lane_off + (int64_t)(16 * i + e) * DV;
                a.ws_s[o] = a.s0 ? a.s0[o] : 0.f;  // S_0
                acc[t][e] = a.ws_r[o];             // S_1 = R_0
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        fetch(x[1], r[1], 1, k);
        fetch(x[2], r[2], 2, k);
    }
    // One step: write S_p; if another follows, S_{p+1} = X_p S_p + R_p from xb, rb, while
    // X_{p+2}, R_{p+2} go out into xn, rn (step p-1's registers). Returns false after the
    // last state.
    auto step = [&](u32x4 (&xb)[TPW][NK][NP], f32x4 (&rb)[TPW], u32x4 (&xn)[TPW][NK][NP],
                    f32x4 (&rn)[TPW], int p) -> bool {
        float *const sp = a.ws_s + (int64_t)p * cstride;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int i = wave + 4 * t;
            if (has(t)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[lane_off + (int64_t)(16 * i + e) * DV] = acc[t][e];
            }
        }
        if (p + 1 >= nseg) return false;
        // S_p into LDS: row lr of the transposed block holds column lr of S_p
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int i = wave + 4 * t;
            if (has(t)) {
                if constexpr (SPLIT) {
                    bf16x4 hd, tl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hd[e] = f32_to_bf16(acc[t][e]);
                        tl[e] = f32_to_bf16(acc[t][e] - static_cast<float>(hd[e]));
                    }
                    *reinterpret_cast<bf16x4 *>(curH[p & 1][0] + lr * LDH + 16 * i + 4 * q4) = hd;
                    *reinterpret_cast<bf16x4 *>(curH[p & 1][1] + lr * LDH + 16 * i + 4 * q4) = tl;
                } else {
                    *reinterpret_cast<f32x4 *>(curT[p & 1] + lr * LDT + 16 * i + 4 * q4) = acc[t];
                }
            }
        }
        __syncthreads();  // S_p complete in LDS (the other buffer's readers finished a step ago)
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] = rb[t];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            fetch(xn, rn, p + 2, k);
            if constexpr (SPLIT) {
                // B: rows 32 k + 8 q4 .. + 7 of S_p's column lr, head and tail
                const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(curH[p & 1][0] + lr * LDH + 32 * k + 8 * q4);
                const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(curH[p & 1][1] + lr * LDH + 32 * k + 8 * q4);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    if (has(t)) {
                        const bf16x8 ah = __builtin_bit_cast(bf16x8, xb[t][k][0]);
                        const bf16x8 al = __builtin_bit_cast(bf16x8, xb[t][k][NP - 1]);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t], 0, 0, 0);
                    }
            } else {
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(curT[p & 1] + lr * LDT + 16 * k + 4 * q4);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    if (has(t)) Mma<float>::mma(acc[t], __builtin_bit_cast(f32x4, xb[t][k][0]), bv);
            }
        }
        return true;
    };
    for (int p = 1;; p += 3) {
        if (!step(x[1], r[1], x[0], r[0], p)) break;
        if (!step(x[2], r[2], x[1], r[1], p + 1)) break;
        if (!step(x[0], r[0], x[2], r[2], p + 2)) break;
    }
}

// Longest-first order of the packed sequences: order[rank] = n, rank = the number of longer
// sequences plus the equal ones before n. One thread per sequence, O(N^2) comparisons.
__global__ __launch_bounds__(256) void order_kernel(const int32_t *cu, int32_t N, int32_t *order) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    const int32_t li = cu[i + 1] - cu[i];
    int rank = 0;
    for (int j = 0; j < N; ++j) {
        const int32_t lj = cu[j + 1] - cu[j];
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

// FIN: the fused input steps; FOUT (unsplit forward and output replay): the output norm.
template <typename Tin, typename OP, int C, int DK, int DV, int NW, bool FIN, bool FOUT>
hipError_t launch_t(const ChunkArgs &a, hipStream_t stream) {
    const int64_t chains = (int64_t)a.n_seqs * a.H;
    if (chains * (a.seg_len ? a.nseg : 1) > 0x7fffffff) return hipErrorInvalidValue;
    constexpr int FUSE = (FIN ? 1 : 0) | (FOUT ? 2 : 0);
    if (!a.seg_len) {
        hipLaunchKernelGGL((chunk_fwd_kernel<Tin, OP, C, DK, DV, NW, false, FUSE>), dim3((unsigned)chains),
                           dim3(64 * NW), 0, stream, a);
        return hipGetLastError();
    }
    hipError_t e;
    if constexpr (DK == DV) {
        // with the output norm every segment's outputs come from the replay (its epilogue
        // is hidden there behind the record reads); otherwise segment 0 writes its own
        hipLaunchKernelGGL((chunk_fwd_kernel<Tin, OP, C, DK, DV, NW, true, FUSE & 1>),
                           dim3((unsigned)(chains * a.nseg)), dim3(64 * NW), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (a.nseg > 2) {
            hipLaunchKernelGGL((replay_kernel<OP, C, DK, DV, NW, true>),
                               dim3((unsigned)(chains * (a.nseg - 2))), dim3(64 * NW), 0, stream, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((split_combine_kernel<DK, DV, !std::is_same<OP, float>::value>), dim3((unsigned)((chains + 7) / 8 * 8 * (DV / 16))),
                           dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((replay_kernel<OP, C, DK, DV, NW, false, FOUT>),
                           dim3((unsigned)(chains * (a.nseg - a.out_from))), dim3(64 * NW), 0, stream, a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;  // the split is planned only for Dk == Dv
    }
}

// Sequence-split plan for B sequences of T tokens. One workgroup fills a compute unit (its
// LDS), so a launch runs in ceil(blocks / CUs) rounds. Without a split that is
// ceil(chains / CUs) rounds of the whole sequence. Cut into P segments, the forward pass runs
// all segments at once (1/P of the sequence per round); the replay passes then re-run the
// state pass alone from the records: X for segments 1..P-2, outputs for segments 1..P-1.
// P is picked by that estimate, in chunk times.
struct SplitPlan {
    int nseg = 1, seg_len = 0;
    size_t bytes = 0;
};

// Compute units of the current device, queried once per device (callers on several host
// threads may race to fill a slot; they all store the same value).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Bytes of one chunk record, from the layout the kernels use (0 for a shape not built).
int64_t record_bytes(int32_t in_dtype, int32_t C, int32_t Dk, int32_t Dv) {
    if (Dk != Dv) return 0;
    if (in_dtype == 1) return C == 64 && Dk == 128 ? Record<_Float16, 64, 128, 128>::BYTES : 0;
    if (C == 16 && Dk == 16) return Record<float, 16, 16, 16>::BYTES;
    if (C == 16 && Dk == 32) return Record<float, 16, 32, 32>::BYTES;
    if (C == 32 && Dk == 128) return Record<float, 32, 128, 128>::BYTES;
    if (C == 64 && Dk == 32) return Record<float, 64, 32, 32>::BYTES;
    if (C == 64 && Dk == 64) return Record<float, 64, 64, 64>::BYTES;
    return 0;
}

SplitPlan plan_split(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                     int32_t in_dtype) {
    SplitPlan sp;
    const int64_t chains = (int64_t)B * H;
    const int64_t cus = device_cus();
    if (chains <= 0 || cus <= 0 || T <= 0 || Dk != Dv) return sp;
    const int64_t nchunks = ((int64_t)T + chunk - 1) / chunk;
    auto rounds = [&](int64_t blocks) { return (double)((blocks + cus - 1) / cus); };
    constexpr double kXCost = 0.15;     // replay chunk, X pass, vs forward chunk
    constexpr double kOutCost = 0.3;    // replay chunk, output pass
    constexpr double kFixedCost = 4.0;  // extra launches and the combine, in chunk times
    double best = rounds(chains) * (double)nchunks;
    for (int64_t P = 2; P <= 16; ++P) {
        const int64_t per = (nchunks + P - 1) / P;  // chunks per segment
        if (per < 4) break;
        const int64_t nseg = (nchunks + per - 1) / per;
        if (nseg < 2) continue;
        const double cost = rounds(chains * nseg) * per + rounds(chains * (nseg - 2)) * per * kXCost +
                            rounds(chains * (nseg - 1)) * per * kOutCost + kFixedCost + 0.25 * (nseg - 2);
        if (cost < (sp.nseg > 1 ? 0.98 : 0.9) * best) {  // a split must gain 10%; more segments 2%
            best = cost;
            sp.nseg = (int)nseg;
            sp.seg_len = (int)(per * chunk);
        }
    }
    if (sp.nseg < 2) return SplitPlan{};
    const int64_t rec_chunks = sp.seg_len / chunk;
    sp.bytes = (size_t)(sp.nseg - 1) * chains * ((size_t)Dk * Dv + (size_t)Dk * Dk) * 4 +  // R, X
               (size_t)sp.nseg * chains * Dk * Dv * 4 +                                  // S_p
               (size_t)sp.nseg * chains * rec_chunks * record_bytes(in_dtype, chunk, Dk, Dv);
    return sp;
}

}  // namespace

constexpr int32_t kMaxOrderedSeqs = 4096;  // packed batches ordered longest first up to this

bool chunk_fwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv) {
    if (Dk != Dv) return false;
    if (in_dtype == 1) return chunk == 64 && Dk == 128;
    if (in_dtype == 0)
        return (chunk == 16 && (Dk == 16 || Dk == 32)) || (chunk == 32 && Dk == 128) ||
               (chunk == 64 && (Dk == 32 || Dk == 64));
    return false;
}

size_t chunk_fwd_split_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                             int32_t chunk, int32_t in_dtype, int32_t num_seqs) {
    if (!chunk_fwd_supported(in_dtype, chunk, Dk, Dv)) return 0;
    if (num_seqs != B)  // packed batch: the longest-first order
        return num_seqs > 1 && num_seqs <= kMaxOrderedSeqs ? (size_t)num_seqs * sizeof(int32_t) : 0;
    return plan_split(B, T, H, Dk, Dv, chunk, in_dtype).bytes;
}

bool chunk_fwd_fused_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv) {
    return in_dtype == 1 && chunk == 64 && Dk == 128 && Dv == 128;
}

hipError_t launch_chunk_fwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv,
                            const ChunkArgs &args, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    if (!chunk_fwd_supported(in_dtype, chunk, Dk, Dv)) return hipErrorInvalidValue;
    if ((args.f.gx || args.f.og) && !chunk_fwd_fused_supported(in_dtype, chunk, Dk, Dv)) return hipErrorInvalidValue;
    if (args.f.og && !args.f.gx) return hipErrorInvalidValue;
    if (args.n_seqs == 0) return hipSuccess;
    ChunkArgs a = args;
    a.seg_len = 0;
    a.nseg = 1;
    if (a.cu_seqlens && workspace && a.n_seqs <= kMaxOrderedSeqs &&
        workspace_bytes >= (size_t)a.n_seqs * sizeof(int32_t)) {
        int32_t *order = static_cast<int32_t *>(workspace);
        hipLaunchKernelGGL(order_kernel, dim3((unsigned)((a.n_seqs + 255) / 256)), dim3(256), 0, stream,
                           a.cu_seqlens, a.n_seqs, order);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        a.order = order;
    }
    if (!a.cu_seqlens && workspace) {
        const SplitPlan sp = plan_split(a.n_seqs, a.seq_len, a.H, Dk, Dv, chunk, in_dtype);
        if (sp.nseg > 1 && workspace_bytes >= sp.bytes) {
            const size_t chains = (size_t)a.n_seqs * a.H;
            a.seg_len = sp.seg_len;
            a.nseg = sp.nseg;
            a.ws_r = static_cast<float *>(workspace);
            a.ws_x = a.ws_r + (size_t)(sp.nseg - 1) * chains * Dk * Dv;
            a.ws_s = a.ws_x + (size_t)(sp.nseg - 1) * chains * Dk * Dk;
            a.rec = reinterpret_cast<uint8_t *>(a.ws_s + (size_t)sp.nseg * chains * Dk * Dv);
            a.rec_chunks = sp.seg_len / chunk;
            a.out_from = a.f.og ? 0 : 1;
        }
    }
    if (in_dtype == 1) {
        if (a.f.gx)
            return a.f.og ? launch_t<bf16_t, _Float16, 64, 128, 128, 8, true, true>(a, stream)
                          : launch_t<bf16_t, _Float16, 64, 128, 128, 8, true, false>(a, stream);
        return launch_t<bf16_t, _Float16, 64, 128, 128, 8, false, false>(a, stream);
    }
    if (chunk == 16)
        return Dk == 16 ? launch_t<float, float, 16, 16, 16, 4, false, false>(a, stream)
                        : launch_t<float, float, 16, 32, 32, 4, false, false>(a, stream);
    if (chunk == 32) return launch_t<float, float, 32, 128, 128, 8, false, false>(a, stream);
    if (Dk == 32) return launch_t<float, float, 64, 32, 32, 4, false, false>(a, stream);
    return launch_t<float, float, 64, 64, 64, 4, false, false>(a, stream);
}

}  // namespace kda
