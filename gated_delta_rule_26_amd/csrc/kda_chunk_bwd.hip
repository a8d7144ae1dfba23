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
// Mapping to the MI355X. Every result is float32-accurate: products run either on the fp32
// matrix cores (v_mfma_f32_16x16x4f32) or, where their operands are stored or staged split into
// bf16 heads and tails, as three bf16 matrix-core products (tail x head, head x tail, head x
// head; about 2^-17 relative). Three launches over a per-(chunk, head) record in the workspace:
//  1. prep    (persistent: one workgroup per compute unit, each taking (chunk, head) items in
//             turn and prefetching the next item's inputs): G, Kd, e^{gC}, A~ and M as 16x16
//             block pairs on the matrix cores (decay split at block boundaries; pair by pair
//             for a block decaying below e^-60), T by blocked substitution, W and U~, and the
//             parts of the reverse state pass that do not depend on dS' (M^T dO, Qg^T dO).
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
// The operands of the state passes' products are stored split and in fragment order: each
// 16x16 tile is 64 lane groups of 16 bytes, lane (lr, q4) holding row lr, columns 4 q4 ..
// 4 q4 + 3 of the tile as four bf16 heads and four bf16 tails, so that one load of a wave
// reads 1 KB in one piece.
template <int C, int DK, int DV> struct BRec {
    static constexpr int64_t oG = 0;                  // [C][DK] G (running sum of g)
    static constexpr int64_t oKd = oG + C * DK;       // [C][DK] Kd = k e^{gC - G} (split tiles)
    static constexpr int64_t oW = oKd + C * DK;       // [C][DK] W (split tiles)
    static constexpr int64_t oU = oW + C * DK;        // [C][DV] U~, then U (fragment order)
    static constexpr int64_t odU = oU + C * DV;       // [C][DV] M^T dO, then dU (fragment order)
    static constexpr int64_t oEg = odU + C * DV;      // [DK]    e^{gC}
    static constexpr int64_t oA = oEg + DK;           // [C][C]  A~ (strictly lower)
    static constexpr int64_t oT = oA + C * C;         // [C][C]  T
    static constexpr int64_t oKdT = oT + C * C;       // [DK][C] Kd^T (split tiles)
    static constexpr int64_t oWT = oKdT + DK * C;     // [DK][C] -W^T (split tiles)
    static constexpr int64_t oQgT = oWT + DK * C;     // [DK][C] Qg^T (split tiles)
    static constexpr int64_t oH = oQgT + DK * C;      // [DK][DV] state entering the chunk (operand tiles)
    static constexpr int64_t odH = oH + DK * DV;      // [DK][DV] Qg^T dO (fragment order), then
                                                      //         dL/d(state leaving the chunk) (operand tiles)
    static constexpr int64_t FLOATS = (odH + DK * DV + 63) & ~int64_t(63);
};

// Offset (floats) of lane `lane`'s 16-byte fragment of tile (rt, ct) of a matrix stored in
// accumulator-fragment order: tile-major over NCT column tiles, each tile 64 lanes x 4 floats,
// lane (lr, q4) holding rows 16 rt + 4 q4 + e (e = 0..3) of column 16 ct + lr.
template <int NCT> __device__ __forceinline__ int64_t afrag(int rt, int ct, int lane) {
    return ((int64_t)(rt * NCT + ct) * 64 + lane) * 4;
}

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

// A float32 4-vector as bf16 heads and bf16 tails (head + tail equals each value to about
// 2^-17 of it), packed in the vector's 16 bytes: [heads 0..3 | tails 0..3]. A product of two
// split factors is three bf16 matrix-core products (tail x head, head x tail, head x head) at
// about float32 accuracy, and bf16 products run several times faster than float32 ones.
struct Split {
    bf16x4 h, t;
};
__device__ __forceinline__ Split split(f32x4 x) {
    Split r;
    r.h = Mma<__bf16>::from_f32(x);
    r.t = Mma<__bf16>::from_f32(x - Mma<__bf16>::to_f32(r.h));
    return r;
}
__device__ __forceinline__ f32x4 pack(Split s) { return __builtin_bit_cast(f32x4, s); }
__device__ __forceinline__ f32x4 split_pack(f32x4 x) { return pack(split(x)); }
__device__ __forceinline__ Split unpack(f32x4 v) { return __builtin_bit_cast(Split, v); }
__device__ __forceinline__ f32x4 unsplit(f32x4 v) {
    const Split s = unpack(v);
    return Mma<__bf16>::to_f32(s.h) + Mma<__bf16>::to_f32(s.t);
}
// Offset (floats) of the 16-byte group holding element (r, c) .. (r, c + 3), c % 4 == 0, of a
// matrix of NCT column tiles stored as split tiles.
template <int NCT> __device__ __forceinline__ int64_t split_at(int r, int c) {
    return afrag<NCT>(r >> 4, c >> 4, (r & 15) + 16 * ((c & 15) >> 2));
}
__device__ __forceinline__ void mma3(f32x4 &acc, Split a, Split b) {
    Mma<__bf16>::mma(acc, a.t, b.h);
    Mma<__bf16>::mma(acc, a.h, b.t);
    Mma<__bf16>::mma(acc, a.h, b.h);
}

// A 16-token block whose decay falls below e^-60 in some channel has diagonal-block factors
// beyond float32's comfortable range; such blocks are summed pair by pair.
constexpr float kExtremeLogDecay = 60.f;
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------------------------------------
// 1. prep
// ------------------------------------------------------------------------------------------
// Four consecutive input elements kept as loaded (bf16: 8 bytes) until they are used, so that a
// load issued early does not make the wave wait for it right away.
template <typename Tin> struct In4;
template <> struct In4<float> {
    typedef f32x4 T;
    static __device__ __forceinline__ T load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
    static __device__ __forceinline__ T zero() { return zero4(); }
    static __device__ __forceinline__ f32x4 f32(T x) { return x; }
};
template <> struct In4<bf16_t> {
    typedef u32x2 T;
    static __device__ __forceinline__ T load(const bf16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
    static __device__ __forceinline__ T zero() { return u32x2{0u, 0u}; }
    static __device__ __forceinline__ f32x4 f32(T u) {
        f32x4 r;
        r.x = __uint_as_float(u.x << 16);
        r.y = __uint_as_float(u.x & 0xffff0000u);
        r.z = __uint_as_float(u.y << 16);
        r.w = __uint_as_float(u.y & 0xffff0000u);
        return r;
    }
};

// Prep runs persistently: each workgroup takes the (slot, head) items b, b + grid, ... and
// loads the next item's inputs into registers while it computes the current one (one
// workgroup fills a compute unit's LDS, so nothing else would hide that load).
template <typename Tin, int C, int DK, int DV>
__global__ __launch_bounds__(512) void bwd_prep_kernel(BwdArgs a) {
    using R = BRec<C, DK, DV>;
    constexpr int NT = 512;
    constexpr int DX = DK > DV ? DK : DV;
    constexpr int LDK = DK + 4, LDX = DX + 4, LDA = C + 4;
    __shared__ __align__(16) float sK[C * LDK];
    __shared__ __align__(16) float sQ[C * LDX];   // q, then beta k e^G
    __shared__ __align__(16) float sG[C * LDX];   // G, then beta v
    // A~ and T; before A~ is formed, the split Qg^T tiles (for Qg^T dO)
    __shared__ __align__(16) float sAT[2 * C * LDA];
    float *const sA = sAT, *const sT = sAT + C * LDA;
    static_assert(DK * C <= 2 * C * LDA, "split Qg^T tiles fit over A~ and T");
    __shared__ __align__(16) f32x4 sMT[(C / 16) * (C / 16) * 64];   // split M^T tiles (for M^T dO)
    __shared__ float sB[C];
    __shared__ int sExt[C / 16];                   // 16-token blocks decaying below e^-60

    const int tid = threadIdx.x;
    const int64_t rsk = (int64_t)a.H * DK, rsv = (int64_t)a.H * DV;
    using I4 = In4<Tin>;
    constexpr int NVL = (C * DV / 4 + NT - 1) / NT, NKL = (C * DK / 4 + NT - 1) / NT;
    constexpr int VTP = DV / 16, ITP = C / 16;
    static_assert(VTP <= NT / 64, "one value-column tile per wave");
    // one item's inputs as loaded: k, q, g rows (4-element groups tid, tid + NT, ...), v rows,
    // beta and this thread's dO values (wave w: value-column tile w, lane (lr, q4): rows
    // 16 ms + 4 q4 + e of column 16 w + lr); zero past the sequence end
    typename I4::T kin4[NKL], qin4[NKL], vin4[NVL];
    f32x4 gin4[NKL];
    f32x4 dpre[ITP];
    float bin;
    auto fetch = [&](int w) {   // w: a valid item
        int n, L;
        int64_t t0;
        const int h = w % a.H;
        locate<C>(a, w / a.H, n, t0, L);
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            const int idx = tid + u * NT, i = idx / (DV / 4), c = 4 * (idx % (DV / 4));
            vin4[u] = idx < C * DV / 4 && i < L ? I4::load(static_cast<const Tin *>(a.v) + (t0 + i) * rsv + (int64_t)h * DV + c)
                                                : I4::zero();
        }
#pragma unroll
        for (int u = 0; u < NKL; ++u) {
            const int idx = tid + u * NT, i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
            const bool in = idx < C * DK / 4 && i < L;
            const int64_t off = (t0 + i) * rsk + (int64_t)h * DK + c;
            kin4[u] = in ? I4::load(static_cast<const Tin *>(a.k) + off) : I4::zero();
            qin4[u] = in ? I4::load(static_cast<const Tin *>(a.q) + off) : I4::zero();
            gin4[u] = in ? *reinterpret_cast<const f32x4 *>(a.g + off) : zero4();
        }
        bin = tid < C && tid < L ? a.beta[(t0 + tid) * a.H + h] : 0.f;
        const int w6 = tid >> 6, l = tid & 63;
        const float *dcol = a.dout + (t0 + 4 * (l >> 4)) * rsv + (int64_t)h * DV + 16 * (w6 < VTP ? w6 : 0) + (l & 15);
#pragma unroll
        for (int ms = 0; ms < ITP; ++ms)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ms + 4 * (l >> 4) + e;
                dpre[ms][e] = w6 < VTP && r < L ? dcol[(int64_t)(16 * ms + e) * rsv] : 0.f;
            }
    };
    const int items = (int)(a.nslots * a.H);   // at most 2^30 (checked by the host)
    // the first item at or after w in this workgroup's sequence that is a chunk (slots past a
    // sequence's last chunk are unused)
    auto next_item = [&](int w) {
        for (; w < items; w += gridDim.x) {
            int n, L;
            int64_t t0;
            if (locate<C>(a, w / a.H, n, t0, L)) break;
        }
        return w;
    };
    // Every input of an item is loaded during the item before it, ahead of that item's record
    // stores, and every wave retires its memory operations in issue order: so an item waits
    // for its own inputs only, never for the previous item's stores, which drain while it
    // computes. (The first item's loads are waited for before the loop, so that the loop's
    // waits count from the loads issued inside it.)
    int w = next_item(blockIdx.x);
    if (w < items) {
        fetch(w);
#pragma unroll
        for (int u = 0; u < NKL; ++u) __asm__ volatile("" : : "v"(kin4[u]), "v"(qin4[u]), "v"(gin4[u]));
#pragma unroll
        for (int u = 0; u < NVL; ++u) __asm__ volatile("" : : "v"(vin4[u]));
#pragma unroll
        for (int ms = 0; ms < ITP; ++ms) __asm__ volatile("" : : "v"(dpre[ms]));
        __asm__ volatile("" : : "v"(bin));
    }
    while (w < items) {
    const int wn = next_item(w + gridDim.x);
    // the thread index through an empty asm statement: the per-thread offsets below are
    // recomputed for each item instead of being hoisted out of the loop and held in registers
    int tid_ = threadIdx.x;
    __asm__ volatile("" : "+v"(tid_));
    const int tid = tid_;
    const int h = w % a.H;
    int n, L;
    int64_t t0;
    locate<C>(a, w / a.H, n, t0, L);
    float *rec = a.ws + (int64_t)w * R::FLOATS;

    // dO as the B fragments of the products below
    Split dOs[ITP];
#pragma unroll
    for (int ms = 0; ms < ITP; ++ms) dOs[ms] = split(dpre[ms]);
    // this item's inputs to LDS (v stays in registers), then the next item's loads
    f32x4 vpre[NVL];
#pragma unroll
    for (int u = 0; u < NVL; ++u) vpre[u] = I4::f32(vin4[u]);
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
        const int idx = tid + u * NT, i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        if (idx < C * DK / 4) {
            *reinterpret_cast<f32x4 *>(sK + i * LDK + c) = I4::f32(kin4[u]);
            *reinterpret_cast<f32x4 *>(sQ + i * LDX + c) = I4::f32(qin4[u]);
            *reinterpret_cast<f32x4 *>(sG + i * LDX + c) = gin4[u];
        }
    }
    if (tid < C) sB[tid] = bin;
    if (wn < items) fetch(wn);
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
    // Record stores go out as whole 1 KB pieces per wave: G row by row, the split tiles
    // fragment by fragment (vector idx is lane idx % 64 of tile idx / 64), each thread
    // gathering its fragment's four values from LDS.
    for (int idx = tid; idx < C * DK / 4; idx += NT) {
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        *reinterpret_cast<f32x4 *>(rec + R::oG + i * DK + c) = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
    }
    for (int idx = tid; idx < C * DK / 4; idx += NT) {
        const int tile = idx >> 6, ln = idx & 63;
        const int i = 16 * (tile / (DK / 16)) + (ln & 15), c = 16 * (tile % (DK / 16)) + 4 * (ln >> 4);
        const f32x4 G = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
        const f32x4 gC = *reinterpret_cast<const f32x4 *>(sG + (C - 1) * LDX + c);
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
        f32x4 kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) kd[e] = kv[e] * __expf(gC[e] - G[e]);
        *reinterpret_cast<f32x4 *>(rec + R::oKd + 4 * idx) = split_pack(kd);   // = split_at<DK / 16>(i, c)
    }
    for (int idx = tid; idx < DK * C / 4; idx += NT) {  // the same, transposed ([channel][row])
        const int tile = idx >> 6, ln = idx & 63;
        const int c = 16 * (tile / (C / 16)) + (ln & 15), i0 = 16 * (tile % (C / 16)) + 4 * (ln >> 4);
        f32x4 qg, kd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float G = sG[(i0 + e) * LDX + c], gC = sG[(C - 1) * LDX + c];
            qg[e] = a.scale * sQ[(i0 + e) * LDX + c] * __expf(G);
            kd[e] = sK[(i0 + e) * LDK + c] * __expf(gC - G);
        }
        const f32x4 qgs = split_pack(qg);
        *reinterpret_cast<f32x4 *>(rec + R::oQgT + split_at<C / 16>(c, i0)) = qgs;
        *reinterpret_cast<f32x4 *>(sAT + split_at<C / 16>(c, i0)) = qgs;
        *reinterpret_cast<f32x4 *>(rec + R::oKdT + split_at<C / 16>(c, i0)) = split_pack(kd);
    }
    // Qg^T dO (the dO part of dS in the reverse state pass) into dH's slot, which that pass
    // reads before it writes it: wave w takes value-column tile w
    constexpr int KTP = DK / 16;
    __syncthreads();
    {
        const int w = tid >> 6, l = tid & 63;
        if (w < VTP) {
            for (int kt = 0; kt < KTP; ++kt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ms = 0; ms < ITP; ++ms)
                    mma3(acc, unpack(*reinterpret_cast<const f32x4 *>(sAT + afrag<ITP>(kt, ms, l))), dOs[ms]);
                *reinterpret_cast<f32x4 *>(rec + R::odH + afrag<VTP>(kt, w, l)) = acc;
            }
        }
    }
    __syncthreads();  // A~ goes over the Qg^T tiles
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
                // lane (jl, ig): column j = 16 I + jl, rows i = 16 I + 4 ig + e (e = 0..3), i.e.
                // one 4-value group of M^T's row j and four values of A~'s column j
                const int jl = lane & 15, ig = lane >> 4, j = 16 * I + jl, i0 = 16 * I + 4 * ig;
                f32x4 mt = zero4();
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + e;
                    float sa = 0.f, sm = 0.f;
                    if (j <= i) {
                        for (int c = 0; c < DK; c += 4) {
                            const f32x4 ki = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
                            const f32x4 kj = *reinterpret_cast<const f32x4 *>(sK + j * LDK + c);
                            const f32x4 qi = *reinterpret_cast<const f32x4 *>(sQ + i * LDX + c);
                            const f32x4 Gi = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
                            const f32x4 Gj = *reinterpret_cast<const f32x4 *>(sG + j * LDX + c);
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const float kjE = kj[u] * __expf(Gi[u] - Gj[u]);
                                sa += ki[u] * kjE;
                                sm += qi[u] * kjE;
                            }
                        }
                    }
                    sA[i * LDA + j] = j < i ? sa : 0.f;
                    mt[e] = j <= i ? a.scale * sm : 0.f;
                }
                sMT[split_at<C / 16>(j, i0) / 4] = split_pack(mt);   // M^T
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
            f32x4 mt;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * q4 + e, j = 16 * J + lr;
                sA[i * LDA + j] = j < i ? accA[e] : 0.f;
                mt[e] = j <= i ? a.scale * accM[e] : 0.f;
            }
            // M^T: row 16 J + lr, the four values of columns 16 I + 4 q4 ..
            sMT[split_at<C / 16>(16 * J + lr, 16 * I + 4 * q4) / 4] = split_pack(mt);
        }
    }
    for (int p = tid; p < C * C; p += NT) {   // A~'s blocks above the diagonal
        const int i = p / C, j = p % C;
        if ((j >> 4) > (i >> 4)) sA[i * LDA + j] = 0.f;
    }
    __syncthreads();
    {   // M^T dO (the dO part of dU in the reverse state pass) into dU's slot: wave w takes
        // value-column tile w; M[m][i] = 0 for m < i
        const int w = tid >> 6, l = tid & 63;
        if (w < VTP) {
#pragma unroll
            for (int it = 0; it < ITP; ++it) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ms = it; ms < ITP; ++ms) mma3(acc, unpack(sMT[afrag<ITP>(it, ms, l) / 4]), dOs[ms]);
                *reinterpret_cast<f32x4 *>(rec + R::odU + afrag<VTP>(it, w, l)) = acc;
            }
        }
    }
    for (int idx = tid; idx < C * DK / 4; idx += NT) {  // beta k e^G over q (k and G die here)
        const int i = idx / (DK / 4), c = 4 * (idx % (DK / 4));
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(sK + i * LDK + c);
        const f32x4 G = *reinterpret_cast<const f32x4 *>(sG + i * LDX + c);
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = sB[i] * kv[e] * __expf(G[e]);
        *reinterpret_cast<f32x4 *>(sQ + i * LDX + c) = r;
    }
    __syncthreads();  // k is dead: its array holds the tiles below
    // T = (I + N)^-1 with N = Diag(beta) A~ (strictly lower): each diagonal 16x16 block by
    // forward substitution (one wave per block, lane = column: 16 dependent steps, the blocks
    // side by side), then block forward substitution T_IJ = -T_II sum_{J <= K < I} N_IK T_KJ on
    // the matrix cores, one block row per level. Intermediate tiles live over k's array.
    {
        constexpr int NBK = C / 16, LDT = 20;         // scratch tile: 16 rows of 20 floats
        // one tile per substituting wave, over k's array where it fits (k is dead), else apart
        constexpr int NSCR = NBK * 16 * LDT;
        constexpr bool kOverK = NSCR <= C * LDK;
        __shared__ __align__(16) float sScr[kOverK ? 4 : NSCR];
        float *const scr = kOverK ? sK : sScr;
        const int wv = tid >> 6, ln = tid & 63, tr = ln & 15, tq = ln >> 4;
        // D (16 x 16: rows 4 tq + e, column tr in this lane) = init + A B, both operands 16 x 16
        // tiles in LDS (A row-major with a per-row scale, B row-major read by columns)
        auto prod = [&](const float *A, int lda, float ascale_row, const float *B, int ldb, f32x4 init) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(A + tr * lda + 4 * tq) * ascale_row;
            f32x4 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = B[(4 * tq + e) * ldb + tr];
            f32x4 acc = init;
            mma(acc, a, b);
            return acc;
        };
        auto put = [&](float *D, int ld, f32x4 v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) D[(4 * tq + e) * ld + tr] = v[e];
        };
        if (wv < NBK && ln < 16) {  // T_II, column ln: x_i = delta_i,col - beta_i sum_{m<i} A~_im x_m
            const int I0 = 16 * wv;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc += sA[(I0 + i) * LDA + I0 + m] * x[m];
                x[i] = (i == ln ? 1.f : 0.f) - sB[I0 + i] * acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(I0 + i) * LDA + I0 + ln] = x[i];
        }
        // the blocks above the diagonal are zero
        for (int idx = tid; idx < C * C; idx += NT) {
            const int i = idx / C, j = idx % C;
            if ((j >> 4) > (i >> 4)) sT[i * LDA + j] = 0.f;
        }
        __syncthreads();
        // block rows I = 1 .. NBK - 1: wave J computes T_IJ, J < I
        for (int I = 1; I < NBK; ++I) {
            const bool act = wv < I;
            const int J = wv;
            float *R = scr + wv * 16 * LDT;             // sum_{K = J}^{I-1} N_IK T_KJ
            if (act) {
                f32x4 r = zero4();
                for (int K = J; K < I; ++K)
                    r = prod(sA + 16 * I * LDA + 16 * K, LDA, sB[16 * I + tr], sT + 16 * K * LDA + 16 * J, LDA, r);
                put(R, LDT, r);
            }
            __syncthreads();
            if (act) put(sT + 16 * I * LDA + 16 * J, LDA, -prod(sT + 16 * I * LDA + 16 * I, LDA, 1.f, R, LDT, zero4()));
            __syncthreads();
        }
        for (int idx = tid; idx < C * C / 4; idx += NT) {   // T and A~ row by row
            const int i = idx / (C / 4), j = 4 * (idx % (C / 4));
            *reinterpret_cast<f32x4 *>(rec + R::oT + i * C + j) = *reinterpret_cast<const f32x4 *>(sT + i * LDA + j);
            *reinterpret_cast<f32x4 *>(rec + R::oA + i * C + j) = *reinterpret_cast<const f32x4 *>(sA + i * LDA + j);
        }
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) {  // beta v over G
        const int idx = tid + u * NT, i = idx / (DV / 4), c = 4 * (idx % (DV / 4));
        if (idx < C * DV / 4) *reinterpret_cast<f32x4 *>(sG + i * LDX + c) = vpre[u] * sB[i];
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
        f32x4 acc = zero4(), accT = zero4();
        for (int ms = 0; ms <= it; ++ms) {
            const int m0 = 16 * ms + 4 * q4;
            const f32x4 A = *reinterpret_cast<const f32x4 *>(sT + (16 * it + lr) * LDA + m0);
            f32x4 B;
#pragma unroll
            for (int e = 0; e < 4; ++e) B[e] = X[(m0 + e) * LDX + 16 * nt + lr];
            mma(acc, A, B);
            if (isW) mma(accT, B, A);   // the same tile transposed: four channels of one row
        }
        if (isW) {
            *reinterpret_cast<f32x4 *>(rec + R::oW + afrag<DK / 16>(it, nt, lane)) = split_pack(accT);
            *reinterpret_cast<f32x4 *>(rec + R::oWT + afrag<C / 16>(nt, it, lane)) = split_pack(-acc);
        } else {
            *reinterpret_cast<f32x4 *>(rec + R::oU + afrag<DV / 16>(it, nt, lane)) = acc;
        }
    }
    __syncthreads();  // the LDS is the next item's
    w = wn;
    }
}

// ------------------------------------------------------------------------------------------
// 2. forward state pass: one workgroup per (chain, 16 value columns); wave w holds the 16x16
//    state tiles of its key-channel tiles in accumulator registers. Every operand but dO is one
//    16-byte load per lane. The next chunk's operands are loaded while this one computes, their
//    loads interleaved with this chunk's products (a wave issues in order: a burst of loads
//    would hold its products back while the CU's memory pipeline drains it), and the chunk after
//    that is touched into the L2 (each of a chain's value-column workgroups touches an eighth of
//    its lines), so those loads hit the cache. The loop body has no branches, so that the
//    scheduling fences below order it.
// ------------------------------------------------------------------------------------------
template <int C, int DK, int DV> struct StatePass {
    static constexpr int KT = DK / 16;
    static constexpr int VT = DV / 16;
    static constexpr int NW = KT < 4 ? KT : 4;
    static constexpr int KTW = KT / NW;
    static constexpr int IT = C / 16;
    static constexpr int NOWN = IT >= NW ? IT / NW : 1;   // row tiles whose U a wave owns
    static_assert(KT % NW == 0, "key tiles spread evenly");
    static_assert(IT % NW == 0 || IT == 1, "row tiles spread evenly");
};

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// A 16x16 tile from accumulator layout (lane (lr, q4): rows 4 q4 + e of column lr) to operand
// layout (lane (lr, q4): row lr, columns 4 q4 + e), through a wave-private LDS tile of 16 rows
// of 20 floats (the reads of one e fall in distinct banks).
__device__ __forceinline__ f32x4 transpose16(f32x4 x, float *t, int lr, int q4) {
    *reinterpret_cast<f32x4 *>(t + lr * 20 + 4 * q4) = x;   // t[c][r] = x[r][c]
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = t[(4 * q4 + e) * 20 + lr];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();   // every lane has read before the tile is written again
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return r;
}

// L2 touch of one step's operands: the 128-byte lines of NR record regions are
// numbered in turn; value-column block vb touches the lines vb, vb + nvb, ..., one load per
// thread (threads past the last line load the first one). The loaded word is kept and consumed
// two steps later, so that the load is issued and nothing waits for it before then.
template <int NR> struct TouchSet {
    const float *base[NR];
    int lines[NR];
};

template <int NR> __device__ __forceinline__ float touch(const TouchSet<NR> &t, int vb, int nvb) {
    int l = vb + nvb * (int)threadIdx.x;
    const float *p = t.base[0];
    bool found = false;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const bool in = !found && l < t.lines[r];
        p = in ? t.base[r] + (int64_t)l * 32 : p;
        found = found || in;
        l = found ? l : l - t.lines[r];
    }
    return *p;
}

template <int C, int DK, int DV> struct FwdOps {
    using P = StatePass<C, DK, DV>;
    f32x4 W[P::IT][P::KTW];     // W rows 16 it + lr, channels 16 kt + 4 q4 ..
    f32x4 KdT[P::KTW][P::IT];   // Kd^T rows 16 kt + lr, tokens 16 it + 4 q4 ..
    f32x4 eg[P::KTW];           // e^{gC} of channels 16 kt + 4 q4 ..
    f32x4 Ut[P::NOWN];          // U~ of the owned row tiles (accumulator fragments)
    float pf;                   // the L2 touch of the chunk two steps ahead
};

template <int C, int DK, int DV>
__device__ __forceinline__ void fwd_state_pass(const BwdArgs &a, int chain, int vb) {
    using R = BRec<C, DK, DV>;
    using P = StatePass<C, DK, DV>;
    constexpr int IT = P::IT, KTW = P::KTW, NW = P::NW, NOWN = P::NOWN, VT = P::VT;
    __shared__ f32x4 sPart[2][NW][IT][64];   // by step parity: one barrier per step
    __shared__ float sTr[NW][16 * 20];        // per-wave transpose tile
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
    // W goes out with this chunk's W S products, Kd^T with its state update: the compute
    // unit's memory pipeline then works through the whole step instead of its first phase
    auto loadW = [&](const float *rec, FwdOps<C, DK, DV> &o, int it) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk)
            o.W[it][kk] = *reinterpret_cast<const f32x4 *>(rec + R::oW + afrag<P::KT>(it, wave * KTW + kk, lane));
    };
    auto loadK = [&](const float *rec, FwdOps<C, DK, DV> &o, int kk, int it) {
        o.KdT[kk][it] = *reinterpret_cast<const f32x4 *>(rec + R::oKdT + afrag<IT>(wave * KTW + kk, it, lane));
    };
    auto loadRest = [&](const float *rec, FwdOps<C, DK, DV> &o) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk)
            o.eg[kk] = *reinterpret_cast<const f32x4 *>(rec + R::oEg + 16 * (wave * KTW + kk) + 4 * q4);
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow) {
            if constexpr (IT >= NW) o.Ut[ow] = *reinterpret_cast<const f32x4 *>(rec + R::oU + afrag<VT>(own(ow), vb, lane));
            else o.Ut[ow] = own(ow) < IT ? *reinterpret_cast<const f32x4 *>(rec + R::oU + afrag<VT>(own(ow), vb, lane)) : zero4();
        }
    };
    auto touch_chunk = [&](int j) {
        const float *rec = rec_of(j);
        TouchSet<4> t;
        t.base[0] = rec + R::oW;   t.lines[0] = C * DK / 32;
        t.base[1] = rec + R::oKdT; t.lines[1] = DK * C / 32;
        t.base[2] = rec + R::oU;   t.lines[2] = C * DV / 32;
        t.base[3] = rec + R::oEg;  t.lines[3] = (DK + 31) / 32;
        return touch(t, vb, DV / 16);
    };

    f32x4 S[KTW];
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
        const int kt = wave * KTW + kk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[kk][e] = a.s0 ? a.s0[(((int64_t)n * a.H + h) * DK + 16 * kt + 4 * q4 + e) * DV + col] : 0.f;
    }
    float sink = 0.f;
    // one chunk with operands `cur`, loading the next chunk's into `nxt` (the last chunk reloads
    // its own: no branch); the loop below alternates the two operand sets
    auto step = [&](int j, FwdOps<C, DK, DV> &cur, FwdOps<C, DK, DV> &nxt) {
        float *rec = rec_of(j);
        const float *nrec = rec_of(j + 1 < nch ? j + 1 : j);
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk)
            *reinterpret_cast<f32x4 *>(rec + R::oH + afrag<VT>(wave * KTW + kk, vb, lane)) =
                transpose16(S[kk], sTr[wave], lr, q4);   // operand layout: row lr, 4 columns
        Split Ss[KTW];
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) Ss[kk] = split(S[kk]);
        f32x4 acc[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            loadW(nrec, nxt, it);
            sched_fence();
            acc[it] = zero4();
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) mma3(acc[it], unpack(cur.W[it][kk]), Ss[kk]);
            sched_fence();
        }
        loadRest(nrec, nxt);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 part = -acc[it];
#pragma unroll
            for (int ow = 0; ow < NOWN; ++ow)
                part += own(ow) == it ? cur.Ut[ow] : zero4();   // the owner of row tile it adds U~
            sPart[j & 1][wave][it][lane] = part;
        }
        __syncthreads();
        f32x4 U[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            U[it] = sPart[j & 1][0][it][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) U[it] += sPart[j & 1][w][it][lane];
        }
        // the touch issued two steps ago is complete (cur's loads came after it): consume it
        // (tied to U so that it stays after them) and touch the chunk two steps ahead
        sink += cur.pf * U[0][0];
        cur.pf = touch_chunk(j + 2 < nch ? j + 2 : nch - 1);
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow) {
            f32x4 u = zero4();
#pragma unroll
            for (int it = 0; it < IT; ++it) u = own(ow) == it ? U[it] : u;
            if (IT >= NW || own(ow) < IT)
                *reinterpret_cast<f32x4 *>(rec + R::oU + afrag<VT>(own(ow), vb, lane)) = u;
        }
        Split Us[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) Us[it] = split(U[it]);
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            S[kk] *= cur.eg[kk];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                loadK(nrec, nxt, kk, it);
                sched_fence();
                mma3(S[kk], unpack(cur.KdT[kk][it]), Us[it]);
                sched_fence();
            }
        }
    };
    FwdOps<C, DK, DV> o0, o1;
    o0.pf = o1.pf = 0.f;
    if (nch > 0) {
        const float *r0 = rec_of(0);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            loadW(r0, o0, it);
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) loadK(r0, o0, kk, it);
        }
        loadRest(r0, o0);
    }
    if (nch > 1) o1.pf = touch_chunk(1);
    int j = 0;
    for (; j + 1 < nch; j += 2) {
        step(j, o0, o1);
        step(j + 1, o1, o0);
    }
    if (j < nch) step(j, o0, o1);
    __asm__ volatile("" : : "v"(sink), "v"(o0.pf), "v"(o1.pf));
}

// ------------------------------------------------------------------------------------------
// 3. reverse state pass: dS held like S above, chunks in reverse order, the same pipeline as
//    the forward pass. With P1 = M^T dO and P2 = Qg^T dO from the prep (in the dU and dH
//    slots), a chunk is dU = Kd dS' + P1 (exchanged like U), then dS = e^{gC} dS' + P2 - W^T dU.
// ------------------------------------------------------------------------------------------
template <int C, int DK, int DV> struct RevOps {
    using P = StatePass<C, DK, DV>;
    f32x4 Kd[P::IT][P::KTW];    // Kd rows 16 it + lr, channels 16 kt + 4 q4 ..
    f32x4 WT[P::KTW][P::IT];    // -W^T rows 16 kt + lr, tokens 16 it + 4 q4 ..
    f32x4 eg[P::KTW];
    f32x4 P1[P::NOWN];          // M^T dO of the owned row tiles (accumulator fragments)
    f32x4 P2[P::KTW];           // Qg^T dO of the wave's key tiles (accumulator fragments)
    float pf;
};

template <int C, int DK, int DV>
__device__ __forceinline__ void rev_state_pass(const BwdArgs &a, int chain, int vb) {
    using R = BRec<C, DK, DV>;
    using P = StatePass<C, DK, DV>;
    constexpr int IT = P::IT, KTW = P::KTW, NW = P::NW, NOWN = P::NOWN, VT = P::VT;
    __shared__ f32x4 sPart[2][NW][IT][64];
    __shared__ float sTr[NW][16 * 20];        // per-wave transpose tile
    const int n = chain / a.H, h = chain % a.H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, q4 = lane >> 4;
    int64_t st, en;
    seq_range(a, n, st, en);
    const int64_t len = en - st;
    const int nch = (int)((len + C - 1) / C);
    const int64_t base = slot_base<C>(a, n);
    const int col = 16 * vb + lr;
    const int64_t sbase = ((int64_t)n * a.H + h) * DK;
    auto rec_of = [&](int j) { return a.ws + ((base + j) * a.H + h) * R::FLOATS; };
    auto own = [&](int o) { return wave + NW * o; };
    // Kd goes out with this chunk's dU products, -W^T with its dS update (as in the forward pass)
    auto loadKd = [&](const float *rec, RevOps<C, DK, DV> &o, int it) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk)
            o.Kd[it][kk] = *reinterpret_cast<const f32x4 *>(rec + R::oKd + afrag<P::KT>(it, wave * KTW + kk, lane));
    };
    auto loadWT = [&](const float *rec, RevOps<C, DK, DV> &o, int kk, int it) {
        o.WT[kk][it] = *reinterpret_cast<const f32x4 *>(rec + R::oWT + afrag<IT>(wave * KTW + kk, it, lane));
    };
    auto loadRest = [&](const float *rec, RevOps<C, DK, DV> &o) {
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const int kt = wave * KTW + kk;
            o.eg[kk] = *reinterpret_cast<const f32x4 *>(rec + R::oEg + 16 * kt + 4 * q4);
            o.P2[kk] = *reinterpret_cast<const f32x4 *>(rec + R::odH + afrag<VT>(kt, vb, lane));
        }
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow) {
            if constexpr (IT >= NW) o.P1[ow] = *reinterpret_cast<const f32x4 *>(rec + R::odU + afrag<VT>(own(ow), vb, lane));
            else o.P1[ow] = own(ow) < IT ? *reinterpret_cast<const f32x4 *>(rec + R::odU + afrag<VT>(own(ow), vb, lane)) : zero4();
        }
    };
    auto touch_chunk = [&](int j) {
        const float *rec = rec_of(j);
        TouchSet<5> t;
        t.base[0] = rec + R::oKd;  t.lines[0] = C * DK / 32;
        t.base[1] = rec + R::oWT;  t.lines[1] = DK * C / 32;
        t.base[2] = rec + R::odU;  t.lines[2] = C * DV / 32;
        t.base[3] = rec + R::odH;  t.lines[3] = DK * DV / 32;
        t.base[4] = rec + R::oEg;  t.lines[4] = (DK + 31) / 32;
        return touch(t, vb, DV / 16);
    };

    f32x4 dS[KTW];
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
        const int kt = wave * KTW + kk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[kk][e] = a.dsT ? a.dsT[(sbase + 16 * kt + 4 * q4 + e) * DV + col] : 0.f;
    }
    float sink = 0.f;
    auto step = [&](int j, RevOps<C, DK, DV> &cur, RevOps<C, DK, DV> &nxt) {
        float *rec = rec_of(j);
        const float *nrec = rec_of(j > 0 ? j - 1 : 0);
        Split dSs[KTW];
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) dSs[kk] = split(dS[kk]);
        f32x4 acc[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            loadKd(nrec, nxt, it);
            sched_fence();
            acc[it] = zero4();
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) mma3(acc[it], unpack(cur.Kd[it][kk]), dSs[kk]);
            sched_fence();
        }
        loadRest(nrec, nxt);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 part = acc[it];
#pragma unroll
            for (int ow = 0; ow < NOWN; ++ow)
                part += own(ow) == it ? cur.P1[ow] : zero4();   // the owner of row tile it adds M^T dO
            sPart[j & 1][wave][it][lane] = part;
        }
        __syncthreads();
        f32x4 dU[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            dU[it] = sPart[j & 1][0][it][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) dU[it] += sPart[j & 1][w][it][lane];
        }
        sink += cur.pf * dU[0][0];
        cur.pf = touch_chunk(j >= 2 ? j - 2 : 0);
        // dU and dS' over this chunk's P1 and P2 (read above, before these stores)
#pragma unroll
        for (int ow = 0; ow < NOWN; ++ow) {
            f32x4 u = zero4();
#pragma unroll
            for (int it = 0; it < IT; ++it) u = own(ow) == it ? dU[it] : u;
            if (IT >= NW || own(ow) < IT)
                *reinterpret_cast<f32x4 *>(rec + R::odU + afrag<VT>(own(ow), vb, lane)) = u;
        }
        Split dUs[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) dUs[it] = split(dU[it]);
#pragma unroll
        for (int kk = 0; kk < KTW; ++kk) {
            const f32x4 dSo = dS[kk];
            dS[kk] = dS[kk] * cur.eg[kk] + cur.P2[kk];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                loadWT(nrec, nxt, kk, it);
                sched_fence();
                mma3(dS[kk], unpack(cur.WT[kk][it]), dUs[it]);   // -W^T dU
                sched_fence();
            }
            *reinterpret_cast<f32x4 *>(rec + R::odH + afrag<VT>(wave * KTW + kk, vb, lane)) =
                transpose16(dSo, sTr[wave], lr, q4);   // operand layout: row lr, 4 columns
        }
    };
    RevOps<C, DK, DV> o0, o1;
    o0.pf = o1.pf = 0.f;
    if (nch > 0) {
        const float *rl = rec_of(nch - 1);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            loadKd(rl, o0, it);
#pragma unroll
            for (int kk = 0; kk < KTW; ++kk) loadWT(rl, o0, kk, it);
        }
        loadRest(rl, o0);
    }
    if (nch > 1) o1.pf = touch_chunk(nch - 2);
    int j = nch - 1;
    for (; j >= 1; j -= 2) {
        step(j, o0, o1);
        step(j - 1, o1, o0);
    }
    if (j == 0) step(0, o0, o1);
    __asm__ volatile("" : : "v"(sink), "v"(o0.pf), "v"(o1.pf));
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
// launch runs both. Workgroup b maps to (direction, chain, value block) so that the value
// blocks of one chain and direction share b mod 8, i.e. one XCD and its L2 (workgroups go to
// the XCDs round robin): pair p = direction * chains + chain takes XCD p mod 8 and, on it,
// the slots (p / 8) * NVB .. + NVB - 1. Slots past the last pair exit at once.
template <int C, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_state_kernel(BwdArgs a) {
    constexpr int NVB = DV / 16;
    const int b = blockIdx.x, k = b >> 3;
    const int p = (k / NVB) * 8 + (b & 7), vb = k % NVB;
    const int chains = a.n_seqs * a.H;
    if (p >= 2 * chains) return;
    if (p < chains) fwd_state_pass<C, DK, DV>(a, p, vb);
    else rev_state_pass<C, DK, DV>(a, p - chains, vb);
}

// The state kernel's grid: 8 XCD lanes x NVB slots per group of 8 (direction, chain) pairs.
template <int DV> unsigned state_blocks(int chains) {
    return (unsigned)(((2 * chains + 7) / 8) * 8 * (DV / 16));
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
    static_assert((IT / 2 + 1) * (IT - IT / 2) <= 2 * NWV, "the dT tile pairs fit the waves");
    constexpr int LDG = DK + 1;
    // the pair-term phase's arrays, over dO / U / T / dT / X once those are done
    constexpr int NG2 = 2 * IT * DK + KT * 768 + C * LDG;
    constexpr int NOU0 = 2 * C * LDV > 3 * C * LDA ? 2 * C * LDV : 3 * C * LDA;
    constexpr int NOU = NOU0 > NG2 ? NOU0 : NG2;
    // dU, and dO then U (both split: 4-column groups of heads and tails), staged once for all
    // waves; T, dT and T^T dT later take dO's and U's space
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

    // Every load of this phase goes out before the first LDS store: dO, U and dU for the
    // staging (NI 16-byte groups per thread), then this wave's rows of S and dS' (key tile
    // ct = wave), which become the split B fragments below.
    constexpr int NG = C * DV / 4, NI = (NG + NT - 1) / NT;
    f32x4 dOv[NI], uv[NI], duv[NI];
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        const int idx = NG % NT == 0 || tid + m * NT < NG ? tid + m * NT : 0;  // past NG: unused
        const int i = idx / (DV / 4), j = 4 * (idx % (DV / 4));
        // rows past the end read the last valid row (L >= 1 here) and are zeroed below
        dOv[m] = *reinterpret_cast<const f32x4 *>(a.dout + (t0 + (i < L ? i : L - 1)) * rsv + (int64_t)h * DV + j);
        uv[m] = *reinterpret_cast<const f32x4 *>(rec + R::oU + 4 * idx);
        duv[m] = *reinterpret_cast<const f32x4 *>(rec + R::odU + 4 * idx);
    }
    const int ct = wave;
    // (without a branch: waves past the last key tile load the last one and do not use it, so
    // that the waits below are counted for the loads in flight on every path)
    const int ctl = ct < KT ? ct : KT - 1;
    f32x4 hraw[VT], dhraw[VT];
#pragma unroll
    for (int js = 0; js < VT; ++js) {
        // S[16 ct + lr][16 js + 4 q4 + e]: the state passes store H and dH tiles in operand
        // layout, so this lane's 4 values are one 16-byte group
        hraw[js] = *reinterpret_cast<const f32x4 *>(rec + R::oH + afrag<VT>(ctl, js, lane));
        dhraw[js] = *reinterpret_cast<const f32x4 *>(rec + R::odH + afrag<VT>(ctl, js, lane));
    }
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        const int idx = tid + m * NT;
        if (NG % NT != 0 && idx >= NG) break;
        const int i = idx / (DV / 4), j = 4 * (idx % (DV / 4));
        // zeroed by a bit mask rather than a select, which the compiler would turn back into
        // a load under a branch (and then wait for every load in flight at the merge)
        const uint32_t keep = i < L ? 0xffffffffu : 0u;
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = __uint_as_float(__float_as_uint(dOv[m][e]) & keep);
        *reinterpret_cast<f32x4 *>(sdO + i * LDV + j) = split_pack(d);
        // U and dU are in fragment order: vector idx is lane idx % 64 of tile idx / 64. U goes
        // to LDS split, element (r, c) as the head and tail at slots c % 4 and 4 + c % 4 of its
        // row's 4-column group
        const int tile = idx >> 6, fl = idx & 63;
        const int r0 = 16 * (tile / VT) + 4 * (fl >> 4), cu = 16 * (tile % VT) + (fl & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            __bf16 *ug = reinterpret_cast<__bf16 *>(sU + (r0 + e) * LDV + (cu & ~3));
            const __bf16 uh = static_cast<__bf16>(uv[m][e]);
            ug[cu & 3] = uh;
            ug[4 + (cu & 3)] = static_cast<__bf16>(uv[m][e] - static_cast<float>(uh));
            sdU[(r0 + e) * LDV + cu] = duv[m][e];
        }
    }
    for (int idx = tid; idx < NSRC * C; idx += NT) (&sDb[0][0])[idx] = 0.f;
    // the split B fragments of this wave's rows of S and dS'
    Split hB[VT], dhB[VT];
#pragma unroll
    for (int js = 0; js < VT; ++js) {
        hB[js] = split(hraw[js]);
        dhB[js] = split(dhraw[js]);
        // formed here, once: without the pin the compiler re-forms them at every use below
        asm volatile("" : "+v"(hB[js].h), "+v"(hB[js].t), "+v"(dhB[js].h), "+v"(dhB[js].t));
    }
    __syncthreads();

    // dQg = dO S^T, dKd = U dS'^T, dW = -dU S^T for key tile ct; d e^{gC} = rowsum(S * dS')
    f32x4 dq_p[IT], dk_p[IT], dG_p[IT];
    // this lane's G (channel 16 ct + lr, rows 16 X + 4 q4 + e), kept for the phases below
    float Gr[IT][4];
#pragma unroll
    for (int X = 0; X < IT; ++X)
#pragma unroll
        for (int e = 0; e < 4; ++e) Gr[X][e] = 0.f;
    if (ct < KT) {
        // this lane's G, Qg, Kd (channel 16 ct + lr, rows 16 it + 4 q4 + e), read before the
        // products so that their latency hides under them
        const int c = 16 * ct + lr;
        // Qg and Kd of rows 16 it + 4 q4 .. + 3: one group of the split Qg^T and Kd^T tiles
        // (head + tail, float32 to about 2^-17)
        const float gC = rec[R::oG + (C - 1) * DK + c];
        f32x4 Ql[IT], Kl[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            Ql[it] = unsplit(*reinterpret_cast<const f32x4 *>(rec + R::oQgT + afrag<IT>(ct, it, lane)));
            Kl[it] = unsplit(*reinterpret_cast<const f32x4 *>(rec + R::oKdT + afrag<IT>(ct, it, lane)));
#pragma unroll
            for (int e = 0; e < 4; ++e) Gr[it][e] = rec[R::oG + (16 * it + 4 * q4 + e) * DK + c];
        }
        const float (&Gl)[IT][4] = Gr;
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
                mma3(aQ[it], unpack(*reinterpret_cast<const f32x4 *>(sdO + i * LDV + j0)), hB[js]);
                mma3(aK[it], unpack(*reinterpret_cast<const f32x4 *>(sU + i * LDV + j0)), dhB[js]);
                mma3(aW[it], split(*reinterpret_cast<const f32x4 *>(sdU + i * LDV + j0)), hB[js]);
            }
            const f32x4 hv = Mma<__bf16>::to_f32(hB[js].h) + Mma<__bf16>::to_f32(hB[js].t);
            const f32x4 dhv = Mma<__bf16>::to_f32(dhB[js].h) + Mma<__bf16>::to_f32(dhB[js].t);
            dgc += hv[0] * dhv[0] + hv[1] * dhv[1] + hv[2] * dhv[2] + hv[3] * dhv[3];
        }
        float cs = 0.f;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * q4 + e;
                const float G = Gl[it][e], Qg = Ql[it][e], Kd = Kl[it][e];
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
    // This lane's rows i = 16 X + 4 q4 + e of k, q (channel 16 ct + lr), of v (column 16 wave
    // + lr) and of beta, for the dKg / dv products and the pair terms (G: Gr above), and the A~ and
    // beta of this wave's lower tiles for dA: all loaded here, so that their latency hides
    // under the products in between (rows past the sequence end read the last row and are
    // zeroed where they are used)
    const int cpr = 16 * (ct < KT ? ct : 0) + lr, jpr = 16 * (wave < VT ? wave : 0) + lr;
    Tin kraw[IT][4], qraw[IT][4], vraw[IT][4];
    float bl[IT][4];
#pragma unroll
    for (int X = 0; X < IT; ++X)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * X + 4 * q4 + e;
            const int64_t row = t0 + (i < L ? i : L - 1);
            const int64_t o = row * rsk + (int64_t)h * DK + cpr;
            kraw[X][e] = kin[o];
            qraw[X][e] = static_cast<const Tin *>(a.q)[o];
            vraw[X][e] = vin[row * rsv + (int64_t)h * DV + jpr];
            bl[X][e] = beta_of(i);
        }
    constexpr int NPT = (NLT + NWV - 1) / NWV;   // lower tiles per wave, at most
    float Atp[NPT][4], btp[NPT][4];
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        int it, jt;
        tile_of(wave + u * NWV < NLT ? wave + u * NWV : 0, it, jt);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * q4 + e;
            Atp[u][e] = rec[R::oA + i * C + 16 * jt + lr];
            btp[u][e] = beta_of(i);
        }
    }
    // dM = tril(dO U^T), written over M
    for (int p = wave; p < NLT; p += NWV) {
        int it, mt;
        tile_of(p, it, mt);
        f32x4 acc = zero4();
#pragma unroll
        for (int js = 0; js < VT; ++js) {
            const int j0 = 16 * js + 4 * q4;
            mma3(acc, unpack(*reinterpret_cast<const f32x4 *>(sdO + (16 * it + lr) * LDV + j0)),
                 unpack(*reinterpret_cast<const f32x4 *>(sU + (16 * mt + lr) * LDV + j0)));
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

    // dT = dU (beta v)^T + dW (beta k e^G)^T, lower tiles. The tiles (it, mt) of one column
    // block mt share their right operands (rows 16 mt .. 16 mt + 15 of beta v and of
    // beta k e^G): they go in pairs to one wave, which loads those rows once for both.
    {
        int g = wave, mt = 0;   // this wave's pair: column block mt, rows it0 (and it0 + 1)
        while (mt < IT && g >= (IT - mt + 1) / 2) {
            g -= (IT - mt + 1) / 2;
            ++mt;
        }
        if (mt < IT) {
            const int it0 = mt + 2 * g;
            const bool two = it0 + 1 < IT;
            const int it1 = two ? it0 + 1 : it0;
            const int m = 16 * mt + lr;
            const float bm = beta_of(m);  // 0 past the sequence end, which zeroes those rows
            // every load goes out before its products (a row past the end reads the last
            // valid row: finite, then zeroed by bm)
            const int64_t mrow = t0 + (m < L ? m : L - 1);
            f32x4 vb[VT];
#pragma unroll
            for (int js = 0; js < VT; ++js) vb[js] = load4(vin + mrow * rsv + (int64_t)h * DV + 16 * js + 4 * q4);
            f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
            for (int js = 0; js < VT; ++js) {
                const f32x4 b = vb[js] * bm;
                mma(acc0, *reinterpret_cast<const f32x4 *>(sdU + (16 * it0 + lr) * LDV + 16 * js + 4 * q4), b);
                if (two) mma(acc1, *reinterpret_cast<const f32x4 *>(sdU + (16 * it1 + lr) * LDV + 16 * js + 4 * q4), b);
            }
            f32x4 kv[KT], Gm[KT];
#pragma unroll
            for (int cs = 0; cs < KT; ++cs) {
                kv[cs] = load4(kin + mrow * rsk + (int64_t)h * DK + 16 * cs + 4 * q4);
                Gm[cs] = *reinterpret_cast<const f32x4 *>(rec + R::oG + m * DK + 16 * cs + 4 * q4);
            }
#pragma unroll
            for (int cs = 0; cs < KT; ++cs) {
                f32x4 kb;
#pragma unroll
                for (int e = 0; e < 4; ++e) kb[e] = bm * kv[cs][e] * __expf(Gm[cs][e]);
                mma(acc0, *reinterpret_cast<const f32x4 *>(sW + (16 * it0 + lr) * LDK + 16 * cs + 4 * q4), kb);
                if (two) mma(acc1, *reinterpret_cast<const f32x4 *>(sW + (16 * it1 + lr) * LDK + 16 * cs + 4 * q4), kb);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sdT[(16 * it0 + 4 * q4 + e) * LDA + m] = acc0[e];
                if (two) sdT[(16 * it1 + 4 * q4 + e) * LDA + m] = acc1[e];
            }
        }
    }
    // dKg = Diag(beta) T^T dW for key tile ct and dv = Diag(beta) T^T dU for value tile vt (both
    // the wave's; T[m][i] = 0 for m < i), with the rows of beta, G, k and v loaded above
    const bool doK = ct < KT, doV = wave < VT;
    if (doK || doV) {
        const int c = cpr, j = jpr;
        float Gl[IT][4], kl[IT][4], vl[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = 16 * it + 4 * q4 + e < L;   // rows past the end: zeroed by beta too
                Gl[it][e] = Gr[it][e];
                kl[it][e] = in ? to_f32(kraw[it][e]) : 0.f;
                vl[it][e] = in ? to_f32(vraw[it][e]) : 0.f;
            }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            f32x4 acc = zero4(), accv = zero4();
#pragma unroll
            for (int ms = 0; ms < IT; ++ms) {
                if (ms < it) continue;
                f32x4 A, B, Bv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 16 * ms + 4 * q4 + e;
                    A[e] = sT[m * LDA + 16 * it + lr];
                    B[e] = sW[m * LDK + c];
                    Bv[e] = sdU[m * LDV + j];
                }
                mma(acc, A, B);
                mma(accv, A, Bv);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * q4 + e;
                const float eG = __expf(Gl[it][e]);
                const float dKg = bl[it][e] * acc[e];
                if (doK) {
                    dk_p[it][e] += eG * dKg;
                    dG_p[it][e] += kl[it][e] * eG * dKg;
                }
                const float rs = sum16(acc[e] * kl[it][e] * eG);
                if (doK && lr == 0) sDb[ct][i] = rs;
                const float rv = sum16(accv[e] * vl[it][e]);
                if (doV && lr == 0) sDb[KT + wave][i] = rv;
                if (doV && i < L) a.dv[(t0 + i) * rsv + (int64_t)h * DV + j] = bl[it][e] * accv[e];
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
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        const int p = wave + u * NWV;
        if (p >= NLT) break;
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
            const float rs = sum16(dA * Atp[u][e]);
            if (lr == 0) sDb[KT + VT + jt][i] = rs;
            sdA[i * LDA + j] = btp[u][e] * dA;
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
        // this lane's rows of k and q (zero past the sequence end; G is constant there). Row
        // 16 X + 4 q4 + e of the token arrays is at lane_off + (16 X + e) * rsk (the stores of
        // dq and dk below).
        const int64_t lane_off = (t0 + 4 * q4) * rsk + (int64_t)h * DK + c;
        float kr[IT][4], qr[IT][4];
#pragma unroll
        for (int X = 0; X < IT; ++X)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = 16 * X + 4 * q4 + e < L;
                kr[X][e] = in ? to_f32(kraw[X][e]) : 0.f;
                qr[X][e] = in ? to_f32(qraw[X][e]) : 0.f;
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

// Compute units of the current device, queried once per device (0 if the query fails).
int64_t compute_units() {
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

template <typename Tin, int C, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
    using P = StatePass<C, DK, DV>;
    const dim3 gs((unsigned)a.nslots, (unsigned)a.H);
    // prep: one persistent workgroup per compute unit (at most one per item)
    const int64_t items = a.nslots * a.H, cus = compute_units();
    const unsigned gp = (unsigned)(cus > 0 && cus < items ? cus : items);
    hipLaunchKernelGGL((bwd_prep_kernel<Tin, C, DK, DV>), dim3(gp), dim3(512), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_state_kernel<C, DK, DV>), dim3(state_blocks<DV>(a.n_seqs * a.H)), dim3(64 * P::NW), 0,
                       stream, a);
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
