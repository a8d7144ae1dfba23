// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Buffer resource (scalar descriptor): base address plus a byte bound. Loads at offsets at
// or past the bound return zero and stores there are dropped, by the hardware.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Storage type of bf16 inputs: raw 16-bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

// Scalar helpers of the fused layer steps.
// softplus(z) = log(1 + e^z) = max(z, 0) + log(1 + e^-|z|), finite for every finite z
__device__ __forceinline__ float softplus_f(float z) {
    return fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
}
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
// 1/sqrt(s) for s > 0, else 0 (a zero vector stays zero)
__device__ __forceinline__ float rsqrt_or_zero(float s) { return s > 0.f ? __builtin_amdgcn_rsqf(s) : 0.f; }

// Token range [start, end) of packed sequence n, from the device-resident offsets cu[n] and
// cu[n + 1] clamped to [0, T] with end >= start. Valid offsets (cu[0] = 0, nondecreasing,
// cu[N] = T) pass unchanged; invalid ones give wrong results but never an access outside
// the caller's [T, ...] arrays.
__device__ __forceinline__ void packed_range(const int32_t *cu, int n, int64_t T, int64_t &start,
                                             int64_t &end) {
    int64_t s = cu[n], e = cu[n + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
    start = s;
    end = e;
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}

// The value of lane (lane ^ M) for M in {1, 2, 4, 8}: lanes of one 16-lane row exchange
// through DPP moves, without the LDS crossbar. quad_perm swaps within quads (M = 1, 2);
// row_shl:M reads lane + M and row_shr:M reads lane - M, picked by the lane's bit M.
template <int M> __device__ __forceinline__ float lane_xor(float x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "within a 16-lane row");
    const int v = __float_as_int(x);
    if constexpr (M == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
    } else if constexpr (M == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
    } else {
        const int below = __builtin_amdgcn_update_dpp(0, v, 0x110 + M, 0xF, 0xF, false);  // row_shr:M
        const int above = __builtin_amdgcn_update_dpp(0, v, 0x100 + M, 0xF, 0xF, false);  // row_shl:M
        return __int_as_float((threadIdx.x & M) ? below : above);
    }
}

// Transposing sum over the 16 lanes of each row: every lane holds 16 values; afterwards v[0] of
// lane l is the row's sum of value index bitrev4(l & 15). Each step keeps one half of the
// values and adds the partner lane's copy of that half.
template <int M, int NH> __device__ __forceinline__ void bfly_step(float (&v)[16]) {
    const bool up = (threadIdx.x & M) != 0;
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const float send = up ? v[i] : v[i + NH], keep = up ? v[i + NH] : v[i];
        v[i] = keep + lane_xor<M>(send);
    }
}
__device__ __forceinline__ void row_transpose_sum16(float (&v)[16]) {
    bfly_step<1, 8>(v);
    bfly_step<2, 4>(v);
    bfly_step<4, 2>(v);
    bfly_step<8, 1>(v);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }

// Two consecutive input elements as floats (8-byte or 4-byte aligned load).
__device__ __forceinline__ f32x2 load2(const float *p) { return *reinterpret_cast<const f32x2 *>(p); }
__device__ __forceinline__ f32x2 load2(const bf16_t *p) {
    const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
    f32x2 r;
    r.x = __uint_as_float(u << 16);
    r.y = __uint_as_float(u & 0xffff0000u);
    return r;
}

// Four consecutive input elements as floats.
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const bf16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    f32x4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
}

// ---------------------------------------------------------------------------------------
// 16x16 matrix-core tiles.
//
// Both operand fragments of a 16 x 16 x 16 product are read the same way: lane l holds
// "row" (l % 16) and the four consecutive reduction indices 4*(l/16) .. 4*(l/16)+3. For the
// A operand the row is an output row; for the B operand it is an output column, so B is
// stored transposed ([n][k]). The accumulator holds D[4*(l/16) + e][l % 16], e = 0..3,
// which is also exactly the B-fragment layout of a [k][n] operand with k = row: a product
// can feed the next one as its B operand without leaving registers.
//
// OP = __bf16: one v_mfma_f32_16x16x16_bf16.
// OP = _Float16: one v_mfma_f32_16x16x16_f16.
// OP = float : four v_mfma_f32_16x16x4_f32; instruction e takes reduction index 4*(l/16)+e
//              from every lane, so the four together cover all 16 indices.
// ---------------------------------------------------------------------------------------
template <typename OP> struct Mma;

template <> struct Mma<__bf16> {
    typedef __bf16 elem;
    typedef bf16x4 frag;
    static __device__ __forceinline__ frag load(const __bf16 *p) {
        return *reinterpret_cast<const frag *>(p);
    }
    static __device__ __forceinline__ frag from_f32(f32x4 x) {
        frag r;
        r.x = f32_to_bf16(x.x);
        r.y = f32_to_bf16(x.y);
        r.z = f32_to_bf16(x.z);
        r.w = f32_to_bf16(x.w);
        return r;
    }
    static __device__ __forceinline__ f32x4 to_f32(frag x) {
        f32x4 r;
        r.x = static_cast<float>(x.x);
        r.y = static_cast<float>(x.y);
        r.z = static_cast<float>(x.z);
        r.w = static_cast<float>(x.w);
        return r;
    }
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), acc, 0, 0, 0);
    }
    // acc += a * b with both factors given in float32, to ~float32 accuracy: each factor is
    // split into a bf16 head and a bf16 tail, and the three leading cross products are summed.
    static __device__ __forceinline__ void mma_split(f32x4 &acc, f32x4 a, f32x4 b) {
        const frag ah = from_f32(a), bh = from_f32(b);
        const frag al = from_f32(a - to_f32(ah)), bl = from_f32(b - to_f32(bh));
        mma(acc, al, bh);
        mma(acc, ah, bl);
        mma(acc, ah, bh);
    }
    static __device__ __forceinline__ void store_pair(__bf16 *p, float a, float b) {
        bf16x2 v;
        v.x = f32_to_bf16(a);
        v.y = f32_to_bf16(b);
        *reinterpret_cast<bf16x2 *>(p) = v;
    }
    static __device__ __forceinline__ void store4(__bf16 *p, f32x4 x) {
        *reinterpret_cast<frag *>(p) = from_f32(x);
    }
};

// OP = _Float16: one v_mfma_f32_16x16x16_f16. Same fragment layouts as bf16; 3 more
// mantissa bits, 8x smaller rounding error, but a narrow exponent range (about 2^+-15).
template <> struct Mma<_Float16> {
    typedef _Float16 elem;
    typedef f16x4 frag;
    static __device__ __forceinline__ frag load(const _Float16 *p) {
        return *reinterpret_cast<const frag *>(p);
    }
    static __device__ __forceinline__ frag from_f32(f32x4 x) {
        frag r;
        r.x = static_cast<_Float16>(x.x);
        r.y = static_cast<_Float16>(x.y);
        r.z = static_cast<_Float16>(x.z);
        r.w = static_cast<_Float16>(x.w);
        return r;
    }
    static __device__ __forceinline__ f32x4 to_f32(frag x) {
        f32x4 r;
        r.x = static_cast<float>(x.x);
        r.y = static_cast<float>(x.y);
        r.z = static_cast<float>(x.z);
        r.w = static_cast<float>(x.w);
        return r;
    }
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    }
    // float32-accurate product with float32's range: bf16 head and tail of each factor
    static __device__ __forceinline__ void mma_split(f32x4 &acc, f32x4 a, f32x4 b) {
        Mma<__bf16>::mma_split(acc, a, b);
    }
    static __device__ __forceinline__ void store_pair(_Float16 *p, float a, float b) {
        f16x2 v;
        v.x = static_cast<_Float16>(a);
        v.y = static_cast<_Float16>(b);
        *reinterpret_cast<f16x2 *>(p) = v;
    }
    static __device__ __forceinline__ void store4(_Float16 *p, f32x4 x) {
        *reinterpret_cast<frag *>(p) = from_f32(x);
    }
};

template <> struct Mma<float> {
    typedef float elem;
    typedef f32x4 frag;
    static __device__ __forceinline__ frag load(const float *p) {
        return *reinterpret_cast<const frag *>(p);
    }
    static __device__ __forceinline__ frag from_f32(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 to_f32(frag x) { return x; }
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ void mma_split(f32x4 &acc, f32x4 a, f32x4 b) { mma(acc, a, b); }
    static __device__ __forceinline__ void store_pair(float *p, float a, float b) {
        f32x2 v;
        v.x = a;
        v.y = b;
        *reinterpret_cast<f32x2 *>(p) = v;
    }
    static __device__ __forceinline__ void store4(float *p, f32x4 x) {
        *reinterpret_cast<f32x4 *>(p) = x;
    }
};

// ---------------------------------------------------------------------------------------
// Reduction steps of the widest matrix-core instruction of each operand type.
//
// A step adds KS reduction indices to a 16x16 float32 accumulator. Lane group q = lane/16
// supplies, for output row/column lane%16, the values of its own KS/4 reduction indices;
// A and B must supply matching indices, which is all the hardware requires. Two index
// assignments are used:
//  * contig: lane group q takes KS/4 consecutive indices starting at k0 + q*KS/4 (one
//    vector load from a row of a [row][k] LDS operand);
//  * split: lane group q takes indices 4q..4q+3 of each 16-index tile in the step, so that
//    a 16x16 accumulator tile held in registers (rows 4q..4q+3) is directly a B fragment
//    (regs()). The matching A fragment is one 8-byte load per tile (split()), or a single
//    16-byte load (permuted()) from an operand stored in perm() order.
// f16 / bf16: one v_mfma_f32_16x16x32 per step (KS = 32, two tiles); float: four
// v_mfma_f32_16x16x4 (KS = 16, one tile).
// ---------------------------------------------------------------------------------------
template <typename OP> struct Step;

template <typename H, typename V8, typename V4> struct Step16 {
    static constexpr int KS = 32;
    static constexpr int TPS = 2;
    typedef V8 frag;
    // Storage position of reduction index k in an operand read with perm(): within each
    // 32-index step the groups of four are ordered 0,4,1,5,2,6,3,7, so that the split index
    // set of lane group q (groups q and q+4) is 8 contiguous elements at 8q.
    static __device__ __forceinline__ int perm(int k) {
        const int g = (k >> 2) & 7;
        return (k & ~31) | (((g & 3) << 1 | (g >> 2)) << 2) | (k & 3);
    }
    static __device__ __forceinline__ frag permuted(const H *row, int k0, int q) {
        return *reinterpret_cast<const V8 *>(row + k0 + 8 * q);
    }
    static __device__ __forceinline__ frag contig(const H *row, int k0, int q) {
        return *reinterpret_cast<const V8 *>(row + k0 + 8 * q);
    }
    static __device__ __forceinline__ frag split(const H *row, int k0, int q) {
        const V4 a = *reinterpret_cast<const V4 *>(row + k0 + 4 * q);
        const V4 b = *reinterpret_cast<const V4 *>(row + k0 + 16 + 4 * q);
        return frag{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    }
    static __device__ __forceinline__ frag regs(const f32x4 *t) {
        return frag{static_cast<H>(t[0].x), static_cast<H>(t[0].y), static_cast<H>(t[0].z),
                    static_cast<H>(t[0].w), static_cast<H>(t[1].x), static_cast<H>(t[1].y),
                    static_cast<H>(t[1].z), static_cast<H>(t[1].w)};
    }
};

template <> struct Step<_Float16> : Step16<_Float16, f16x8, f16x4> {
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
};

template <> struct Step<__bf16> : Step16<__bf16, bf16x8, bf16x4> {
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};

template <> struct Step<float> {
    static constexpr int KS = 16;
    static constexpr int TPS = 1;
    typedef f32x4 frag;
    static __device__ __forceinline__ frag contig(const float *row, int k0, int q) {
        return *reinterpret_cast<const f32x4 *>(row + k0 + 4 * q);
    }
    static __device__ __forceinline__ frag split(const float *row, int k0, int q) {
        return contig(row, k0, q);
    }
    static __device__ __forceinline__ frag regs(const f32x4 *t) { return t[0]; }
    static __device__ __forceinline__ int perm(int k) { return k; }
    static __device__ __forceinline__ frag permuted(const float *row, int k0, int q) {
        return contig(row, k0, q);
    }
    static __device__ __forceinline__ void mma(f32x4 &acc, frag a, frag b) { Mma<float>::mma(acc, a, b); }
};

}  // namespace kda
