// C ABI of libkda (include/kda.h): host-side argument validation and kernel dispatch.
// Every check runs before any HIP call, so invalid requests launch nothing and leave the
// outputs untouched.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

kda_status ok() {
    g_err[0] = '\0';
    return KDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }

kda_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char *kda_status_string(int32_t status) {
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: return "KDA_ERR_UNKNOWN";
    }
}

const char *kda_last_error(void) { return g_err; }

int32_t kda_version(void) { return (1 << 16) | 0; }

size_t kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                     int32_t chunk, int32_t in_dtype, int32_t num_seqs) {
    if (B < 1 || T < 0 || H < 1 || !valid_dtype(in_dtype) ||
        !kda::chunk_fwd_supported(in_dtype, chunk, Dk, Dv))
        return 0;
    return kda::chunk_fwd_split_bytes(B, T, H, Dk, Dv, chunk, in_dtype, num_seqs);
}

kda_status kda_chunk_fwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                         int32_t in_dtype, int32_t out_dtype, float scale,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state, float *final_state, void *o,
                         const int32_t *cu_seqlens, int32_t num_seqs,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || chunk < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d T=%d H=%d Dk=%d Dv=%d chunk=%d)",
                    B, T, H, Dk, Dv, chunk);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d out=%d)", in_dtype, out_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
        if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
    } else if (num_seqs != B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    const int64_t tokens = (int64_t)B * T;
    if (tokens * H * (Dk > Dv ? Dk : Dv) > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    if (tokens > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o are required");
    const void *ptrs[] = {q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (workspace_bytes > 0 && !workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace_bytes > 0 with a NULL workspace");
    if (out_dtype != KDA_F32) return fail(KDA_ERR_UNSUPPORTED, "only float32 o is supported");
    if (!kda::chunk_fwd_supported(in_dtype, chunk, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no instantiation for in_dtype=%d chunk=%d Dk=%d Dv=%d",
                    in_dtype, chunk, Dk, Dv);
    if (num_seqs == 0) return ok();

    kda::ChunkArgs a;
    a.n_seqs = num_seqs;
    a.seq_len = T;
    a.cu_seqlens = cu_seqlens;
    a.H = H;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.s0 = initial_state;
    a.s_out = final_state;
    a.o = o;
    a.f = kda::Fusion{};
    a.seg_len = 0;
    a.nseg = 1;
    a.ws_r = a.ws_x = a.ws_s = nullptr;
    a.rec = nullptr;
    a.rec_chunks = 0;
    a.out_from = 0;
    a.order = nullptr;
    return hip_status(kda::launch_chunk_fwd(in_dtype, chunk, Dk, Dv, a, workspace, workspace_bytes,
                                            static_cast<hipStream_t>(stream)),
                      "kda_chunk_fwd launch");
}

size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                     int32_t chunk, int32_t in_dtype, int32_t num_seqs) {
    if (!valid_dtype(in_dtype)) return 0;
    return kda::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, num_seqs);
}

}  // extern "C"

namespace {

// Checks of kda_chunk_bwd's arguments other than the workspace, before any HIP call; fills
// `a` (all but the workspace) on success.
kda_status check_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                     int32_t in_dtype, float scale, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const float *initial_state,
                     const float *d_o, const float *d_final_state, float *dq, float *dk, float *dv,
                     float *dg, float *dbeta, float *d_initial_state, const int32_t *cu_seqlens,
                     int32_t num_seqs, kda::BwdArgs &a) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || chunk < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d T=%d H=%d Dk=%d Dv=%d chunk=%d)",
                    B, T, H, Dk, Dv, chunk);
    if (!valid_dtype(in_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d)", in_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
        if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
    } else if (num_seqs != B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    const int64_t tokens = (int64_t)B * T;
    if (tokens * H * (Dk > Dv ? Dk : Dv) > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    if (tokens > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, d_o, dq, dk, dv, dg and dbeta are required");
    const void *ptrs[] = {q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                          d_initial_state, cu_seqlens};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (!kda::chunk_bwd_supported(in_dtype, chunk, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no backward instantiation for in_dtype=%d chunk=%d Dk=%d Dv=%d",
                    in_dtype, chunk, Dk, Dv);
    a.n_seqs = num_seqs;
    a.seq_len = T;
    a.cu_seqlens = cu_seqlens;
    a.H = H;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.s0 = initial_state;
    a.dout = d_o;
    a.dsT = d_final_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dg = dg;
    a.dbeta = dbeta;
    a.ds0 = d_initial_state;
    a.ws = nullptr;
    a.nslots = num_seqs + (tokens + chunk - 1) / chunk;
    // record slots x heads index the kernels' work items in 32 bits (far beyond any workspace)
    if (a.nslots * H > ((int64_t)1 << 30)) return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                         int32_t in_dtype, float scale,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *initial_state,
                         const float *d_o, const float *d_final_state,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta,
                         float *d_initial_state,
                         const int32_t *cu_seqlens, int32_t num_seqs,
                         void *workspace, size_t workspace_bytes, void *stream) {
    kda::BwdArgs a;
    const kda_status st = check_bwd(B, T, H, Dk, Dv, chunk, in_dtype, scale, q, k, v, g, beta, initial_state,
                                    d_o, d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, cu_seqlens,
                                    num_seqs, a);
    if (st != KDA_OK) return st;
    if (workspace && !aligned16(workspace))
        return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    const size_t need = kda::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, num_seqs);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "kda_chunk_bwd needs %zu workspace bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (num_seqs == 0) return ok();
    a.ws = static_cast<float *>(workspace);
    return hip_status(kda::launch_chunk_bwd(in_dtype, chunk, Dk, Dv, a, static_cast<hipStream_t>(stream)),
                      "kda_chunk_bwd launch");
}

kda_status kda_chunk_bwd_noalloc(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                                 int32_t in_dtype, float scale,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, const float *initial_state,
                                 const float *d_o, const float *d_final_state,
                                 float *dq, float *dk, float *dv, float *dg, float *dbeta,
                                 float *d_initial_state,
                                 const int32_t *cu_seqlens, int32_t num_seqs, void *stream) {
    kda::BwdArgs a;
    const kda_status st = check_bwd(B, T, H, Dk, Dv, chunk, in_dtype, scale, q, k, v, g, beta, initial_state,
                                    d_o, d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, cu_seqlens,
                                    num_seqs, a);
    if (st != KDA_OK) return st;
    const size_t need = kda::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, in_dtype, num_seqs);
    if (need > kda::kBwdScratchBytes)
        return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                    "kda_chunk_bwd_noalloc: this problem needs %zu bytes of records, beyond the fixed "
                    "scratch of %zu bytes (call kda_chunk_bwd with a workspace instead)",
                    need, kda::kBwdScratchBytes);
    if (num_seqs == 0) return ok();
    void *scratch = nullptr;
    const kda_status ss = hip_status(kda::bwd_scratch(&scratch), "kda_chunk_bwd_noalloc scratch lookup");
    if (ss != KDA_OK) return ss;
    a.ws = static_cast<float *>(scratch);
    return hip_status(kda::launch_chunk_bwd(in_dtype, chunk, Dk, Dv, a, static_cast<hipStream_t>(stream)),
                      "kda_chunk_bwd_noalloc launch");
}

kda_status kda_decode_step(int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                           int32_t in_dtype, int32_t out_dtype, float scale,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, void *o, void *stream) {
    if (N < 0 || H < 1 || Dk < 1 || Dv < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes (N=%d H=%d Dk=%d Dv=%d)", N, H, Dk, Dv);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d out=%d)", in_dtype, out_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if ((int64_t)N * H > 0x7fffffff) return fail(KDA_ERR_INVALID_ARGUMENT, "N*H too large");
    if (N > 0 && (!q || !k || !v || !g || !beta || !state || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, state and o are required");
    const void *ptrs[] = {q, k, v, g, beta, state, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (out_dtype != KDA_F32) return fail(KDA_ERR_UNSUPPORTED, "only float32 o is supported");
    if (!kda::decode_supported(in_dtype, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no decode instantiation for in_dtype=%d Dk=%d Dv=%d",
                    in_dtype, Dk, Dv);
    if (N == 0) return ok();
    kda::DecodeArgs a;
    a.N = N;
    a.H = H;
    a.L = 1;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.f = kda::Fusion{};
    return hip_status(kda::launch_decode(in_dtype, Dk, Dv, a, static_cast<hipStream_t>(stream)),
                      "kda_decode_step launch");
}

}  // extern "C"

namespace {

// Checks of a kda_fusion shared by both fused entry points; fills `f`.
kda_status check_fusion(const kda_fusion *fusion, int32_t out_dtype, kda::Fusion &f) {
    if (!fusion) return fail(KDA_ERR_INVALID_ARGUMENT, "fusion is required");
    if (!fusion->gate_x || !fusion->A_log || !fusion->dt_bias)
        return fail(KDA_ERR_INVALID_ARGUMENT, "gate_x, A_log and dt_bias are required");
    if (fusion->o_gate && !fusion->o_weight)
        return fail(KDA_ERR_INVALID_ARGUMENT, "o_weight is required with o_gate");
    if (fusion->o_gate && !(fusion->o_eps >= 0.f && std::isfinite(fusion->o_eps)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "o_eps must be finite and >= 0");
    if (out_dtype == KDA_BF16 && !fusion->o_gate)
        return fail(KDA_ERR_UNSUPPORTED, "bf16 o needs the output norm (o_gate)");
    const void *ptrs[] = {fusion->gate_x, fusion->A_log, fusion->dt_bias, fusion->o_gate, fusion->o_weight};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    f.gx = fusion->gate_x;
    f.A_log = fusion->A_log;
    f.dt_bias = fusion->dt_bias;
    f.norm_qk = fusion->normalize_qk ? 1 : 0;
    f.og = fusion->o_gate;
    f.ow = fusion->o_gate ? fusion->o_weight : nullptr;
    f.oeps = fusion->o_gate ? fusion->o_eps : 0.f;
    f.o_bf16 = out_dtype == KDA_BF16 ? 1 : 0;
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_fused(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                               int32_t in_dtype, int32_t out_dtype, float scale,
                               const void *q, const void *k, const void *v,
                               const kda_fusion *fusion, const float *beta,
                               const float *initial_state, float *final_state, void *o,
                               const int32_t *cu_seqlens, int32_t num_seqs,
                               void *workspace, size_t workspace_bytes, void *stream) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || chunk < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d T=%d H=%d Dk=%d Dv=%d chunk=%d)",
                    B, T, H, Dk, Dv, chunk);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d out=%d)", in_dtype, out_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
        if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
    } else if (num_seqs != B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    const int64_t tokens = (int64_t)B * T;
    if (tokens * H * (Dk > Dv ? Dk : Dv) > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    kda::Fusion f;
    const kda_status fs = check_fusion(fusion, out_dtype, f);
    if (fs != KDA_OK) return fs;
    if (tokens > 0 && (!q || !k || !v || !beta || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, beta and o are required");
    const void *ptrs[] = {q, k, v, beta, initial_state, final_state, o, cu_seqlens, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (workspace_bytes > 0 && !workspace)
        return fail(KDA_ERR_INVALID_ARGUMENT, "workspace_bytes > 0 with a NULL workspace");
    if (!kda::chunk_fwd_fused_supported(in_dtype, chunk, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no fused instantiation for in_dtype=%d chunk=%d Dk=%d Dv=%d",
                    in_dtype, chunk, Dk, Dv);
    if (num_seqs == 0) return ok();

    kda::ChunkArgs a;
    a.n_seqs = num_seqs;
    a.seq_len = T;
    a.cu_seqlens = cu_seqlens;
    a.H = H;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = nullptr;
    a.beta = beta;
    a.s0 = initial_state;
    a.s_out = final_state;
    a.o = o;
    a.f = f;
    a.seg_len = 0;
    a.nseg = 1;
    a.ws_r = a.ws_x = a.ws_s = nullptr;
    a.rec = nullptr;
    a.rec_chunks = 0;
    a.out_from = 0;
    a.order = nullptr;
    return hip_status(kda::launch_chunk_fwd(in_dtype, chunk, Dk, Dv, a, workspace, workspace_bytes,
                                            static_cast<hipStream_t>(stream)),
                      "kda_chunk_fwd_fused launch");
}

kda_status kda_decode_step_fused(int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                                 int32_t in_dtype, int32_t out_dtype, float scale,
                                 const void *q, const void *k, const void *v,
                                 const kda_fusion *fusion, const float *beta,
                                 float *state, void *o, void *stream) {
    if (N < 0 || H < 1 || Dk < 1 || Dv < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes (N=%d H=%d Dk=%d Dv=%d)", N, H, Dk, Dv);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d out=%d)", in_dtype, out_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if ((int64_t)N * H > 0x7fffffff) return fail(KDA_ERR_INVALID_ARGUMENT, "N*H too large");
    kda::Fusion f;
    const kda_status fs = check_fusion(fusion, out_dtype, f);
    if (fs != KDA_OK) return fs;
    if (N > 0 && (!q || !k || !v || !beta || !state || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, beta, state and o are required");
    const void *ptrs[] = {q, k, v, beta, state, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (!kda::decode_supported(in_dtype, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no decode instantiation for in_dtype=%d Dk=%d Dv=%d",
                    in_dtype, Dk, Dv);
    if (N == 0) return ok();
    kda::DecodeArgs a;
    a.N = N;
    a.H = H;
    a.L = 1;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = nullptr;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.f = f;
    return hip_status(kda::launch_decode(in_dtype, Dk, Dv, a, static_cast<hipStream_t>(stream)),
                      "kda_decode_step_fused launch");
}

}  // extern "C"

extern "C" {

kda_status kda_short_conv_fwd(int32_t B, int32_t T, int32_t C, int32_t W, int32_t dtype,
                              int32_t activation, const void *x, const float *weight,
                              const float *bias, const void *initial_state, void *final_state,
                              void *y, const int32_t *cu_seqlens, int32_t num_seqs, void *stream) {
    if (B < 1 || T < 0 || C < 1 || W < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes (B=%d T=%d C=%d W=%d)", B, T, C, W);
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code %d", dtype);
    if (activation != KDA_ACT_NONE && activation != KDA_ACT_SILU)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown activation %d", activation);
    if (cu_seqlens) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens requires B == 1 (got B=%d)", B);
        if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
    } else if (num_seqs != B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                    num_seqs, B);
    }
    const int64_t tokens = (int64_t)B * T;
    if (tokens * C > ((int64_t)1 << 40)) return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    if (!weight) return fail(KDA_ERR_INVALID_ARGUMENT, "weight is required");
    if (tokens > 0 && (!x || !y)) return fail(KDA_ERR_INVALID_ARGUMENT, "x and y are required");
    const void *ptrs[] = {x, weight, bias, initial_state, final_state, y, cu_seqlens};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (!kda::conv_supported(dtype, C, W))
        return fail(KDA_ERR_UNSUPPORTED, "no short-convolution instantiation for dtype=%d C=%d W=%d "
                    "(W = 4, C a multiple of 8)", dtype, C, W);
    if (num_seqs == 0) return ok();
    kda::ConvArgs a;
    a.n_seqs = num_seqs;
    a.seq_len = T;
    a.cu_seqlens = cu_seqlens;
    a.tokens = tokens;
    a.C = C;
    a.x = x;
    a.w = weight;
    a.bias = bias;
    a.s0 = initial_state;
    a.s_out = final_state;
    a.y = y;
    a.silu = activation == KDA_ACT_SILU ? 1 : 0;
    return hip_status(kda::launch_conv(dtype, a, false, static_cast<hipStream_t>(stream)),
                      "kda_short_conv_fwd launch");
}

kda_status kda_short_conv_update(int32_t N, int32_t C, int32_t W, int32_t dtype, int32_t activation,
                                 const void *x, const float *weight, const float *bias, void *state,
                                 void *y, void *stream) {
    if (N < 0 || C < 1 || W < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes (N=%d C=%d W=%d)", N, C, W);
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code %d", dtype);
    if (activation != KDA_ACT_NONE && activation != KDA_ACT_SILU)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown activation %d", activation);
    if ((int64_t)N * C > ((int64_t)1 << 40)) return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    if (!weight) return fail(KDA_ERR_INVALID_ARGUMENT, "weight is required");
    if (N > 0 && (!x || !state || !y)) return fail(KDA_ERR_INVALID_ARGUMENT, "x, state and y are required");
    const void *ptrs[] = {x, weight, bias, state, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (!kda::conv_supported(dtype, C, W))
        return fail(KDA_ERR_UNSUPPORTED, "no short-convolution instantiation for dtype=%d C=%d W=%d "
                    "(W = 4, C a multiple of 8)", dtype, C, W);
    if (N == 0) return ok();
    kda::ConvArgs a;
    a.n_seqs = N;
    a.seq_len = 1;
    a.cu_seqlens = nullptr;
    a.tokens = N;
    a.C = C;
    a.x = x;
    a.w = weight;
    a.bias = bias;
    a.s0 = state;
    a.s_out = state;
    a.y = y;
    a.silu = activation == KDA_ACT_SILU ? 1 : 0;
    return hip_status(kda::launch_conv(dtype, a, true, static_cast<hipStream_t>(stream)),
                      "kda_short_conv_update launch");
}

}  // extern "C"

extern "C" {

kda_status kda_recurrent_fwd(int32_t N, int32_t L, int32_t H, int32_t Dk, int32_t Dv,
                             int32_t in_dtype, int32_t out_dtype, float scale,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             float *state, void *o, void *stream) {
    if (N < 0 || L < 0 || H < 1 || Dk < 1 || Dv < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes (N=%d L=%d H=%d Dk=%d Dv=%d)", N, L, H, Dk, Dv);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown dtype code (in=%d out=%d)", in_dtype, out_dtype);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if ((int64_t)N * H > 0x7fffffff) return fail(KDA_ERR_INVALID_ARGUMENT, "N*H too large");
    if ((int64_t)N * L * H * (Dk > Dv ? Dk : Dv) > ((int64_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "problem too large");
    if ((int64_t)N * L > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o are required");
    if (N > 0 && !state) return fail(KDA_ERR_INVALID_ARGUMENT, "state is required");
    const void *ptrs[] = {q, k, v, g, beta, state, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (out_dtype != KDA_F32) return fail(KDA_ERR_UNSUPPORTED, "only float32 o is supported");
    if (!kda::decode_supported(in_dtype, Dk, Dv))
        return fail(KDA_ERR_UNSUPPORTED, "no recurrent instantiation for in_dtype=%d Dk=%d Dv=%d",
                    in_dtype, Dk, Dv);
    if (N == 0 || L == 0) return ok();
    kda::DecodeArgs a;
    a.N = N;
    a.H = H;
    a.L = L;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.f = kda::Fusion{};
    return hip_status(kda::launch_decode(in_dtype, Dk, Dv, a, static_cast<hipStream_t>(stream)),
                      "kda_recurrent_fwd launch");
}

kda_status kda_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "src, dst and a positive multiple of 16 bytes are required");
    if (!aligned16(src) || !aligned16(dst))
        return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    return hip_status(kda::launch_probe_copy(src, dst, (int64_t)bytes, static_cast<hipStream_t>(stream)),
                      "kda_probe_copy launch");
}

kda_status kda_probe_read(const void *src, size_t bytes, void *stream) {
    if (!src || bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "src and a positive multiple of 16 bytes are required");
    if (!aligned16(src)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    return hip_status(kda::launch_probe_read(src, (int64_t)bytes, static_cast<hipStream_t>(stream)),
                      "kda_probe_read launch");
}

kda_status kda_probe_rmw(void *buf, size_t bytes, float factor, void *stream) {
    if (!buf || bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
        return fail(KDA_ERR_INVALID_ARGUMENT, "buf and a positive multiple of 16 bytes are required");
    if (!aligned16(buf)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    if (!std::isfinite(factor)) return fail(KDA_ERR_INVALID_ARGUMENT, "factor must be finite");
    return hip_status(kda::launch_probe_rmw(buf, (int64_t)bytes, factor, static_cast<hipStream_t>(stream)),
                      "kda_probe_rmw launch");
}

static kda_status probe_mfma(int32_t bf16, int32_t shape, int32_t iters, int32_t blocks, float *sink,
                             void *stream) {
    if (shape < 0 || shape > 1 || iters < 1 || blocks < 1 || !sink)
        return fail(KDA_ERR_INVALID_ARGUMENT, "shape 0 or 1, positive iters and blocks, and sink are required");
    if (!aligned16(sink)) return fail(KDA_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
    return hip_status(kda::launch_probe_mfma(bf16, shape, iters, blocks, sink, static_cast<hipStream_t>(stream)),
                      bf16 ? "kda_probe_mfma_bf16 launch" : "kda_probe_mfma_f16 launch");
}

kda_status kda_probe_mfma_f16(int32_t shape, int32_t iters, int32_t blocks, float *sink, void *stream) {
    return probe_mfma(0, shape, iters, blocks, sink, stream);
}

kda_status kda_probe_mfma_bf16(int32_t shape, int32_t iters, int32_t blocks, float *sink, void *stream) {
    return probe_mfma(1, shape, iters, blocks, sink, stream);
}

double kda_probe_mfma_f16_flops(int32_t iters, int32_t blocks) {
    return (double)iters * (double)blocks * 256.0 * (double)kda::probe_mfma_flops_per_iter_and_thread();
}

}  // extern "C"
