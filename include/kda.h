/*
 * kda.h - C ABI of the MI355X (gfx950) KDA core: Kimi Delta Attention, the gated delta rule
 * with a per-channel (fine-grained) forget gate.
 *
 * The operation (per sequence n and head h, over its tokens t = 1..L_n):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (scale * q_t)
 *
 * Sources (web pages on Kimi Linear; short names used throughout this code):
 *   [KV-cache page]  "Starting from the KV-cache explosion: what KimiLinear's linear
 *                    attention solves" (hands-on guide, sections 1-6)
 *   [loading page]   "Starting from a loading error: configuring Kimi Linear's KDA and
 *                    NoPE" (walk-through of the modelling code, sections 1-6)
 *   [overview page]  "How to fit a million tokens on an ordinary GPU with Kimi Linear"
 *   [revolution page] "Linear attention revolution: Kimi Linear ..." (model overview)
 *
 * S is a d_k x d_v state per (sequence, head) whose rows are key channels: KDA keeps a
 * fixed-size state matrix that does not grow with the sequence ([KV-cache page] section 2).
 * exp(g_t) is KDA's channel-wise forget gate, the fine-grained gating that refines Gated
 * DeltaNet ([revolution page], the KDA section; [overview page], "How Kimi Delta Attention
 * works"). (I - beta k k^T) is the delta-rule erase term, which keeps the state bounded only
 * for unit-norm keys ([KV-cache page] section 5: without L2-normalised q and k the state
 * blows up to NaN). The library does not normalise: callers pass normalised q and k.
 *
 * Two entry points do the work; kda_recurrent_fwd runs several tokens per sequence in the
 * decode kernel's way; two fused variants add the KDA layer's steps on either side of the
 * core (kda_chunk_fwd_fused, kda_decode_step_fused); two more run the layer's short
 * convolution with its conv state (kda_short_conv_fwd, kda_short_conv_update); kda_chunk_bwd
 * is the backward pass of kda_chunk_fwd (training), and kda_chunk_bwd_noalloc the same for
 * callers that cannot allocate a workspace; and two measurement probes report the
 * device's practical bandwidth and matrix-core peaks (kda_probe_copy/read/rmw, kda_probe_mfma_f16/bf16, at the
 * end of this file):
 *   kda_chunk_fwd    prefill: the chunkwise-parallel form of the recurrence ([KV-cache page]
 *                    section 3: chunk_size 64; section 6: chunked parallel form with a WY
 *                    representation), over fixed-length batches or packed variable-length
 *                    sequences, with optional initial and final states. It computes exactly
 *                    the recurrence above, up to floating-point rounding.
 *   kda_decode_step  one token per (sequence, head) on a persistent float32 state, updated in
 *                    place (the token-by-token "fused_recurrent" mode and the recurrent state
 *                    that the decode cache carries across calls: [loading page] sections 2,
 *                    5 and 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers. Every tensor pointer is a DEVICE pointer (HIP device memory) owned by the
 *   caller; the library allocates nothing and keeps no per-call state (scratch space, where
 *   a call needs it, is the caller's workspace argument; the one exception,
 *   kda_chunk_bwd_noalloc, uses a fixed device array the library holds instead). Tensors
 *   are dense and contiguous with the last dimension innermost ("... h d" layout), and
 *   16-byte aligned.
 * - Dtypes. q, k, v are KDA_F32 or KDA_BF16 (in_dtype); g (log-decay, <= 0), beta, states
 *   and o are float32 (out_dtype must be KDA_F32, except after the fused output norm); the
 *   backward pass's gradients are float32.
 * - Streams. `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work on
 *   it and never synchronise the host. Calls on different streams are independent.
 * - Errors. Arguments are validated on the host before any HIP call: on an error nothing is
 *   launched and no output is touched. A failed launch returns KDA_ERR_HIP. The message of
 *   the last error on the calling thread is available from kda_last_error().
 * - Not checked (preconditions): the contents of device arrays (cu_seqlens values, NaN or
 *   Inf inputs, which propagate), and overlaps between outputs and inputs other than the
 *   allowed final_state == initial_state aliasing. The kernels clamp packed offsets: sequence
 *   n covers [s, e) with s = cu[n] and e = cu[n+1] clamped to [0, T] and e >= s, so offsets
 *   that break the precondition give the result of those clamped ranges (wrong, and racy
 *   where two ranges overlap) but never an access outside the caller's arrays.
 * - Supported sizes: see kda_chunk_fwd and kda_decode_step.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

/* Bytes of the fixed device scratch behind kda_chunk_bwd_noalloc (per device). */
#define KDA_BWD_SCRATCH_BYTES ((size_t)512 << 20)

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* NULL or misaligned pointer, bad size, bad dtype code */
    KDA_ERR_UNSUPPORTED = 2,      /* valid request with no compiled instantiation */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Human-readable name of a status code (static storage). */
const char *kda_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread (static, thread-local
 * storage; empty string if none). */
const char *kda_last_error(void);

/* Library version, (major << 16) | minor. */
int32_t kda_version(void);

/*
 * kda_chunk_fwd_workspace_bytes - optional device workspace for kda_chunk_fwd with these
 * sizes on the current device (0 when it would not be used).
 *
 * Fixed-length batches (num_seqs == B): with few (sequence, head) chains the recurrence
 * would occupy only a few compute units, so each sequence may be cut into segments. The
 * chunked forward runs all segments at once: segment 0 from the initial state (writing its
 * outputs, except with the fused output norm), the others from zero, recording each chunk's
 * operands. A replay pass computes each later segment's linear state map from the records,
 * the maps are chained into the true start state of every segment, and a second replay pass
 * produces the remaining outputs and the final state. The workspace holds the records, maps
 * and states (about 74 KB per chunk and head for the bf16 instantiation, plus three states
 * per segment).
 * Packed batches (cu_seqlens): num_seqs int32 for running the sequences longest first.
 * The workspace is optional: with less (or NULL) the call runs unsplit / in the given order,
 * with the same result up to rounding.
 */
size_t kda_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                     int32_t chunk, int32_t in_dtype, int32_t num_seqs);

/*
 * kda_chunk_fwd - chunked prefill.
 *
 * Sequences. Without cu_seqlens: B sequences of T tokens each (num_seqs must equal B), and
 * the token index of (b, t) is b*T + t. With cu_seqlens (device int32 [num_seqs + 1],
 * cu[0] = 0, non-decreasing, cu[num_seqs] = T): B must be 1 and sequence n is tokens
 * cu[n] .. cu[n+1]-1 of the packed batch; zero-length sequences are allowed (their final
 * state is their initial state). T = 0 is allowed.
 *
 *   q, k          [B*T, H, Dk]  in_dtype, unit L2 norm per (token, head)
 *   v             [B*T, H, Dv]  in_dtype
 *   g             [B*T, H, Dk]  float32 log-decay (the gate is exp(g) <= 1)
 *   beta          [B*T, H]      float32 write strength in [0, 1]
 *   initial_state [N, H, Dk, Dv] float32, or NULL for zeros (N = num_seqs)
 *   final_state   [N, H, Dk, Dv] float32 output, or NULL to skip; may equal initial_state
 *                 (exact aliasing: each state is read before it is overwritten)
 *   o             [B*T, H, Dv]  out_dtype (KDA_F32)
 *   chunk         tokens per chunk of the chunkwise form (a tuning choice: every chunk
 *                 size gives the same result up to rounding)
 *   scale         multiplies q (finite)
 *   workspace     optional device buffer (see kda_chunk_fwd_workspace_bytes); its contents
 *                 are scratch, overwritten by the call
 *
 * Compiled instantiations (in_dtype, chunk, Dk = Dv):
 *   (KDA_BF16, 64, 128)   bf16 inputs; fp16 matrix-core operands (decay factors balanced
 *                         by powers of two into fp16's range), float32 accumulation and
 *                         state; exact for any finite g <= 0 (chunks whose 16-token decay
 *                         falls below e^-12 sum their diagonal blocks pair by pair).
 *                         Range precondition (not checked): the state S, the intra-chunk
 *                         values U~ = T Diag(beta) V and U = U~ - W S, and v itself enter the
 *                         matrix cores as fp16, so their magnitudes must stay below fp16's
 *                         largest value, 65504; beyond it the outputs turn non-finite. With
 *                         unit-norm keys and beta in [0, 1] the state stays within a small
 *                         multiple of max |v| and of the initial state (the erase term has
 *                         spectral norm <= 1), so |v| and |initial_state| up to about 10^3 are
 *                         far inside it. The float32 instantiations have no such limit.
 *   (KDA_F32, 16, 16), (KDA_F32, 16, 32), (KDA_F32, 32, 128), (KDA_F32, 64, 32),
 *   (KDA_F32, 64, 64)     float32 matrix-core path (reference-precision instantiations;
 *                         D = 32 runs at two chunk sizes, which give the same result up to
 *                         rounding; at D = 128 the float32 operands fit one CU's LDS with
 *                         32-token chunks)
 * Other combinations return KDA_ERR_UNSUPPORTED.
 */
kda_status kda_chunk_fwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                         int32_t in_dtype, int32_t out_dtype, float scale,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state, float *final_state, void *o,
                         const int32_t *cu_seqlens, int32_t num_seqs,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step - one recurrent step for N independent (sequence, head) states.
 *
 *   q, k    [N, H, Dk] in_dtype (unit L2 norm)     v [N, H, Dv] in_dtype
 *   g       [N, H, Dk] float32 log-decay             beta [N, H] float32
 *   state   [N, H, Dk, Dv] float32, read and updated in place (S_{t-1} -> S_t)
 *   o       [N, H, Dv] out_dtype (KDA_F32): S_t^T (scale * q)
 *
 * Dk = Dv in {16, 32, 64, 128}; in_dtype KDA_F32 or KDA_BF16.
 */
kda_status kda_decode_step(int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                           int32_t in_dtype, int32_t out_dtype, float scale,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, void *o, void *stream);

/*
 * kda_recurrent_fwd - L tokens per (sequence, head), token by token, on a persistent float32
 * state: the recurrent ("fused_recurrent") mode that the layer uses for short queries
 * ([loading page] section 5), e.g. several tokens per decode step. The state is read once and
 * written once per call, whatever L is; kda_decode_step is the case L = 1.
 *
 *   q, k, g [N, L, H, Dk]; v [N, L, H, Dv]; beta [N, L, H]  (in_dtype / float32 as in
 *   kda_decode_step; token t of sequence n is row n*L + t)
 *   state   [N, H, Dk, Dv] float32, S_0 in, S_L out (in place)
 *   o       [N, L, H, Dv] out_dtype (KDA_F32)
 *
 * The same result as kda_chunk_fwd over those L tokens with initial_state = final_state =
 * state, up to rounding. Dk = Dv in {16, 32, 64, 128}; L >= 0 (L = 0 leaves the state as it
 * is). Errors as kda_decode_step.
 */
kda_status kda_recurrent_fwd(int32_t N, int32_t L, int32_t H, int32_t Dk, int32_t Dv,
                             int32_t in_dtype, int32_t out_dtype, float scale,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             float *state, void *o, void *stream);

/*
 * kda_fusion - the KDA layer's steps on either side of the core, done inside the kernels.
 *
 * Input side ([loading page] section 3: the KDA layer's gate parameters A_log, the decay
 * rate, and dt_bias, a time-step bias; [KV-cache page] sections 3 and 5: q and k must be
 * L2-normalised):
 *   gate_x        [tokens, H, Dk] in_dtype, the forget gate's pre-activation (required):
 *                 g = -exp(A_log[h]) * softplus(gate_x + dt_bias[h, c]) replaces the g input
 *   A_log         [H] float32 (required)
 *   dt_bias       [H, Dk] float32 (required)
 *   normalize_qk  nonzero: q and k are divided by their L2 norm per (token, head) (a zero
 *                 vector stays zero); zero: q and k are used as given
 * Output side ([loading page] section 3: o_norm, a gated RMSNorm with a sigmoid gate):
 *   o_gate        [tokens, H, Dv] in_dtype, the output gate's pre-activation, or NULL for
 *                 the raw read-out o_t
 *   o_weight      [Dv] float32 gain (required with o_gate)
 *   o_eps         >= 0; with o_gate the output is, per (token, head),
 *                 y = o / sqrt(mean(o^2) + o_eps) * o_weight * sigmoid(o_gate)
 * Every pointer is a 16-byte aligned device pointer owned by the caller.
 */
typedef struct kda_fusion {
    const void *gate_x;
    const float *A_log;
    const float *dt_bias;
    int32_t normalize_qk;
    const void *o_gate;
    const float *o_weight;
    float o_eps;
} kda_fusion;

/*
 * kda_chunk_fwd_fused - kda_chunk_fwd with the fused layer steps: the gate from gate_x
 * (no g argument), optional q/k normalisation, and optionally the output norm, written as
 * float32 or bf16 (out_dtype KDA_BF16 requires o_gate). Every other argument, the
 * workspace (kda_chunk_fwd_workspace_bytes), the sequence layout and the errors are those of
 * kda_chunk_fwd; fusion == NULL or a NULL required field is KDA_ERR_INVALID_ARGUMENT.
 * Compiled instantiation: (KDA_BF16, chunk 64, Dk = Dv = 128); others are UNSUPPORTED.
 */
kda_status kda_chunk_fwd_fused(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                               int32_t in_dtype, int32_t out_dtype, float scale,
                               const void *q, const void *k, const void *v,
                               const kda_fusion *fusion, const float *beta,
                               const float *initial_state, float *final_state, void *o,
                               const int32_t *cu_seqlens, int32_t num_seqs,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step_fused - kda_decode_step with the fused layer steps (gate from gate_x,
 * optional q/k normalisation, optional output norm with float32 or bf16 output). Sizes,
 * dtypes and errors as kda_decode_step.
 */
kda_status kda_decode_step_fused(int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                                 int32_t in_dtype, int32_t out_dtype, float scale,
                                 const void *q, const void *k, const void *v,
                                 const kda_fusion *fusion, const float *beta,
                                 float *state, void *o, void *stream);

/*
 * The short causal convolution in front of the core ([loading page] section 3: the KDA
 * layer's short convolution, kernel size 4; section 6: the decode cache carries its
 * conv_states beside the recurrent states). Depthwise over the channels of a [tokens, C]
 * tensor (the layer's q, k or v projections, or several side by side), per sequence:
 *
 *     y_t[c] = act(bias[c] + sum_{j < W} weight[c][j] * x_{t-W+1+j}[c])
 *
 * where the inputs before a sequence's first token come from its conv state, the W - 1
 * previous inputs oldest first (zeros without one). act: KDA_ACT_NONE or KDA_ACT_SILU (the
 * pages name no activation). Computed in float32, stored in dtype.
 */
typedef enum kda_activation { KDA_ACT_NONE = 0, KDA_ACT_SILU = 1 } kda_activation;

/*
 * kda_chunk_bwd - the backward pass of kda_chunk_fwd (the training side of the layer, which
 * runs in chunk mode: [loading page] section 5, the mode switch): the gradients of a scalar
 * loss L with respect to every input of the forward, given dL/do and dL/dS_final. It is the
 * reverse-mode derivative of the recurrence S_t = (I - beta k k^T) Diag(e^g) S_{t-1} + beta k v^T,
 * o_t = S_t^T (scale q) ([KV-cache page] section 5), evaluated in its chunkwise form
 * ([KV-cache page] section 6).
 *   B, T, H, Dk, Dv, chunk, in_dtype, scale, q, k, v, g, beta, initial_state, cu_seqlens,
 *   num_seqs     exactly as in the kda_chunk_fwd call being differentiated (the forward's
 *                outputs are not needed: the states are recomputed)
 *   d_o          [B*T, H, Dv] float32, dL/do
 *   d_final_state [N, H, Dk, Dv] float32 or NULL (zero)
 *   dq, dk, dg   [B*T, H, Dk] float32 outputs (dL/dq, dL/dk, dL/dg)
 *   dv           [B*T, H, Dv] float32 output
 *   dbeta        [B*T, H] float32 output
 *   d_initial_state [N, H, Dk, Dv] float32 output or NULL (not written); written also when
 *                initial_state is NULL (the gradient at a zero initial state)
 *   workspace    device buffer of at least kda_chunk_bwd_workspace_bytes(...) bytes (required);
 *                it holds per-(chunk, head) intermediates and is overwritten
 * Every result is float32-accurate: products run on the fp32 matrix cores or as three bf16
 * products of factors split into bf16 heads and tails (about 2^-17 relative). Compiled
 * instantiations (in_dtype, chunk, Dk = Dv): (KDA_BF16, 64, 128), (KDA_F32, 64, 128) and
 * (KDA_F32, 16, 16); others return KDA_ERR_UNSUPPORTED (the forward need not have an
 * instantiation of its own at the same sizes). Output buffers must not overlap the inputs or
 * each other. Errors as kda_chunk_fwd (KDA_ERR_WORKSPACE_TOO_SMALL for a short workspace;
 * KDA_ERR_INVALID_ARGUMENT also when the record slots times heads, (num_seqs +
 * ceil(B*T / chunk)) * H, exceed 2^30); nothing is launched and no output is written on an
 * error.
 */
size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                     int32_t chunk, int32_t in_dtype, int32_t num_seqs);
kda_status kda_chunk_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                         int32_t in_dtype, float scale,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *initial_state,
                         const float *d_o, const float *d_final_state,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta,
                         float *d_initial_state,
                         const int32_t *cu_seqlens, int32_t num_seqs,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_bwd_noalloc - kda_chunk_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight training loops, harnesses that forbid hipMalloc): the same
 * arguments, results and errors, minus the workspace. The per-(chunk, head) records live in a
 * fixed device array inside the library instead, KDA_BWD_SCRATCH_BYTES (512 MiB) per device,
 * which each device holds from the library's load until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine): the outputs are the
 * caller's.
 *   A problem whose records need more than KDA_BWD_SCRATCH_BYTES, i.e. whose
 *   kda_chunk_bwd_workspace_bytes(...) exceeds it (at chunk 64, Dk = Dv = 128: 1258 record
 *   slots x heads, where a sequence takes one slot more than its chunks; e.g. 4096 tokens
 *   fit with up to 19 heads), returns KDA_ERR_WORKSPACE_TOO_SMALL with nothing launched.
 *   Every call on one device uses that device's single array: calls that overlap on one
 *   device (on different streams, or from several host threads) race and give wrong
 *   results; calls in one stream's order do not. Nothing in the array needs to start at zero
 *   (every record is written before it is read), so a call never depends on what an earlier
 *   one left there.
 */
kda_status kda_chunk_bwd_noalloc(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                                 int32_t in_dtype, float scale,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, const float *initial_state,
                                 const float *d_o, const float *d_final_state,
                                 float *dq, float *dk, float *dv, float *dg, float *dbeta,
                                 float *d_initial_state,
                                 const int32_t *cu_seqlens, int32_t num_seqs, void *stream);

/*
 * kda_short_conv_fwd - the convolution over a prefill batch.
 *   x, y           [B*T, C] dtype (KDA_F32 or KDA_BF16); sequences as in kda_chunk_fwd
 *                  (B sequences of T tokens, or packed with cu_seqlens, B = 1)
 *   weight         [C, W] float32; weight[c][W-1] multiplies the current token
 *   bias           [C] float32 or NULL
 *   initial_state  [N, W-1, C] dtype or NULL (zeros)
 *   final_state    [N, W-1, C] dtype or NULL: each sequence's last W - 1 inputs (shifted in
 *                  from the initial state for sequences shorter than W - 1); may equal
 *                  initial_state
 * y must not overlap x or the states. Supported: W = 4, C a multiple of 8. Errors as
 * kda_chunk_fwd.
 */
kda_status kda_short_conv_fwd(int32_t B, int32_t T, int32_t C, int32_t W, int32_t dtype,
                              int32_t activation, const void *x, const float *weight,
                              const float *bias, const void *initial_state, void *final_state,
                              void *y, const int32_t *cu_seqlens, int32_t num_seqs, void *stream);

/*
 * kda_short_conv_update - one decode token per sequence: x, y [N, C] dtype; state
 * [N, W-1, C] dtype, read and shifted in place (the oldest input drops out, x comes in).
 */
kda_status kda_short_conv_update(int32_t N, int32_t C, int32_t W, int32_t dtype, int32_t activation,
                                 const void *x, const float *weight, const float *bias, void *state,
                                 void *y, void *stream);

/*
 * Measurement probes: the device's practical peaks, which the benchmark reports the kernels'
 * roofline fractions against (next to the published peaks). Not part of the KDA path.
 *
 * kda_probe_copy - dst = src over `bytes` (a multiple of 16; both 16-byte aligned device
 *   pointers, not overlapping), read with non-temporal 16-byte loads: the HBM bandwidth of a
 *   kernel that reads and writes each byte once is 2 * bytes / time.
 * kda_probe_read - reads `bytes` at src (a multiple of 16, 16-byte aligned) with
 *   non-temporal 16-byte loads, 64 KB per workgroup, and writes nothing: the practical read
 *   bandwidth is bytes / time.
 * kda_probe_rmw - buf *= factor in place over `bytes` (a multiple of 16, 16-byte aligned),
 *   non-temporal loads and stores, 16 KB per workgroup: the access pattern of the decode
 *   step's state (each byte read once, then written once in place), whose practical bandwidth
 *   is 2 * bytes / time.
 * kda_probe_mfma_f16 - `blocks` workgroups of 256 threads each run `iters` iterations of
 *   independent fp16 matrix-core products per wave: eight v_mfma_f32_16x16x32_f16 (shape 0)
 *   or four v_mfma_f32_32x32x16_f16 (shape 1), the same flops; sink [blocks * 256] float32
 *   receives the accumulators (so nothing is optimised away). kda_probe_mfma_f16_flops gives
 *   the launch's dense flops.
 * kda_probe_mfma_bf16 - the same loop with bf16 operands (v_mfma_f32_16x16x32_bf16 or
 *   v_mfma_f32_32x32x16_bf16) and the same flops (kda_probe_mfma_f16_flops).
 * Errors as kda_chunk_fwd (invalid sizes or pointers, nothing launched).
 */
kda_status kda_probe_copy(const void *src, void *dst, size_t bytes, void *stream);
kda_status kda_probe_read(const void *src, size_t bytes, void *stream);
kda_status kda_probe_rmw(void *buf, size_t bytes, float factor, void *stream);
kda_status kda_probe_mfma_f16(int32_t shape, int32_t iters, int32_t blocks, float *sink, void *stream);
kda_status kda_probe_mfma_bf16(int32_t shape, int32_t iters, int32_t blocks, float *sink, void *stream);
double kda_probe_mfma_f16_flops(int32_t iters, int32_t blocks);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
