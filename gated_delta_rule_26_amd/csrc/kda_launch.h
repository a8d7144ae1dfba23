// Host-side launchers of the KDA kernels (internal to libkda; the public ABI is kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// The layer's steps fused into the kernels (kda_chunk_fwd_fused / kda_decode_step_fused).
struct Fusion {
    const void *gx;              // [tokens, H, Dk] in_dtype gate pre-activation (replaces g), or nullptr
    const float *A_log;          // [H]     g = -exp(A_log[h]) * softplus(gx + dt_bias[h, c])
    const float *dt_bias;        // [H, Dk]
    int32_t norm_qk;             // q and k divided by their L2 norm per (token, head)
    const void *og;              // [tokens, H, Dv] in_dtype output-gate pre-activation, or nullptr
    const float *ow;             // [Dv] output norm gain
    float oeps;                  // output norm epsilon
    int32_t o_bf16;              // o is stored as bf16 (only with og)
};

struct ChunkArgs {
    int32_t n_seqs;              // number of sequences N
    int32_t seq_len;             // tokens per sequence when cu_seqlens == nullptr
    const int32_t *cu_seqlens;   // device [N+1] or nullptr
    const int32_t *order;        // device [N]: sequence of each rank (longest first), or nullptr
    int32_t H;
    float scale;
    const void *q, *k, *v;       // [tokens, H, Dk] / [tokens, H, Dv], in_dtype
    const float *g, *beta;       // [tokens, H, Dk], [tokens, H]
    const float *s0;             // [N, H, Dk, Dv] or nullptr
    float *s_out;                // [N, H, Dk, Dv] or nullptr
    void *o;                     // [tokens, H, Dv] float32 (bf16 only with the output norm)
    Fusion f;                    // the layer steps fused around the core (all null: none)
    // sequence split (fixed-length batches with few chains): each sequence is cut into nseg
    // segments of seg_len tokens (a multiple of the chunk); seg_len 0 = no split
    int32_t seg_len, nseg;
    float *ws_r;                 // [nseg-1][N*H][Dk][Dv] R_p: segment p's final state (p = 0:
                                 //   from the initial state; p > 0: from zero)
    float *ws_x;                 // [nseg-1][N*H][Dk*Dk] X_p: segment p's linear part (p >= 1), in the combine's operand order
    float *ws_s;                 // [nseg][N*H][Dk][Dv]   S_p: segment p's true start state
    uint8_t *rec;                // [nseg][N*H][rec_chunks] chunk records of segments out_from..
    int32_t out_from;            // first segment whose outputs come from the output replay
    int32_t rec_chunks;          // chunks per segment (seg_len / chunk)
};

struct DecodeArgs {
    int32_t N, H;
    int32_t L;                   // tokens per sequence ([N, L, H, D] inputs; 1 = decode step)
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    void *o;
    Fusion f;
};

struct ConvArgs {
    int32_t n_seqs;              // sequences N (decode: tokens, one per sequence)
    int32_t seq_len;             // tokens per sequence when cu_seqlens == nullptr
    const int32_t *cu_seqlens;   // device [N+1] or nullptr
    int64_t tokens;              // rows of x and y
    int32_t C;                   // channels per row (a multiple of 8)
    const void *x;               // [tokens, C] dtype
    const float *w;              // [C, 4] taps, the last on the current token
    const float *bias;           // [C] or nullptr
    const void *s0;              // [N, 3, C] dtype conv state, or nullptr (zeros)
    void *s_out;                 // [N, 3, C] final conv state (decode: the state, in place)
    void *y;                     // [tokens, C] dtype
    int32_t silu;                // SiLU after the convolution
};

struct BwdArgs {
    int32_t n_seqs;              // number of sequences N
    int32_t seq_len;             // tokens per sequence when cu_seqlens == nullptr
    const int32_t *cu_seqlens;   // device [N+1] or nullptr
    int32_t H;
    float scale;
    const void *q, *k, *v;       // [tokens, H, Dk] / [tokens, H, Dv], in_dtype
    const float *g, *beta;       // [tokens, H, Dk], [tokens, H]
    const float *s0;             // [N, H, Dk, Dv] or nullptr (zeros)
    const float *dout;           // [tokens, H, Dv] dL/do
    const float *dsT;            // [N, H, Dk, Dv] dL/dS_final or nullptr (zero)
    float *dq, *dk, *dg;         // [tokens, H, Dk]
    float *dv;                   // [tokens, H, Dv]
    float *dbeta;                // [tokens, H]
    float *ds0;                  // [N, H, Dk, Dv] dL/dS_init or nullptr (not written)
    float *ws;                   // per-(chunk, head) records, chunk_bwd_workspace_bytes(...)
    int64_t nslots;              // N + ceil(tokens / chunk) record slots per head
};

// Workspace bytes the sequence split needs for this problem on the current device (0: no
// split). The split is used only when the call provides at least this much workspace.
size_t chunk_fwd_split_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                             int32_t chunk, int32_t in_dtype, int32_t num_seqs);

// True if an instantiation exists for these parameters (in_dtype is a kda_dtype code).
bool chunk_fwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv);
bool chunk_fwd_fused_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv);
bool decode_supported(int32_t in_dtype, int32_t Dk, int32_t Dv);
bool conv_supported(int32_t dtype, int32_t C, int32_t W);
bool chunk_bwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv);
// Workspace bytes of the backward pass (always required; 0: unsupported parameters).
size_t chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t chunk,
                                 int32_t in_dtype, int32_t num_seqs);

// Enqueue the kernel on `stream`; returns the launch status (hipGetLastError).
// Enqueue kda_chunk_fwd. `workspace` (may be null) enables the sequence split when it holds
// chunk_fwd_split_bytes(...) bytes and the batch has no cu_seqlens.
hipError_t launch_chunk_fwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv,
                            const ChunkArgs &a, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);
hipError_t launch_decode(int32_t in_dtype, int32_t Dk, int32_t Dv, const DecodeArgs &a,
                         hipStream_t stream);
// The short convolution: the prefill over packed/batched sequences (then the final states when
// s_out is given), or (update) one decode token per sequence with the state shifted in place.
hipError_t launch_conv(int32_t dtype, const ConvArgs &a, bool update, hipStream_t stream);
// Measurement probes (the device's practical peaks): a 16-byte-vector copy and a pure fp16
// matrix-core loop (shape 0: 16x16x32, 1: 32x32x16) over `blocks` workgroups of 256 threads.
hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);
// A read-only stream and an in-place read-modify-write stream (buf *= factor) over `bytes`.
hipError_t launch_probe_read(const void *src, int64_t bytes, hipStream_t stream);
hipError_t launch_probe_rmw(void *buf, int64_t bytes, float factor, hipStream_t stream);
hipError_t launch_probe_mfma(int32_t bf16, int32_t shape, int32_t iters, int32_t blocks, float *sink,
                             hipStream_t stream);
int64_t probe_mfma_flops_per_iter_and_thread();
// Fixed scratch of kda_chunk_bwd_noalloc: a device array of this many bytes per device,
// which holds the backward pass's records in place of a caller-provided workspace.
constexpr size_t kBwdScratchBytes = (size_t)512 << 20;
// Device address of the current device's scratch array (looked up once per device).
hipError_t bwd_scratch(void **ptr);
// The chunked backward pass: three kernels in stream order over the workspace records.
hipError_t launch_chunk_bwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv, const BwdArgs &a,
                            hipStream_t stream);

}  // namespace kda
