// Host-side launchers of the KDA kernels (internal to libkda; the public ABI is kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ChunkArgs {
    int32_t n_seqs;              // number of sequences N
    int32_t seq_len;             // tokens per sequence when cu_seqlens == nullptr
    const int32_t *cu_seqlens;   // device [N+1] or nullptr
    int32_t H;
    float scale;
    const void *q, *k, *v;       // [tokens, H, Dk] / [tokens, H, Dv], in_dtype
    const float *g, *beta;       // [tokens, H, Dk], [tokens, H]
    const float *s0;             // [N, H, Dk, Dv] or nullptr
    float *s_out;                // [N, H, Dk, Dv] or nullptr
    float *o;                    // [tokens, H, Dv]
};

struct DecodeArgs {
    int32_t N, H;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    float *o;
};

// True if an instantiation exists for these parameters (in_dtype is a kda_dtype code).
bool chunk_fwd_supported(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv);
bool decode_supported(int32_t in_dtype, int32_t Dk, int32_t Dv);

// Enqueue the kernel on `stream`; returns the launch status (hipGetLastError).
hipError_t launch_chunk_fwd(int32_t in_dtype, int32_t chunk, int32_t Dk, int32_t Dv,
                            const ChunkArgs &a, hipStream_t stream);
hipError_t launch_decode(int32_t in_dtype, int32_t Dk, int32_t Dv, const DecodeArgs &a,
                         hipStream_t stream);

}  // namespace kda
