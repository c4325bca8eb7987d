// Internal launch interface between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

struct ChunkArgs {
    const void *q, *k, *v;          // [B*T, H, K] / [B*T, H, V], bf16 or fp32
    const float *gate;              // [B*T, H, K]
    const float *beta;              // [B*T, H]
    const float *initial_state;     // [N, H, K, V] or null
    float *final_state;             // [N, H, K, V] or null
    const int32_t *cu_seqlens;      // [N+1] or null
    void *out;                      // [B*T, H, V]
    int64_t T;                      // tokens per batch row (unused with cu_seqlens)
    int H;
    int gate_is_log;
    int out_bf16;
    float scale;
};

struct StepArgs {
    const void *q, *k, *v;          // [B, H, K] / [B, H, V]
    const float *gate;              // [B, H, K]
    const float *beta;              // [B, H]
    float *state;                   // [B, H, K, V], in place
    void *out;                      // [B, H, V]
    int gate_is_log;
    int out_bf16;
    float scale;
};

struct GateArgs {
    const void *logits;
    const float *log_scale;
    const float *bias;
    float *out;
    int64_t n;                      // rows * H * K
    int H, K;
    float lower_bound;
    int out_log;
    int vec8;                       // K % 8 == 0 and 16-byte aligned logits/out
};

hipError_t launch_chunk_fwd(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                            hipStream_t stream, int *bv);
// value-block width the chunk kernel uses for this shape, 0 if the shape is not compiled
// (its LDS layout would exceed 160 KB)
int chunk_fwd_value_block(bool fp32_inputs, int K, int V, int C);
hipError_t launch_recurrent_step(const StepArgs &a, bool fp32_inputs, int K, int V, int pairs,
                                 hipStream_t stream);
hipError_t launch_bounded_decay(const GateArgs &a, bool fp32_logits, hipStream_t stream);
// dst[i] = src ? src[i] : 0 for i < n
hipError_t launch_fill_copy(float *dst, const float *src, int64_t n, hipStream_t stream);

}  // namespace kda
