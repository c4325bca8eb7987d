// Internal launch interface between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

namespace kda {

// How the per-channel retention reaches a kernel: alpha itself, its log, or the raw gate
// logits z, turned into alpha = exp(lower * sigmoid(e^A (z + bias))) on the fly.
enum GateMode { GATE_ALPHA = 0, GATE_LOG = 1, GATE_LOGITS = 2 };

struct GateIn {
    int mode;                       // GateMode
    const float *gate;              // ALPHA / LOG: [rows, H, K] float32
    const void *logits;             // LOGITS: [rows, H, K], same dtype as q, k, v
    const float *log_scale;         // LOGITS: [H] (A; the applied scale is e^A)
    const float *bias;              // LOGITS: [H*K] or null
    float lower_bound;              // LOGITS: g_min < 0
};

struct ChunkArgs {
    const void *q, *k, *v;          // [B*T, H, K] / [B*T, H, V], bf16 or fp32
    GateIn gate;
    const float *beta;              // [B*T, H]
    const float *initial_state;     // [N, H, K, V] or null
    float *final_state;             // [N, H, K, V] or null
    const int32_t *cu_seqlens;      // [N+1] or null
    void *out;                      // [B*T, H, V]
    int64_t T;                      // tokens per batch row (unused with cu_seqlens)
    int H;
    int out_bf16;
    float scale;
    int qk_l2norm;                  // q, k divided by their L2 norm over K in the kernel
    int beta_logits;                // beta holds logits; the kernel applies sigmoid
    int state_vk;                   // states are [N, H, V, K] (K contiguous)
    int num_seqs;                   // N with cu_seqlens
    unsigned char *pack;            // two-kernel form: per (chunk slot, head) packages, or null
    int pack_slots;                 // chunk slots per head in `pack`
    int c_begin, c_end;             // two-kernel form, without cu_seqlens: chunks [c_begin, c_end) of
                                    // every sequence (the pre-pass's items, the chain's steps)
    int pack_paired;                // two-kernel form: packages in the paired column order
};

struct StepArgs {
    const void *q, *k, *v;          // [B, H, K] / [B, H, V]
    GateIn gate;                    // rows = B
    const float *beta;              // [B, H]
    float *state;                   // [B, H, K, V], in place
    void *out;                      // [B, H, V]
    int H;
    int out_bf16;
    float scale;
    int qk_l2norm, beta_logits, state_vk;  // as in ChunkArgs
};

struct RecurrentArgs {
    const void *q, *k, *v;          // [B*T, H, K] / [B*T, H, V], bf16 or fp32
    GateIn gate;
    const float *beta;              // [B*T, H]
    const float *initial_state;     // [N, H, K, V] or null
    float *final_state;             // [N, H, K, V] or null
    const int32_t *cu_seqlens;      // [N+1] or null
    void *out;                      // [B*T, H, V]
    int64_t T;
    int H;
    int out_bf16;
    float scale;
    int qk_l2norm, beta_logits, state_vk;  // as in ChunkArgs
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
    int vec4;                       // K % 4 == 0, 256 % (K / 4) == 0, logits aligned to 4 elements, out to 16 bytes
};

// Intermediates of the chunkwise backward, each [slots * H, ...] float32 (slot = chunk slot)
struct BwdWork {
    float *W, *Kd, *Qg, *Kg, *PS, *PdK, *PW;  // [.., C, K]
    float *U, *Vt, *dVt;                      // [.., C, V]
    float *Aqk, *Tm, *Abar, *MA, *MT;         // [.., C, C]
    float *h, *dh;                            // [.., K, V] chunk start state, end-state gradient
    float *gC, *rs;                           // [.., K]
    float *dbv;                               // [.., C]
};

struct BwdArgs {
    const void *q, *k, *v;          // [B*T, H, K] / [B*T, H, V], bf16 or fp32
    GateIn gate;                    // GATE_ALPHA or GATE_LOG
    const float *beta;              // [B*T, H]
    const float *initial_state;     // [N, H, K, V] or null
    const int32_t *cu_seqlens;      // [N+1] or null
    int num_seqs;                   // N with cu_seqlens
    int64_t T;
    int H;
    float scale;
    const void *d_out;              // [B*T, H, V]
    int dout_bf16;
    const float *d_final_state;     // [N, H, K, V] or null
    void *dq, *dk, *dv;             // like q, k, v
    int grad_bf16;
    float *dgate;                   // [B*T, H, K]
    float *dbeta;                   // [B*T, H]
    float *d_initial_state;         // [N, H, K, V] or null
    int slots;                      // chunk slots per head
    BwdWork w;
};

// chunk slots per head, workspace floats per (slot, head), and the carving of a workspace
int64_t chunk_bwd_slots(int B, int64_t T, int num_seqs, bool varlen);
size_t chunk_bwd_floats_per_slot(int K, int V);
void chunk_bwd_carve(BwdWork &w, float *base, int64_t slot_heads, int K, int V);
hipError_t launch_chunk_bwd(const BwdArgs &a, bool fp32_inputs, int K, int V, int num_seqs, hipStream_t stream);

struct GateBwdArgs {
    const void *logits;
    const float *log_scale, *bias;
    const float *grad;              // dL/dalpha or dL/dg
    void *d_logits;
    float *d_log_scale, *d_bias;    // [H], [H*K]; either may be null
    int64_t rows;
    int H, K;
    float lower_bound;
    int grad_is_log;
    int dlogits_bf16;
};
hipError_t launch_bounded_decay_bwd(const GateBwdArgs &a, bool fp32_logits, hipStream_t stream);

hipError_t launch_chunk_fwd(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                            hipStream_t stream, int *bv);
// the same for a.gate.mode == GATE_LOGITS (kernels that evaluate the gate themselves),
// without and with the in-kernel L2 normalisation of q and k
hipError_t launch_chunk_fwd_logits_norm(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                        hipStream_t stream, int *bv);
hipError_t launch_chunk_fwd_logits(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                   hipStream_t stream, int *bv);
// value-block width the chunk kernel uses for this shape, 0 if the shape is not compiled
// (its LDS layout would exceed 160 KB)
int chunk_fwd_value_block(bool fp32_inputs, int K, int V, int C);
// Two-kernel form (a.pack != null): the pre-pass writes one package per (chunk slot, head),
// the chain kernel consumes them.  Chunk slots per head, package bytes (0 if the form does
// not support the shape), and the launch of both kernels.
int64_t chunk_fwd_slots(int B, int64_t T, int num_seqs, bool varlen, int C);
size_t chunk_pack_bytes(bool fp32_inputs, int K, int V, int C);
// workspace bytes of the two-kernel form: the packages, then one float32 state per
// (sequence, head) carried between the chunk segments of one call
size_t chunk_fwd_workspace_bytes(bool fp32_inputs, int64_t slots, int64_t N, int H, int K, int V, int C);
hipError_t launch_chunk_fwd_two_pass(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                     int64_t slots, hipStream_t stream, int *bv);
// the pre-pass alone over `items` (chunk, head) items, at most max_wgs workgroups (0: as
// many as fit); by gate mode (float32 gate, logits, logits with q/k normalisation)
hipError_t launch_chunk_pack(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items, int max_wgs,
                             hipStream_t stream);
hipError_t launch_chunk_pack_logits(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items,
                                    int max_wgs, hipStream_t stream);
hipError_t launch_chunk_pack_logits_norm(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items,
                                         int max_wgs, hipStream_t stream);
hipError_t launch_chunk_chain(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                              hipStream_t stream, int *bv);
// one launch holding the chain over the chunks of `ca` and the pre-pass of `pa` (`items`
// items on at most pack_wgs workgroups), by the pre-pass's gate mode as above
hipError_t launch_chunk_segment(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V, int C,
                                int num_pairs, int64_t items, int pack_wgs, hipStream_t stream);
hipError_t launch_chunk_segment_logits(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V,
                                       int C, int num_pairs, int64_t items, int pack_wgs, hipStream_t stream);
hipError_t launch_chunk_segment_logits_norm(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V,
                                            int C, int num_pairs, int64_t items, int pack_wgs, hipStream_t stream);
hipError_t launch_recurrent_step(const StepArgs &a, bool fp32_inputs, int K, int V, int pairs,
                                 hipStream_t stream);
hipError_t launch_recurrent_fwd(const RecurrentArgs &a, bool fp32_inputs, int K, int V, int num_pairs,
                                hipStream_t stream);
hipError_t launch_bounded_decay(const GateArgs &a, bool fp32_logits, hipStream_t stream);
// dst[i] = src ? src[i] : 0 for i < n
hipError_t launch_fill_copy(float *dst, const float *src, int64_t n, hipStream_t stream);
// compute units of the current device (queried once per device; 256 if the query fails)
int device_cu_count();

}  // namespace kda
