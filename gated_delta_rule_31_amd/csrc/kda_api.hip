// kda_api.hip -- the C ABI (include/kda.h): argument validation, the empty-sequence
// path, and dispatch onto the kernels.  Nothing here allocates, synchronises or
// prints; every launch goes onto the caller's stream.
#include <string.h>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

kda_status hip_fail(hipError_t e) {
    const char *msg = hipGetErrorString(e);
    strncpy(g_last_hip_error, msg ? msg : "unknown HIP error", sizeof(g_last_hip_error) - 1);
    g_last_hip_error[sizeof(g_last_hip_error) - 1] = 0;
    return e == hipErrorNotSupported ? KDA_ERR_UNSUPPORTED : KDA_ERR_HIP;
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(kda_dtype t) { return t == KDA_F32 || t == KDA_BF16; }
bool gate_ok(kda_gate_kind g) { return g == KDA_GATE_ALPHA || g == KDA_GATE_LOG; }

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_POINTER: return "a required pointer is NULL";
        case KDA_ERR_BAD_SHAPE: return "bad shape";
        case KDA_ERR_BAD_DTYPE: return "bad dtype or gate kind";
        case KDA_ERR_UNSUPPORTED: return "unsupported size combination";
        case KDA_ERR_BAD_ARGUMENT: return "bad argument";
        case KDA_ERR_ALIAS: return "an output aliases an input";
        case KDA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_chunk_fwd_supported(kda_dtype in_dtype, int K, int V, int chunk_size) {
    if (!dtype_ok(in_dtype) || !dim_ok(K) || !dim_ok(V)) return 0;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    return kda::chunk_fwd_value_block(in_dtype == KDA_F32, K, V, chunk_size);
}

const char *kda_last_hip_error(void) { return g_last_hip_error; }

kda_status kda_bounded_decay(const void *logits, kda_dtype logits_dtype, const float *log_scale,
                             const float *bias, float lower_bound, int64_t rows, int H, int K,
                             kda_gate_kind out_kind, float *out, hipStream_t stream) {
    if (rows < 0 || H <= 0 || K <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(logits_dtype) || !gate_ok(out_kind)) return KDA_ERR_BAD_DTYPE;
    if (!(lower_bound < 0.f)) return KDA_ERR_BAD_ARGUMENT;
    if (rows == 0) return KDA_OK;
    if (!logits || !log_scale || !out) return KDA_ERR_NULL_POINTER;
    if ((const void *)out == logits || (const void *)out == (const void *)log_scale ||
        (bias && (const void *)out == (const void *)bias))
        return KDA_ERR_ALIAS;
    kda::GateArgs a;
    a.logits = logits;
    a.log_scale = log_scale;
    a.bias = bias;
    a.out = out;
    a.n = rows * (int64_t)H * K;
    a.H = H;
    a.K = K;
    a.lower_bound = lower_bound;
    a.out_log = out_kind == KDA_GATE_LOG;
    const size_t esz = logits_dtype == KDA_F32 ? 4 : 2;
    a.vec4 = (K % 4 == 0) && (256 % (K / 4) == 0) && ((uintptr_t)logits % (4 * esz) == 0) &&
             ((uintptr_t)out % 16 == 0);
    hipError_t e = kda::launch_bounded_decay(a, logits_dtype == KDA_F32, stream);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Shared body of the chunk entry points; `gate` says how the retention arrives.
kda_status chunk_fwd_impl(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                          const kda::GateIn &gate, unsigned flags, const float *beta, const float *initial_state,
                          float *final_state, const int32_t *cu_seqlens, int num_seqs, int B, int64_t T,
                          int H, int K, int V, int chunk_size, float scale, void *out, kda_dtype out_dtype,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_BAD_DTYPE;
    if (flags & ~(unsigned)(KDA_QK_L2NORM | KDA_BETA_LOGITS | KDA_STATE_VK)) return KDA_ERR_BAD_ARGUMENT;
    if (!dim_ok(K) || !dim_ok(V)) return KDA_ERR_UNSUPPORTED;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return KDA_ERR_BAD_ARGUMENT;
    const int64_t N = cu_seqlens ? num_seqs : B;
    const size_t state_bytes = (size_t)N * H * K * V * sizeof(float);

    if (B == 0 || T == 0 || N == 0) {
        // Empty sequence (PaperLeet contract, "Empty sequence"): nothing to scan;
        // the final state is the supplied state, or zeros.
        if (final_state && N > 0 && initial_state != final_state) {
            hipError_t e = kda::launch_fill_copy(final_state, initial_state, (int64_t)(state_bytes / 4), stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        return KDA_OK;
    }
    const void *gin = gate.mode == kda::GATE_LOGITS ? gate.logits : (const void *)gate.gate;
    if (!q || !k || !v || !gin || !beta || !out) return KDA_ERR_NULL_POINTER;
    if (gate.mode == kda::GATE_LOGITS && !gate.log_scale) return KDA_ERR_NULL_POINTER;
    const void *ins[] = {q, k, v, gin, beta, initial_state, cu_seqlens, gate.log_scale, gate.bias};
    for (const void *p : ins) {
        if (p && (p == out || p == (const void *)final_state)) {
            if (p == (const void *)initial_state && p == (const void *)final_state) continue;
            return KDA_ERR_ALIAS;
        }
    }
    if ((const void *)out == (const void *)final_state) return KDA_ERR_ALIAS;
    if (N > (int64_t)(1 << 30) / H) return KDA_ERR_UNSUPPORTED;
    // the kernels write four value columns of a token per store (8 or 16 bytes)
    if ((uintptr_t)out % (out_dtype == KDA_BF16 ? 8 : 16) != 0) return KDA_ERR_BAD_ARGUMENT;
    int64_t slots = 0;
    if (workspace) {
        // the two-kernel form: one package per (chunk slot, head) in the workspace
        const size_t pb = kda::chunk_pack_bytes(in_dtype == KDA_F32, K, V, chunk_size);
        if (pb == 0) return KDA_ERR_UNSUPPORTED;
        slots = kda::chunk_fwd_slots(B, T, num_seqs, cu_seqlens != nullptr, chunk_size);
        if (slots * H > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;  // (slot, head) indexes as int
        if (workspace_bytes < kda::chunk_fwd_workspace_bytes(in_dtype == KDA_F32, slots, N, H, K, V, chunk_size) ||
            (uintptr_t)workspace % 16 != 0)
            return KDA_ERR_BAD_ARGUMENT;
        for (const void *p : ins)
            if (p == workspace) return KDA_ERR_ALIAS;
        if (workspace == out || workspace == (const void *)final_state) return KDA_ERR_ALIAS;
    }

    kda::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gate = gate;
    a.beta = beta;
    a.initial_state = initial_state;
    a.final_state = final_state;
    a.cu_seqlens = cu_seqlens;
    a.out = out;
    a.T = T;
    a.H = H;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.scale = scale;
    a.qk_l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.beta_logits = (flags & KDA_BETA_LOGITS) != 0;
    a.state_vk = (flags & KDA_STATE_VK) != 0;
    a.num_seqs = (int)N;
    a.pack = static_cast<unsigned char *>(workspace);
    a.pack_slots = (int)slots;
    a.c_begin = 0;
    a.c_end = INT32_MAX;
    a.pack_paired = 0;
    int bv = 0;
    hipError_t e = workspace ? kda::launch_chunk_fwd_two_pass(a, in_dtype == KDA_F32, K, V, chunk_size, (int)(N * H),
                                                              slots, stream, &bv)
                             : kda::launch_chunk_fwd(a, in_dtype == KDA_F32, K, V, chunk_size, (int)(N * H), stream, &bv);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

kda_status recurrent_step_impl(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                               const kda::GateIn &gate, unsigned flags, const float *beta, float *state, int B, int H,
                               int K, int V, float scale, void *out, kda_dtype out_dtype,
                               hipStream_t stream) {
    if (B < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_BAD_DTYPE;
    if (flags & ~(unsigned)(KDA_QK_L2NORM | KDA_BETA_LOGITS | KDA_STATE_VK)) return KDA_ERR_BAD_ARGUMENT;
    if (!dim_ok(K) || !dim_ok(V)) return KDA_ERR_UNSUPPORTED;
    if (B == 0) return KDA_OK;
    const void *gin = gate.mode == kda::GATE_LOGITS ? gate.logits : (const void *)gate.gate;
    if (!q || !k || !v || !gin || !beta || !state || !out) return KDA_ERR_NULL_POINTER;
    if (gate.mode == kda::GATE_LOGITS && !gate.log_scale) return KDA_ERR_NULL_POINTER;
    const void *ins[] = {q, k, v, gin, beta, gate.log_scale, gate.bias};
    for (const void *p : ins)
        if (p && (p == out || p == (const void *)state)) return KDA_ERR_ALIAS;
    if ((const void *)out == (const void *)state) return KDA_ERR_ALIAS;
    if ((uintptr_t)state % 16 != 0) return KDA_ERR_BAD_ARGUMENT;
    if ((int64_t)B * H > (int64_t)0x7fffffff) return KDA_ERR_UNSUPPORTED;
    kda::StepArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gate = gate;
    a.beta = beta;
    a.state = state;
    a.out = out;
    a.H = H;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.scale = scale;
    a.qk_l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.beta_logits = (flags & KDA_BETA_LOGITS) != 0;
    a.state_vk = (flags & KDA_STATE_VK) != 0;
    hipError_t e = kda::launch_recurrent_step(a, in_dtype == KDA_F32, K, V, B * H, stream);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

// Shared body of the token-recurrent entry points (same contract as the chunk ones,
// without a chunk size and without the chunk path's log-decay bound).
kda_status recurrent_fwd_impl(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                              const kda::GateIn &gate, unsigned flags, const float *beta, const float *initial_state,
                              float *final_state, const int32_t *cu_seqlens, int num_seqs, int B, int64_t T,
                              int H, int K, int V, float scale, void *out, kda_dtype out_dtype,
                              hipStream_t stream) {
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_BAD_DTYPE;
    if (flags & ~(unsigned)(KDA_QK_L2NORM | KDA_BETA_LOGITS | KDA_STATE_VK)) return KDA_ERR_BAD_ARGUMENT;
    if (!dim_ok(K) || !dim_ok(V)) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return KDA_ERR_BAD_ARGUMENT;
    const int64_t N = cu_seqlens ? num_seqs : B;
    if (B == 0 || T == 0 || N == 0) {
        if (final_state && N > 0 && initial_state != final_state) {
            hipError_t e = kda::launch_fill_copy(final_state, initial_state, N * H * K * V, stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        return KDA_OK;
    }
    const void *gin = gate.mode == kda::GATE_LOGITS ? gate.logits : (const void *)gate.gate;
    if (!q || !k || !v || !gin || !beta || !out) return KDA_ERR_NULL_POINTER;
    if (gate.mode == kda::GATE_LOGITS && !gate.log_scale) return KDA_ERR_NULL_POINTER;
    const void *ins[] = {q, k, v, gin, beta, initial_state, cu_seqlens, gate.log_scale, gate.bias};
    for (const void *p : ins) {
        if (p && (p == out || p == (const void *)final_state)) {
            if (p == (const void *)initial_state && p == (const void *)final_state) continue;
            return KDA_ERR_ALIAS;
        }
    }
    if ((const void *)out == (const void *)final_state) return KDA_ERR_ALIAS;
    if (N > (int64_t)(1 << 28) / H) return KDA_ERR_UNSUPPORTED;
    // the kernel moves states and outputs in 16-byte (8-byte for bf16 outputs) pieces
    const uintptr_t oal = out_dtype == KDA_BF16 ? 8 : 16;
    if ((uintptr_t)initial_state % 16 != 0 || (uintptr_t)final_state % 16 != 0 || (uintptr_t)out % oal != 0)
        return KDA_ERR_BAD_ARGUMENT;
    kda::RecurrentArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gate = gate;
    a.beta = beta;
    a.initial_state = initial_state;
    a.final_state = final_state;
    a.cu_seqlens = cu_seqlens;
    a.out = out;
    a.T = T;
    a.H = H;
    a.out_bf16 = out_dtype == KDA_BF16;
    a.scale = scale;
    a.qk_l2norm = (flags & KDA_QK_L2NORM) != 0;
    a.beta_logits = (flags & KDA_BETA_LOGITS) != 0;
    a.state_vk = (flags & KDA_STATE_VK) != 0;
    hipError_t e = kda::launch_recurrent_fwd(a, in_dtype == KDA_F32, K, V, (int)(N * H), stream);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

kda::GateIn gate_given(const float *gate, kda_gate_kind kind) {
    kda::GateIn g{};
    g.mode = kind == KDA_GATE_LOG ? kda::GATE_LOG : kda::GATE_ALPHA;
    g.gate = gate;
    return g;
}

kda::GateIn gate_logits(const void *logits, const float *log_scale, const float *bias, float lower_bound) {
    kda::GateIn g{};
    g.mode = kda::GATE_LOGITS;
    g.logits = logits;
    g.log_scale = log_scale;
    g.bias = bias;
    g.lower_bound = lower_bound;
    return g;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                         const float *gate, kda_gate_kind gate_kind, const float *beta,
                         const float *initial_state, float *final_state,
                         const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H, int K,
                         int V, int chunk_size, float scale, void *out, kda_dtype out_dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!gate_ok(gate_kind)) return KDA_ERR_BAD_DTYPE;
    return chunk_fwd_impl(q, k, v, in_dtype, gate_given(gate, gate_kind), 0u, beta, initial_state, final_state,
                          cu_seqlens, num_seqs, B, T, H, K, V, chunk_size, scale, out, out_dtype, workspace,
                          workspace_bytes, stream);
}

kda_status kda_chunk_fwd_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                    const void *logits, const float *log_scale, const float *bias,
                                    float lower_bound, unsigned flags, const float *beta, const float *initial_state,
                                    float *final_state, const int32_t *cu_seqlens, int num_seqs, int B,
                                    int64_t T, int H, int K, int V, int chunk_size, float scale, void *out,
                                    kda_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    // the chunk path needs every log-decay >= -5, which the bound guarantees when
    // lower_bound >= -5
    if (!(lower_bound < 0.f) || lower_bound < -5.f) return KDA_ERR_BAD_ARGUMENT;
    return chunk_fwd_impl(q, k, v, in_dtype, gate_logits(logits, log_scale, bias, lower_bound), flags, beta,
                          initial_state, final_state, cu_seqlens, num_seqs, B, T, H, K, V, chunk_size, scale,
                          out, out_dtype, workspace, workspace_bytes, stream);
}

size_t kda_chunk_fwd_workspace_size(kda_dtype in_dtype, int B, int64_t T, int num_seqs, int varlen, int H, int K,
                                    int V, int chunk_size) {
    if (!dtype_ok(in_dtype) || !dim_ok(K) || !dim_ok(V) || B < 0 || T < 0 || H <= 0 || num_seqs < 0) return 0;
    if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    const size_t pb = kda::chunk_pack_bytes(in_dtype == KDA_F32, K, V, chunk_size);
    if (pb == 0) return 0;
    const int64_t slots = kda::chunk_fwd_slots(B, T, num_seqs, varlen != 0, chunk_size);
    if (slots * H > (int64_t)INT32_MAX) return 0;
    const int64_t N = varlen ? num_seqs : B;
    return kda::chunk_fwd_workspace_bytes(in_dtype == KDA_F32, slots, N, H, K, V, chunk_size);
}

kda_status kda_recurrent_fwd(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                             const float *gate, kda_gate_kind gate_kind, const float *beta,
                             const float *initial_state, float *final_state, const int32_t *cu_seqlens,
                             int num_seqs, int B, int64_t T, int H, int K, int V, float scale, void *out,
                             kda_dtype out_dtype, hipStream_t stream) {
    if (!gate_ok(gate_kind)) return KDA_ERR_BAD_DTYPE;
    return recurrent_fwd_impl(q, k, v, in_dtype, gate_given(gate, gate_kind), 0u, beta, initial_state, final_state,
                              cu_seqlens, num_seqs, B, T, H, K, V, scale, out, out_dtype, stream);
}

kda_status kda_recurrent_fwd_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                        const void *logits, const float *log_scale, const float *bias,
                                        float lower_bound, unsigned flags, const float *beta,
                                        const float *initial_state,
                                        float *final_state, const int32_t *cu_seqlens, int num_seqs, int B,
                                        int64_t T, int H, int K, int V, float scale, void *out,
                                        kda_dtype out_dtype, hipStream_t stream) {
    if (!(lower_bound < 0.f)) return KDA_ERR_BAD_ARGUMENT;
    return recurrent_fwd_impl(q, k, v, in_dtype, gate_logits(logits, log_scale, bias, lower_bound), flags, beta,
                              initial_state, final_state, cu_seqlens, num_seqs, B, T, H, K, V, scale, out,
                              out_dtype, stream);
}

kda_status kda_recurrent_step(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                              const float *gate, kda_gate_kind gate_kind, const float *beta,
                              float *state, int B, int H, int K, int V, float scale, void *out,
                              kda_dtype out_dtype, hipStream_t stream) {
    if (!gate_ok(gate_kind)) return KDA_ERR_BAD_DTYPE;
    return recurrent_step_impl(q, k, v, in_dtype, gate_given(gate, gate_kind), 0u, beta, state, B, H, K, V, scale,
                               out, out_dtype, stream);
}

kda_status kda_recurrent_step_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                         const void *logits, const float *log_scale, const float *bias,
                                         float lower_bound, unsigned flags, const float *beta, float *state, int B,
                                         int H,
                                         int K, int V, float scale, void *out, kda_dtype out_dtype,
                                         hipStream_t stream) {
    if (!(lower_bound < 0.f)) return KDA_ERR_BAD_ARGUMENT;
    return recurrent_step_impl(q, k, v, in_dtype, gate_logits(logits, log_scale, bias, lower_bound), flags, beta,
                               state,
                               B, H, K, V, scale, out, out_dtype, stream);
}

}  // extern "C"

extern "C" {

size_t kda_chunk_bwd_workspace_size(int B, int64_t T, int H, int K, int V, int num_seqs, int varlen) {
    if (B < 0 || T < 0 || H <= 0 || !dim_ok(K) || !dim_ok(V) || num_seqs < 0) return 0;
    const int64_t slots = kda::chunk_bwd_slots(B, T, num_seqs, varlen != 0);
    return (size_t)slots * (size_t)H * kda::chunk_bwd_floats_per_slot(K, V) * sizeof(float);
}

kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, kda_dtype in_dtype, const float *gate,
                         kda_gate_kind gate_kind, const float *beta, const float *initial_state,
                         const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H, int K, int V,
                         float scale, const void *d_out, kda_dtype dout_dtype, const float *d_final_state,
                         void *dq, void *dk, void *dv, kda_dtype grad_dtype, float *dgate, float *dbeta,
                         float *d_initial_state, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(in_dtype) || !dtype_ok(dout_dtype) || !dtype_ok(grad_dtype) || !gate_ok(gate_kind))
        return KDA_ERR_BAD_DTYPE;
    if (!dim_ok(K) || !dim_ok(V)) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return KDA_ERR_BAD_ARGUMENT;
    const int64_t N = cu_seqlens ? num_seqs : B;
    if (B == 0 || T == 0 || N == 0) {
        // empty scan: final = initial, so the initial state's gradient is the final state's
        if (d_initial_state && N > 0 && (const float *)d_initial_state != d_final_state) {
            hipError_t e = kda::launch_fill_copy(d_initial_state, d_final_state, N * H * (int64_t)K * V, stream);
            if (e != hipSuccess) return hip_fail(e);
        }
        return KDA_OK;
    }
    if (!q || !k || !v || !gate || !beta || !d_out || !dq || !dk || !dv || !dgate || !dbeta || !workspace)
        return KDA_ERR_NULL_POINTER;
    const size_t need = kda_chunk_bwd_workspace_size(B, T, H, K, V, num_seqs, cu_seqlens != nullptr);
    if (workspace_bytes < need) return KDA_ERR_BAD_ARGUMENT;
    if (N > 65535 || H > 65535) return KDA_ERR_UNSUPPORTED;
    const void *ins[] = {q, k, v, gate, beta, initial_state, cu_seqlens, d_out, d_final_state};
    const void *outs[] = {dq, dk, dv, dgate, dbeta, d_initial_state, workspace};
    for (int i = 0; i < 7; ++i) {
        if (!outs[i]) continue;
        for (const void *p : ins)
            if (p == outs[i]) return KDA_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return KDA_ERR_ALIAS;
    }
    const int64_t slots = kda::chunk_bwd_slots(B, T, num_seqs, cu_seqlens != nullptr);
    if (slots * H > (int64_t)INT32_MAX) return KDA_ERR_UNSUPPORTED;  // (chunk slot, head) units index as int

    kda::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gate = gate_given(gate, gate_kind);
    a.beta = beta;
    a.initial_state = initial_state;
    a.cu_seqlens = cu_seqlens;
    a.num_seqs = (int)N;
    a.T = T;
    a.H = H;
    a.scale = scale;
    a.d_out = d_out;
    a.dout_bf16 = dout_dtype == KDA_BF16;
    a.d_final_state = d_final_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.grad_bf16 = grad_dtype == KDA_BF16;
    a.dgate = dgate;
    a.dbeta = dbeta;
    a.d_initial_state = d_initial_state;
    a.slots = (int)slots;
    kda::chunk_bwd_carve(a.w, static_cast<float *>(workspace), slots * H, K, V);
    hipError_t e = kda::launch_chunk_bwd(a, in_dtype == KDA_F32, K, V, (int)N, stream);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

kda_status kda_bounded_decay_bwd(const void *logits, kda_dtype logits_dtype, const float *log_scale,
                                 const float *bias, float lower_bound, int64_t rows, int H, int K,
                                 const float *grad, kda_gate_kind grad_kind, void *d_logits,
                                 kda_dtype dlogits_dtype, float *d_log_scale, float *d_bias, hipStream_t stream) {
    if (rows < 0 || H <= 0 || K <= 0) return KDA_ERR_BAD_SHAPE;
    if (!dtype_ok(logits_dtype) || !dtype_ok(dlogits_dtype) || !gate_ok(grad_kind)) return KDA_ERR_BAD_DTYPE;
    if (!(lower_bound < 0.f)) return KDA_ERR_BAD_ARGUMENT;
    if (!log_scale) return KDA_ERR_NULL_POINTER;
    if (rows > 0 && (!logits || !grad || !d_logits)) return KDA_ERR_NULL_POINTER;
    const void *ins[] = {logits, log_scale, bias, grad};
    const void *outs[] = {d_logits, d_log_scale, d_bias};
    for (int i = 0; i < 3; ++i) {
        if (!outs[i]) continue;
        for (const void *p : ins)
            if (p == outs[i]) return KDA_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return KDA_ERR_ALIAS;
    }
    if (rows == 0 && !d_log_scale && !d_bias) return KDA_OK;
    kda::GateBwdArgs a;
    a.logits = logits;
    a.log_scale = log_scale;
    a.bias = bias;
    a.grad = grad;
    a.d_logits = d_logits;
    a.d_log_scale = d_log_scale;
    a.d_bias = d_bias;
    a.rows = rows;
    a.H = H;
    a.K = K;
    a.lower_bound = lower_bound;
    a.grad_is_log = grad_kind == KDA_GATE_LOG;
    a.dlogits_bf16 = dlogits_dtype == KDA_BF16;
    hipError_t e = kda::launch_bounded_decay_bwd(a, logits_dtype == KDA_F32, stream);
    return e == hipSuccess ? KDA_OK : hip_fail(e);
}

}  // extern "C"
