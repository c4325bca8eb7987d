// kda_noalloc.hip -- kda_chunk_fwd_fused_gate_noalloc: the chunked prefill with the gate in
// its kernels, in its two-kernel form, with the pre-pass packages and the carried state in a
// fixed device array of this library instead of a caller-provided workspace.  For callers
// that cannot allocate device memory (code under graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/kda.h"

// The workspace of every call on a device.  Each GPU the library runs on holds its own copy
// until the process ends; calls that overlap in time on one GPU race on it.
static constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up once per device; the
// array's name is a host-side stand-in, never a device address).
kda_status scratch_for_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return kScratchBytes; }

kda_status kda_chunk_fwd_fused_gate_noalloc(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                            const void *logits, const float *log_scale, const float *bias,
                                            float lower_bound, unsigned flags, const float *beta,
                                            const float *initial_state, float *final_state,
                                            const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H,
                                            int K, int V, int chunk_size, float scale, void *out,
                                            kda_dtype out_dtype, hipStream_t stream) {
    if (B < 0 || T < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
    if (B == 0 || T == 0 || (cu_seqlens && num_seqs == 0))  // empty: no workspace is touched
        return kda_chunk_fwd_fused_gate(q, k, v, in_dtype, logits, log_scale, bias, lower_bound, flags, beta,
                                        initial_state, final_state, cu_seqlens, num_seqs, B, T, H, K, V,
                                        chunk_size, scale, out, out_dtype, nullptr, 0, stream);
    const size_t need = kda_chunk_fwd_workspace_size(in_dtype, B, T, num_seqs, cu_seqlens != nullptr, H, K, V,
                                                     chunk_size);
    if (need == 0) return KDA_ERR_UNSUPPORTED;             // no two-kernel form for this shape
    if (need > kScratchBytes) return KDA_ERR_UNSUPPORTED;  // beyond the fixed scratch array
    void *ws = nullptr;
    const kda_status st = scratch_for_current_device(&ws);
    if (st != KDA_OK) return st;
    return kda_chunk_fwd_fused_gate(q, k, v, in_dtype, logits, log_scale, bias, lower_bound, flags, beta,
                                    initial_state, final_state, cu_seqlens, num_seqs, B, T, H, K, V, chunk_size,
                                    scale, out, out_dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
