// kda_chunk.hip -- chunkwise prefill entry into the kernels of kda_chunk_kernel.h and the
// pre-pass of kda_chunk_pack.h, with the gate given as a float32 tensor (alpha or ln
// alpha); a gate given as logits goes to the instantiations in kda_chunk_logits.hip (and
// kda_chunk_logits_norm.hip when q and k are normalised in the kernel).
#include "kda_chunk_pack.h"

namespace kda {

int chunk_fwd_value_block(bool fp32_inputs, int K, int V, int C) {
    ChunkArgs q{};  // q == nullptr: query
    int bv = 0;
    (void)(fp32_inputs ? launch_p<PrecF32, 0>(q, K, V, C, 0, nullptr, &bv)
                       : launch_p<PrecMixed, 0>(q, K, V, C, 0, nullptr, &bv));
    return bv;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                            hipStream_t stream, int *bv) {
    if (a.gate.mode == GATE_LOGITS)
        return a.qk_l2norm ? launch_chunk_fwd_logits_norm(a, fp32_inputs, K, V, C, num_pairs, stream, bv)
                           : launch_chunk_fwd_logits(a, fp32_inputs, K, V, C, num_pairs, stream, bv);
    return fp32_inputs ? launch_p<PrecF32, 0>(a, K, V, C, num_pairs, stream, bv)
                       : launch_p<PrecMixed, 0>(a, K, V, C, num_pairs, stream, bv);
}

hipError_t launch_chunk_pack(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items, int max_wgs,
                             hipStream_t stream) {
    return fp32_inputs ? launch_pack_p<PrecF32, 0>(a, K, C, items, max_wgs, stream)
                       : launch_pack_p<PrecMixed, 0>(a, K, C, items, max_wgs, stream);
}

hipError_t launch_chunk_segment(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V, int C,
                                int num_pairs, int64_t items, int pack_wgs, hipStream_t stream) {
    return fp32_inputs ? launch_segment_p<PrecF32, 0>(ca, pa, K, V, C, num_pairs, items, pack_wgs, stream)
                       : launch_segment_p<PrecMixed, 0>(ca, pa, K, V, C, num_pairs, items, pack_wgs, stream);
}

}  // namespace kda
