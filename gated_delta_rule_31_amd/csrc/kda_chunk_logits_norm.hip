// kda_chunk_logits_norm.hip -- the chunk kernels of kda_chunk_kernel.h that evaluate the
// bounded gate from its logits and divide q and k by their L2 norms over K while
// staging each chunk (the preparation the model's layer asks its kernels to do).
#include "kda_chunk_pack.h"

namespace kda {

hipError_t launch_chunk_fwd_logits_norm(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                        hipStream_t stream, int *bv) {
    return fp32_inputs ? launch_p<PrecF32, 2>(a, K, V, C, num_pairs, stream, bv)
                       : launch_p<PrecMixed, 2>(a, K, V, C, num_pairs, stream, bv);
}

hipError_t launch_chunk_pack_logits_norm(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items, int max_wgs,
                                         hipStream_t stream) {
    return fp32_inputs ? launch_pack_p<PrecF32, 2>(a, K, C, items, max_wgs, stream)
                       : launch_pack_p<PrecMixed, 2>(a, K, C, items, max_wgs, stream);
}

hipError_t launch_chunk_segment_logits_norm(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V, int C,
                                            int num_pairs, int64_t items, int pack_wgs, hipStream_t stream) {
    return fp32_inputs ? launch_segment_p<PrecF32, 2>(ca, pa, K, V, C, num_pairs, items, pack_wgs, stream)
                       : launch_segment_p<PrecMixed, 2>(ca, pa, K, V, C, num_pairs, items, pack_wgs, stream);
}

}  // namespace kda
