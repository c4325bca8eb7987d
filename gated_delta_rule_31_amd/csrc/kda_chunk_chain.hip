// kda_chunk_chain.hip -- the two-kernel form of the chunkwise prefill (kda_chunk_pack.h):
// the chain kernels, the package size and the launch of pre-pass plus chain.
#include "kda_chunk_chain2.h"
#include "kda_chunk_pack.h"

namespace kda {

static_assert(PackLayout<PrecMixed, 128, 32>::bytes == 2 * (3 * 32 * 128 + 3 * 32 * 32) + 4 * 128 + 4 * 32,
              "chunk_pack_bytes follows PackLayout");
static_assert(PackLayout<PrecF32, 64, 16>::bytes == 4 * (3 * 16 * 64 + 2 * 16 * 16) + 4 * 64 + 4 * 16,
              "chunk_pack_bytes follows PackLayout");

int64_t chunk_fwd_slots(int B, int64_t T, int num_seqs, bool varlen, int C) {
    return varlen ? T / C + num_seqs : (int64_t)B * ((T + C - 1) / C);
}

hipError_t launch_chunk_chain(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                              hipStream_t stream, int *bv) {
    return fp32_inputs ? launch_chain_p<PrecF32>(a, K, V, C, num_pairs, stream, bv)
                       : launch_chain_p<PrecMixed>(a, K, V, C, num_pairs, stream, bv);
}

size_t chunk_pack_bytes(bool fp32_inputs, int K, int V, int C) {
    ChunkArgs q{};  // q == nullptr: query
    int bv = 0;
    if (launch_chunk_chain(q, fp32_inputs, K, V, C, 0, nullptr, &bv) != hipSuccess || bv == 0) return 0;
    const size_t tm = fp32_inputs ? 4 : 2;  // matrix-operand bytes (PackLayout)
    const size_t aq = fp32_inputs ? 1 : 2;  // A_qk parts (PackLayout)
    return tm * (3 * (size_t)C * K + (1 + aq) * (size_t)C * C) + 4 * (size_t)K + 4 * (size_t)C;
}

size_t chunk_fwd_workspace_bytes(bool fp32_inputs, int64_t slots, int64_t N, int H, int K, int V, int C) {
    const size_t pb = chunk_pack_bytes(fp32_inputs, K, V, C);
    if (pb == 0) return 0;
    return (size_t)slots * (size_t)H * pb + (size_t)N * (size_t)H * (size_t)K * (size_t)V * sizeof(float);
}

namespace {

hipError_t launch_pack_any(const ChunkArgs &a, bool fp32_inputs, int K, int C, int64_t items, int max_wgs,
                           hipStream_t stream) {
    if (a.gate.mode == GATE_LOGITS)
        return a.qk_l2norm ? launch_chunk_pack_logits_norm(a, fp32_inputs, K, C, items, max_wgs, stream)
                           : launch_chunk_pack_logits(a, fp32_inputs, K, C, items, max_wgs, stream);
    return launch_chunk_pack(a, fp32_inputs, K, C, items, max_wgs, stream);
}

hipError_t launch_segment_any(const ChunkArgs &ca, const ChunkArgs &pa, bool fp32_inputs, int K, int V, int C,
                              int num_pairs, int64_t items, int pack_wgs, hipStream_t stream) {
    if (pa.gate.mode == GATE_LOGITS)
        return pa.qk_l2norm
                   ? launch_chunk_segment_logits_norm(ca, pa, fp32_inputs, K, V, C, num_pairs, items, pack_wgs, stream)
                   : launch_chunk_segment_logits(ca, pa, fp32_inputs, K, V, C, num_pairs, items, pack_wgs, stream);
    return launch_chunk_segment(ca, pa, fp32_inputs, K, V, C, num_pairs, items, pack_wgs, stream);
}

// The 16-bit chain kernel with direct global-to-LDS copies (kda_chunk_chain2.h), where its
// layout fits; else hipErrorNotSupported.
template <int K, int V, int C, int NW>
hipError_t launch_chain2_kvcw(const ChunkArgs &a, int num_pairs, hipStream_t stream) {
    using L2 = Chain2Layout<K, V, C, NW>;
    if constexpr (!L2::ok) {
        return hipErrorNotSupported;
    } else {
        if (!a.q) return hipSuccess;  // query only
        // the kernel's LDS is static (its chunk buffers)
        auto kern = chunk_chain2_kernel<K, V, C, NW>;
        hipLaunchKernelGGL(kern, dim3(num_pairs * (V / L2::BV)), dim3(64 * NW), 0, stream, a);
        return hipGetLastError();
    }
}

// Four waves (64 value columns, one wave per SIMD) give the shortest step, so they serve
// when the workgroups fit on the device at once; with at least two rounds of workgroups the
// device is throughput-bound, and eight waves (128 value columns, two waves per SIMD, each
// package copied once per head) do more per compute unit.
template <int K, int V, int C>
hipError_t launch_chain2_kvc(const ChunkArgs &a, int num_pairs, hipStream_t stream) {
    if constexpr (Chain2Layout<K, V, C, 8>::ok) {
        if (a.q && (int64_t)num_pairs * (V / 128) >= 2 * (int64_t)device_cu_count())
            return launch_chain2_kvcw<K, V, C, 8>(a, num_pairs, stream);
    }
    return launch_chain2_kvcw<K, V, C, 4>(a, num_pairs, stream);
}

hipError_t launch_chain2(const ChunkArgs &a, int K, int V, int C, int num_pairs, hipStream_t stream) {
#define KDA_CHAIN2_C(KK, VV)                                                       \
    switch (C) {                                                                   \
        case 32: return launch_chain2_kvc<KK, VV, 32>(a, num_pairs, stream);       \
        case 64: return launch_chain2_kvc<KK, VV, 64>(a, num_pairs, stream);       \
        default: return hipErrorNotSupported;                                      \
    }
#define KDA_CHAIN2_V(KK)                        \
    switch (V) {                                \
        case 64: KDA_CHAIN2_C(KK, 64)           \
        case 128: KDA_CHAIN2_C(KK, 128)         \
        default: return hipErrorNotSupported;   \
    }
    switch (K) {
        case 32: KDA_CHAIN2_V(32)
        case 64: KDA_CHAIN2_V(64)
        case 128: KDA_CHAIN2_V(128)
        default: return hipErrorNotSupported;
    }
#undef KDA_CHAIN2_V
#undef KDA_CHAIN2_C
}

bool chain2_supported(int K, int V, int C) {
    ChunkArgs q{};  // q == nullptr: query
    return launch_chain2(q, K, V, C, 0, nullptr) == hipSuccess;
}

}  // namespace

hipError_t launch_chunk_fwd_two_pass(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                     int64_t slots, hipStream_t stream, int *bv) {
    // 16-bit operands: the whole pre-pass, then the chain kernel fed by direct copies (one
    // pass each over the full device; the same schedule with and without cu_seqlens).
    if (!fp32_inputs && chain2_supported(K, V, C)) {
        ChunkArgs b = a;
        b.pack_paired = 1;
        hipError_t e = launch_pack_any(b, fp32_inputs, K, C, slots * a.H, 0, stream);
        if (e != hipSuccess) return e;
        if (bv) *bv = 64;
        return launch_chain2(b, K, V, C, num_pairs, stream);
    }
    const int64_t NC = (a.T + C - 1) / C;  // chunks per sequence (fixed-length batches)
    // Packed sequences, or few chunks: the pre-pass over every slot, then the chain.
    constexpr int64_t SEG_MIN = 32;  // chunks per segment, at least
    constexpr int64_t MAX_SEG = 16;
    if (a.cu_seqlens || NC < 2 * SEG_MIN) {
        hipError_t e = launch_pack_any(a, fp32_inputs, K, C, slots * a.H, 0, stream);
        if (e != hipSuccess) return e;
        return launch_chunk_chain(a, fp32_inputs, K, V, C, num_pairs, stream, bv);
    }
    // Fixed-length sequences: chunk segments, all on the caller's stream.  Launch 0 is the
    // pre-pass of segment 0; launch s + 1 holds the chain over segment s and the pre-pass
    // of segment s + 1, so the chain (bound by its serial dependence, LDS and HBM) runs
    // beside the pre-pass (bound by vector arithmetic).  The chain's workgroups come first
    // in each launch and the pre-pass is held to about 1.25 workgroups per compute unit,
    // so every chain workgroup is placed at once.  The state passes from segment to
    // segment through the workspace's state area (or final_state when the caller keeps
    // one).
    const int64_t seg = NC / SEG_MIN >= MAX_SEG ? (NC + MAX_SEG - 1) / MAX_SEG : SEG_MIN;
    const int nseg = (int)((NC + seg - 1) / seg);
    const size_t pb = chunk_pack_bytes(fp32_inputs, K, V, C);
    float *carry = reinterpret_cast<float *>(a.pack + (size_t)slots * (size_t)a.H * pb);
    float *mid = a.final_state ? a.final_state : carry;  // state between segments
    const int64_t B = slots / NC;
    const int cus = device_cu_count();
    auto seg_args = [&](int s) {
        ChunkArgs x = a;
        x.c_begin = (int)(s * seg);
        x.c_end = (int)((s + 1) * seg < NC ? (s + 1) * seg : NC);
        return x;
    };
    auto items_of = [&](const ChunkArgs &x) { return B * (x.c_end - x.c_begin) * a.H; };
    ChunkArgs p0 = seg_args(0);
    hipError_t e = launch_pack_any(p0, fp32_inputs, K, C, items_of(p0), 0, stream);
    if (e != hipSuccess) return e;
    for (int s = 0; s < nseg; ++s) {
        ChunkArgs c = seg_args(s);
        c.initial_state = s == 0 ? a.initial_state : mid;
        c.final_state = s == nseg - 1 ? a.final_state : mid;
        if (s + 1 < nseg) {
            const ChunkArgs p = seg_args(s + 1);
            e = launch_segment_any(c, p, fp32_inputs, K, V, C, num_pairs, items_of(p), cus + cus / 4, stream);
        } else {
            e = launch_chunk_chain(c, fp32_inputs, K, V, C, num_pairs, stream, bv);  // the last: chain alone
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
