// kda_chunk_chain.hip -- the two-kernel form of the chunkwise prefill (kda_chunk_pack.h):
// the chain kernels, the package size and the launch of pre-pass plus chain.
#include "kda_chunk_pack.h"

namespace kda {

static_assert(PackLayout<PrecMixed, 128, 32>::bytes == 2 * (3 * 32 * 128 + 2 * 32 * 32) + 4 * 128 + 4 * 32,
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
    return tm * (3 * (size_t)C * K + 2 * (size_t)C * C) + 4 * (size_t)K + 4 * (size_t)C;
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

// A second stream and events per (host thread, device), made on first use, for running the
// pre-pass of later chunk segments beside the chain kernel of earlier ones.
constexpr int MAX_SEG = 16;
struct Side {
    hipStream_t stream = nullptr;
    hipEvent_t start = nullptr;
    hipEvent_t done[MAX_SEG] = {};
};

hipError_t side_of_current_device(Side *&out) {
    static thread_local Side side[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorNotSupported;
    Side &x = side[dev];
    if (!x.stream) {
        // default priority (the only one this library uses), no implicit sync with stream 0
        if ((e = hipStreamCreateWithFlags(&x.stream, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&x.start, hipEventDisableTiming)) != hipSuccess) return e;
        for (int i = 0; i < MAX_SEG; ++i)
            if ((e = hipEventCreateWithFlags(&x.done[i], hipEventDisableTiming)) != hipSuccess) return e;
    }
    out = &x;
    return hipSuccess;
}

}  // namespace

hipError_t launch_chunk_fwd_two_pass(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                                     int64_t slots, hipStream_t stream, int *bv) {
    const int64_t NC = (a.T + C - 1) / C;  // chunks per sequence (fixed-length batches)
    // Packed sequences, or few chunks: the pre-pass over every slot, then the chain.
    constexpr int64_t SEG_MIN = 32;  // chunks per segment, at least
    if (a.cu_seqlens || NC < 2 * SEG_MIN) {
        hipError_t e = launch_pack_any(a, fp32_inputs, K, C, slots * a.H, 0, stream);
        if (e != hipSuccess) return e;
        return launch_chunk_chain(a, fp32_inputs, K, V, C, num_pairs, stream, bv);
    }
    // Fixed-length sequences: chunk segments.  The side stream runs the pre-pass of segment
    // 0, 1, ... back to back; the caller's stream runs the chain over segment s once the
    // pre-pass of s is done, so the chain of s overlaps the pre-pass of s + 1 (the chain
    // is bound by its serial dependence, the pre-pass by vector arithmetic).  The state
    // passes from segment to segment through the workspace's state area (or final_state
    // when the caller keeps one).  Segments after the first keep the pre-pass to about
    // 1.25 workgroups per compute unit, so every chain workgroup still finds room.
    Side *sd = nullptr;
    hipError_t e = side_of_current_device(sd);
    if (e != hipSuccess) return e;
    const int64_t seg = NC / SEG_MIN >= MAX_SEG ? (NC + MAX_SEG - 1) / MAX_SEG : SEG_MIN;
    const int nseg = (int)((NC + seg - 1) / seg);
    const size_t pb = chunk_pack_bytes(fp32_inputs, K, V, C);
    float *carry = reinterpret_cast<float *>(a.pack + (size_t)slots * (size_t)a.H * pb);
    float *mid = a.final_state ? a.final_state : carry;  // state between segments
    const int64_t B = slots / NC;
    const int cus = device_cu_count();
    if ((e = hipEventRecord(sd->start, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sd->stream, sd->start, 0)) != hipSuccess) return e;
    for (int s = 0; s < nseg; ++s) {
        ChunkArgs x = a;
        x.c_begin = (int)(s * seg);
        x.c_end = (int)((s + 1) * seg < NC ? (s + 1) * seg : NC);
        const int64_t items = B * (x.c_end - x.c_begin) * a.H;
        if ((e = launch_pack_any(x, fp32_inputs, K, C, items, s == 0 ? 0 : cus + cus / 4, sd->stream)) != hipSuccess)
            return e;
        if ((e = hipEventRecord(sd->done[s], sd->stream)) != hipSuccess) return e;
    }
    for (int s = 0; s < nseg; ++s) {
        ChunkArgs x = a;
        x.c_begin = (int)(s * seg);
        x.c_end = (int)((s + 1) * seg < NC ? (s + 1) * seg : NC);
        x.initial_state = s == 0 ? a.initial_state : mid;
        x.final_state = s == nseg - 1 ? a.final_state : mid;
        if ((e = hipStreamWaitEvent(stream, sd->done[s], 0)) != hipSuccess) return e;
        if ((e = launch_chunk_chain(x, fp32_inputs, K, V, C, num_pairs, stream, bv)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
