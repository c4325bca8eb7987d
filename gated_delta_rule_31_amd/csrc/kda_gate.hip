// kda_gate.hip -- the bounded per-channel decay gate (gfx950).
//
// PaperLeet "Formula and conventions" (bounded_decay) and the KDA cheat sheet gate
// table (Kimi K3 column): g = g_min * sigmoid(e^A (z + bias)), alpha = e^g, so
// alpha lies in [e^g_min, 1] whatever z is.  The bias is the featurewise offset the
// KDARecurrent page adds to the gate input before the positive per-head scale.
// Elementwise and bound by HBM: each thread converts 8 consecutive channels (one
// 16-byte load of bf16 logits, two 16-byte stores of float32), in float32 with a
// sigmoid that evaluates exp only of a non-positive argument.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ float bounded_gate(float x, float scale, float lower, int out_log) {
    const float u = scale * x;
    const float e = expf(-fabsf(u));                    // in (0, 1]
    const float sg = u >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
    const float g = lower * sg;
    return out_log ? g : expf(g);
}

template <typename TIn>
__global__ __launch_bounds__(256) void bounded_decay_kernel(GateArgs a) {
    const TIn *z = static_cast<const TIn *>(a.logits);
    const int64_t n8 = a.n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (a.vec8) {
        // 8 consecutive channels of one (row, head) per thread
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
            const int64_t e0 = i * 8;
            const int c0 = (int)(e0 % a.K);
            const int h = (int)((e0 / a.K) % a.H);
            const float sc = expf(a.log_scale[h]);
            float x[8];
            if constexpr (sizeof(TIn) == 2) {
                const bf16x8 zz = *reinterpret_cast<const bf16x8 *>(z + e0);
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = (float)zz[j];
            } else {
                const float4 z0 = *reinterpret_cast<const float4 *>(z + e0);
                const float4 z1 = *reinterpret_cast<const float4 *>(z + e0 + 4);
                x[0] = z0.x; x[1] = z0.y; x[2] = z0.z; x[3] = z0.w;
                x[4] = z1.x; x[5] = z1.y; x[6] = z1.z; x[7] = z1.w;
            }
            if (a.bias) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] += a.bias[h * a.K + c0 + j];
            }
            float4 o0, o1;
            o0.x = bounded_gate(x[0], sc, a.lower_bound, a.out_log);
            o0.y = bounded_gate(x[1], sc, a.lower_bound, a.out_log);
            o0.z = bounded_gate(x[2], sc, a.lower_bound, a.out_log);
            o0.w = bounded_gate(x[3], sc, a.lower_bound, a.out_log);
            o1.x = bounded_gate(x[4], sc, a.lower_bound, a.out_log);
            o1.y = bounded_gate(x[5], sc, a.lower_bound, a.out_log);
            o1.z = bounded_gate(x[6], sc, a.lower_bound, a.out_log);
            o1.w = bounded_gate(x[7], sc, a.lower_bound, a.out_log);
            *reinterpret_cast<float4 *>(a.out + e0) = o0;
            *reinterpret_cast<float4 *>(a.out + e0 + 4) = o1;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += stride) {
            const int c = (int)(i % a.K);
            const int h = (int)((i / a.K) % a.H);
            float x = ld_f32(z, i);
            if (a.bias) x += a.bias[h * a.K + c];
            a.out[i] = bounded_gate(x, expf(a.log_scale[h]), a.lower_bound, a.out_log);
        }
    }
}

}  // namespace

hipError_t launch_bounded_decay(const GateArgs &a, bool fp32_logits, hipStream_t stream) {
    const int64_t work = a.vec8 ? a.n / 8 : a.n;
    int64_t blocks = (work + 255) / 256;
    const int64_t cap = 256 * 32;  // enough resident waves to saturate HBM; the kernel grid-strides
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (fp32_logits)
        hipLaunchKernelGGL(bounded_decay_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bounded_decay_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
