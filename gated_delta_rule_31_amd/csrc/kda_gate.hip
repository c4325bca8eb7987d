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

// Gradients of the gate (the chain rule through g = lower sigmoid(x), x = e^A (z + bias),
// alpha = e^g): dx = dg lower sigmoid'(x), with dg = grad (grad is dL/dg) or grad alpha,
// sigmoid'(x) = e^{-|x|} / (1 + e^{-|x|})^2 (no cancellation at either end); dz = e^A dx,
// d bias[h,c] = sum over rows of dz, d log_scale[h] = sum over rows and channels of x dx.
// One workgroup per head: thread (row group, channel) walks its rows, the sums over rows
// are finished in a fixed order in LDS, so every result is reproducible bit for bit.
template <typename TIn>
__global__ __launch_bounds__(256) void bounded_decay_bwd_kernel(GateBwdArgs a) {
    __shared__ float sPart[256];
    const TIn *z = static_cast<const TIn *>(a.logits);
    const int h = blockIdx.x, tid = threadIdx.x, K = a.K, H = a.H;
    const int CW = K < 256 ? K : 256, RG = 256 / CW;  // channels per pass, row groups
    const int cl = tid % CW, rg = tid / CW;
    const float sc = expf(a.log_scale[h]), lo = a.lower_bound;
    float ls = 0.f;
    for (int cb = 0; cb < K; cb += CW) {
        const int c = cb + cl;
        float bsum = 0.f;
        if (rg < RG && c < K) {
            const float b = a.bias ? a.bias[h * K + c] : 0.f;
#pragma unroll 4
            for (int64_t r = rg; r < a.rows; r += RG) {
                const int64_t i = (r * H + h) * K + c;
                const float x = sc * (ld_f32(z, i) + b);
                const float ex = expf(-fabsf(x));
                const float inv = 1.f / (1.f + ex);
                const float sg = x >= 0.f ? inv : ex * inv;
                const float dg = a.grad_is_log ? a.grad[i] : a.grad[i] * expf(lo * sg);
                const float dx = dg * lo * ex * inv * inv;
                const float dz = dx * sc;
                st_out(a.d_logits, a.dlogits_bf16, i, dz);
                bsum += dz;
                ls += dx * x;
            }
        }
        __syncthreads();
        sPart[tid] = bsum;
        __syncthreads();
        if (a.d_bias && tid < CW && cb + tid < K) {
            float acc = 0.f;
            for (int j = 0; j < RG; ++j) acc += sPart[j * CW + tid];
            a.d_bias[h * K + cb + tid] = acc;
        }
    }
    __syncthreads();
    sPart[tid] = ls;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) sPart[tid] += sPart[tid + s];
        __syncthreads();
    }
    if (tid == 0 && a.d_log_scale) a.d_log_scale[h] = sPart[0];
}

}  // namespace

hipError_t launch_bounded_decay_bwd(const GateBwdArgs &a, bool fp32_logits, hipStream_t stream) {
    if (fp32_logits)
        hipLaunchKernelGGL(bounded_decay_bwd_kernel<float>, dim3(a.H), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bounded_decay_bwd_kernel<__bf16>, dim3(a.H), dim3(256), 0, stream, a);
    return hipGetLastError();
}

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
