// kda_gate.hip -- the bounded per-channel decay gate (gfx950).
//
// PaperLeet "Formula and conventions" (bounded_decay) and the KDA cheat sheet gate
// table (Kimi K3 column): g = g_min * sigmoid(e^A (z + bias)), alpha = e^g, so
// alpha lies in [e^g_min, 1] whatever z is.  The bias is the featurewise offset the
// KDARecurrent page adds to the gate input before the positive per-head scale.
// Elementwise and bound by HBM: each thread converts 4 consecutive channels (one 8-byte
// load of bf16 logits, one 16-byte store of float32), in float32 with a sigmoid that
// evaluates exp only of a non-positive argument.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

// The hardware exponential (2^x of a product with log2 e) and reciprocal: for alpha = e^g
// with g in [g_min, 0] the relative error stays below a few 1e-7; for g itself the error of
// e^-|u| at large |u| is relative to a term that is then below e^-|u| |u| g_min, far under
// any useful absolute tolerance.
__device__ __forceinline__ float bounded_gate(float x, float scale, float lower, int out_log) {
    const float u = scale * x;
    const float e = __expf(-fabsf(u));                  // in (0, 1]
    const float r = __builtin_amdgcn_rcpf(1.f + e);     // 1 / (1 + e), 1 + e in [1, 2]
    const float sg = u >= 0.f ? r : e * r;
    const float g = lower * sg;
    return out_log ? g : __expf(g);
}

// Heads whose per-head scale e^A the vectorised path keeps in LDS (one exponential per
// head per workgroup instead of one per unit); more heads take it from memory per unit.
constexpr int GATE_SC_HEADS = 1024;

template <typename TIn>
__global__ __launch_bounds__(256) void bounded_decay_kernel(GateArgs a) {
    const TIn *z = static_cast<const TIn *>(a.logits);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (a.vec4) {
        __shared__ float s_sc[GATE_SC_HEADS];
        const bool sc_lds = a.H <= GATE_SC_HEADS;  // workgroup-uniform
        if (sc_lds) {
            for (int i = threadIdx.x; i < a.H; i += 256) s_sc[i] = expf(a.log_scale[i]);
            __syncthreads();
        }
        // 4 consecutive channels of one (row, head) per thread: K / 4 threads per (row, head)
        // unit, 256 / (K / 4) units per workgroup (the host asks K / 4 to divide 256), so a
        // wave reads one contiguous run of logits and writes one contiguous 1 KB run of
        // retention.  The thread's channels stay fixed over the grid-stride loop and its head
        // advances by a constant step, so the loop needs no division.
        const int K4 = a.K >> 2;
        const int upb = 256 / K4;                              // units per workgroup
        const int c0 = (int)(threadIdx.x % K4) * 4;
        const int64_t units = a.n / a.K;                       // rows * H
        const int64_t ustride = (int64_t)gridDim.x * upb;
        int64_t u = (int64_t)blockIdx.x * upb + threadIdx.x / K4;
        int h = (int)(u % a.H);
        const int dh = (int)(ustride % a.H);
        const bool bias16 = a.bias && ((uintptr_t)a.bias % 16 == 0);
        for (; u < units; u += ustride) {
            const int64_t e0 = u * a.K + c0;
            const float sc = sc_lds ? s_sc[h] : expf(a.log_scale[h]);
            float x[4];
            if constexpr (sizeof(TIn) == 2) {
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                const bf16x4 zz = *reinterpret_cast<const bf16x4 *>(z + e0);
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = (float)zz[j];
            } else {
                const float4 z0 = *reinterpret_cast<const float4 *>(z + e0);
                x[0] = z0.x; x[1] = z0.y; x[2] = z0.z; x[3] = z0.w;
            }
            if (bias16) {
                const float4 b0 = *reinterpret_cast<const float4 *>(a.bias + h * a.K + c0);
                x[0] += b0.x; x[1] += b0.y; x[2] += b0.z; x[3] += b0.w;
            } else if (a.bias) {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] += a.bias[h * a.K + c0 + j];
            }
            float4 o;
            o.x = bounded_gate(x[0], sc, a.lower_bound, a.out_log);
            o.y = bounded_gate(x[1], sc, a.lower_bound, a.out_log);
            o.z = bounded_gate(x[2], sc, a.lower_bound, a.out_log);
            o.w = bounded_gate(x[3], sc, a.lower_bound, a.out_log);
            // streamed: written once, read by a later kernel
            __builtin_nontemporal_store(f4{o.x, o.y, o.z, o.w}, reinterpret_cast<f4 *>(a.out + e0));
            h += dh;
            if (h >= a.H) h -= a.H;
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
    // (vectorised: one thread per 4 channels of a (row, head) unit, whole units per workgroup)
    const int64_t work = a.vec4 ? a.n / 4 : a.n;
    int64_t blocks = (work + 255) / 256;
    // one round of resident workgroups (2048 of four waves: 32 waves per compute unit); the
    // kernel grid-strides.  Four rounds (8192 workgroups) measured 2-3% slower.
    const int64_t cap = 256 * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (fp32_logits)
        hipLaunchKernelGGL(bounded_decay_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bounded_decay_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
