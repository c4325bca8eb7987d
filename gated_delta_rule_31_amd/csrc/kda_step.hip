// kda_step.hip -- fused single-token KDA decode step over a kept state (gfx950).
//
// Per (batch row, head), with the float32 state S [K x V] kept in HBM and
// updated in place (Kept-memory page: a decode call updates the kept per-head state
// with one token and leaves the result for the next call; PaperLeet
// "Formula and conventions" for the recurrence):
//   Sbar  = Diag(alpha) S
//   p     = Sbar^T k,  r = Sbar^T q                    (two reductions over K, one pass)
//   delta = beta (v - p)
//   S_t   = Sbar + k delta^T
//   o     = scale S_t^T q = scale (r + (k . q) delta)  (no second pass over the state)
// The step is bound by the state stream: 2*K*V*4 bytes per head against ~7*K*V
// flops.  Each workgroup owns one state: it reads it once with 16-byte coalesced
// loads into registers, reduces across threads through LDS, and writes it back
// once.  No atomics: every output element has one writer.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

template <int K, int V>
struct StepCfg {
    static constexpr int CQ = V / 4;                              // float4 column groups
    static constexpr int RPT = (K * CQ) / 256 > 0 ? (K * CQ) / 256 : 1;  // rows per thread
    static constexpr int NRG = K / RPT;                           // row groups
    static constexpr int NT = CQ * NRG;                           // threads
    static_assert(NT <= 256 && NRG * RPT == K, "step mapping");
};

// ZG: the gate arrives as logits and is evaluated here; otherwise as alpha or ln alpha.
template <typename TIn, int K, int V, bool ZG>
__global__ __launch_bounds__((StepCfg<K, V>::NT)) void recurrent_step_kernel(StepArgs a) {
    using Cf = StepCfg<K, V>;
    constexpr int CQ = Cf::CQ, RPT = Cf::RPT, NRG = Cf::NRG;
    __shared__ float red_p[NRG][V];
    __shared__ float red_r[NRG][V];
    __shared__ float red_kq[3][NRG];  // k.q, k.k, q.q partials
    __shared__ float dlt[V];
    __shared__ float kq_s, ik_s, iq_s;

    const int pair = blockIdx.x;  // b * H + h
    const int tid = threadIdx.x;
    const int cq = tid % CQ;  // this thread's 4 value columns: 4*cq .. 4*cq+3
    const int rg = tid / CQ;  // this thread's key rows: rg + NRG * i
    const TIn *q = static_cast<const TIn *>(a.q) + (int64_t)pair * K;
    const TIn *k = static_cast<const TIn *>(a.k) + (int64_t)pair * K;
    const TIn *v = static_cast<const TIn *>(a.v) + (int64_t)pair * V;
    const int h = pair % a.H;
    const bool glog = a.gate.mode == GATE_LOG;
    const float *gate = a.gate.gate + (int64_t)pair * K;
    const TIn *zl = static_cast<const TIn *>(a.gate.logits) + (int64_t)pair * K;
    float s2 = 0.f, l2 = 0.f;
    if constexpr (ZG) {
        s2 = expf(a.gate.log_scale[h]) * 1.44269504088896341f;
        l2 = a.gate.lower_bound * 1.44269504088896341f;
    }
    float4 *S = reinterpret_cast<float4 *>(a.state + (int64_t)pair * K * V);

    // the state is streamed: read once and written once per step.  The stores are
    // non-temporal (nothing gains from allocating the state in the caches); the loads are
    // ordinary ones, which on this GPU stream faster than non-temporal loads (measured:
    // 123 against 143 us per B=64, H=96 step)
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const f4 x = *reinterpret_cast<const f4 *>(&S[(rg + NRG * i) * CQ + cq]);
        s[i] = float4{x[0], x[1], x[2], x[3]};
    }

    float4 pp = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f, kk = 0.f, qq = 0.f;
    float kr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + NRG * i;
        float al;
        if constexpr (ZG) {
            const float z = ld_f32(zl, row) + (a.gate.bias ? a.gate.bias[h * K + row] : 0.f);
            al = fast_bounded_alpha(z, s2, l2);
        } else {
            const float g = gate[row];
            al = glog ? expf(g) : g;
        }
        const float kv = ld_f32(k, row), qv = ld_f32(q, row);
        kr[i] = kv;
        kq += kv * qv;
        kk += kv * kv;
        qq += qv * qv;
        s[i].x *= al; s[i].y *= al; s[i].z *= al; s[i].w *= al;
        pp.x += s[i].x * kv; pp.y += s[i].y * kv; pp.z += s[i].z * kv; pp.w += s[i].w * kv;
        rr.x += s[i].x * qv; rr.y += s[i].y * qv; rr.z += s[i].z * qv; rr.w += s[i].w * qv;
    }
    red_p[rg][4 * cq + 0] = pp.x; red_p[rg][4 * cq + 1] = pp.y;
    red_p[rg][4 * cq + 2] = pp.z; red_p[rg][4 * cq + 3] = pp.w;
    red_r[rg][4 * cq + 0] = rr.x; red_r[rg][4 * cq + 1] = rr.y;
    red_r[rg][4 * cq + 2] = rr.z; red_r[rg][4 * cq + 3] = rr.w;
    if (cq == 0) {
        red_kq[0][rg] = kq;
        red_kq[1][rg] = kk;
        red_kq[2][rg] = qq;
    }
    __syncthreads();
    if (tid == 0) {
        float x = 0.f, nk = 0.f, nq = 0.f;
        for (int g2 = 0; g2 < NRG; ++g2) {
            x += red_kq[0][g2];
            nk += red_kq[1][g2];
            nq += red_kq[2][g2];
        }
        // with in-kernel normalisation the reductions above used the raw k and q:
        // S^T (k/|k|) = (S^T k)/|k|, so only the results are rescaled
        const float ik = a.qk_l2norm ? 1.f / fmaxf(sqrtf(nk), 1e-6f) : 1.f;
        const float iq = a.qk_l2norm ? 1.f / fmaxf(sqrtf(nq), 1e-6f) : 1.f;
        kq_s = x * ik * iq;
        ik_s = ik;
        iq_s = iq;
    }
    __syncthreads();
    if (tid < V) {
        float p = 0.f, r = 0.f;
        for (int g2 = 0; g2 < NRG; ++g2) {
            p += red_p[g2][tid];
            r += red_r[g2][tid];
        }
        const float bl = a.beta[pair];
        const float bt = a.beta_logits ? 1.f / (1.f + __expf(-bl)) : bl;
        const float d = bt * (ld_f32(v, tid) - p * ik_s);
        dlt[tid] = d * ik_s;  // the state update adds (k/|k|) d^T
        st_out(a.out, a.out_bf16, (int64_t)pair * V + tid, a.scale * (r * iq_s + kq_s * d));
    }
    __syncthreads();
    const float4 d4 = {dlt[4 * cq], dlt[4 * cq + 1], dlt[4 * cq + 2], dlt[4 * cq + 3]};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        float4 x = s[i];
        x.x += kr[i] * d4.x; x.y += kr[i] * d4.y; x.z += kr[i] * d4.z; x.w += kr[i] * d4.w;
        __builtin_nontemporal_store(f4{x.x, x.y, x.z, x.w}, reinterpret_cast<f4 *>(&S[(rg + NRG * i) * CQ + cq]));
    }
}

// The same step with the state stored [V, K] (K contiguous, the transposed layout some
// model code keeps).  Thread (cq, rg) holds KPT keys of each of its value rows rg + NRG*i:
// float4 piece g covers keys 4 (cq + CQ g) .. + 3, so the CQ lanes of a row read one
// contiguous run per piece.  The reductions over K are in-thread sums over the KPT keys,
// then log2(CQ) exchanges across the row's lanes; every lane ends with the sums it needs,
// with no LDS round trip.  With 16 keys per thread (K >= 64) a row takes 8 lanes (3
// exchange steps for each of its 4 rows at K = V = 128) instead of 32 (5 steps for each
// of 16 rows at 4 keys per thread).  The token's k, q and retention are formed once per
// key into a small LDS table (every row group needs all of them) behind one barrier.
template <int K, int V>
struct StepVkCfg {
    static constexpr int KPT = K >= 64 ? 16 : 4;              // keys per thread
    static constexpr int G = KPT / 4;                         // float4 pieces per row
    static constexpr int CQ = K / KPT;                        // lanes per value row
    static constexpr int NT0 = V * CQ < 256 ? V * CQ : 256;
    static constexpr int NRG = NT0 / CQ;                      // row groups
    static constexpr int RPT = V / NRG;                       // rows per thread
    static constexpr int NT = NRG * CQ;                       // threads
    static_assert(64 % CQ == 0 && RPT * NRG == V && RPT >= 1, "vk step mapping");
};

template <typename TIn, int K, int V, bool ZG>
__global__ __launch_bounds__((StepVkCfg<K, V>::NT)) void recurrent_step_vk_kernel(StepArgs a) {
    using Cf = StepVkCfg<K, V>;
    constexpr int G = Cf::G, CQ = Cf::CQ, RPT = Cf::RPT, NRG = Cf::NRG;
    const int pair = blockIdx.x;  // b * H + h
    const int tid = threadIdx.x;
    const int cq = tid % CQ;      // keys 4 (cq + CQ g) .. + 3 of piece g
    const int rg = tid / CQ;      // value rows rg + NRG * i
    const int h = pair % a.H;
    const TIn *q = static_cast<const TIn *>(a.q) + (int64_t)pair * K;
    const TIn *k = static_cast<const TIn *>(a.k) + (int64_t)pair * K;
    const TIn *v = static_cast<const TIn *>(a.v) + (int64_t)pair * V;
    float4 *S = reinterpret_cast<float4 *>(a.state + (int64_t)pair * K * V);
    constexpr int R4 = K / 4;     // float4 pieces per value row

    float4 s[RPT][G];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const f4 x = *reinterpret_cast<const f4 *>(&S[(rg + NRG * i) * R4 + cq + CQ * g]);
            s[i][g] = float4{x[0], x[1], x[2], x[3]};
        }
    // The token's k, q and retention, once per key for the whole workgroup (every row group
    // needs the same keys): formed by the first K threads into LDS, behind an LDS-only
    // barrier, so the state loads above stay in flight across it.
    __shared__ __align__(16) float sh_k[K];
    __shared__ __align__(16) float sh_q[K];
    __shared__ __align__(16) float sh_al[K];
    {
        float s2 = 0.f, l2 = 0.f;
        if constexpr (ZG) {
            s2 = expf(a.gate.log_scale[h]) * 1.44269504088896341f;
            l2 = a.gate.lower_bound * 1.44269504088896341f;
        }
        for (int c = tid; c < K; c += Cf::NT) {
            sh_k[c] = ld_f32(k, c);
            sh_q[c] = ld_f32(q, c);
            if constexpr (ZG) {
                const float z = ld_f32(static_cast<const TIn *>(a.gate.logits) + (int64_t)pair * K, c) +
                                (a.gate.bias ? a.gate.bias[h * K + c] : 0.f);
                sh_al[c] = fast_bounded_alpha(z, s2, l2);
            } else {
                const float gg = a.gate.gate[(int64_t)pair * K + c];
                sh_al[c] = a.gate.mode == GATE_LOG ? expf(gg) : gg;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    float al[G][4], kv[G][4], qv[G][4];
    float kq = 0.f, nk = 0.f, nq = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int c = 4 * (cq + CQ * g);
        const float4 k4 = *reinterpret_cast<const float4 *>(sh_k + c);
        const float4 q4 = *reinterpret_cast<const float4 *>(sh_q + c);
        const float4 a4 = *reinterpret_cast<const float4 *>(sh_al + c);
        kv[g][0] = k4.x; kv[g][1] = k4.y; kv[g][2] = k4.z; kv[g][3] = k4.w;
        qv[g][0] = q4.x; qv[g][1] = q4.y; qv[g][2] = q4.z; qv[g][3] = q4.w;
        al[g][0] = a4.x; al[g][1] = a4.y; al[g][2] = a4.z; al[g][3] = a4.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kq += kv[g][e] * qv[g][e];
            nk += kv[g][e] * kv[g][e];
            nq += qv[g][e] * qv[g][e];
        }
    }
#pragma unroll
    for (int m = 1; m < CQ; m <<= 1) {
        kq += __shfl_xor(kq, m);
        nk += __shfl_xor(nk, m);
        nq += __shfl_xor(nq, m);
    }
    const float ik = a.qk_l2norm ? 1.f / fmaxf(sqrtf(nk), 1e-6f) : 1.f;
    const float iq = a.qk_l2norm ? 1.f / fmaxf(sqrtf(nq), 1e-6f) : 1.f;
    kq *= ik * iq;
    const float bl = a.beta[pair];
    const float bt = a.beta_logits ? 1.f / (1.f + __expf(-bl)) : bl;
    float p[RPT], r[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        p[i] = 0.f;
        r[i] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float4 &x = s[i][g];
            x.x *= al[g][0]; x.y *= al[g][1]; x.z *= al[g][2]; x.w *= al[g][3];
            p[i] += x.x * kv[g][0] + x.y * kv[g][1] + x.z * kv[g][2] + x.w * kv[g][3];
            r[i] += x.x * qv[g][0] + x.y * qv[g][1] + x.z * qv[g][2] + x.w * qv[g][3];
        }
    }
#pragma unroll
    for (int m = 1; m < CQ; m <<= 1)
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            p[i] += __shfl_xor(p[i], m);
            r[i] += __shfl_xor(r[i], m);
        }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + NRG * i;
        const float d = bt * (ld_f32(v, row) - p[i] * ik);
        if (cq == 0) st_out(a.out, a.out_bf16, (int64_t)pair * V + row, a.scale * (r[i] * iq + kq * d));
        const float dk = d * ik;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float4 x = s[i][g];
            x.x += kv[g][0] * dk; x.y += kv[g][1] * dk; x.z += kv[g][2] * dk; x.w += kv[g][3] * dk;
            __builtin_nontemporal_store(f4{x.x, x.y, x.z, x.w}, reinterpret_cast<f4 *>(&S[row * R4 + cq + CQ * g]));
        }
    }
}

template <typename TIn, int K>
hipError_t launch_k(const StepArgs &a, int V, int pairs, hipStream_t stream) {
    switch (V) {
#define KDA_STEP_CASE(VV)                                                                         \
    case VV:                                                                                      \
        if (a.state_vk) {                                                                         \
            if (a.gate.mode == GATE_LOGITS)                                                       \
                hipLaunchKernelGGL((recurrent_step_vk_kernel<TIn, K, VV, true>), dim3(pairs),     \
                                   dim3(StepVkCfg<K, VV>::NT), 0, stream, a);                     \
            else                                                                                  \
                hipLaunchKernelGGL((recurrent_step_vk_kernel<TIn, K, VV, false>), dim3(pairs),    \
                                   dim3(StepVkCfg<K, VV>::NT), 0, stream, a);                     \
        } else if (a.gate.mode == GATE_LOGITS) {                                                  \
            hipLaunchKernelGGL((recurrent_step_kernel<TIn, K, VV, true>), dim3(pairs),            \
                               dim3(StepCfg<K, VV>::NT), 0, stream, a);                           \
        } else {                                                                                  \
            hipLaunchKernelGGL((recurrent_step_kernel<TIn, K, VV, false>), dim3(pairs),           \
                               dim3(StepCfg<K, VV>::NT), 0, stream, a);                           \
        }                                                                                         \
        return hipGetLastError();
        KDA_STEP_CASE(16)
        KDA_STEP_CASE(32)
        KDA_STEP_CASE(64)
        KDA_STEP_CASE(128)
#undef KDA_STEP_CASE
        default: return hipErrorNotSupported;
    }
}

template <typename TIn>
hipError_t launch_t(const StepArgs &a, int K, int V, int pairs, hipStream_t stream) {
    switch (K) {
        case 16: return launch_k<TIn, 16>(a, V, pairs, stream);
        case 32: return launch_k<TIn, 32>(a, V, pairs, stream);
        case 64: return launch_k<TIn, 64>(a, V, pairs, stream);
        case 128: return launch_k<TIn, 128>(a, V, pairs, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_recurrent_step(const StepArgs &a, bool fp32_inputs, int K, int V, int pairs,
                                 hipStream_t stream) {
    return fp32_inputs ? launch_t<float>(a, K, V, pairs, stream) : launch_t<__bf16>(a, K, V, pairs, stream);
}

}  // namespace kda
