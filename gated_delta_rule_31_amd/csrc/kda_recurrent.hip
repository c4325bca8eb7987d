// kda_recurrent.hip -- multi-token fused recurrent KDA forward (gfx950).
//
// The recurrence itself, token after token, for short sequences (speculative decode,
// short prompts) where the chunked form's per-chunk set-up does not pay off
// (PaperLeet "Formula and conventions"; the model excerpt on the Kept-memory page has a
// token-recurrent kernel beside the chunked one, taking any length and packed sequences):
//   Sbar  = Diag(alpha_t) S
//   delta = beta_t (v_t - Sbar^T k_t)
//   S     = Sbar + k_t delta^T
//   o_t   = scale S^T q_t = scale (Sbar^T q_t + (k_t . q_t) delta)
// Any alpha in [0, 1] is allowed (no rescaling is involved).
//
// Mapping: one workgroup per (sequence, head, block of BV value columns), one wave per
// 16 columns.  Lane l of a wave owns the four columns 4 (l / 16) .. + 3 and the key rows
// [RL (l % 16), RL (l % 16) + RL) with RL = K / 16, so the state stays in registers for
// the whole sequence, each token reads only the lane's RL rows of k, q and alpha from
// LDS (shared by its four columns), and the reductions over K are a sum over the lane's
// rows plus a DPP sum inside the 16-lane row.  The token inputs arrive in blocks of TB
// tokens: the workgroup loads block b+1 with 16-byte loads while it runs block b from
// LDS, and converts it to float32 (alpha and k.q included) once for all its columns.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int RW = 4;  // waves per workgroup (at most; fewer when V < 64)
constexpr int TB = 8;  // tokens per staged block

typedef __attribute__((ext_vector_type(8))) float f4x2;

__device__ __forceinline__ f4x2 to_f4x2(f4x2 x) { return x; }
__device__ __forceinline__ f4x2 to_f4x2(bf16x8 x) {
    f4x2 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)x[e];
    return y;
}

// Four waves per SIMD (at most 128 registers; five would spill): more workgroups in
// flight hide the state loads at their start.
template <typename TIn, int K, int V, bool ZG>
__global__ __launch_bounds__(64 * RW) __attribute__((amdgpu_waves_per_eu(4))) void recurrent_fwd_kernel(
    RecurrentArgs a) {
    constexpr int RL = K / 16;                      // key rows per lane
    constexpr int NW = V / 16 < RW ? V / 16 : RW;   // waves per workgroup
    constexpr int NTH = 64 * NW;
    constexpr int BV = 16 * NW;                     // value columns per workgroup
    constexpr int NVB = V / BV;
    constexpr int UK = K / 8;                       // 8-element units per key row
    constexpr int NU = TB * UK;                     // key-row units of one block (per tensor)
    constexpr int UPT = (NU + NTH - 1) / NTH;       // units per thread and tensor
    constexpr int VU = TB * BV / 8;                 // value units of one block
    constexpr int VPT = (VU + NTH - 1) / NTH;
    using RawU = typename std::conditional<std::is_same<TIn, float>::value, f4x2, bf16x8>::type;
    using RawG = typename std::conditional<ZG, RawU, f4x2>::type;

    // two blocks of TB tokens staged in float32: k, q and alpha rows, k.q, v, beta
    __shared__ __align__(16) float sk[2][TB][K];
    __shared__ __align__(16) float sq[2][TB][K];
    __shared__ __align__(16) float sa[2][TB][K];
    __shared__ __align__(16) float sv[2][TB][BV];
    __shared__ float skq[2][TB], sbeta[2][TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = lane & 15;                       // key-row group: rows RL rg .. RL rg + RL - 1
    const int cg = lane >> 4;                       // column group: columns 4 cg .. 4 cg + 3
    const int vb = blockIdx.x % NVB;
    const int pair = blockIdx.x / NVB;
    const int H = a.H;
    const int h = pair % H;
    const int s = pair / H;
    int64_t bos, eos;
    if (a.cu_seqlens) {
        bos = a.cu_seqlens[s];
        eos = a.cu_seqlens[s + 1];
    } else {
        bos = (int64_t)s * a.T;
        eos = bos + a.T;
    }
    const int col = wave * 16 + 4 * cg;             // first of the lane's columns within the block
    const int gcol = vb * BV + col;
    const int r0 = RL * rg;

    // the lane's RL x 4 block of the state: 16-byte accesses along V ([K, V] states) or
    // along K ([V, K] states, RL a multiple of 4) keep a row of 16 lanes on 64 contiguous bytes
    float S[RL][4];
    const float *s0 = a.initial_state ? a.initial_state + ((int64_t)s * H + h) * K * V : nullptr;
#pragma unroll
    for (int i = 0; i < RL; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) S[i][c] = 0.f;
    if (s0) {
        if (!a.state_vk) {
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                const float4 x = *reinterpret_cast<const float4 *>(s0 + (int64_t)(r0 + i) * V + gcol);
                S[i][0] = x.x; S[i][1] = x.y; S[i][2] = x.z; S[i][3] = x.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < RL; ++i) S[i][c] = s0[(int64_t)(gcol + c) * K + r0 + i];
        }
    }

    const bool glog = a.gate.mode == GATE_LOG;
    float s2 = 0.f, l2 = 0.f;
    float zbias[UPT][8];
#pragma unroll
    for (int w = 0; w < UPT; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) zbias[w][e] = 0.f;
    if constexpr (ZG) {
        s2 = expf(a.gate.log_scale[h]) * 1.44269504088896341f;
        l2 = a.gate.lower_bound * 1.44269504088896341f;
        if (a.gate.bias) {
#pragma unroll
            for (int w = 0; w < UPT; ++w) {
                const int c = 8 * ((tid + NTH * w) % UK);  // the same column for every block
#pragma unroll
                for (int e = 0; e < 8; ++e) zbias[w][e] = a.gate.bias[h * K + c + e];
            }
        }
    }
    const TIn *q = static_cast<const TIn *>(a.q);
    const TIn *k = static_cast<const TIn *>(a.k);
    const TIn *v = static_cast<const TIn *>(a.v);
    const TIn *zl = static_cast<const TIn *>(a.gate.logits);
    const int nblk = (int)((eos - bos + TB - 1) / TB);

    // raw units of one block, held in registers between their load and their staging
    RawU rk[UPT], rq[UPT], rv[VPT];
    RawG ra[UPT];
    float rb = 0.f;
    auto load_block = [&](int b) {
        const int64_t t0 = bos + (int64_t)b * TB;
        const int64_t last = eos - 1;  // rows past the end read the last row (not used)
#pragma unroll
        for (int w = 0; w < UPT; ++w) {
            const int u = tid + NTH * w < NU ? tid + NTH * w : 0;
            const int j = u / UK, c = 8 * (u % UK);
            const int64_t t = t0 + j < last ? t0 + j : last;
            const int64_t o = (t * H + h) * K + c;
            rk[w] = *reinterpret_cast<const RawU *>(k + o);
            rq[w] = *reinterpret_cast<const RawU *>(q + o);
            if constexpr (ZG)
                ra[w] = *reinterpret_cast<const RawU *>(zl + o);
            else
                ra[w] = *reinterpret_cast<const f4x2 *>(a.gate.gate + o);
        }
#pragma unroll
        for (int w = 0; w < VPT; ++w) {
            const int u = tid + NTH * w < VU ? tid + NTH * w : 0;
            const int j = u / (BV / 8), c = 8 * (u % (BV / 8));
            const int64_t t = t0 + j < last ? t0 + j : last;
            rv[w] = *reinterpret_cast<const RawU *>(v + (t * H + h) * V + vb * BV + c);
        }
        if (tid < TB) rb = a.beta[(t0 + tid < last ? t0 + tid : last) * H + h];
    };
    // convert the held units into LDS buffer `buf`; alpha and k.q are formed here, once
    // per workgroup rather than once per value column
    auto stage_block = [&](int buf) {
#pragma unroll
        for (int w = 0; w < UPT; ++w) {
            const int u = tid + NTH * w;
            const int j = u / UK, c = 8 * (u % UK);
            f4x2 kk = to_f4x2(rk[w]), qq = to_f4x2(rq[w]);
            f4x2 al = to_f4x2(ra[w]);
            float dot = 0.f, nk = 0.f, nq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (ZG)
                    al[e] = fast_bounded_alpha(al[e] + zbias[w][e], s2, l2);
                else if (glog)
                    al[e] = expf(al[e]);
                dot += kk[e] * qq[e];
                nk += kk[e] * kk[e];
                nq += qq[e] * qq[e];
            }
            // row sums over the token: the UK units of a row sit in UK consecutive lanes
#pragma unroll
            for (int m = 1; m < UK; m <<= 1) {
                dot += __shfl_xor(dot, m);
                nk += __shfl_xor(nk, m);
                nq += __shfl_xor(nq, m);
            }
            if (a.qk_l2norm) {
                const float ik = 1.f / fmaxf(sqrtf(nk), 1e-6f), iq = 1.f / fmaxf(sqrtf(nq), 1e-6f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kk[e] *= ik;
                    qq[e] *= iq;
                }
                dot *= ik * iq;
            }
            if (u < NU) {
                *reinterpret_cast<f4x2 *>(&sk[buf][j][c]) = kk;
                *reinterpret_cast<f4x2 *>(&sq[buf][j][c]) = qq;
                *reinterpret_cast<f4x2 *>(&sa[buf][j][c]) = al;
                if (c == 0) skq[buf][j] = dot;
            }
        }
#pragma unroll
        for (int w = 0; w < VPT; ++w) {
            const int u = tid + NTH * w;
            if (u < VU) {
                const int j = u / (BV / 8), c = 8 * (u % (BV / 8));
                *reinterpret_cast<f4x2 *>(&sv[buf][j][c]) = to_f4x2(rv[w]);
            }
        }
        if (tid < TB) sbeta[buf][tid] = a.beta_logits ? 1.f / (1.f + __expf(-rb)) : rb;
    };

    if (nblk > 0) {
        load_block(0);
        stage_block(0);
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
        const int buf = b & 1;
        if (b + 1 < nblk) load_block(b + 1);  // in flight while this block runs
        const int64_t t0 = bos + (int64_t)b * TB;
        for (int j = 0; j < TB; ++j) {
            const int64_t t = t0 + j;
            if (t >= eos) break;
            float kx[RL], qx[RL], ax[RL];
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                kx[i] = sk[buf][j][r0 + i];
                qx[i] = sq[buf][j][r0 + i];
                ax[i] = sa[buf][j][r0 + i];
            }
            float p[4], r[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                p[c] = 0.f;
                r[c] = 0.f;
#pragma unroll
                for (int i = 0; i < RL; ++i) {
                    S[i][c] *= ax[i];
                    p[c] += S[i][c] * kx[i];
                    r[c] += S[i][c] * qx[i];
                }
                // sum over the 16 row groups (the lanes of this DPP row)
                p[c] = row16_sum(p[c]);
                r[c] = row16_sum(r[c]);
            }
            const float4 v4 = *reinterpret_cast<const float4 *>(&sv[buf][j][col]);
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            const float bj = sbeta[buf][j], kq = skq[buf][j];
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float d = bj * (vv[c] - p[c]);
                o[c] = a.scale * (r[c] + kq * d);
#pragma unroll
                for (int i = 0; i < RL; ++i) S[i][c] += kx[i] * d;
            }
            if (rg == 0) {  // the row's four columns in one store
                const int64_t oi = (t * H + h) * V + gcol;
                if (a.out_bf16) {
                    typedef __attribute__((ext_vector_type(4))) __bf16 bf4;
                    *reinterpret_cast<bf4 *>(static_cast<__bf16 *>(a.out) + oi) =
                        bf4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + oi) = float4{o[0], o[1], o[2], o[3]};
                }
            }
        }
        if (b + 1 < nblk) stage_block(buf ^ 1);
        __syncthreads();
    }
    if (a.final_state) {
        float *sf = a.final_state + ((int64_t)s * H + h) * K * V;
        if (!a.state_vk) {
#pragma unroll
            for (int i = 0; i < RL; ++i)
                *reinterpret_cast<float4 *>(sf + (int64_t)(r0 + i) * V + gcol) = float4{S[i][0], S[i][1], S[i][2], S[i][3]};
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < RL; ++i) sf[(int64_t)(gcol + c) * K + r0 + i] = S[i][c];
        }
    }
}

template <typename TIn, bool ZG, int K>
hipError_t launch_k(const RecurrentArgs &a, int V, int num_pairs, hipStream_t stream) {
    switch (V) {
#define KDA_REC_CASE(VV)                                                                          \
    case VV: {                                                                                    \
        constexpr int NW = VV / 16 < RW ? VV / 16 : RW;                                           \
        hipLaunchKernelGGL((recurrent_fwd_kernel<TIn, K, VV, ZG>), dim3(num_pairs * (VV / (16 * NW))), \
                           dim3(64 * NW), 0, stream, a);                                          \
        return hipGetLastError();                                                                 \
    }
        KDA_REC_CASE(16)
        KDA_REC_CASE(32)
        KDA_REC_CASE(64)
        KDA_REC_CASE(128)
#undef KDA_REC_CASE
        default: return hipErrorNotSupported;
    }
}

template <typename TIn, bool ZG>
hipError_t launch_t(const RecurrentArgs &a, int K, int V, int num_pairs, hipStream_t stream) {
    switch (K) {
        case 16: return launch_k<TIn, ZG, 16>(a, V, num_pairs, stream);
        case 32: return launch_k<TIn, ZG, 32>(a, V, num_pairs, stream);
        case 64: return launch_k<TIn, ZG, 64>(a, V, num_pairs, stream);
        case 128: return launch_k<TIn, ZG, 128>(a, V, num_pairs, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_recurrent_fwd(const RecurrentArgs &a, bool fp32_inputs, int K, int V, int num_pairs,
                                hipStream_t stream) {
    const bool zg = a.gate.mode == GATE_LOGITS;
    if (fp32_inputs)
        return zg ? launch_t<float, true>(a, K, V, num_pairs, stream) : launch_t<float, false>(a, K, V, num_pairs, stream);
    return zg ? launch_t<__bf16, true>(a, K, V, num_pairs, stream) : launch_t<__bf16, false>(a, K, V, num_pairs, stream);
}

}  // namespace kda
