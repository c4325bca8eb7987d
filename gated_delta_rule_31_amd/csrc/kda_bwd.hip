// Backward of the chunkwise KDA recurrence: gradients of
//   L = <d_out, out> + <d_final_state, final_state>
// with respect to q, k, v, the gate (retention alpha or its log), beta and the initial
// state (PaperLeet "Return requirements": gradients reach every input of the scan).
//
// The chunkwise forward (KDA cheat sheet, "Chunkwise parallel form"), per chunk of C
// tokens with start state S and in-chunk cumulative log-decay Gamma:
//   Abar[r,s] = sum_c k_rc k_sc e^{Gamma_rc - Gamma_sc} (s < r),  T = (I + diag(beta) Abar)^-1
//   W = T (beta K e^Gamma),  U = T (beta V),  Vt = U - W S
//   A_qk[r,s] = sum_c q_rc k_sc e^{Gamma_rc - Gamma_sc} (s <= r)
//   O = scale [(Q e^Gamma) S + A_qk Vt],   S' = gamma_C S + Kd^T Vt,  Kd = K e^{Gamma_C - Gamma}
// differentiated in reverse (dO here already carries the scale):
//   dVt = Kd dS' + A_qk^T dO,   dS = gamma_C dS' + (Q e^Gamma)^T dO - W^T dVt
//   dQ = (dO S^T) e^Gamma + adj_X(tril(dO Vt^T); Q, K)
//   dW = -dVt S^T,  dT = dVt (beta V)^T + dW (beta K e^Gamma)^T,  dV = beta (T^T dVt)
//   dA = -strict_tril(T^T dT T^T),  dbeta = rowsum(V T^T dVt) + rowsum(K e^Gamma T^T dW) + rowsum(dA Abar)
//   dK = adj_Y(tril(dO Vt^T)) + (Vt dS'^T) e^{Gamma_C - Gamma} + beta e^Gamma T^T dW
//        + adj_X(beta dA; K, K) + adj_Y(beta dA; K, K)
//   dGamma = Q dQ + K (dK_row-side - dK_col-side); d ln alpha = its reverse in-chunk sum
//            + gamma_C rowsum(S dS') + the forward (exclusive) sum of K (Vt dS'^T) e^{Gamma_C - Gamma}
// where for A[r,s] = sum_c X_rc Y_sc e^{Gamma_rc - Gamma_sc} and dL/dA = M:
//   adj_X(M)[r] = sum_s M[r,s] Y_s e^{Gamma_r - Gamma_s},  adj_Y(M)[s] = sum_r M[r,s] X_r e^{Gamma_r - Gamma_s}.
// Every such decayed product is split at the middle row m of the 16-row tile of r:
// e^{Gamma_r - Gamma_m} e^{Gamma_m - Gamma_s}; with every log-decay >= -5 (the K3 bound of
// the cheat sheet's gate table) neither factor exceeds e^40 on the kept entries.
//
// Five launches on one stream, all float32 on the matrix cores (16x16x4) and vector units:
//   prep    (chunk, head)          Gamma, Abar, T (blocked 16x16 inverse), A_qk, W, U, Kd, Q e^Gamma, K e^Gamma
//   states  (value block, head, seq) serial over chunks: keeps each chunk's start state and Vt
//   dstates (value block, head, seq) serial backwards: keeps each chunk's end-state gradient,
//                                  dVt, and writes the initial-state gradient
//   vgrads  (chunk, head)          the contractions over V; writes dv
//   kgrads  (chunk, head)          dT, dA and the decayed adjoints; writes dq, dk, dgate, dbeta
// Chunk slots: without cu_seqlens slot b*NT + j is chunk j of batch row b; with them,
// sequence s owns slots floor(cu[s]/C) + s + j, j < ceil(len_s / C) (disjoint, fewer than
// T/C + N in all); a slot no sequence owns is skipped.
#include "kda_chunk_kernel.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BC = 64;          // tokens per chunk
constexpr int NP = BC / 16;     // 16-row tiles per chunk
constexpr int NTH = 256;        // four waves
constexpr int LDC = BC + 4;     // LDS row stride of a C x C matrix

__device__ __forceinline__ f4 mf(float a, float b, f4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

struct ChunkPos {
    int64_t t0;  // first token row
    int L;       // tokens in the chunk (0: slot unused)
};

__device__ __forceinline__ ChunkPos slot_chunk(int n, const int32_t *cu, int N, int64_t T) {
    ChunkPos p;
    if (!cu) {
        const int NT = (int)((T + BC - 1) / BC);
        const int b = n / NT, j = n - b * NT;
        p.t0 = (int64_t)b * T + (int64_t)j * BC;
        p.L = (int)min((int64_t)BC, T - (int64_t)j * BC);
        return p;
    }
    int lo = 0, hi = N - 1;  // last sequence whose first slot is <= n
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / BC + mid <= n) lo = mid;
        else hi = mid - 1;
    }
    const int64_t a0 = cu[lo], len = (int64_t)cu[lo + 1] - a0;
    const int64_t off = (int64_t)(n - (cu[lo] / BC + lo)) * BC;
    p.t0 = a0 + off;
    p.L = off < len ? (int)min((int64_t)BC, len - off) : 0;
    return p;
}

__device__ __forceinline__ void seq_range(int s, const int32_t *cu, int64_t T, int64_t &t0, int64_t &len,
                                          int &base) {
    if (cu) {
        t0 = cu[s];
        len = (int64_t)cu[s + 1] - t0;
        base = (int)(t0 / BC) + s;
    } else {
        t0 = (int64_t)s * T;
        len = T;
        base = s * (int)((T + BC - 1) / BC);
    }
}

__device__ __forceinline__ float gate_log(const GateIn &g, int64_t i) {
    return g.mode == GATE_LOG ? g.gate[i] : logf(g.gate[i]);
}

__device__ __forceinline__ float ld_any(const void *p, int is_bf16, int64_t i) {
    return is_bf16 ? (float)static_cast<const __bf16 *>(p)[i] : static_cast<const float *>(p)[i];
}

// sum over the 16 lanes that share lane >> 4 (one accumulator row)
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// ------------------------------------------------------------------------------------
// prep: one workgroup per (chunk slot, head)
template <int K>
struct PrepLds {
    static constexpr int LK = K + 4;
    static constexpr size_t bytes = sizeof(float) * (3 * BC * LK + 2 * BC * LDC + BC + K);
};

template <typename TIn, int K, int V>
__global__ __launch_bounds__(NTH) void bwd_prep_kernel(BwdArgs a) {
    constexpr int LK = PrepLds<K>::LK;
    extern __shared__ __align__(16) unsigned char smem[];
    float *sQ = reinterpret_cast<float *>(smem);  // q, later beta k e^Gamma
    float *sK = sQ + BC * LK;
    float *sG = sK + BC * LK;                     // log-decay, then Gamma
    float *sA = sG + BC * LK;                     // Abar
    float *sT = sA + BC * LDC;                    // T
    float *sB = sT + BC * LDC;                    // beta
    float *sE = sB + BC;                          // Gamma at the chunk end

    const int n = blockIdx.x, h = blockIdx.y, H = a.H;
    const ChunkPos cp = slot_chunk(n, a.cu_seqlens, a.num_seqs, a.T);
    if (cp.L == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, i16 = lane & 15;
    const int64_t sh = (int64_t)n * H + h;
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k);
    const TIn *v = static_cast<const TIn *>(a.v);

    for (int i = tid; i < BC * K; i += NTH) {
        const int r = i / K, c = i % K;
        float qv = 0.f, kv = 0.f, gv = 0.f;  // rows past the chunk: no token, no decay
        if (r < cp.L) {
            const int64_t gi = ((cp.t0 + r) * H + h) * K + c;
            qv = ld_f32(q, gi);
            kv = ld_f32(k, gi);
            gv = gate_log(a.gate, gi);
        }
        sQ[r * LK + c] = qv;
        sK[r * LK + c] = kv;
        sG[r * LK + c] = gv;
    }
    if (tid < BC) sB[tid] = tid < cp.L ? a.beta[(cp.t0 + tid) * H + h] : 0.f;
    __syncthreads();
    if (tid < K) {
        float run = 0.f;
        for (int r = 0; r < BC; ++r) {
            run += sG[r * LK + tid];
            sG[r * LK + tid] = run;
        }
        sE[tid] = run;
    }
    __syncthreads();

    // Abar (strictly lower) and A_qk (lower) in 16x16 tiles, split at the row tile's middle
    float *Aqk = a.w.Aqk + sh * BC * BC, *Abar = a.w.Abar + sh * BC * BC;
    for (int t = w; t < NP * NP; t += 4) {
        const int p = t / NP, qt = t % NP;
        f4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
        if (qt <= p) {
            const float *mref = sG + (16 * p + 7) * LK;
            const int r = 16 * p + i16, s = 16 * qt + i16;
#pragma unroll 4
            for (int c0 = 0; c0 < K; c0 += 4) {
                const int c = c0 + g4;
                const float m = mref[c];
                const float er = expf(sG[r * LK + c] - m);
                const float b = sK[s * LK + c] * expf(m - sG[s * LK + c]);
                ak = mf(sK[r * LK + c] * er, b, ak);
                aq = mf(sQ[r * LK + c] * er, b, aq);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e, col = 16 * qt + i16;
            const float vk = row > col ? ak[e] : 0.f;  // selects: masked entries may be inf
            const float vq = row >= col ? aq[e] : 0.f;
            sA[row * LDC + col] = vk;
            Abar[row * BC + col] = vk;
            Aqk[row * BC + col] = vq;
        }
    }
    __syncthreads();

    // T = (I + diag(beta) Abar)^-1: diagonal 16x16 blocks by the blocked inverse, then
    // block forward substitution T_pq = -T_pp sum_{q<=u<p} A_pu T_uq
    if (w < NP) {
        const int p = w;
        f4 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            av[e] = sB[row] * sA[row * LDC + 16 * p + i16];
        }
        const f4 tb = unit_lower_inverse16<float>(av, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * p + 4 * g4 + e) * LDC + 16 * p + i16] = tb[e];
    }
    for (int i = tid; i < BC * BC; i += NTH) {
        const int r = i / BC, c = i % BC;
        if ((c >> 4) > (r >> 4)) sT[r * LDC + c] = 0.f;
    }
    __syncthreads();
    for (int p = 1; p < NP; ++p) {
        if (w < p) {
            const int qb = w;
            f4 x = {0.f, 0.f, 0.f, 0.f};
            for (int u = qb; u < p; ++u) {
#pragma unroll
                for (int s0 = 0; s0 < 16; s0 += 4) {
                    const int r = 16 * p + i16, s = 16 * u + s0 + g4;
                    x = mf(sB[r] * sA[r * LDC + s], sT[s * LDC + 16 * qb + i16], x);
                }
            }
            f4 xr;  // row-operand form of T_pp: lane (g, r) holds T_pp[r][4g + s]
#pragma unroll
            for (int s = 0; s < 4; ++s) xr[s] = sT[(16 * p + i16) * LDC + 16 * p + 4 * g4 + s];
            const f4 y = mma16_reg<float>(xr, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * p + 4 * g4 + e) * LDC + 16 * qb + i16] = -y[e];
        }
        __syncthreads();
    }

    // elementwise products and the chunk-end decay; beta K e^Gamma replaces q in LDS
    float *Qg = a.w.Qg + sh * BC * K, *Kd = a.w.Kd + sh * BC * K, *Kg = a.w.Kg + sh * BC * K;
    for (int i = tid; i < BC * K; i += NTH) {
        const int r = i / K, c = i % K;
        const float G = sG[r * LK + c], eg = expf(G), kv = sK[r * LK + c];
        Qg[r * K + c] = sQ[r * LK + c] * eg;
        Kd[r * K + c] = kv * expf(sE[c] - G);
        Kg[r * K + c] = kv * eg;
        sQ[r * LK + c] = sB[r] * kv * eg;
    }
    if (tid < K) a.w.gC[sh * K + tid] = expf(sE[tid]);
    float *Tm = a.w.Tm + sh * BC * BC;
    for (int i = tid; i < BC * BC; i += NTH) Tm[i] = sT[(i / BC) * LDC + i % BC];
    __syncthreads();

    // W = T (beta K e^Gamma), U = T (beta V); T is lower triangular
    float *W = a.w.W + sh * BC * K, *U = a.w.U + sh * BC * V;
    for (int t = w; t < NP * (K / 16); t += 4) {
        const int p = t / (K / 16), ct = t % (K / 16);
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < 16 * (p + 1); s0 += 4)
            acc = mf(sT[(16 * p + i16) * LDC + s0 + g4], sQ[(s0 + g4) * LK + 16 * ct + i16], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) W[(16 * p + 4 * g4 + e) * K + 16 * ct + i16] = acc[e];
    }
    for (int t = w; t < NP * (V / 16); t += 4) {
        const int p = t / (V / 16), ct = t % (V / 16);
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < 16 * (p + 1); s0 += 4) {
            const int s = s0 + g4;
            const float bv = s < cp.L ? sB[s] * ld_f32(v, ((cp.t0 + s) * H + h) * V + 16 * ct + i16) : 0.f;
            acc = mf(sT[(16 * p + i16) * LDC + s], bv, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) U[(16 * p + 4 * g4 + e) * V + 16 * ct + i16] = acc[e];
    }
}

// ------------------------------------------------------------------------------------
// states: the forward over chunks, one workgroup per (value block, head, sequence)
constexpr int SBV = 16;  // value columns per workgroup in the serial passes

template <int K, int V>
__global__ __launch_bounds__(NTH) void bwd_states_kernel(BwdArgs a) {
    constexpr int LB = SBV + 4;
    __shared__ float sS[K * LB];
    __shared__ float sV[BC * LB];
    const int vb = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, i16 = lane & 15;
    const int j0 = vb * SBV;
    int64_t t0, len;
    int base;
    seq_range(s, a.cu_seqlens, a.T, t0, len, base);
    const int nch = (int)((len + BC - 1) / BC);
    for (int i = tid; i < K * SBV; i += NTH) {
        const int r = i / SBV, c = i % SBV;
        sS[r * LB + c] = a.initial_state ? a.initial_state[(((int64_t)s * H + h) * K + r) * V + j0 + c] : 0.f;
    }
    for (int j = 0; j < nch; ++j) {
        const int64_t sh = (int64_t)(base + j) * H + h;
        __syncthreads();
        float *hp = a.w.h + sh * K * V;
        for (int i = tid; i < K * SBV; i += NTH) {
            const int r = i / SBV, c = i % SBV;
            hp[r * V + j0 + c] = sS[r * LB + c];
        }
        const float *W = a.w.W + sh * BC * K, *U = a.w.U + sh * BC * V;
        float *Vt = a.w.Vt + sh * BC * V;
        for (int t = w; t < NP * (SBV / 16); t += 4) {
            const int p = t / (SBV / 16), ct = t % (SBV / 16);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k0 = 0; k0 < K; k0 += 4)
                acc = mf(W[(16 * p + i16) * K + k0 + g4], sS[(k0 + g4) * LB + 16 * ct + i16], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * p + 4 * g4 + e, col = 16 * ct + i16;
                const float vt = U[row * V + j0 + col] - acc[e];
                sV[row * LB + col] = vt;
                Vt[row * V + j0 + col] = vt;
            }
        }
        __syncthreads();
        const float *Kd = a.w.Kd + sh * BC * K, *gC = a.w.gC + sh * K;
        for (int t = w; t < (K / 16) * (SBV / 16); t += 4) {
            const int rt = t / (SBV / 16), ct = t % (SBV / 16);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int r0 = 0; r0 < BC; r0 += 4)
                acc = mf(Kd[(r0 + g4) * K + 16 * rt + i16], sV[(r0 + g4) * LB + 16 * ct + i16], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * rt + 4 * g4 + e, col = 16 * ct + i16;
                sS[m * LB + col] = gC[m] * sS[m * LB + col] + acc[e];
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// dstates: the reverse over chunks
template <int K, int V>
__global__ __launch_bounds__(NTH) void bwd_dstates_kernel(BwdArgs a) {
    constexpr int LB = SBV + 4;
    __shared__ float sD[K * LB];
    __shared__ float sO[BC * LB];
    __shared__ float sV[BC * LB];
    const int vb = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = a.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, i16 = lane & 15;
    const int j0 = vb * SBV;
    int64_t t0, len;
    int base;
    seq_range(s, a.cu_seqlens, a.T, t0, len, base);
    const int nch = (int)((len + BC - 1) / BC);
    const int64_t st = ((int64_t)s * H + h) * K;
    for (int i = tid; i < K * SBV; i += NTH) {
        const int r = i / SBV, c = i % SBV;
        sD[r * LB + c] = a.d_final_state ? a.d_final_state[(st + r) * V + j0 + c] : 0.f;
    }
    for (int j = nch - 1; j >= 0; --j) {
        const int64_t sh = (int64_t)(base + j) * H + h;
        const int64_t tc = t0 + (int64_t)j * BC;
        const int L = (int)min((int64_t)BC, len - (int64_t)j * BC);
        __syncthreads();
        float *dhp = a.w.dh + sh * K * V;
        for (int i = tid; i < K * SBV; i += NTH) {
            const int r = i / SBV, c = i % SBV;
            dhp[r * V + j0 + c] = sD[r * LB + c];
        }
        for (int i = tid; i < BC * SBV; i += NTH) {
            const int r = i / SBV, c = i % SBV;
            sO[r * LB + c] = r < L ? a.scale * ld_any(a.d_out, a.dout_bf16, ((tc + r) * H + h) * V + j0 + c) : 0.f;
        }
        __syncthreads();
        const float *Kd = a.w.Kd + sh * BC * K, *Aqk = a.w.Aqk + sh * BC * BC;
        float *dVt = a.w.dVt + sh * BC * V;
        for (int t = w; t < NP * (SBV / 16); t += 4) {
            const int p = t / (SBV / 16), ct = t % (SBV / 16);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k0 = 0; k0 < K; k0 += 4)
                acc = mf(Kd[(16 * p + i16) * K + k0 + g4], sD[(k0 + g4) * LB + 16 * ct + i16], acc);
            // A_qk^T dO: A_qk[s][r] is zero for s < r
            for (int s0 = 16 * p; s0 < BC; s0 += 4)
                acc = mf(Aqk[(s0 + g4) * BC + 16 * p + i16], sO[(s0 + g4) * LB + 16 * ct + i16], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * p + 4 * g4 + e, col = 16 * ct + i16;
                sV[row * LB + col] = acc[e];
                dVt[row * V + j0 + col] = acc[e];
            }
        }
        __syncthreads();
        const float *Qg = a.w.Qg + sh * BC * K, *W = a.w.W + sh * BC * K, *gC = a.w.gC + sh * K;
        for (int t = w; t < (K / 16) * (SBV / 16); t += 4) {
            const int rt = t / (SBV / 16), ct = t % (SBV / 16);
            f4 acc = {0.f, 0.f, 0.f, 0.f}, neg = acc;
#pragma unroll 8
            for (int r0 = 0; r0 < BC; r0 += 4) {
                const int r = r0 + g4;
                acc = mf(Qg[r * K + 16 * rt + i16], sO[r * LB + 16 * ct + i16], acc);
                neg = mf(W[r * K + 16 * rt + i16], sV[r * LB + 16 * ct + i16], neg);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * rt + 4 * g4 + e, col = 16 * ct + i16;
                sD[m * LB + col] = gC[m] * sD[m * LB + col] + acc[e] - neg[e];
            }
        }
    }
    __syncthreads();
    if (a.d_initial_state)
        for (int i = tid; i < K * SBV; i += NTH) {
            const int r = i / SBV, c = i % SBV;
            a.d_initial_state[(st + r) * V + j0 + c] = sD[r * LB + c];
        }
}

// ------------------------------------------------------------------------------------
// vgrads: contractions over the value dimension, one workgroup per (chunk slot, head)
template <int V>
struct VgLds {
    static constexpr int LV = V + 4;
    static constexpr size_t bytes = sizeof(float) * (2 * BC * LV + BC + (V / 16) * BC);
};

template <typename TIn, int K, int V>
__global__ __launch_bounds__(NTH) void bwd_vgrads_kernel(BwdArgs a) {
    constexpr int LV = VgLds<V>::LV;
    extern __shared__ __align__(16) unsigned char smem[];
    float *sO = reinterpret_cast<float *>(smem);  // scale * dO
    float *sVr = sO + BC * LV;                     // v
    float *sB = sVr + BC * LV;                     // beta
    float *sRed = sB + BC;                         // [V/16][BC] partial row sums
    const int n = blockIdx.x, h = blockIdx.y, H = a.H;
    const ChunkPos cp = slot_chunk(n, a.cu_seqlens, a.num_seqs, a.T);
    if (cp.L == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, i16 = lane & 15;
    const int64_t sh = (int64_t)n * H + h;
    const TIn *v = static_cast<const TIn *>(a.v);
    for (int i = tid; i < BC * V; i += NTH) {
        const int r = i / V, c = i % V;
        float ov = 0.f, vv = 0.f;
        if (r < cp.L) {
            const int64_t gi = ((cp.t0 + r) * H + h) * V + c;
            ov = a.scale * ld_any(a.d_out, a.dout_bf16, gi);
            vv = ld_f32(v, gi);
        }
        sO[r * LV + c] = ov;
        sVr[r * LV + c] = vv;
    }
    if (tid < BC) sB[tid] = tid < cp.L ? a.beta[(cp.t0 + tid) * H + h] : 0.f;
    __syncthreads();

    const float *hp = a.w.h + sh * K * V, *dhp = a.w.dh + sh * K * V;
    const float *Vt = a.w.Vt + sh * BC * V, *dVt = a.w.dVt + sh * BC * V, *Tm = a.w.Tm + sh * BC * BC;
    float *PS = a.w.PS + sh * BC * K, *PW = a.w.PW + sh * BC * K, *PdK = a.w.PdK + sh * BC * K;
    // dO S^T, dVt S^T and Vt dS'^T  [C x K]
    for (int t = w; t < NP * (K / 16); t += 4) {
        const int p = t / (K / 16), ct = t % (K / 16);
        f4 ps = {0.f, 0.f, 0.f, 0.f}, pw = ps, pd = ps;
        const int r = 16 * p + i16, c = 16 * ct + i16;
#pragma unroll 4
        for (int j0 = 0; j0 < V; j0 += 4) {
            const int j = j0 + g4;
            const float hb = hp[c * V + j], db = dhp[c * V + j];
            ps = mf(sO[r * LV + j], hb, ps);
            pw = mf(dVt[r * V + j], hb, pw);
            pd = mf(Vt[r * V + j], db, pd);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            PS[row * K + c] = ps[e];
            PW[row * K + c] = pw[e];
            PdK[row * K + c] = pd[e];
        }
    }
    // dO Vt^T and dVt (beta V)^T  [C x C]
    float *MA = a.w.MA + sh * BC * BC, *MT = a.w.MT + sh * BC * BC;
    for (int t = w; t < NP * NP; t += 4) {
        const int p = t / NP, qt = t % NP;
        f4 ma = {0.f, 0.f, 0.f, 0.f}, mt = ma;
        const int r = 16 * p + i16, s = 16 * qt + i16;
        const float bs = sB[s];
#pragma unroll 4
        for (int j0 = 0; j0 < V; j0 += 4) {
            const int j = j0 + g4;
            ma = mf(sO[r * LV + j], Vt[s * V + j], ma);
            mt = mf(dVt[r * V + j], bs * sVr[s * LV + j], mt);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            MA[row * BC + s] = ma[e];
            MT[row * BC + s] = mt[e];
        }
    }
    // T^T dVt: dv = beta T^T dVt, and its beta part rowsum(V T^T dVt)
    void *dv = a.dv;
    for (int t = w; t < NP * (V / 16); t += 4) {
        const int p = t / (V / 16), ct = t % (V / 16);
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        const int c = 16 * ct + i16;
        for (int s0 = 16 * p; s0 < BC; s0 += 4)
            acc = mf(Tm[(s0 + g4) * BC + 16 * p + i16], dVt[(s0 + g4) * V + c], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            if (row < cp.L) st_out(dv, a.grad_bf16, ((cp.t0 + row) * H + h) * V + c, sB[row] * acc[e]);
            const float part = row16_sum(sVr[row * LV + c] * acc[e]);
            if (i16 == 0) sRed[ct * BC + row] = part;
        }
    }
    // gamma_C's partner: rowsum(S dS') per key channel
    for (int c = tid; c < K; c += NTH) {
        float acc = 0.f;
        for (int j = 0; j < V; ++j) acc += hp[c * V + j] * dhp[c * V + j];
        a.w.rs[sh * K + c] = acc;
    }
    __syncthreads();
    if (tid < BC) {
        float acc = 0.f;
        for (int ct = 0; ct < V / 16; ++ct) acc += sRed[ct * BC + tid];
        a.w.dbv[sh * BC + tid] = acc;
    }
}

// ------------------------------------------------------------------------------------
// kgrads: everything in key space, one workgroup per (chunk slot, head)
template <int K>
struct KgLds {
    static constexpr int LK = K + 4;
    static constexpr size_t bytes = sizeof(float) * (3 * BC * LK + 3 * BC * LDC + BC + K + (K / 16) * BC + NP * BC);
};

template <typename TIn, int K, int V>
__global__ __launch_bounds__(NTH) void bwd_kgrads_kernel(BwdArgs a) {
    constexpr int LK = KgLds<K>::LK;
    constexpr int KT = K / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    float *sQ = reinterpret_cast<float *>(smem);
    float *sK = sQ + BC * LK;
    float *sG = sK + BC * LK;
    float *sT = sG + BC * LK;
    float *sM = sT + BC * LDC;   // dT, then beta dA
    float *sY = sM + BC * LDC;   // dT T^T
    float *sB = sY + BC * LDC;
    float *sE = sB + BC;
    float *sRk = sE + K;         // [K/16][BC] partial rowsum(K e^Gamma dBk)
    float *sRa = sRk + KT * BC;  // [NP][BC] partial rowsum(dA Abar)

    const int n = blockIdx.x, h = blockIdx.y, H = a.H;
    const ChunkPos cp = slot_chunk(n, a.cu_seqlens, a.num_seqs, a.T);
    if (cp.L == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, i16 = lane & 15;
    const int64_t sh = (int64_t)n * H + h;
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k);

    for (int i = tid; i < BC * K; i += NTH) {
        const int r = i / K, c = i % K;
        float qv = 0.f, kv = 0.f, gv = 0.f;
        if (r < cp.L) {
            const int64_t gi = ((cp.t0 + r) * H + h) * K + c;
            qv = ld_f32(q, gi);
            kv = ld_f32(k, gi);
            gv = gate_log(a.gate, gi);
        }
        sQ[r * LK + c] = qv;
        sK[r * LK + c] = kv;
        sG[r * LK + c] = gv;
    }
    if (tid < BC) sB[tid] = tid < cp.L ? a.beta[(cp.t0 + tid) * H + h] : 0.f;
    const float *Tm = a.w.Tm + sh * BC * BC;
    for (int i = tid; i < BC * BC; i += NTH) sT[(i / BC) * LDC + i % BC] = Tm[i];
    __syncthreads();
    if (tid < K) {
        float run = 0.f;
        for (int r = 0; r < BC; ++r) {
            run += sG[r * LK + tid];
            sG[r * LK + tid] = run;
        }
        sE[tid] = run;
    }

    // dT = dVt (beta V)^T + dW (beta K e^Gamma)^T, dW = -dVt S^T
    const float *PW = a.w.PW + sh * BC * K, *Kg = a.w.Kg + sh * BC * K, *MT = a.w.MT + sh * BC * BC;
    for (int t = w; t < NP * NP; t += 4) {
        const int p = t / NP, qt = t % NP;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * p + i16, s = 16 * qt + i16;
        const float bs = sB[s];
#pragma unroll 4
        for (int c0 = 0; c0 < K; c0 += 4) {
            const int c = c0 + g4;
            acc = mf(PW[r * K + c], bs * Kg[s * K + c], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            sM[row * LDC + s] = MT[row * BC + s] - acc[e];
        }
    }
    __syncthreads();
    // Y = dT T^T
    for (int t = w; t < NP * NP; t += 4) {
        const int p = t / NP, qt = t % NP;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * p + i16, s = 16 * qt + i16;
#pragma unroll 4
        for (int j0 = 0; j0 < BC; j0 += 4) acc = mf(sM[r * LDC + j0 + g4], sT[s * LDC + j0 + g4], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[(16 * p + 4 * g4 + e) * LDC + s] = acc[e];
    }
    __syncthreads();
    // dA = -strict_tril(T^T Y); rowsum(dA Abar) for dbeta; beta dA replaces dT
    const float *Abar = a.w.Abar + sh * BC * BC;
    for (int t = w; t < NP * NP; t += 4) {
        const int p = t / NP, qt = t % NP;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        const int s = 16 * qt + i16;
        if (qt <= p) {
#pragma unroll 4
            for (int j0 = 0; j0 < BC; j0 += 4)
                acc = mf(sT[(j0 + g4) * LDC + 16 * p + i16], sY[(j0 + g4) * LDC + s], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * p + 4 * g4 + e;
            const float da = row > s ? -acc[e] : 0.f;
            const float part = row16_sum(da * Abar[row * BC + s]);
            if (i16 == 0) sRa[qt * BC + row] = part;
            sM[row * LDC + s] = sB[row] * da;
        }
    }
    __syncthreads();

    // per owned C x K tile: dq, dk and the per-row terms of d ln alpha
    const float *PS = a.w.PS + sh * BC * K, *PdK = a.w.PdK + sh * BC * K, *MA = a.w.MA + sh * BC * BC;
    float *dGt = a.w.PS + sh * BC * K;   // overwritten element by element by its only reader
    float *eSt = a.w.PdK + sh * BC * K;
    for (int t = w; t < NP * KT; t += 4) {
        const int rt = t / KT, ct = t % KT;
        const int c = 16 * ct + i16;
        // T^T dW = -T^T (dVt S^T)
        f4 bk = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 16 * rt; s0 < BC; s0 += 4)
            bk = mf(sT[(s0 + g4) * LDC + 16 * rt + i16], PW[(s0 + g4) * K + c], bk);
        // row side of the decayed adjoints (rows of tile rt): A_qk -> dq, beta dA -> dk
        f4 xq = {0.f, 0.f, 0.f, 0.f}, xk = xq;
        {
            const float m = sG[(16 * rt + 7) * LK + c];
            const int r = 16 * rt + i16;
            for (int s0 = 0; s0 < 16 * rt + 16; s0 += 4) {
                const int s = s0 + g4;
                const float b = sK[s * LK + c] * expf(m - sG[s * LK + c]);
                const float ma = s <= r ? MA[r * BC + s] : 0.f;
                xq = mf(ma, b, xq);
                xk = mf(sM[r * LDC + s], b, xk);
            }
        }
        // column side (rows of tile rt as the later index s): sums over every row tile p >= rt
        f4 yq = {0.f, 0.f, 0.f, 0.f}, yk = yq;
        for (int p = rt; p < NP; ++p) {
            const float m = sG[(16 * p + 7) * LK + c];
            f4 aq = {0.f, 0.f, 0.f, 0.f}, akk = aq;
            const int s = 16 * rt + i16;
#pragma unroll
            for (int r0 = 0; r0 < 16; r0 += 4) {
                const int r = 16 * p + r0 + g4;
                const float er = expf(sG[r * LK + c] - m);
                const float ma = r >= s ? MA[r * BC + s] : 0.f;
                aq = mf(ma, sQ[r * LK + c] * er, aq);
                akk = mf(sM[r * LDC + s], sK[r * LK + c] * er, akk);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float fs = expf(m - sG[(16 * rt + 4 * g4 + e) * LK + c]);
                yq[e] += fs * aq[e];
                yk[e] += fs * akk[e];
            }
        }
        const float mr = sG[(16 * rt + 7) * LK + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * rt + 4 * g4 + e;
            const float G = sG[row * LK + c], eg = expf(G), kv = sK[row * LK + c], qv = sQ[row * LK + c];
            const float fr = expf(G - mr);
            const float dBk = -bk[e];
            const float dKW = sB[row] * eg * dBk;
            const float dQ = PS[row * K + c] * eg + fr * xq[e];
            const float dKS = PdK[row * K + c] * expf(sE[c] - G);
            const float dK1 = fr * xk[e];
            const float dK = yq[e] + dKS + dKW + dK1 + yk[e];
            dGt[row * K + c] = qv * dQ + kv * (dK1 + dKW - yq[e] - yk[e]);
            eSt[row * K + c] = kv * dKS;
            const float part = row16_sum(kv * eg * dBk);
            if (i16 == 0) sRk[ct * BC + row] = part;
            if (row < cp.L) {
                const int64_t gi = ((cp.t0 + row) * H + h) * K + c;
                st_out(a.dq, a.grad_bf16, gi, dQ);
                st_out(a.dk, a.grad_bf16, gi, dK);
            }
        }
    }
    __syncthreads();
    if (tid < cp.L) {
        float acc = a.w.dbv[sh * BC + tid];
        for (int ct = 0; ct < KT; ++ct) acc += sRk[ct * BC + tid];
        for (int qt = 0; qt < NP; ++qt) acc += sRa[qt * BC + tid];
        a.dbeta[(cp.t0 + tid) * H + h] = acc;
    }
    // d ln alpha per key channel: reverse in-chunk sum of the row terms, plus the
    // chunk-end terms gamma_C rowsum(S dS') and the exclusive forward sum of the Kd terms
    if (tid < K) {
        const int c = tid;
        float dl[BC];
        float f = a.w.gC[sh * K + c] * a.w.rs[sh * K + c];
#pragma unroll
        for (int r = 0; r < BC; ++r) {
            dl[r] = f;
            f += eSt[r * K + c];
        }
        float rv = 0.f;
#pragma unroll
        for (int r = BC - 1; r >= 0; --r) {
            rv += dGt[r * K + c];
            dl[r] += rv;
        }
#pragma unroll
        for (int r = 0; r < BC; ++r)
            if (r < cp.L) {
                const int64_t gi = ((cp.t0 + r) * H + h) * K + c;
                a.dgate[gi] = a.gate.mode == GATE_LOG ? dl[r] : dl[r] / a.gate.gate[gi];
            }
    }
}

template <int K, int V>
hipError_t set_lds(const void *kern, size_t bytes) {
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const BwdArgs &a, int num_seqs, hipStream_t stream) {
    static bool attr = false;  // per instantiation, once per process
    auto kprep = bwd_prep_kernel<TIn, K, V>;
    auto kvg = bwd_vgrads_kernel<TIn, K, V>;
    auto kkg = bwd_kgrads_kernel<TIn, K, V>;
    if (!attr) {
        hipError_t e = set_lds<K, V>(reinterpret_cast<const void *>(kprep), PrepLds<K>::bytes);
        if (e == hipSuccess) e = set_lds<K, V>(reinterpret_cast<const void *>(kvg), VgLds<V>::bytes);
        if (e == hipSuccess) e = set_lds<K, V>(reinterpret_cast<const void *>(kkg), KgLds<K>::bytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const dim3 gp(a.slots, a.H), gs(V / SBV, a.H, num_seqs);
    hipLaunchKernelGGL(kprep, gp, dim3(NTH), PrepLds<K>::bytes, stream, a);
    hipLaunchKernelGGL((bwd_states_kernel<K, V>), gs, dim3(NTH), 0, stream, a);
    hipLaunchKernelGGL((bwd_dstates_kernel<K, V>), gs, dim3(NTH), 0, stream, a);
    hipLaunchKernelGGL(kvg, gp, dim3(NTH), VgLds<V>::bytes, stream, a);
    hipLaunchKernelGGL(kkg, gp, dim3(NTH), KgLds<K>::bytes, stream, a);
    return hipGetLastError();
}

template <typename TIn, int K>
hipError_t launch_k(const BwdArgs &a, int V, int num_seqs, hipStream_t stream) {
    switch (V) {
        case 16: return launch_kv<TIn, K, 16>(a, num_seqs, stream);
        case 32: return launch_kv<TIn, K, 32>(a, num_seqs, stream);
        case 64: return launch_kv<TIn, K, 64>(a, num_seqs, stream);
        case 128: return launch_kv<TIn, K, 128>(a, num_seqs, stream);
    }
    return hipErrorNotSupported;
}

template <typename TIn>
hipError_t launch_t(const BwdArgs &a, int K, int V, int num_seqs, hipStream_t stream) {
    switch (K) {
        case 16: return launch_k<TIn, 16>(a, V, num_seqs, stream);
        case 32: return launch_k<TIn, 32>(a, V, num_seqs, stream);
        case 64: return launch_k<TIn, 64>(a, V, num_seqs, stream);
        case 128: return launch_k<TIn, 128>(a, V, num_seqs, stream);
    }
    return hipErrorNotSupported;
}

}  // namespace

int64_t chunk_bwd_slots(int B, int64_t T, int num_seqs, bool varlen) {
    return varlen ? T / BC + num_seqs : (int64_t)B * ((T + BC - 1) / BC);
}

size_t chunk_bwd_floats_per_slot(int K, int V) {
    return (size_t)7 * BC * K + (size_t)3 * BC * V + (size_t)5 * BC * BC + (size_t)2 * K * V + 2 * K + BC;
}

void chunk_bwd_carve(BwdWork &w, float *base, int64_t slot_heads, int K, int V) {
    const int64_t ck = slot_heads * BC * K, cv = slot_heads * BC * V, cc = slot_heads * BC * BC;
    const int64_t kv = slot_heads * K * V, kk = slot_heads * K, cb = slot_heads * BC;
    float *p = base;
    float **ck_arr[] = {&w.W, &w.Kd, &w.Qg, &w.Kg, &w.PS, &w.PdK, &w.PW};
    for (float **x : ck_arr) { *x = p; p += ck; }
    float **cv_arr[] = {&w.U, &w.Vt, &w.dVt};
    for (float **x : cv_arr) { *x = p; p += cv; }
    float **cc_arr[] = {&w.Aqk, &w.Tm, &w.Abar, &w.MA, &w.MT};
    for (float **x : cc_arr) { *x = p; p += cc; }
    w.h = p; p += kv;
    w.dh = p; p += kv;
    w.gC = p; p += kk;
    w.rs = p; p += kk;
    w.dbv = p;
    (void)cb;
}

hipError_t launch_chunk_bwd(const BwdArgs &a, bool fp32_inputs, int K, int V, int num_seqs, hipStream_t stream) {
    return fp32_inputs ? launch_t<float>(a, K, V, num_seqs, stream) : launch_t<__bf16>(a, K, V, num_seqs, stream);
}

}  // namespace kda
