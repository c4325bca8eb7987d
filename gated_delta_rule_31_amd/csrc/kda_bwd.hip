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
//   prep    (chunk, head) units, persistent, eight waves:
//                                  Gamma, Abar, T (blocked 16x16 inverse), A_qk, W, U, Kd, Q e^Gamma, K e^Gamma
//   states  (value block, head, seq) serial over chunks: keeps each chunk's start state and Vt
//   dstates (value block, head, seq) serial backwards: keeps each chunk's end-state gradient,
//                                  dVt, and writes the initial-state gradient
//   vgrads  (chunk, head), eight waves: the contractions over V, dT, dA and T^T dW; writes dv, dbeta
//   kgrads  (chunk, head, block of 32 key channels): the decayed adjoints; writes dq, dk, dgate
// The waves of a workgroup exchange data through LDS only (global memory is read, or
// written for later launches, never read back in the same kernel), so every workgroup
// barrier is an LDS-only barrier: global loads and stores stay in flight across it.
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

// gate values of four consecutive elements as log-decay (rows past the chunk: 0, no decay);
// a retention alpha goes through the hardware base-2 logarithm (1 ulp) times ln 2
__device__ __forceinline__ float ln_alpha(float x) { return __builtin_amdgcn_logf(x) * 0.69314718055994531f; }
__device__ __forceinline__ float4 gate_log4(const GateIn &g, float4 x, bool ok) {
    if (!ok) return make_float4(0.f, 0.f, 0.f, 0.f);
    if (g.mode == GATE_LOG) return x;
    return make_float4(ln_alpha(x.x), ln_alpha(x.y), ln_alpha(x.z), ln_alpha(x.w));
}

// Workgroups go to the 8 XCDs round-robin by block index, and each XCD has its own L2.
// Block b is mapped to (unit, sub) so that the nsub blocks of one unit, which read the same
// per-chunk data, run on the same XCD one after another: the grid is 8 * nsub * ceil(units / 8)
// blocks and a unit index past the last unit has no work.
__device__ __forceinline__ void xcd_map(int b, int nsub, int &unit, int &sub) {
    const int x = b & 7, j = b >> 3;
    sub = j % nsub;
    unit = (j / nsub) * 8 + x;
}

// four consecutive elements as float (16-byte / 8-byte aligned loads)
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 ld4(const __bf16 *p) {
    const s16x4 x = *reinterpret_cast<const s16x4 *>(p);
    return make_float4(__builtin_bit_cast(float, (uint32_t)(uint16_t)x[0] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[1] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[2] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[3] << 16));
}
// Four elements of a tensor given in either format, without a branch: both loads are issued
// (the unused one reads the tensor's first four elements, valid for any tensor of at least 16
// bytes) and the wanted value is selected.  A branch per format would wait for the load
// inside it, and with it for every load issued before.
__device__ __forceinline__ float4 ld4_any(const void *p, int is_bf16, int64_t i) {
    const float4 f = ld4(static_cast<const float *>(p) + (is_bf16 ? 0 : i));
    const float4 b = ld4(static_cast<const __bf16 *>(p) + (is_bf16 ? i : 0));
    return is_bf16 ? b : f;
}
__device__ __forceinline__ void st4(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }
__device__ __forceinline__ void st2(float *p, float2 x) { *reinterpret_cast<float2 *>(p) = x; }
// two consecutive elements as float (8-byte / 4-byte aligned loads)
__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }
__device__ __forceinline__ float2 ld2(const __bf16 *p) {
    const uint32_t x = *reinterpret_cast<const uint32_t *>(p);
    return make_float2(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, x & 0xffff0000u));
}
// two elements of a tensor given in either format, without a branch (as ld4_any)
__device__ __forceinline__ float2 ld2_any(const void *p, int is_bf16, int64_t i) {
    const float2 f = ld2(static_cast<const float *>(p) + (is_bf16 ? 0 : i));
    const float2 b = ld2(static_cast<const __bf16 *>(p) + (is_bf16 ? i : 0));
    return is_bf16 ? b : f;
}
// e^x for |x| <= 40 (a log-decay difference inside one 16-row tile): the hardware base-2
// exponential of x log2(e); the rounding of the product adds at most 3e-6 relative error
__device__ __forceinline__ float exp_in_tile(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
// four loaded elements as float: float4 as is, bf16 by widening
__device__ __forceinline__ float4 raw_f4(float4 x) { return x; }
__device__ __forceinline__ float4 raw_f4(s16x4 x) {
    return make_float4(__builtin_bit_cast(float, (uint32_t)(uint16_t)x[0] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[1] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[2] << 16),
                       __builtin_bit_cast(float, (uint32_t)(uint16_t)x[3] << 16));
}

// Loads are issued from addresses that are always valid (rows past the chunk read its last
// row) and masked where the value is used: a load under a per-lane condition is compiled
// into its own branch with a wait for it, which would serialise a batch of loads.
__device__ __forceinline__ int crow(int r, int L) { return r < L ? r : L - 1; }
__device__ __forceinline__ float4 mask4(float4 x, bool ok) { return ok ? x : make_float4(0.f, 0.f, 0.f, 0.f); }

// (row16_sum, the DPP sum over one 16-lane row of an accumulator tile, is in kda_device.h)

// ------------------------------------------------------------------------------------
// prep: per (chunk slot, head) unit.  After the in-chunk cumulative sum, Gamma is
// replaced in LDS by F1 = e^{Gamma - m_tile} (m_p: Gamma at the middle row of row tile p);
// every decay factor is then a product of F1, its reciprocal and per-channel tables
// (e^{m_p - m_q}, e^{m_p}, e^{Gamma_C - m_p}), so no exponential is taken in the products.
template <int K, int V>
struct PrepLds {
    static constexpr int LK = K + 4;                 // q, k, F1: 16-row fragment reads
    // beta K e^Gamma, beta v: read as B fragments whose rows are 4 apart (k = 16 m + 4 (lane/16) + u),
    // which a row stride of 4 mod 16 words keeps on distinct banks
    static constexpr int LW = K + 4, LV = V + 4;
    static constexpr int R0 = 3 * BC * LK, RW = BC * LW + BC * LV;
    static constexpr int R = R0 > RW ? R0 : RW;
    static constexpr int TAB = (NP * NP + 3 * NP) * K;
    static constexpr size_t bytes = sizeof(float) * (R + 2 * BC * LDC + BC + TAB + K);
};

// Persistent: workgroup b takes the (chunk slot, head) units b, b + G, b + 2G, ... (G the
// grid size, one workgroup of eight waves per CU: LDS allows no more) and loads the next
// unit's q, k, gate and beta while it processes the current one.
constexpr int PNW = 8, PNT = 64 * PNW;  // prep waves and threads
template <typename TIn, int K, int V>
__global__ __launch_bounds__(PNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_prep_kernel(BwdArgs a) {
    constexpr int LK = PrepLds<K, V>::LK, LW = PrepLds<K, V>::LW, LV = PrepLds<K, V>::LV;
    constexpr int NV4 = (BC * V / 4 + PNT - 1) / PNT;  // float4 groups of v per thread
    constexpr int NK4 = (BC * K / 4 + PNT - 1) / PNT;  // float4 groups of a C x K tile per thread
    extern __shared__ __align__(16) unsigned char smem[];
    float *sQ = reinterpret_cast<float *>(smem);     // q
    float *sK = sQ + BC * LK;                          // k
    float *sG = sK + BC * LK;                          // log-decay, Gamma, then F1
    float *sW = reinterpret_cast<float *>(smem);     // beta K e^Gamma  (after the element-wise phase)
    float *sBV = sW + BC * LW;                         // beta v          (after the element-wise phase)
    float *sA = reinterpret_cast<float *>(smem) + PrepLds<K, V>::R;  // Abar
    float *sT = sA + BC * LDC;                         // T
    float *sB = sT + BC * LDC;                         // beta
    float *sEpq = sB + BC;                             // [NP][NP][K] e^{m_p - m_q}
    float *sEm = sEpq + NP * NP * K;                   // [NP][K] e^{m_p}
    float *sEe = sEm + NP * K;                         // [NP][K] e^{Gamma_C - m_p}
    float *sMid = sEe + NP * K;                        // [NP][K] m_p
    float *sE = sMid + NP * K;                         // [K] Gamma_C

    const int H = a.H;
    const int units = a.slots * H;  // below 2^31 (checked by the host)
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k);
    const TIn *v = static_cast<const TIn *>(a.v);
    // q, k, gate and beta of the next unit (four elements per load; rows past the chunk
    // read its last row and are masked when stored), kept in the input format until then
    using Raw4 = typename std::conditional<std::is_same<TIn, float>::value, float4, s16x4>::type;
    Raw4 rq[NK4], rk[NK4];
    float4 rg[NK4];
    float rb = 0.f;
    // Unconditional, so that the loads land directly in the registers the next iteration
    // reads (a load under a condition would be merged through copies that wait for it);
    // an unused slot, or a unit past the last one, reads row 0.
    auto fetch = [&](int un, ChunkPos c) {
        const int h = un % H, tid = threadIdx.x;
        if (c.L == 0) c = ChunkPos{0, 1};
#pragma unroll
        for (int i = 0; i < NK4; ++i) {
            const int idx = min(tid + PNT * i, BC * K / 4 - 1), r = (4 * idx) / K, col = (4 * idx) % K;
            const int64_t gi = ((c.t0 + crow(r, c.L)) * H + h) * K + col;
            rq[i] = *reinterpret_cast<const Raw4 *>(q + gi);
            rk[i] = *reinterpret_cast<const Raw4 *>(k + gi);
            rg[i] = ld4(a.gate.gate + gi);
        }
        rb = a.beta[(c.t0 + crow(tid & (BC - 1), c.L)) * H + h];
    };
    int unit = blockIdx.x;
    ChunkPos cpn = {0, 0};
    if (unit < units) cpn = slot_chunk(unit / H, a.cu_seqlens, a.num_seqs, a.T);
    fetch(unit, cpn);
    for (; unit < units; unit += gridDim.x) {
    // The thread index is re-read in every iteration through an opaque copy, so that the
    // compiler does not hoist the unit's many index computations out of the loop and keep
    // them all in registers.
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 4, i16 = lane & 15;
    const ChunkPos cp = cpn;
    const int n = unit / H, h = unit % H;
    const int un = unit + (int)gridDim.x;
    cpn = un < units ? slot_chunk(un / H, a.cu_seqlens, a.num_seqs, a.T) : ChunkPos{0, 0};
    if (cp.L == 0) {  // an unused slot (uniform): only the next unit's loads
        fetch(un, cpn);
        continue;
    }
    const int64_t sh = (int64_t)n * H + h;
    Raw4 rv[NV4];  // this chunk's v, in flight (in the input format) until U is formed
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int idx = min(tid + PNT * i, BC * V / 4 - 1), r = (4 * idx) / V, c = (4 * idx) % V;
        rv[i] = *reinterpret_cast<const Raw4 *>(v + ((cp.t0 + crow(r, cp.L)) * H + h) * V + c);
    }
#pragma unroll
    for (int i = 0; i < NK4; ++i) {  // rows past the chunk: no token, no decay
        const int idx = tid + PNT * i, r = (4 * idx) / K, c = (4 * idx) % K;
        if (idx < BC * K / 4) {
            st4(sQ + r * LK + c, mask4(raw_f4(rq[i]), r < cp.L));
            st4(sK + r * LK + c, mask4(raw_f4(rk[i]), r < cp.L));
            st4(sG + r * LK + c, gate_log4(a.gate, rg[i], r < cp.L));
        }
    }
    if (tid < BC) sB[tid] = tid < cp.L ? rb : 0.f;
    lds_barrier();
    fetch(un, cpn);  // in flight while this unit is processed
    {
        // Gamma: inclusive prefix sums over the chunk's rows per channel, in NSEG segments of
        // SEG rows (each read into registers at once), offset by the earlier segments' totals
        constexpr int NSEG = PNT / K < BC ? PNT / K : BC, SEG = BC / NSEG;
        const int c = tid % K, sg = tid / K;
        float x[SEG];
        if (sg < NSEG) {
#pragma unroll
            for (int j = 0; j < SEG; ++j) x[j] = sG[(sg * SEG + j) * LK + c];
#pragma unroll
            for (int j = 1; j < SEG; ++j) x[j] += x[j - 1];
            sA[sg * K + c] = x[SEG - 1];  // segment totals (sA is free until the A tiles)
        }
        lds_barrier();
        if (sg < NSEG) {
            float off = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < NSEG - 1; ++s2)
                if (s2 < sg) off += sA[s2 * K + c];
#pragma unroll
            for (int j = 0; j < SEG; ++j) sG[(sg * SEG + j) * LK + c] = x[j] + off;
            if (sg == NSEG - 1) {
                sE[c] = x[SEG - 1] + off;
                a.w.gC[sh * K + c] = expf(x[SEG - 1] + off);
            }
        }
    }
    lds_barrier();
    for (int i = tid; i < (NP * NP + 3 * NP) * K; i += PNT) {
        const int c = i % K, j = i / K;
        if (j < NP * NP) {
            const int pp = j / NP, qq = j % NP;
            sEpq[j * K + c] = qq <= pp ? expf(sG[(16 * pp + 7) * LK + c] - sG[(16 * qq + 7) * LK + c]) : 0.f;
        } else if (j < NP * NP + NP) {
            sEm[(j - NP * NP) * K + c] = expf(sG[(16 * (j - NP * NP) + 7) * LK + c]);
        } else if (j < NP * NP + 2 * NP) {
            const int pp = j - NP * NP - NP;
            sEe[pp * K + c] = expf(sE[c] - sG[(16 * pp + 7) * LK + c]);
        } else {
            const int pp = j - NP * NP - 2 * NP;
            sMid[pp * K + c] = sG[(16 * pp + 7) * LK + c];
        }
    }
    lds_barrier();
    for (int i = tid; i < BC * K; i += PNT) {  // F1 replaces Gamma, element by element
        const int r = i / K, c = i % K;
        sG[r * LK + c] = exp_in_tile(sG[r * LK + c] - sMid[(r >> 4) * K + c]);
    }
    lds_barrier();
    float *sF1 = sG;

    // Abar (strictly lower) and A_qk (lower): the ten tiles on or below the diagonal, spread
    // over the waves.  Row r of tile p enters as k_r F1_r (q_r F1_r); column s of tile q as
    // k_s / F1_s * e^{m_p - m_q}; the channel axis is read four at a time.
    float *Aqk = a.w.Aqk + sh * BC * BC, *Abar = a.w.Abar + sh * BC * BC;
    for (int t = w; t < NP * (NP + 1) / 2; t += PNW) {
        int p = 0;
        while ((p + 1) * (p + 2) / 2 <= t) ++p;
        const int qt = t - p * (p + 1) / 2;
        f4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
        const int r = 16 * p + i16, sc = 16 * qt + i16;
        const float *e = sEpq + (p * NP + qt) * K + 4 * g4;
#pragma unroll 2
        for (int c0 = 0; c0 < K; c0 += 16) {
            const float4 f1r = *reinterpret_cast<const float4 *>(sF1 + r * LK + c0 + 4 * g4);
            const float4 kr = *reinterpret_cast<const float4 *>(sK + r * LK + c0 + 4 * g4);
            const float4 qr = *reinterpret_cast<const float4 *>(sQ + r * LK + c0 + 4 * g4);
            const float4 f1s = *reinterpret_cast<const float4 *>(sF1 + sc * LK + c0 + 4 * g4);
            const float4 ks = *reinterpret_cast<const float4 *>(sK + sc * LK + c0 + 4 * g4);
            const float4 ep = *reinterpret_cast<const float4 *>(e + c0);
            const float b0 = ks.x * __builtin_amdgcn_rcpf(f1s.x) * ep.x, b1 = ks.y * __builtin_amdgcn_rcpf(f1s.y) * ep.y;
            const float b2 = ks.z * __builtin_amdgcn_rcpf(f1s.z) * ep.z, b3 = ks.w * __builtin_amdgcn_rcpf(f1s.w) * ep.w;
            ak = mf(kr.x * f1r.x, b0, ak);
            aq = mf(qr.x * f1r.x, b0, aq);
            ak = mf(kr.y * f1r.y, b1, ak);
            aq = mf(qr.y * f1r.y, b1, aq);
            ak = mf(kr.z * f1r.z, b2, ak);
            aq = mf(qr.z * f1r.z, b2, aq);
            ak = mf(kr.w * f1r.w, b3, ak);
            aq = mf(qr.w * f1r.w, b3, aq);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * p + 4 * g4 + u, col = 16 * qt + i16;
            const float vk = row > col ? ak[u] : 0.f;  // selects: masked entries may be inf
            const float vq = row >= col ? aq[u] : 0.f;
            sA[row * LDC + col] = vk;
            Abar[row * BC + col] = vk;
            Aqk[row * BC + col] = vq;
        }
    }
    for (int i = tid; i < BC * BC; i += PNT) {  // the tiles above the diagonal are zero
        const int r = i / BC, c = i % BC;
        if ((c >> 4) > (r >> 4)) {
            sA[r * LDC + c] = 0.f;
            sT[r * LDC + c] = 0.f;
            Abar[i] = 0.f;
            Aqk[i] = 0.f;
        }
    }
    lds_barrier();

    // T = (I + diag(beta) Abar)^-1: diagonal 16x16 blocks by the blocked inverse, then
    // block forward substitution T_pq = -T_pp sum_{q<=u<p} A_pu T_uq
    if (w < NP) {
        const int pb = w;
        f4 av;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * pb + 4 * g4 + u;
            av[u] = sB[row] * sA[row * LDC + 16 * pb + i16];
        }
        const f4 tb = unit_lower_inverse16<float>(av, lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) sT[(16 * pb + 4 * g4 + u) * LDC + 16 * pb + i16] = tb[u];
    }
    lds_barrier();
    for (int pb = 1; pb < NP; ++pb) {
        if (w < pb) {
            const int qb = w;
            f4 x = {0.f, 0.f, 0.f, 0.f};
            for (int u = qb; u < pb; ++u) {
#pragma unroll
                for (int s0 = 0; s0 < 16; s0 += 4) {
                    const int r = 16 * pb + i16, sc = 16 * u + s0 + g4;
                    x = mf(sB[r] * sA[r * LDC + sc], sT[sc * LDC + 16 * qb + i16], x);
                }
            }
            f4 xr;  // row-operand form of T_pp: lane (g, r) holds T_pp[r][4g + s]
#pragma unroll
            for (int u = 0; u < 4; ++u) xr[u] = sT[(16 * pb + i16) * LDC + 16 * pb + 4 * g4 + u];
            const f4 y = mma16_reg<float>(xr, x);
#pragma unroll
            for (int u = 0; u < 4; ++u) sT[(16 * pb + 4 * g4 + u) * LDC + 16 * qb + i16] = -y[u];
        }
        lds_barrier();
    }

    // element-wise products: e^Gamma = F1 e^{m_p}, e^{Gamma_C - Gamma} = e^{Gamma_C - m_p} / F1
    float *Qg = a.w.Qg + sh * BC * K, *Kd = a.w.Kd + sh * BC * K, *Kg = a.w.Kg + sh * BC * K;
    float4 bkg[NK4];
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
        const int idx = tid + PNT * i, r = (4 * idx) / K, c = (4 * idx) % K;
        if (idx < BC * K / 4) {
            const int pp = r >> 4;
            const float4 f1 = *reinterpret_cast<const float4 *>(sF1 + r * LK + c);
            const float4 kv = *reinterpret_cast<const float4 *>(sK + r * LK + c);
            const float4 qv = *reinterpret_cast<const float4 *>(sQ + r * LK + c);
            const float4 em = *reinterpret_cast<const float4 *>(sEm + pp * K + c);
            const float4 ee = *reinterpret_cast<const float4 *>(sEe + pp * K + c);
            const float4 eg = make_float4(f1.x * em.x, f1.y * em.y, f1.z * em.z, f1.w * em.w);
            const float4 ed = make_float4(ee.x * __builtin_amdgcn_rcpf(f1.x), ee.y * __builtin_amdgcn_rcpf(f1.y),
                                          ee.z * __builtin_amdgcn_rcpf(f1.z), ee.w * __builtin_amdgcn_rcpf(f1.w));
            const float4 kg = make_float4(kv.x * eg.x, kv.y * eg.y, kv.z * eg.z, kv.w * eg.w);
            st4(Qg + r * K + c, make_float4(qv.x * eg.x, qv.y * eg.y, qv.z * eg.z, qv.w * eg.w));
            st4(Kd + r * K + c, make_float4(kv.x * ed.x, kv.y * ed.y, kv.z * ed.z, kv.w * ed.w));
            st4(Kg + r * K + c, kg);
            const float b = sB[r];
            bkg[i] = make_float4(b * kg.x, b * kg.y, b * kg.z, b * kg.w);
        }
    }
    float *Tm = a.w.Tm + sh * BC * BC;
    for (int i = tid; i < BC * BC / 4; i += PNT) {
        const int e = 4 * i;
        st4(Tm + e, *reinterpret_cast<const float4 *>(sT + (e / BC) * LDC + e % BC));
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NK4; ++i) {  // q, k and F1 are consumed: their LDS takes beta K e^Gamma
        const int idx = tid + PNT * i, r = (4 * idx) / K, c = (4 * idx) % K;
        if (idx < BC * K / 4) st4(sW + r * LW + c, bkg[i]);
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {  // and beta v (beta is zero past the chunk)
        const int idx = tid + PNT * i, r = (4 * idx) / V, c = (4 * idx) % V;
        if (idx < BC * V / 4) {
            const float b = sB[r];
            const float4 x = raw_f4(rv[i]);
            st4(sBV + r * LV + c, make_float4(b * x.x, b * x.y, b * x.z, b * x.w));
        }
    }
    lds_barrier();

    // W = T (beta K e^Gamma), U = T (beta V); T is lower triangular.  Wave w owns the
    // column tiles w, w + 8, ... of W and of U over all four row tiles, so one read of a
    // T fragment serves every column tile and one B read every row tile; the reduction
    // runs in 16-row groups m with k = 16 m + 4 (lane / 16) + u, and group m only feeds
    // row tiles p >= m.
    constexpr int NWT = (K / 16 + PNW - 1) / PNW, NUT = (V / 16 + PNW - 1) / PNW;
    float *W = a.w.W + sh * BC * K, *U = a.w.U + sh * BC * V;
    f4 aw[NP][NWT], au[NP][NUT];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
#pragma unroll
        for (int i = 0; i < NWT; ++i) aw[pp][i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NUT; ++i) au[pp][i] = f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        float4 ta[NP];
#pragma unroll
        for (int pp = m; pp < NP; ++pp)
            ta[pp] = *reinterpret_cast<const float4 *>(sT + (16 * pp + i16) * LDC + 16 * m + 4 * g4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 16 * m + 4 * g4 + u;
            float bw[NWT], bu[NUT];
#pragma unroll
            for (int i = 0; i < NWT; ++i) bw[i] = sW[r * LW + 16 * min(w + PNW * i, K / 16 - 1) + i16];
#pragma unroll
            for (int i = 0; i < NUT; ++i) bu[i] = sBV[r * LV + 16 * min(w + PNW * i, V / 16 - 1) + i16];
#pragma unroll
            for (int pp = m; pp < NP; ++pp) {
                const float av = u == 0 ? ta[pp].x : u == 1 ? ta[pp].y : u == 2 ? ta[pp].z : ta[pp].w;
#pragma unroll
                for (int i = 0; i < NWT; ++i) aw[pp][i] = mf(av, bw[i], aw[pp][i]);
#pragma unroll
                for (int i = 0; i < NUT; ++i) au[pp][i] = mf(av, bu[i], au[pp][i]);
            }
        }
    }
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
#pragma unroll
        for (int i = 0; i < NWT; ++i) {
            const int ct = w + PNW * i;
            if (ct < K / 16) {
#pragma unroll
                for (int u = 0; u < 4; ++u) W[(16 * pp + 4 * g4 + u) * K + 16 * ct + i16] = aw[pp][i][u];
            }
        }
#pragma unroll
        for (int i = 0; i < NUT; ++i) {
            const int ct = w + PNW * i;
            if (ct < V / 16) {
#pragma unroll
                for (int u = 0; u < 4; ++u) U[(16 * pp + 4 * g4 + u) * V + 16 * ct + i16] = au[pp][i][u];
            }
        }
    }
    lds_barrier();  // this unit's LDS is consumed before the next unit's inputs are stored
    }
}

// ------------------------------------------------------------------------------------
// states: the forward over chunks, one workgroup per (value block, head, sequence).
// A chunk step has two phases: the pseudo-values Vt = U - W S (wave w: rows of tile w),
// then S = gamma_C S + Kd^T Vt (wave w: key tiles w, w + 4, ...).  Each phase's matrix
// operands go straight from memory into registers in fragment order (the reduction index
// permuted as k = 16 q + 4 (lane / 16) + s on both operands), and each wave loads one
// phase's operands while the other phase computes.
constexpr int SBV = 16;  // value columns per workgroup in the serial passes

template <int K, int V>
// (three workgroups per CU)
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(3, 3))) void bwd_states_kernel(BwdArgs a) {
    constexpr int LB = SBV + 4, KQ = K / 16, NST = (K / 16 + 3) / 4;
    __shared__ __align__(16) float sS[K * LB];
    __shared__ float sV[BC * LB];
    int hs, vb;  // (sequence, head) unit; the value blocks of one unit share an XCD
    xcd_map(blockIdx.x, V / SBV, hs, vb);
    const int H = a.H;
    if (hs >= a.num_seqs * H) return;
    const int h = hs % H, s = hs / H;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 4, i16 = lane & 15;
    const int j0 = vb * SBV, p = w;
    int64_t t0, len;
    int base;
    seq_range(s, a.cu_seqlens, a.T, t0, len, base);
    const int nch = (int)((len + BC - 1) / BC);
    {
        constexpr int N4 = (K * SBV / 4 + NTH - 1) / NTH;
        float4 x[N4];
#pragma unroll
        for (int i = 0; i < N4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / SBV, c = (4 * idx) % SBV;
            x[i] = (idx < K * SBV / 4 && a.initial_state)
                       ? ld4(a.initial_state + (((int64_t)s * H + h) * K + r) * V + j0 + c)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < N4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / SBV, c = (4 * idx) % SBV;
            if (idx < K * SBV / 4) st4(sS + r * LB + c, x[i]);
        }
    }
    float4 wf[KQ];
    float uf[4], kdf[NST][16], gcf[NST][4];
    auto loadA = [&](int64_t sh) {  // W rows of tile p, U on the tile's outputs
        const float *W = a.w.W + sh * BC * K + (16 * p + i16) * K + 4 * g4;
#pragma unroll
        for (int q = 0; q < KQ; ++q) wf[q] = ld4(W + 16 * q);
        const float *U = a.w.U + sh * BC * V + j0 + i16;
#pragma unroll
        for (int e = 0; e < 4; ++e) uf[e] = U[(16 * p + 4 * g4 + e) * V];
    };
    auto loadB = [&](int64_t sh) {  // Kd columns of this wave's key tiles, gamma_C on their rows
        const float *Kd = a.w.Kd + sh * BC * K, *gC = a.w.gC + sh * K;
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int rt = w + 4 * i;
            if (rt < K / 16) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u) kdf[i][4 * q + u] = Kd[(16 * q + 4 * g4 + u) * K + 16 * rt + i16];
#pragma unroll
                for (int e = 0; e < 4; ++e) gcf[i][e] = gC[16 * rt + 4 * g4 + e];
            }
        }
    };
    if (nch > 0) loadA((int64_t)base * H + h);
    for (int j = 0; j < nch; ++j) {
        const int64_t sh = (int64_t)(base + j) * H + h;
        loadB(sh);
        lds_barrier();
        float *hp = a.w.h + sh * K * V;
        for (int i = tid; i < K * SBV / 4; i += NTH) {
            const int r = (4 * i) / SBV, c = (4 * i) % SBV;
            st4(hp + r * V + j0 + c, *reinterpret_cast<const float4 *>(sS + r * LB + c));
        }
        {
            // two accumulators (even and odd key tiles), so consecutive products overlap
            f4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int q = 0; q < KQ; ++q) {
                const float *b = sS + (16 * q + 4 * g4) * LB + i16;
                acc[q & 1] = mf(wf[q].x, b[0], acc[q & 1]);
                acc[q & 1] = mf(wf[q].y, b[LB], acc[q & 1]);
                acc[q & 1] = mf(wf[q].z, b[2 * LB], acc[q & 1]);
                acc[q & 1] = mf(wf[q].w, b[3 * LB], acc[q & 1]);
            }
            float *Vt = a.w.Vt + sh * BC * V + j0 + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * p + 4 * g4 + e;
                const float vt = uf[e] - (acc[0][e] + acc[1][e]);
                sV[row * LB + i16] = vt;
                Vt[row * V] = vt;
            }
        }
        lds_barrier();
        if (j + 1 < nch) loadA(sh + H);
        {
            // this wave's key tiles side by side, so their products overlap
            float bv[16];  // the pseudo-value column of this lane, read before the products
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) bv[4 * q + u] = sV[(16 * q + 4 * g4 + u) * LB + i16];
            __builtin_amdgcn_sched_barrier(0);
            f4 acc[NST];
#pragma unroll
            for (int i = 0; i < NST; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < 16; ++x)
#pragma unroll
                for (int i = 0; i < NST; ++i)
                    if (w + 4 * i < K / 16) acc[i] = mf(kdf[i][x], bv[x], acc[i]);
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const int rt = w + 4 * i;
                if (rt < K / 16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * rt + 4 * g4 + e;
                        sS[m * LB + i16] = gcf[i][e] * sS[m * LB + i16] + acc[i][e];
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// dstates: the reverse over chunks, the same two-phase structure:
//   dVt = Kd dS' + A_qk^T dO (wave w: rows of tile w),
//   dS  = gamma_C dS' + Qg^T dO - W^T dVt (wave w: key tiles w, w + 4, ...)
// on DBV value columns per workgroup (the prefetched fragments serve every column tile).
template <int V>
struct DstCfg {
    static constexpr int DBV = V < 32 ? V : 32, NCT = DBV / 16;
};

template <int K, int V>
// (two workgroups per CU: the register allocation stays within half a SIMD's file)
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dstates_kernel(BwdArgs a) {
    constexpr int DBV = DstCfg<V>::DBV, NCT = DstCfg<V>::NCT;
    constexpr int LB = DBV + 4, KQ = K / 16, NST = (K / 16 + 3) / 4;
    __shared__ __align__(16) float sD[K * LB];
    __shared__ float sO[BC * LB];
    __shared__ float sV[BC * LB];
    int hs, vb;
    xcd_map(blockIdx.x, V / DBV, hs, vb);
    const int H = a.H;
    if (hs >= a.num_seqs * H) return;
    const int h = hs % H, s = hs / H;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 4, i16 = lane & 15;
    const int j0 = vb * DBV, p = w;
    int64_t t0, len;
    int base;
    seq_range(s, a.cu_seqlens, a.T, t0, len, base);
    const int nch = (int)((len + BC - 1) / BC);
    const int64_t st = ((int64_t)s * H + h) * K;
    static_assert(BC * DBV / 4 % NTH == 0, "whole float4 groups per thread");
    {
        constexpr int N4 = (K * DBV / 4 + NTH - 1) / NTH;
        float4 x[N4];
        if (a.d_final_state) {
#pragma unroll
            for (int i = 0; i < N4; ++i) {
                const int idx = min(tid + NTH * i, K * DBV / 4 - 1), r = (4 * idx) / DBV, c = (4 * idx) % DBV;
                x[i] = ld4(a.d_final_state + (st + r) * V + j0 + c);
            }
        } else {
#pragma unroll
            for (int i = 0; i < N4; ++i) x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < N4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / DBV, c = (4 * idx) % DBV;
            if (idx < K * DBV / 4) st4(sD + r * LB + c, x[i]);
        }
    }
    constexpr int NO4 = BC * DBV / 4 / NTH;  // dO staging: float4 groups per thread
    float4 kdf[KQ], dof[NO4];
    bool dok[NO4];
    float aqf[16], qgf[NST][16], wwf[NST][16], gcf[NST][4];
    auto loadA = [&](int j) {  // Kd rows and A_qk columns of tile p, and this chunk's dO block
        const int64_t sh = (int64_t)(base + j) * H + h;
        const float *Kd = a.w.Kd + sh * BC * K + (16 * p + i16) * K + 4 * g4;
#pragma unroll
        for (int q = 0; q < KQ; ++q) kdf[q] = ld4(Kd + 16 * q);
        const float *Aqk = a.w.Aqk + sh * BC * BC + 16 * p + i16;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) aqf[4 * q + u] = Aqk[(16 * q + 4 * g4 + u) * BC];  // used for q >= p
        const int64_t tc = t0 + (int64_t)j * BC;
        const int L = (int)min((int64_t)BC, len - (int64_t)j * BC);
#pragma unroll
        for (int i = 0; i < NO4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / DBV, c = (4 * idx) % DBV;
            dof[i] = ld4_any(a.d_out, a.dout_bf16, ((tc + crow(r, L)) * H + h) * V + j0 + c);
            dok[i] = r < L;
        }
    };
    auto loadB = [&](int j) {  // Qg and W columns of this wave's key tiles, gamma_C on their rows
        const int64_t sh = (int64_t)(base + j) * H + h;
        const float *Qg = a.w.Qg + sh * BC * K, *W = a.w.W + sh * BC * K, *gC = a.w.gC + sh * K;
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int rt = min(w + 4 * i, K / 16 - 1);  // a wave with no second tile reloads its first
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = 16 * q + 4 * g4 + u;
                    qgf[i][4 * q + u] = Qg[r * K + 16 * rt + i16];
                    wwf[i][4 * q + u] = W[r * K + 16 * rt + i16];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) gcf[i][e] = gC[16 * rt + 4 * g4 + e];
        }
    };
    if (nch > 0) loadA(nch - 1);
    for (int j = nch - 1; j >= 0; --j) {
        const int64_t sh = (int64_t)(base + j) * H + h;
        loadB(j);
        lds_barrier();
        float *dhp = a.w.dh + sh * K * V;
        for (int i = tid; i < K * DBV / 4; i += NTH) {
            const int r = (4 * i) / DBV, c = (4 * i) % DBV;
            st4(dhp + r * V + j0 + c, *reinterpret_cast<const float4 *>(sD + r * LB + c));
        }
        const float sc = a.scale;
#pragma unroll
        for (int i = 0; i < NO4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / DBV, c = (4 * idx) % DBV;
            const float f = dok[i] ? sc : 0.f;
            st4(sO + r * LB + c, make_float4(f * dof[i].x, f * dof[i].y, f * dof[i].z, f * dof[i].w));
        }
        lds_barrier();
        {
            f4 acc[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < KQ; ++q) {
                const float *b = sD + (16 * q + 4 * g4) * LB + i16;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    acc[ct] = mf(kdf[q].x, b[16 * ct], acc[ct]);
                    acc[ct] = mf(kdf[q].y, b[16 * ct + LB], acc[ct]);
                    acc[ct] = mf(kdf[q].z, b[16 * ct + 2 * LB], acc[ct]);
                    acc[ct] = mf(kdf[q].w, b[16 * ct + 3 * LB], acc[ct]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= p) {  // A_qk[s][r] is zero for s < r
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
                            acc[ct] = mf(aqf[4 * q + u], sO[(16 * q + 4 * g4 + u) * LB + 16 * ct + i16], acc[ct]);
                }
            }
            float *dVt = a.w.dVt + sh * BC * V + j0 + i16;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * p + 4 * g4 + e;
                    sV[row * LB + 16 * ct + i16] = acc[ct][e];
                    dVt[row * V + 16 * ct] = acc[ct][e];
                }
        }
        lds_barrier();
        if (j > 0) loadA(j - 1);
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int rt = w + 4 * i;
            if (rt < K / 16) {
                f4 acc[NCT], neg[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc[ct] = neg[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 16 * q + 4 * g4 + u;
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            acc[ct] = mf(qgf[i][4 * q + u], sO[r * LB + 16 * ct + i16], acc[ct]);
                            neg[ct] = mf(wwf[i][4 * q + u], sV[r * LB + 16 * ct + i16], neg[ct]);
                        }
                    }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * rt + 4 * g4 + e, col = 16 * ct + i16;
                        sD[m * LB + col] = gcf[i][e] * sD[m * LB + col] + acc[ct][e] - neg[ct][e];
                    }
            }
        }
    }
    lds_barrier();
    if (a.d_initial_state)
        for (int i = tid; i < K * DBV / 4; i += NTH) {
            const int r = (4 * i) / DBV, c = (4 * i) % DBV;
            st4(a.d_initial_state + (st + r) * V + j0 + c, *reinterpret_cast<const float4 *>(sD + r * LB + c));
        }
}

// ------------------------------------------------------------------------------------
// vgrads: contractions over the value dimension, one workgroup of eight waves per (chunk
// slot, head).  The value axis is walked in 16-column slices staged in LDS (the next slice
// is loaded into registers while the matrix cores work on the current one and stored into
// the other of two slice buffers, so one barrier per slice suffices); the C x K and C x C
// results accumulate in registers over the slices.  Two waves share each SIMD, so one
// wave's LDS reads and stores overlap the other's products.
constexpr int VNW = 8, VNT = 64 * VNW;  // vgrads waves and threads
template <int K>
struct VgLds {
    static constexpr int JS = 16, LJ = JS + 4;  // slice width; row stride 20 keeps fragment reads conflict-free
    static constexpr int LK = K + 4;
    static constexpr int SL = 2 * K * LJ + 4 * BC * LJ;               // one slice buffer
    static constexpr int SLICES = 2 * SL;                              // two slice buffers
    static constexpr int TAIL = 2 * BC * LK + 2 * BC * LDC;           // PW, beta Kg, MT / Y, dT (after the slices)
    static constexpr int R1 = SLICES > TAIL ? SLICES : TAIL;
    static constexpr size_t bytes = sizeof(float) * (R1 + 2 * BC * LDC + BC + VNT + (1 + K / 16 + NP) * BC);
};

// Tiles of wave w: C x K tiles t = w + 8 i (row tile t / (K/16), column tile t % (K/16)),
// C x C tiles (2 i + w / 4, w % 4) for i = 0, 1; T^T dVt on row tile w for w < 4.
// (LDS limits this kernel to one workgroup per CU: each wave may use half a SIMD's registers)
template <typename TIn, int K, int V>
__global__ __launch_bounds__(VNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_vgrads_kernel(BwdArgs a) {
    constexpr int JS = VgLds<K>::JS, LJ = VgLds<K>::LJ, KT = K / 16, SL = VgLds<K>::SL;
    constexpr int NCK = NP * KT, NOWN = (NCK + VNW - 1) / VNW;  // C x K tiles, per wave
    constexpr int KP = (K * 4 + VNT - 1) / VNT;  // 4-column groups of the K x 16 slices per thread
    static_assert(NP == 4, "four 16-row tiles per chunk");
    extern __shared__ __align__(16) unsigned char smem[];
    // slice buffer b: S [K][16], dS' [K][16], scale dO [C][16], Vt [C][16], dVt [C][16], v [C][16]
    constexpr int oDH = K * LJ, oO = 2 * K * LJ, oVt = oO + BC * LJ, odVt = oVt + BC * LJ, oVr = odVt + BC * LJ;
    float *sT = reinterpret_cast<float *>(smem) + VgLds<K>::R1;  // T [C][C]
    float *sTt = sT + BC * LDC;                    // T^T [C][C]: the A operand of the T^T products
    float *sB = sTt + BC * LDC;                    // beta
    float *sRs = sB + BC;                          // partial rowsum(S dS')
    float *sRv = sRs + VNT;                        // [C] rowsum(V T^T dVt)
    float *sRk = sRv + BC;                         // [K/16][C] partial rowsum(K e^Gamma dBk)
    float *sRa = sRk + KT * BC;                    // [NP][C] partial rowsum(dA Abar)
    const int n = blockIdx.x, h = blockIdx.y, H = a.H;
    const ChunkPos cp = slot_chunk(n, a.cu_seqlens, a.num_seqs, a.T);
    if (cp.L == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, i16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int wq = w & 3, wh = w >> 2;                        // C x C tiles: column tile, row parity
    const int64_t sh = (int64_t)n * H + h;
    const TIn *v = static_cast<const TIn *>(a.v);
    const float *hp = a.w.h + sh * K * V, *dhp = a.w.dh + sh * K * V;
    const float *Vtp = a.w.Vt + sh * BC * V, *dVtp = a.w.dVt + sh * BC * V, *Tm = a.w.Tm + sh * BC * BC;

    // slice staging: K x 16 of S and dS' in 16-byte groups, C x 16 of dO, Vt, dVt, v in
    // 8-byte pairs (row tid / 8, columns 2 (tid % 8) + 0, 1)
    float4 rh[KP], rdh[KP];
    float2 ro, rvt, rdvt, rv;
    const int sr = tid >> 3, sg = 2 * (tid & 7);
    const int64_t tok = ((cp.t0 + crow(sr, cp.L)) * H + h) * V + sg;
    auto load = [&](int j0) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int idx = min(tid + VNT * i, K * 4 - 1);
            const int c = idx >> 2, g = 4 * (idx & 3);
            rh[i] = ld4(hp + c * V + j0 + g);
            rdh[i] = ld4(dhp + c * V + j0 + g);
        }
        rvt = ld2(Vtp + sr * V + j0 + sg);
        rdvt = ld2(dVtp + sr * V + j0 + sg);
        ro = ld2_any(a.d_out, a.dout_bf16, tok + j0);  // masked past the chunk when stored
        rv = ld2(v + tok + j0);
    };
    auto store = [&](float *sb) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int idx = tid + VNT * i;
            if (idx < K * 4) {
                const int c = idx >> 2, g = 4 * (idx & 3);
                st4(sb + c * LJ + g, rh[i]);
                st4(sb + oDH + c * LJ + g, rdh[i]);
            }
        }
        const bool ok = sr < cp.L;
        const float sc = ok ? a.scale : 0.f;
        st2(sb + oO + sr * LJ + sg, make_float2(sc * ro.x, sc * ro.y));
        st2(sb + oVt + sr * LJ + sg, rvt);
        st2(sb + odVt + sr * LJ + sg, rdvt);
        st2(sb + oVr + sr * LJ + sg, ok ? rv : make_float2(0.f, 0.f));
    };

    load(0);
    {
        float4 x[BC * BC / 4 / VNT];
#pragma unroll
        for (int i = 0; i < BC * BC / 4 / VNT; ++i) x[i] = ld4(Tm + 4 * (tid + VNT * i));
#pragma unroll
        for (int i = 0; i < BC * BC / 4 / VNT; ++i) {
            const int e = 4 * (tid + VNT * i), r = e / BC, c = e % BC;
            st4(sT + r * LDC + c, x[i]);
            sTt[c * LDC + r] = x[i].x;
            sTt[(c + 1) * LDC + r] = x[i].y;
            sTt[(c + 2) * LDC + r] = x[i].z;
            sTt[(c + 3) * LDC + r] = x[i].w;
        }
    }
    if (tid < BC) sB[tid] = tid < cp.L ? a.beta[(cp.t0 + tid) * H + h] : 0.f;
    store(reinterpret_cast<float *>(smem));
    lds_barrier();

    f4 ps[NOWN], pw[NOWN], pd[NOWN], ma[2], mt[2];
#pragma unroll
    for (int i = 0; i < NOWN; ++i) ps[i] = pw[i] = pd[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) ma[i] = mt[i] = f4{0.f, 0.f, 0.f, 0.f};
    float dbacc[4] = {0.f, 0.f, 0.f, 0.f}, rsacc = 0.f;
    // rowsum(S dS'): PARTS threads per key row, CW columns each
    constexpr int PARTS = VNT / K < 16 ? VNT / K : 16, CW = JS / PARTS;

    for (int js = 0; js < V / JS; ++js) {
        float *sb = reinterpret_cast<float *>(smem) + (js & 1) * SL;
        const float *sH = sb, *sDH = sb + oDH, *sO = sb + oO, *sVt = sb + oVt, *sdVt = sb + odVt, *sVr = sb + oVr;
        const bool more = js + 1 < V / JS;
        if (more) load((js + 1) * JS);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products they overlap
        // Operands of T^T dVt (waves 0..3, below), read first so that they arrive during the
        // products.  k = s = 16 m + 4 (lane/16) + u over every m: the blocks m < p of T^T
        // are zero, and the wave with p = 0, which needs them all, sets the pace anyway.
        float4 at[NP];
        float bt[NP][4], bs[4], vr[4];
        const int pt = wq;  // row tile of T^T dVt (used by waves 0..3)
        if (w < 4) {
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                at[m] = *reinterpret_cast<const float4 *>(sTt + (16 * pt + i16) * LDC + 16 * m + 4 * g4);
#pragma unroll
                for (int u = 0; u < 4; ++u) bt[m][u] = sdVt[(16 * m + 4 * g4 + u) * LJ + i16];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bs[e] = sB[16 * pt + 4 * g4 + e];
                vr[e] = sVr[(16 * pt + 4 * g4 + e) * LJ + i16];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep these reads here, ahead of the products
        // dO S^T, dVt S^T, Vt dS'^T on this wave's C x K tiles and dO Vt^T, dVt V^T on its
        // C x C tiles.  The slice's 16-wide reduction is split as k = 4*(lane/16) + s on both
        // operands, so one 16-byte LDS read per operand feeds four matrix-core steps.
        {
            const int rq = (16 * wq + i16) * LJ + 4 * g4;
            const float4 bvt = *reinterpret_cast<const float4 *>(sVt + rq);
            const float4 bv = *reinterpret_cast<const float4 *>(sVr + rq);
            float4 fa[2][3];
            auto frag = [&](int p, float4 (&f)[3]) {
                const int ra = (16 * p + i16) * LJ + 4 * g4;
                f[0] = *reinterpret_cast<const float4 *>(sO + ra);
                f[1] = *reinterpret_cast<const float4 *>(sVt + ra);
                f[2] = *reinterpret_cast<const float4 *>(sdVt + ra);
            };
            if constexpr (KT % VNW == 0) {
                // Column tiles w + 8 c of every row tile p: row tile p's fragments of dO, Vt and
                // dVt serve them all and, when p = 2 i + w/4, the C x C tile (p, w % 4); the next
                // row tile's fragments are read while the current one's products run.
                constexpr int CT = KT / VNW;
                float4 bh[CT], bdh[CT];
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const int rb = (16 * (w + VNW * c) + i16) * LJ + 4 * g4;
                    bh[c] = *reinterpret_cast<const float4 *>(sH + rb);
                    bdh[c] = *reinterpret_cast<const float4 *>(sDH + rb);
                }
                frag(0, fa[0]);
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    if (p + 1 < NP) frag(p + 1, fa[(p + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);  // the next row tile's reads go out first
                    const float4 ao = fa[p & 1][0], avt = fa[p & 1][1], adv = fa[p & 1][2];
#pragma unroll
                    for (int c = 0; c < CT; ++c) {
                        const int i = p * CT + c;  // tile w + 8 i: row tile p, column tile w + 8 c
                        ps[i] = mf(ao.x, bh[c].x, ps[i]); pw[i] = mf(adv.x, bh[c].x, pw[i]); pd[i] = mf(avt.x, bdh[c].x, pd[i]);
                        ps[i] = mf(ao.y, bh[c].y, ps[i]); pw[i] = mf(adv.y, bh[c].y, pw[i]); pd[i] = mf(avt.y, bdh[c].y, pd[i]);
                        ps[i] = mf(ao.z, bh[c].z, ps[i]); pw[i] = mf(adv.z, bh[c].z, pw[i]); pd[i] = mf(avt.z, bdh[c].z, pd[i]);
                        ps[i] = mf(ao.w, bh[c].w, ps[i]); pw[i] = mf(adv.w, bh[c].w, pw[i]); pd[i] = mf(avt.w, bdh[c].w, pd[i]);
                    }
                    if ((p & 1) == wh) {
                        const int i = p >> 1;
                        ma[i] = mf(ao.x, bvt.x, ma[i]); mt[i] = mf(adv.x, bv.x, mt[i]);
                        ma[i] = mf(ao.y, bvt.y, ma[i]); mt[i] = mf(adv.y, bv.y, mt[i]);
                        ma[i] = mf(ao.z, bvt.z, ma[i]); mt[i] = mf(adv.z, bv.z, mt[i]);
                        ma[i] = mf(ao.w, bvt.w, ma[i]); mt[i] = mf(adv.w, bv.w, mt[i]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NOWN; ++i) {
                    const int t = w + VNW * i;
                    if (t < NCK) {
                        const int p = t / KT, ct = t % KT;
                        const int rb = (16 * ct + i16) * LJ + 4 * g4;
                        frag(p, fa[0]);
                        const float4 ao = fa[0][0], avt = fa[0][1], adv = fa[0][2];
                        const float4 bh = *reinterpret_cast<const float4 *>(sH + rb);
                        const float4 bdh = *reinterpret_cast<const float4 *>(sDH + rb);
                        ps[i] = mf(ao.x, bh.x, ps[i]); pw[i] = mf(adv.x, bh.x, pw[i]); pd[i] = mf(avt.x, bdh.x, pd[i]);
                        ps[i] = mf(ao.y, bh.y, ps[i]); pw[i] = mf(adv.y, bh.y, pw[i]); pd[i] = mf(avt.y, bdh.y, pd[i]);
                        ps[i] = mf(ao.z, bh.z, ps[i]); pw[i] = mf(adv.z, bh.z, pw[i]); pd[i] = mf(avt.z, bdh.z, pd[i]);
                        ps[i] = mf(ao.w, bh.w, ps[i]); pw[i] = mf(adv.w, bh.w, pw[i]); pd[i] = mf(avt.w, bdh.w, pd[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    frag(2 * i + wh, fa[1]);
                    const float4 ao = fa[1][0], adv = fa[1][2];
                    ma[i] = mf(ao.x, bvt.x, ma[i]); mt[i] = mf(adv.x, bv.x, mt[i]);
                    ma[i] = mf(ao.y, bvt.y, ma[i]); mt[i] = mf(adv.y, bv.y, mt[i]);
                    ma[i] = mf(ao.z, bvt.z, ma[i]); mt[i] = mf(adv.z, bv.z, mt[i]);
                    ma[i] = mf(ao.w, bvt.w, ma[i]); mt[i] = mf(adv.w, bv.w, mt[i]);
                }
            }
        }
        // T^T dVt on row tile p = w of this slice (waves 0..3): dv = beta T^T dVt,
        // rowsum(V T^T dVt) for dbeta (even and odd k blocks in two accumulators)
        if (w < 4) {
            f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NP; m += 2) {
                acc0 = mf(at[m].x, bt[m][0], acc0);
                acc1 = mf(at[m + 1].x, bt[m + 1][0], acc1);
                acc0 = mf(at[m].y, bt[m][1], acc0);
                acc1 = mf(at[m + 1].y, bt[m + 1][1], acc1);
                acc0 = mf(at[m].z, bt[m][2], acc0);
                acc1 = mf(at[m + 1].z, bt[m + 1][2], acc1);
                acc0 = mf(at[m].w, bt[m][3], acc0);
                acc1 = mf(at[m + 1].w, bt[m + 1][3], acc1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * pt + 4 * g4 + e;
                const float x = acc0[e] + acc1[e];
                if (row < cp.L)
                    st_out(a.dv, a.grad_bf16, ((cp.t0 + row) * H + h) * V + js * JS + i16, bs[e] * x);
                dbacc[e] += vr[e] * x;  // summed over the row's lanes at the end
            }
        }
        if (tid < K * PARTS) {
            const int c = tid % K, part = tid / K;
            if constexpr (CW == 4) {  // one 16-byte read of each (rows 80 bytes apart: no bank conflict)
                const float4 x = *reinterpret_cast<const float4 *>(sH + c * LJ + 4 * part);
                const float4 y = *reinterpret_cast<const float4 *>(sDH + c * LJ + 4 * part);
                rsacc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            } else {
#pragma unroll
                for (int j = 0; j < CW; ++j) rsacc += sH[c * LJ + part * CW + j] * sDH[c * LJ + part * CW + j];
            }
        }
        if (more) store(reinterpret_cast<float *>(smem) + ((js + 1) & 1) * SL);
        lds_barrier();
    }

    // the slices are done: their LDS now holds PW (-dW), beta K e^Gamma, MT and the C x C work
    constexpr int LK = VgLds<K>::LK;
    float *sPW = reinterpret_cast<float *>(smem);  // [C][K+4]
    float *sKg = sPW + BC * LK;                    // [C][K+4] K e^Gamma
    float *sM = sKg + BC * LK;                     // [C][C] beta MT, then Y = dT T^T
    float *sY = sM + BC * LDC;                     // [C][C] dT
    const float *Kg = a.w.Kg + sh * BC * K, *Abar = a.w.Abar + sh * BC * BC;
    float abr[2][4];  // Abar on this wave's C x C tiles, for rowsum(dA Abar)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) abr[i][e] = Abar[(16 * (2 * i + wh) + 4 * g4 + e) * BC + 16 * wq + i16];
    constexpr int NKG = (BC * K / 4 + VNT - 1) / VNT;
    float4 kg4[NKG];
#pragma unroll
    for (int i = 0; i < NKG; ++i) kg4[i] = ld4(Kg + 4 * min(tid + VNT * i, BC * K / 4 - 1));
    float *PS = a.w.PS + sh * BC * K, *PdK = a.w.PdK + sh * BC * K, *MA = a.w.MA + sh * BC * BC;
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
        const int t = w + VNW * i;
        if (t < NCK) {
            const int p = t / KT, c = 16 * (t % KT) + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * p + 4 * g4 + e;
                PS[row * K + c] = ps[i][e];
                PdK[row * K + c] = pd[i][e];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) MA[(16 * (2 * i + wh) + 4 * g4 + e) * BC + 16 * wq + i16] = ma[i][e];
    if (w < 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dbacc[e] = row16_sum(dbacc[e]);
        if (i16 == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sRv[16 * w + 4 * g4 + e] = dbacc[e];
        }
    }
    sRs[tid] = rsacc;
    lds_barrier();  // every wave is past the slices
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
        const int t = w + VNW * i;
        if (t < NCK) {
            const int p = t / KT, c = 16 * (t % KT) + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) sPW[(16 * p + 4 * g4 + e) * LK + c] = pw[i][e];
        }
    }
    {
        const int s = 16 * wq + i16;
        const float bs = sB[s];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) sM[(16 * (2 * i + wh) + 4 * g4 + e) * LDC + s] = bs * mt[i][e];
    }
#pragma unroll
    for (int i = 0; i < NKG; ++i) {
        const int idx = tid + VNT * i;
        if (idx < BC * K / 4) {
            const int r = (4 * idx) / K, c = (4 * idx) % K;
            st4(sKg + r * LK + c, kg4[i]);
        }
    }
    if (tid < K) {
        float acc = 0.f;
        for (int part = 0; part < PARTS; ++part) acc += sRs[part * K + tid];
        a.w.rs[sh * K + tid] = acc;
    }
    lds_barrier();
    // The C x C tiles of a wave share their column tile w % 4; the products below run the
    // two tiles side by side and share the operand of that column tile.
    // dT = MT + dW (beta K e^Gamma)^T with dW = -PW (beta_s applied to the column)
    {
        f4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const float *br = sKg + (16 * wq + i16) * LK + 4 * g4;
#pragma unroll 2
        for (int c0 = 0; c0 < K; c0 += 16) {
            const float4 y = *reinterpret_cast<const float4 *>(br + c0);
            float4 x[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                x[i] = *reinterpret_cast<const float4 *>(sPW + (16 * (2 * i + wh) + i16) * LK + 4 * g4 + c0);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].x, y.x, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].y, y.y, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].z, y.z, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].w, y.w, acc[i]);
        }
        const int s = 16 * wq + i16;
        const float bs = sB[s];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * (2 * i + wh) + 4 * g4 + e;
                sY[row * LDC + s] = sM[row * LDC + s] - bs * acc[i][e];
            }
    }
    // dBk = T^T dW = -T^T PW on this wave's C x K tiles; rowsum(K e^Gamma dBk) for dbeta.
    float *dBk = a.w.PW + sh * BC * K;
    {
        f4 acc[NOWN];
#pragma unroll
        for (int i = 0; i < NOWN; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NP; ++m) {
#pragma unroll
            for (int i = 0; i < NOWN; ++i) {
                const int t = w + VNW * i, p = KT % VNW == 0 ? (VNW * i) / KT : t / KT, c = 16 * (t % KT) + i16;
                if (t < NCK && m >= p) {
                    const float4 at = *reinterpret_cast<const float4 *>(sTt + (16 * p + i16) * LDC + 16 * m + 4 * g4);
                    const float *br = sPW + (16 * m + 4 * g4) * LK + c;
                    acc[i] = mf(at.x, br[0], acc[i]);
                    acc[i] = mf(at.y, br[LK], acc[i]);
                    acc[i] = mf(at.z, br[2 * LK], acc[i]);
                    acc[i] = mf(at.w, br[3 * LK], acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NOWN; ++i) {
            const int t = w + VNW * i;
            if (t < NCK) {
                const int p = t / KT, ct = t % KT, c = 16 * ct + i16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * p + 4 * g4 + e;
                    dBk[row * K + c] = -acc[i][e];
                    const float part = row16_sum(-acc[i][e] * sKg[row * LK + c]);
                    if (i16 == 0) sRk[ct * BC + row] = part;
                }
            }
        }
    }
    lds_barrier();
    // Y = dT T^T
    {
        f4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const float *br = sT + (16 * wq + i16) * LDC + 4 * g4;
#pragma unroll
        for (int j0 = 0; j0 < BC; j0 += 16) {
            const float4 y = *reinterpret_cast<const float4 *>(br + j0);
            float4 x[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                x[i] = *reinterpret_cast<const float4 *>(sY + (16 * (2 * i + wh) + i16) * LDC + 4 * g4 + j0);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].x, y.x, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].y, y.y, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].z, y.z, acc[i]);
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] = mf(x[i].w, y.w, acc[i]);
        }
        const int s = 16 * wq + i16;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) sM[(16 * (2 * i + wh) + 4 * g4 + e) * LDC + s] = acc[i][e];
    }
    lds_barrier();
    // dA = -strict_tril(T^T Y); rowsum(dA Abar) for dbeta; beta dA is what the key space needs
    float *dAb = a.w.MT + sh * BC * BC;
    {
        f4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int s = 16 * wq + i16;
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            const float *br = sM + (16 * m + 4 * g4) * LDC + s;
            const float b0 = br[0], b1 = br[LDC], b2 = br[2 * LDC], b3 = br[3 * LDC];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = 2 * i + wh;
                if (wq <= p && p <= m) {  // tiles on or below the diagonal; T^T is upper
                    const float4 at = *reinterpret_cast<const float4 *>(sTt + (16 * p + i16) * LDC + 16 * m + 4 * g4);
                    acc[i] = mf(at.x, b0, acc[i]);
                    acc[i] = mf(at.y, b1, acc[i]);
                    acc[i] = mf(at.z, b2, acc[i]);
                    acc[i] = mf(at.w, b3, acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * (2 * i + wh) + 4 * g4 + e;
                const float da = row > s ? -acc[i][e] : 0.f;
                const float part = row16_sum(da * abr[i][e]);
                if (i16 == 0) sRa[wq * BC + row] = part;
                dAb[row * BC + s] = sB[row] * da;
            }
    }
    lds_barrier();
    if (tid < cp.L) {
        float acc = sRv[tid];
        for (int ct = 0; ct < KT; ++ct) acc += sRk[ct * BC + tid];
        for (int qt = 0; qt < NP; ++qt) acc += sRa[qt * BC + tid];
        a.dbeta[(cp.t0 + tid) * H + h] = acc;
    }
}

// ------------------------------------------------------------------------------------
// kgrads: the key-space gradients, one workgroup per (chunk slot, head, block of KB key
// channels).  The products over tokens (the decayed adjoints) are independent per key
// channel, so a block needs only its own columns of q, k and Gamma, plus the two C x C
// matrices tril(dO Vt^T) and beta dA; everything is staged in LDS.  No exponential is
// taken inside the products: with m_p = Gamma at the middle row of row tile p,
//   e^{Gamma_r - Gamma_s} = F1_r E[p][q] F2_s,  F1 = e^{Gamma - m_tile(r)}, F2 = e^{m_tile(s) - Gamma},
//   E[p][q] = e^{m_p - m_q}  (q <= p: at most 1),
// and e^Gamma, e^{Gamma_C - Gamma} come from the same factors and two per-tile tables.
template <int K>
struct KgLds {
    static constexpr int KB = K < 32 ? K : 32, LKB = KB + 4;
    static constexpr size_t bytes = sizeof(float) * (4 * BC * LKB + 2 * BC * LDC + BC + (NP * NP + 3 * NP) * KB);
};

template <typename TIn, int K, int V>
// Persistent: workgroup b takes the work items b, b + G, ... (G the grid size, a multiple
// of 8 so that an item's XCD does not change), and loads the next item's inputs while it
// processes the current one.  Two workgroups per CU.
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_kgrads_kernel(BwdArgs a) {
    constexpr int KB = KgLds<K>::KB, LKB = KgLds<K>::LKB, NCB = K / KB, KBT = KB / 16;
    constexpr int NOWN = NP * KBT / 4;
    extern __shared__ __align__(16) unsigned char smem[];
    float *sQ = reinterpret_cast<float *>(smem);  // q, later the row terms of d ln alpha
    float *sK = sQ + BC * LKB;                     // k, later the Kd terms
    float *sF1 = sK + BC * LKB;                    // e^{Gamma - m_tile}
    float *sF2 = sF1 + BC * LKB;                   // Gamma, then e^{m_tile - Gamma}
    float *sMA = sF2 + BC * LKB;                   // tril(dO Vt^T)
    float *sdA = sMA + BC * LDC;                   // beta dA (strictly lower)
    float *sB = sdA + BC * LDC;
    float *sEpq = sB + BC;                         // [NP][NP][KB] e^{m_p - m_q}
    float *sEm = sEpq + NP * NP * KB;              // [NP][KB] e^{m_p}
    float *sEe = sEm + NP * KB;                    // [NP][KB] e^{Gamma_C - m_p}
    float *sMid = sEe + NP * KB;                   // [NP][KB] m_p

    const int H = a.H, units = a.slots * H;
    const int items = 8 * NCB * ((units + 7) / 8);
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k);
    // An item: its (chunk slot, head) unit, channel block and chunk; an item with no work
    // (past the last unit, or an unused slot) reads unit 0, row 0 (valid addresses).
    struct Item {
        int n, h, c0;
        ChunkPos cp;
        bool work;
    };
    auto item_of = [&](int it) {
        Item x{0, 0, 0, ChunkPos{0, 0}, false};
        if (it < items) {
            int u, cb;  // the channel blocks of one unit share an XCD
            xcd_map(it, NCB, u, cb);
            if (u < units) {
                x.n = u / H;
                x.h = u % H;
                x.c0 = cb * KB;
                x.cp = slot_chunk(x.n, a.cu_seqlens, a.num_seqs, a.T);
                x.work = x.cp.L > 0;
            }
        }
        if (!x.work) x = Item{0, 0, 0, ChunkPos{0, 1}, false};
        return x;
    };
    // inputs of the next item, kept in the input format until they are stored in LDS;
    // fetched unconditionally so that the loads land in the registers the next iteration
    // reads (a load under a condition is merged through copies that wait for it)
    using Raw4 = typename std::conditional<std::is_same<TIn, float>::value, float4, s16x4>::type;
    constexpr int NK4 = (BC * KB / 4 + NTH - 1) / NTH, NM4 = BC * BC / 4 / NTH;
    static_assert(BC * KB / 4 % NTH == 0, "whole float4 groups per thread");
    Raw4 rq[NK4], rk[NK4];
    float4 rg[NK4], rm[NM4], rd[NM4];
    float rb;
    auto fetch_in = [&](const Item &x) {
        const int tid = threadIdx.x;
        const int64_t sh = (int64_t)x.n * H + x.h;
#pragma unroll
        for (int i = 0; i < NK4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / KB, c = (4 * idx) % KB;
            const int64_t gi = ((x.cp.t0 + crow(r, x.cp.L)) * H + x.h) * K + x.c0 + c;
            rq[i] = *reinterpret_cast<const Raw4 *>(q + gi);
            rk[i] = *reinterpret_cast<const Raw4 *>(k + gi);
            rg[i] = ld4(a.gate.gate + gi);
        }
        const float *MA = a.w.MA + sh * BC * BC, *dAb = a.w.MT + sh * BC * BC;
#pragma unroll
        for (int i = 0; i < NM4; ++i) {
            rm[i] = ld4(MA + 4 * (tid + NTH * i));
            rd[i] = ld4(dAb + 4 * (tid + NTH * i));
        }
        rb = a.beta[(x.cp.t0 + crow(tid & (BC - 1), x.cp.L)) * H + x.h];
    };
    // element-wise inputs of this thread's output tiles (dO S^T, Vt dS'^T, T^T dW): loaded
    // once the current item's are used, in flight until the next item's products
    float pre[NOWN][3][4];
    auto fetch_pre = [&](const Item &x) {
        const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g4 = lane >> 4, i16 = lane & 15;
        const int64_t sh = (int64_t)x.n * H + x.h;
        const float *PS = a.w.PS + sh * BC * K, *PdK = a.w.PdK + sh * BC * K, *dBk = a.w.PW + sh * BC * K;
#pragma unroll
        for (int i = 0; i < NOWN; ++i) {
            const int t = w + 4 * i, rt = t / KBT, ct = t % KBT, gc = x.c0 + 16 * ct + i16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * rt + 4 * g4 + e;
                pre[i][0][e] = PS[row * K + gc];
                pre[i][1][e] = PdK[row * K + gc];
                pre[i][2][e] = dBk[row * K + gc];
            }
        }
    };
    int item = blockIdx.x;
    Item nx = item_of(item);
    fetch_in(nx);
    fetch_pre(nx);
    for (; item < items; item += gridDim.x) {
    // the thread index is re-read through an opaque copy in every iteration, so that the
    // item's index computations are not hoisted out of the loop into registers
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g4 = lane >> 4, i16 = lane & 15;
    const Item cur = nx;
    nx = item_of(item + gridDim.x);
    if (!cur.work) {  // uniform: only the next item's loads
        fetch_in(nx);
        fetch_pre(nx);
        continue;
    }
    const int n = cur.n, h = cur.h, c0 = cur.c0;
    const ChunkPos cp = cur.cp;
    const int64_t sh = (int64_t)n * H + h;
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
        const int idx = tid + NTH * i, r = (4 * idx) / KB, c = (4 * idx) % KB;
        st4(sQ + r * LKB + c, mask4(raw_f4(rq[i]), r < cp.L));
        st4(sK + r * LKB + c, mask4(raw_f4(rk[i]), r < cp.L));
        st4(sF2 + r * LKB + c, gate_log4(a.gate, rg[i], r < cp.L));
    }
#pragma unroll
    for (int i = 0; i < NM4; ++i) {
        const int e = 4 * (tid + NTH * i), r = e / BC, c = e % BC;
        const float4 m = rm[i];  // tril(dO Vt^T): entries with s > r are dropped
        st4(sMA + r * LDC + c, make_float4(c <= r ? m.x : 0.f, c + 1 <= r ? m.y : 0.f, c + 2 <= r ? m.z : 0.f,
                                           c + 3 <= r ? m.w : 0.f));
        st4(sdA + r * LDC + c, rd[i]);
    }
    if (tid < BC) sB[tid] = tid < cp.L ? rb : 0.f;
    // kept for the end: the gate values (alpha, for dgate = d ln alpha / alpha) and the
    // chunk-end term gamma_C rowsum(S dS') of this thread's channel, read before the next
    // item's loads go out
    float4 al[NK4];
#pragma unroll
    for (int i = 0; i < NK4; ++i) al[i] = rg[i];
    const float gcrs = a.w.gC[sh * K + c0 + tid % KB] * a.w.rs[sh * K + c0 + tid % KB];
    lds_barrier();
    fetch_in(nx);  // in flight while this item is processed
    {
        // Gamma: inclusive prefix sums over the chunk's rows per channel, in NSEG segments of
        // SEG rows (each read into registers at once), offset by the earlier segments' totals
        constexpr int NSEG = NTH / KB < BC ? NTH / KB : BC, SEG = BC / NSEG;
        const int c = tid % KB, sg = tid / KB;
        float x[SEG];
        if (sg < NSEG) {
#pragma unroll
            for (int j = 0; j < SEG; ++j) x[j] = sF2[(sg * SEG + j) * LKB + c];
#pragma unroll
            for (int j = 1; j < SEG; ++j) x[j] += x[j - 1];
            sEpq[sg * KB + c] = x[SEG - 1];  // segment totals (the tables are written later)
        }
        lds_barrier();
        if (sg < NSEG) {
            float off = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < NSEG - 1; ++s2)
                if (s2 < sg) off += sEpq[s2 * KB + c];
#pragma unroll
            for (int j = 0; j < SEG; ++j) sF2[(sg * SEG + j) * LKB + c] = x[j] + off;
        }
    }
    lds_barrier();
    // tables per channel, from the tile middles m_p and the chunk end
    for (int i = tid; i < (NP * NP + 3 * NP) * KB; i += NTH) {
        const int c = i % KB, j = i / KB;
        if (j < NP * NP) {
            const int pp = j / NP, qq = j % NP;
            sEpq[j * KB + c] = qq <= pp ? expf(sF2[(16 * pp + 7) * LKB + c] - sF2[(16 * qq + 7) * LKB + c]) : 0.f;
        } else if (j < NP * NP + NP) {
            sEm[(j - NP * NP) * KB + c] = expf(sF2[(16 * (j - NP * NP) + 7) * LKB + c]);
        } else if (j < NP * NP + 2 * NP) {
            const int pp = j - NP * NP - NP;
            sEe[pp * KB + c] = expf(sF2[(BC - 1) * LKB + c] - sF2[(16 * pp + 7) * LKB + c]);
        } else {
            const int pp = j - NP * NP - 2 * NP;
            sMid[pp * KB + c] = sF2[(16 * pp + 7) * LKB + c];
        }
    }
    lds_barrier();
    for (int i = tid; i < BC * KB; i += NTH) {  // each element rewritten by the thread that reads it
        const int r = i / KB, c = i % KB;
        const float d = sF2[r * LKB + c] - sMid[(r >> 4) * KB + c];
        sF1[r * LKB + c] = exp_in_tile(d);
        sF2[r * LKB + c] = exp_in_tile(-d);
    }
    lds_barrier();

    float dgt[NOWN][4], est[NOWN][4];
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
        const int t = w + 4 * i, rt = t / KBT, ct = t % KBT;
        const int c = 16 * ct + i16, gc = c0 + c;
        const float *ps_ = pre[i][0], *pdk_ = pre[i][1], *dbk_ = pre[i][2];
        // row side of the decayed adjoints (rows of tile rt): A_qk -> dq, beta dA -> dk;
        // column s of tile qs enters as k_s F2_s E[rt][qs], the result is scaled by F1_r
        f4 xq = {0.f, 0.f, 0.f, 0.f}, xk = xq;
        {
            const int r = 16 * rt + i16;
            for (int qs = 0; qs <= rt; ++qs) {
                const float epq = sEpq[(rt * NP + qs) * KB + c];
                // k = 16 qs + 4 (lane/16) + u: one 16-byte read of each A row, B rows 4 apart
                const float4 ma = *reinterpret_cast<const float4 *>(sMA + r * LDC + 16 * qs + 4 * g4);
                const float4 da = *reinterpret_cast<const float4 *>(sdA + r * LDC + 16 * qs + 4 * g4);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int s = 16 * qs + 4 * g4 + u;
                    const float b = sK[s * LKB + c] * sF2[s * LKB + c] * epq;
                    xq = mf(u == 0 ? ma.x : u == 1 ? ma.y : u == 2 ? ma.z : ma.w, b, xq);
                    xk = mf(u == 0 ? da.x : u == 1 ? da.y : u == 2 ? da.z : da.w, b, xk);
                }
            }
        }
        // column side (rows of tile rt as the earlier index s): row r of tile p >= rt enters
        // as q_r F1_r (k_r F1_r), the result for row s is scaled by E[p][rt] F2_s
        f4 yq = {0.f, 0.f, 0.f, 0.f}, yk = yq;
        for (int p = rt; p < NP; ++p) {
            f4 aq = {0.f, 0.f, 0.f, 0.f}, akk = aq;
            const int s = 16 * rt + i16;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 16 * p + 4 * g4 + u;  // rows 4 apart per lane group
                const float f1 = sF1[r * LKB + c];
                aq = mf(sMA[r * LDC + s], sQ[r * LKB + c] * f1, aq);
                akk = mf(sdA[r * LDC + s], sK[r * LKB + c] * f1, akk);
            }
            const float epr = sEpq[(p * NP + rt) * KB + c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float fs = epr * sF2[(16 * rt + 4 * g4 + e) * LKB + c];
                yq[e] += fs * aq[e];
                yk[e] += fs * akk[e];
            }
        }
        const float em = sEm[rt * KB + c], ee = sEe[rt * KB + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * rt + 4 * g4 + e;
            const float fr = sF1[row * LKB + c], kv = sK[row * LKB + c], qv = sQ[row * LKB + c];
            const float eg = fr * em;                          // e^Gamma
            const float dKW = sB[row] * eg * dbk_[e];
            const float dQ = ps_[e] * eg + fr * xq[e];
            const float dKS = pdk_[e] * (ee * sF2[row * LKB + c]);  // e^{Gamma_C - Gamma}
            const float dK1 = fr * xk[e];
            const float dK = yq[e] + dKS + dKW + dK1 + yk[e];
            dgt[i][e] = qv * dQ + kv * (dK1 + dKW - yq[e] - yk[e]);
            est[i][e] = kv * dKS;
            if (row < cp.L) {
                const int64_t gi = ((cp.t0 + row) * H + h) * K + gc;
                st_out(a.dq, a.grad_bf16, gi, dQ);
                st_out(a.dk, a.grad_bf16, gi, dK);
            }
        }
    }
    lds_barrier();  // q, k are no longer read: their LDS takes the row terms
    fetch_pre(nx);  // this item's tile inputs are used
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
        const int t = w + 4 * i, rt = t / KBT, ct = t % KBT, c = 16 * ct + i16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * rt + 4 * g4 + e;
            sQ[row * LKB + c] = dgt[i][e];
            sK[row * LKB + c] = est[i][e];
        }
    }
    lds_barrier();
    // d ln alpha per key channel: reverse in-chunk sum of the row terms, plus the chunk-end
    // terms gamma_C rowsum(S dS') and the exclusive forward sum of the Kd terms; the result
    // replaces the row terms in LDS
    // (in NSEG segments of SEG rows per channel: segment sums first, then the offsets from
    // the other segments)
    {
        constexpr int NSEG = NTH / KB < BC ? NTH / KB : BC, SEG = BC / NSEG;
        float *sTot = sMA;  // [2][NSEG][KB] segment totals (tril(dO Vt^T) is consumed)
        const int c = tid % KB, sg = tid / KB;
        float kd[SEG], rw[SEG];
        if (sg < NSEG) {
            float tk = 0.f, tr = 0.f;
#pragma unroll
            for (int j = 0; j < SEG; ++j) {
                kd[j] = sK[(sg * SEG + j) * LKB + c];
                rw[j] = sQ[(sg * SEG + j) * LKB + c];
                tk += kd[j];
                tr += rw[j];
            }
            sTot[sg * KB + c] = tk;
            sTot[(NSEG + sg) * KB + c] = tr;
        }
        lds_barrier();
        if (sg < NSEG) {
            const int gc = c0 + c;
            // forward exclusive sum of the Kd terms (from the chunk-end term), reverse
            // inclusive sum of the row terms
            float f = gcrs, rv = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < NSEG; ++s2) {
                if (s2 < sg) f += sTot[s2 * KB + c];
                if (s2 > sg) rv += sTot[(NSEG + s2) * KB + c];
            }
            float dl[SEG];
#pragma unroll
            for (int j = 0; j < SEG; ++j) {
                dl[j] = f;
                f += kd[j];
            }
#pragma unroll
            for (int j = SEG - 1; j >= 0; --j) {
                rv += rw[j];
                sQ[(sg * SEG + j) * LKB + c] = dl[j] + rv;
            }
        }
    }
    lds_barrier();
    // dgate in four-element groups over the whole workgroup (alpha kept from the staging)
    {
        constexpr int NK4 = (BC * KB / 4 + NTH - 1) / NTH;
        const bool log_gate = a.gate.mode == GATE_LOG;
#pragma unroll
        for (int i = 0; i < NK4; ++i) {
            const int idx = tid + NTH * i, r = (4 * idx) / KB, c = (4 * idx) % KB;
            if (r < cp.L) {
                const float *x = sQ + r * LKB + c;
                float4 o = make_float4(x[0], x[1], x[2], x[3]);
                if (!log_gate) {
                    o.x *= __builtin_amdgcn_rcpf(al[i].x);
                    o.y *= __builtin_amdgcn_rcpf(al[i].y);
                    o.z *= __builtin_amdgcn_rcpf(al[i].z);
                    o.w *= __builtin_amdgcn_rcpf(al[i].w);
                }
                st4(a.dgate + ((cp.t0 + r) * H + h) * K + c0 + c, o);
            }
        }
    }
    lds_barrier();  // this item's LDS is consumed before the next item's inputs are stored
    }
}

int num_cus() { return device_cu_count(); }

template <int K, int V>
hipError_t set_lds(const void *kern, size_t bytes) {
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const BwdArgs &a, int num_seqs, hipStream_t stream) {
    static std::atomic<bool> attr{false};  // per instantiation, once per process
    auto kprep = bwd_prep_kernel<TIn, K, V>;
    auto kvg = bwd_vgrads_kernel<TIn, K, V>;
    auto kkg = bwd_kgrads_kernel<TIn, K, V>;
    if (!attr) {
        hipError_t e = set_lds<K, V>(reinterpret_cast<const void *>(kprep), PrepLds<K, V>::bytes);
        if (e == hipSuccess) e = set_lds<K, V>(reinterpret_cast<const void *>(kvg), VgLds<K>::bytes);
        if (e == hipSuccess) e = set_lds<K, V>(reinterpret_cast<const void *>(kkg), KgLds<K>::bytes);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int hs8 = (num_seqs * a.H + 7) / 8, sh8 = (int)(((int64_t)a.slots * a.H + 7) / 8);
    const dim3 gp(a.slots, a.H), gs(8 * (V / SBV) * hs8), gd(8 * (V / DstCfg<V>::DBV) * hs8);
    const int64_t units = (int64_t)a.slots * a.H;
    const dim3 gpp((unsigned)(units < num_cus() ? units : num_cus()));  // persistent prep
    const dim3 gk(8 * (K / KgLds<K>::KB) * sh8);
    const int gk_max = 2 * num_cus() / 8 * 8 > 8 ? 2 * num_cus() / 8 * 8 : 8;  // two per CU, a multiple of 8
    const dim3 gkp(gk.x < (unsigned)gk_max ? gk.x : (unsigned)gk_max);         // persistent kgrads
    constexpr size_t prep_bytes = PrepLds<K, V>::bytes;
    hipLaunchKernelGGL(kprep, gpp, dim3(PNT), prep_bytes, stream, a);
    hipLaunchKernelGGL((bwd_states_kernel<K, V>), gs, dim3(NTH), 0, stream, a);
    hipLaunchKernelGGL((bwd_dstates_kernel<K, V>), gd, dim3(NTH), 0, stream, a);
    hipLaunchKernelGGL(kvg, gp, dim3(VNT), VgLds<K>::bytes, stream, a);
    hipLaunchKernelGGL(kkg, gkp, dim3(NTH), KgLds<K>::bytes, stream, a);
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
