// kda_chunk_kernel.h -- chunkwise-parallel KDA prefill on gfx950 matrix cores: the
// kernel template and its launch helpers, instantiated by kda_chunk.hip (gate given as
// a float32 tensor) and kda_chunk_logits.hip (gate computed from its logits in the
// kernel), two translation units so the two sets compile in parallel.
//
// Method (KDA cheat sheet, "Chunkwise parallel form", with the UT transform the
// page names written out): for a chunk of C tokens with start state S and in-chunk
// cumulative decay gamma_i = prod_{r<=i} alpha_r (per key channel),
//   A_kk[i,j] = beta_i sum_c k_ic k_jc gamma_ic / gamma_jc   (j < i),  T = (I + A_kk)^-1
//   Vt = T (beta V - (beta gamma K) S)                     (= U - W S, the pseudo-values)
//   A_qk[i,j] = sum_c q_ic k_jc gamma_ic / gamma_jc         (j <= i: each read follows
//                                                          its own write, so the diagonal stays)
//   O  = (gamma Q) S + A_qk Vt                              (inter + intra chunk)
//   S' = gamma_C S + (K gamma_C / gamma)^T Vt
// which equals the token recurrence exactly in real arithmetic.
//
// Rescaling (cheat sheet gate table): with every log-decay >= -5, a 16-token tile
// decays by at most e^-80, so each ratio gamma_i / gamma_j is split at a per-tile
// reference into two factors inside [e^-80, e^80] -- within float and bf16 range --
// and every tile of A_kk and A_qk is a dense matrix-core product.  With R_p / E_p
// the cumulative decay before / at the end of 16-row tile p:
//   diagonal tile p:         (gamma_i / R_p) * (R_p / gamma_j)
//   off-diagonal tile (p,q): (gamma_i / R_p) * (R_p / gamma_j), the right factor built
//                            as (E_q / gamma_j) * (R_p / E_q) so nothing underflows early.
// All factors are products of retention factors (in-tile prefix and suffix
// products), so no per-element exponential is needed.
//
// Work decomposition: one workgroup of 12 waves (three per SIMD) per (sequence, head,
// block of BV value columns); value columns evolve independently, so the split is exact.
// Each chunk period has two workgroup barriers, B1 and B2.
//  * 4 state waves own the float32 state S[K x BV] in registers (one 16-column tile
//    each).  Before B1 they compute the A-matrix tiles and T's diagonal blocks of the
//    chunk staged in the previous period; after it, T's off-diagonal blocks (every
//    state wave computes all of them, so no further barrier is needed) and the serial
//    part for that chunk: Y = beta V - Bw S, Vt = T Y, O = Qt S + A_qk Vt,
//    S = gamma_C S + Kt^T Vt.  Their matrix-core operands come straight from the
//    accumulators of the previous product (the k order of each product is permuted to
//    match the accumulator layout), so the state never round-trips through LDS.
//  * 8 prep waves form the next chunk's decay products before B1; after it they stage
//    the A-matrix operands, send the prefetch of the chunk after, and store the package
//    (Qt, -Bw, Kt, beta V, gamma_C) in the other half of a double-buffered LDS area.
//
// Precision (bf16 inputs): the A-matrix operands carry factors up to e^80 and use
// bf16; A_qk, which carries each token's own value to its output, is formed from
// hi+lo bf16 splits of both operands.  Every other product has operands bounded by
// ~1 or by the state/value magnitude and uses fp16 (3 more mantissa bits than
// bf16).  fp32 inputs use fp32 matrix cores throughout.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int NSW = 4;           // state waves: 0..3
constexpr int NPW = 8;           // prep waves: 4..11
constexpr int NPT = 64 * NPW;    // prep threads
constexpr int NT = 64 * NSW + NPT;  // threads per workgroup (three waves per SIMD)

constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }

// kSegWaves: waves per SIMD the segment kernel (chain beside pre-pass) is compiled for --
// four on the 16-bit path, so a chain workgroup and a pre-pass workgroup share a compute
// unit; two with float32 operands, whose fragments take twice the registers.
struct PrecMixed {
    using TA = __bf16;    // operands of the decay-rescaled key/query products
    using TM = _Float16;  // every other matrix-core operand
    static constexpr bool kSplit = true;
    static constexpr int kSegWaves = 4;
    // A_qk reaches the serial part as hi + lo fp16 parts: the product that carries each
    // token's own pseudo-value to its output needs more than fp16's 11 mantissa bits
    static constexpr int kAqParts = 2;
};
struct PrecF32 {
    using TA = float;
    using TM = float;
    static constexpr bool kSplit = false;
    static constexpr int kSegWaves = 2;
    static constexpr int kAqParts = 1;
};

template <class P, int K, int V, int C, int BV>
struct Layout {
    using TA = typename P::TA;
    using TM = typename P::TM;
    static constexpr int NP = C / 16;                                  // 16-row tiles per chunk
    static constexpr int NX = NP >= 3 ? (NP - 1) * (NP - 2) / 2 : 0;  // tiles (p,q) with q <= p-2
    // 64-token chunks at K = 128 with 16-bit operands: the operand staging holds half of the
    // key columns at a time (the A-matrix products accumulate over the two halves), and the
    // package rows of token index (Kt, T, A_qk, v) go unpadded, so that the staging, and two
    // packages, fit the 160 KB of LDS
    static constexpr bool kWide = C >= 64 && K >= 128 && sizeof(TM) == 2;
    static constexpr int KS = kWide ? K / 2 : K;                 // key columns staged at once
    static constexpr int LKA = KS + 16 / (int)sizeof(TA);  // padded row strides (elements)
    static constexpr int LKM = K + 16 / (int)sizeof(TM);
    static constexpr int LCM = C + (kWide ? 0 : 16 / (int)sizeof(TM));
    static constexpr int LCF = C + 4;
    static constexpr int LKS = KS + 16 / (int)sizeof(TA);       // staging rows
    static constexpr int NJT = BV / 16;                         // value column tiles
    static constexpr int MJ = (NJT + NSW - 1) / NSW;            // column tiles per state wave

    // operand staging of the A-matrix products, in the A-operand type: Lk, then one block
    // holding Lq, Rd, Ro and the extra right-operand versions X (element offsets sLq..sX).
    // With a split precision the block is followed by a copy of the same shape holding
    // the low parts (x - hi), NST elements further on.
    static constexpr size_t oLk = 0;
    static constexpr size_t oSt = oLk + al16((size_t)C * LKA * sizeof(TA));
    static constexpr int sLq = 0;
    static constexpr int sRd = sLq + C * LKS;
    static constexpr int sRo = sRd + C * LKS;
    static constexpr int sX = sRo + (C > 16 ? C - 16 : 0) * LKS;
    static constexpr int NST = sX + NX * 16 * LKS;
    static constexpr size_t oAkk = oSt + al16((size_t)NST * sizeof(TA) * (P::kSplit ? 2 : 1));
    static constexpr size_t oTf = oAkk + al16((size_t)C * LCF * 4);
    // per-row partial sums of q^2 and k^2 from each wave that holds part of a tile's row
    static constexpr int NPART = K / 2 > 16 ? K / 32 : 1;
    static constexpr int NNRM = NP * 2 * 16 * NPART;                  // floats per buffer
    static constexpr size_t oNrm = oTf + al16((size_t)C * LCF * 4);  // [2][NP][2][16][NPART], by chunk parity
    static constexpr size_t oTP = oNrm + al16((size_t)2 * NNRM * 4);
    static constexpr size_t oBt = oTP + al16((size_t)NP * K * 4);
    static constexpr size_t oPkg = oBt + al16((size_t)C * 4);
    // package (two copies)
    static constexpr size_t pQt = 0;
    static constexpr size_t pBw = pQt + al16((size_t)C * LKM * sizeof(TM));
    static constexpr size_t pKt = pBw + al16((size_t)C * LKM * sizeof(TM));
    static constexpr size_t pTm = pKt + al16((size_t)K * LCM * sizeof(TM));
    static constexpr size_t pAqk = pTm + al16((size_t)C * LCM * sizeof(TM));
    static constexpr size_t pAql = pAqk + al16((size_t)C * LCM * sizeof(TM));  // low part (16-bit path)
    // the raw values of the chunk's value block, [BV][LCM] in the input type (same size
    // as TM); gamma_C [K] and beta [C] in float32, adjacent as in the workspace package
    static constexpr size_t pbV = pAql + (P::kAqParts - 1) * al16((size_t)C * LCM * sizeof(TM));
    static constexpr size_t pGC = pbV + al16((size_t)BV * LCM * sizeof(TM));
    static constexpr size_t pBt = pGC + (size_t)K * 4;
    static constexpr size_t szPkg = al16(pBt + (size_t)C * 4);
    static constexpr size_t total = oPkg + 2 * szPkg;
    static constexpr bool fits = total <= 160 * 1024;
};

// ---- matrix-core products whose B operand comes from accumulator tiles ----------------
//
// A D-layout accumulator tile (lane l holds rows 4*(l/16)+e, column l%16) is, after
// conversion, directly a B operand when the k order is permuted: a 16x16x32 step over
// k tiles (2m, 2m+1) takes k = 32m + 4g + i (i < 4) and 32m + 16 + 4g + (i-4) (i >= 4)
// for lane group g = l/16; an odd last tile takes k = 16t + 4g + i in the lower half of
// the same instruction (upper half zero); an fp32 16x16x4 step s over tile t takes
// k = 16t + 4g + s.  The A operand is read from LDS
// (k contiguous) in the same order.
template <typename TM, int NKT>
struct BFrag;  // packed B operands for NKT consecutive 16-k tiles

template <int NKT>
struct BFrag<_Float16, NKT> {
    f16x8 pair[NKT / 2 > 0 ? NKT / 2 : 1];
    f16x4 tail;
    __device__ __forceinline__ void set(const f4 *t) {
#pragma unroll
        for (int m = 0; m < NKT / 2; ++m) {
            f16x8 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (_Float16)t[2 * m][e];
                x[4 + e] = (_Float16)t[2 * m + 1][e];
            }
            pair[m] = x;
        }
        if constexpr (NKT % 2 == 1) {
            f16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (_Float16)t[NKT - 1][e];
            tail = y;
        }
    }
};

template <int NKT>
struct BFrag<float, NKT> {
    f4 t[NKT];
    __device__ __forceinline__ void set(const f4 *x) {
#pragma unroll
        for (int i = 0; i < NKT; ++i) t[i] = x[i];
    }
};

// acc += A[16 x 16*nkt] * B, A rows in LDS (arow = this lane's row, k contiguous), over
// the first nkt (<= NKT) k tiles of b.  Callers pass nkt rounded up to even on the
// 16-bit path only when the extra tile of A is zero.  With SW the row is stored
// swizzled: in rows whose index has bit 3 set (this lane's row, lane & 8) the two 8-byte
// halves of every 16-byte piece are swapped, so the 16 rows one instruction reads fall
// in distinct banks.
template <int NKT, bool SW = false>
__device__ __forceinline__ void mma_bfrag(f4 &acc, const _Float16 *arow, const BFrag<_Float16, NKT> &b,
                                          int nkt, int lane) {
    const int g = lane >> 4;
    const int kg = (4 * g) ^ (SW && (lane & 8) ? 4 : 0);  // this lane's 4-element k group
#pragma unroll
    for (int m = 0; m < NKT / 2; ++m) {
        if (2 * m < nkt) {
            const f16x4 lo = *reinterpret_cast<const f16x4 *>(arow + 32 * m + kg);
            const f16x4 hi = *reinterpret_cast<const f16x4 *>(arow + 32 * m + 16 + kg);
            const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b.pair[m], acc, 0, 0, 0);
        }
    }
    if constexpr (NKT % 2 == 1) {
        // an odd last tile goes through the same 16x16x32 instruction with its upper half
        // zero, so one accumulation chain never mixes instruction shapes
        if (NKT - 1 < nkt) {
            const f16x4 lo = *reinterpret_cast<const f16x4 *>(arow + 16 * (NKT - 1) + kg);
            const f16x8 a = {lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
            const f16x8 bb = {b.tail[0], b.tail[1], b.tail[2], b.tail[3], 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb, acc, 0, 0, 0);
        }
    }
}

template <int NKT, bool SW = false>
__device__ __forceinline__ void mma_bfrag(f4 &acc, const float *arow, const BFrag<float, NKT> &b, int nkt,
                                          int lane) {
    const int g = lane >> 4;
    const int sw = SW && (lane & 8) ? 2 : 0;  // 8-byte halves swapped: element ^ 2
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        if (t < nkt) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[16 * t + 4 * g + (s ^ sw)], b.t[t][s], acc, 0, 0, 0);
        }
    }
}

// The A operand of mma_bfrag held in registers: this lane's part of one 16-row tile over
// NKT k tiles, in the permuted k order of BFrag.  Loading a whole phase's fragments before
// its products keeps the LDS reads in flight together instead of one read per product.
template <typename TM, int NKT>
struct AFrag;

template <int NKT>
struct AFrag<_Float16, NKT> {
    f16x8 pair[NKT / 2 > 0 ? NKT / 2 : 1];
    f16x4 tail;
    // the first nkt k tiles of row `arow` (rows with bit 3 set swizzled when SW)
    template <bool SW>
    __device__ __forceinline__ void load(const _Float16 *arow, int nkt, int lane) {
        const int kg = (4 * (lane >> 4)) ^ (SW && (lane & 8) ? 4 : 0);
#pragma unroll
        for (int m = 0; m < NKT / 2; ++m) {
            if (2 * m < nkt) {
                const f16x4 lo = *reinterpret_cast<const f16x4 *>(arow + 32 * m + kg);
                const f16x4 hi = *reinterpret_cast<const f16x4 *>(arow + 32 * m + 16 + kg);
                pair[m] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        }
        if constexpr (NKT % 2 == 1) {
            if (NKT - 1 < nkt) tail = *reinterpret_cast<const f16x4 *>(arow + 16 * (NKT - 1) + kg);
        }
    }
};

template <int NKT>
struct AFrag<float, NKT> {
    f4 t[NKT];
    template <bool SW>
    __device__ __forceinline__ void load(const float *arow, int nkt, int lane) {
        const int g = lane >> 4;
        const int sw = SW && (lane & 8) ? 2 : 0;
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            if (i < nkt) {
                f4 x;
#pragma unroll
                for (int s = 0; s < 4; ++s) x[s] = arow[16 * i + 4 * g + (s ^ sw)];
                t[i] = x;
            }
        }
    }
};

// acc += A B over the first nkt k tiles, A from registers (AFrag), B from accumulators
// (BFrag): rows of the result are A's rows.  With TR the operands trade places, giving
// the transposed tile (B^T A^T): rows are B's columns and columns are A's rows.
template <bool TR, int NKT>
__device__ __forceinline__ void mma_frag(f4 &acc, const AFrag<_Float16, NKT> &a, const BFrag<_Float16, NKT> &b,
                                         int nkt) {
#pragma unroll
    for (int m = 0; m < NKT / 2; ++m)
        if (2 * m < nkt)
            acc = TR ? __builtin_amdgcn_mfma_f32_16x16x32_f16(b.pair[m], a.pair[m], acc, 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_16x16x32_f16(a.pair[m], b.pair[m], acc, 0, 0, 0);
    if constexpr (NKT % 2 == 1) {
        if (NKT - 1 < nkt) {
            const f16x8 x = {a.tail[0], a.tail[1], a.tail[2], a.tail[3], 0, 0, 0, 0};
            const f16x8 y = {b.tail[0], b.tail[1], b.tail[2], b.tail[3], 0, 0, 0, 0};
            acc = TR ? __builtin_amdgcn_mfma_f32_16x16x32_f16(y, x, acc, 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
        }
    }
}

template <bool TR, int NKT>
__device__ __forceinline__ void mma_frag(f4 &acc, const AFrag<float, NKT> &a, const BFrag<float, NKT> &b, int nkt) {
#pragma unroll
    for (int i = 0; i < NKT; ++i)
        if (i < nkt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = TR ? __builtin_amdgcn_mfma_f32_16x16x4f32(b.t[i][s], a.t[i][s], acc, 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_16x16x4f32(a.t[i][s], b.t[i][s], acc, 0, 0, 0);
}

// Compiler scheduling fence: no instruction moves across it, so LDS reads issued before
// it stay ahead of the products after it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// store two consecutive elements (a at p[0], b at p[1]) as one packed write
template <typename T>
__device__ __forceinline__ void st2(T *p, float a, float b);
template <>
__device__ __forceinline__ void st2<float>(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = float2{a, b};
}
template <>
__device__ __forceinline__ void st2<__bf16>(__bf16 *p, float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 v2;
    *reinterpret_cast<v2 *>(p) = v2{(__bf16)a, (__bf16)b};
}
template <>
__device__ __forceinline__ void st2<_Float16>(_Float16 *p, float a, float b) {
    typedef __attribute__((ext_vector_type(2))) _Float16 v2;
    *reinterpret_cast<v2 *>(p) = v2{(_Float16)a, (_Float16)b};
}

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS traffic only.  The waves exchange data through LDS alone,
// so global loads may stay in flight across it (the prep waves' prefetch of the next
// chunk does); __syncthreads() would drain them at every barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Load a T at a 32-bit byte offset from a workgroup-uniform base: the address is formed by
// the load itself (scalar base + vector offset), with no 64-bit address arithmetic.
template <typename T>
__device__ __forceinline__ T ld_at(const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Store two consecutive T at a 32-bit byte offset from a workgroup-uniform base.
template <typename T>
__device__ __forceinline__ void st2_at(void *base, uint32_t byte_off, float a, float b) {
    st2<T>(reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off), a, b);
}

// acc += A[16 x kdim] * B[kdim x 16] for the A-matrix tiles: A rows and B^T rows staged
// in the A-operand type (k contiguous).  With SPLIT both operands also have low parts
// (x - hi) `lo` elements further on, and the product is hi*hi + hi*lo + lo*hi (about 16
// mantissa bits).
template <class P, bool SPLIT, int kdim>
__device__ __forceinline__ void mma_stage(f4 &acc, const typename P::TA *A, int lda, const typename P::TA *B,
                                          int ldb, int lo, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if constexpr (std::is_same<typename P::TA, float>::value) {
#pragma unroll
        for (int k0 = 0; k0 < kdim; k0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + g], B[r * ldb + k0 + g], acc, 0, 0, 0);
    } else {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
        const bf16x4 z4 = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
        auto ld = [&](const __bf16 *p, int k0) -> bf16x8 {
            if (k0 + 32 > kdim) {
                // a 16-wide tail fills the lower half of the operand, the upper half is zero
                const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p + k0 + 4 * g);
                return __builtin_shufflevector(x, z4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return *reinterpret_cast<const bf16x8 *>(p + k0 + 8 * g);
        };
#pragma unroll
        for (int k0 = 0; k0 < kdim; k0 += 32) {
            const bf16x8 ah = ld(A + r * lda, k0), bh = ld(B + r * ldb, k0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
            if constexpr (SPLIT) {
                const bf16x8 al = ld(A + lo + r * lda, k0), bl = ld(B + lo + r * ldb, k0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
            }
        }
    }
}

// Store two staged values in the A-operand type; with a split precision also their low
// parts (x - hi), `lo` elements further on.
template <class P>
__device__ __forceinline__ void st2_stage(typename P::TA *p, int lo, float a, float b) {
    if constexpr (std::is_same<typename P::TA, float>::value) {
        *reinterpret_cast<float2 *>(p) = float2{a, b};
    } else {
        typedef __attribute__((ext_vector_type(2))) __bf16 v2;
        const v2 h = {(__bf16)a, (__bf16)b};
        *reinterpret_cast<v2 *>(p) = h;
        if constexpr (P::kSplit) {
            // the hi parts back in float32 straight from the packed pair (no second rounding)
            uint32_t hw = __builtin_bit_cast(uint32_t, h);
            asm("" : "+v"(hw));  // keeps the compiler from converting each hi part once more
            const float ha = __builtin_bit_cast(float, hw << 16), hb = __builtin_bit_cast(float, hw & 0xffff0000u);
            *reinterpret_cast<v2 *>(p + lo) = v2{(__bf16)(a - ha), (__bf16)(b - hb)};
        }
    }
}

// acc = X Y for 16x16 X, Y whose 16-wide reduction is held in registers: lane (g, r) gives
// xr[s] = X[r][4g+s] and lane (g, n) gives yc[s] = Y[4g+s][n] (k = 4g + s on both sides;
// the result is in the accumulator layout).  T is the operand type: float runs four fp32
// steps, _Float16 one 16x16x32 step with the upper half of each operand zero.
template <typename T>
__device__ __forceinline__ f4 mma16_reg(f4 xr, f4 yc);
template <>
__device__ __forceinline__ f4 mma16_reg<float>(f4 xr, f4 yc) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[s], yc[s], acc, 0, 0, 0);
    return acc;
}
template <>
__device__ __forceinline__ f4 mma16_reg<_Float16>(f4 xr, f4 yc) {
    const f16x8 a = {(_Float16)xr[0], (_Float16)xr[1], (_Float16)xr[2], (_Float16)xr[3], 0, 0, 0, 0};
    const f16x8 b = {(_Float16)yc[0], (_Float16)yc[1], (_Float16)yc[2], (_Float16)yc[3], 0, 0, 0, 0};
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, z, 0, 0, 0);
}

// Value of `v` in lane J of this lane's group of four.
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), J * 0x55, 0xf, 0xf, false));
}

// (I + A)^-1 for a 16x16 strictly lower triangular A given as an accumulator tile (lane
// (g, n) holds A[4g+e][n]; entries on and above the diagonal are ignored).  Returns the
// inverse in the same layout.  Blocked: with Ad the 4x4 diagonal blocks of A and Ao the
// rest, I + A = (I + Ad)(I + N), N = D Ao, D = (I + Ad)^-1; N is strictly lower at
// 4x4-block level, so N^4 = 0 and (I + A)^-1 = (I - N + N^2 - N^3) D.  The four 4x4
// inverses come from forward and backward substitution inside groups of four lanes; the
// rest is six 16x16 products on the matrix cores in operand type T.
template <typename T>
__device__ __forceinline__ f4 unit_lower_inverse16(const f4 a, int lane) {
    const int g = lane >> 4, n = lane & 15, c = n & 3;
    const bool diag = (n >> 2) == g;  // lanes holding column c of diagonal block g
    // entries a_ej = A[4g+e][4g+j] (e > j) of the diagonal block, from quad lane j
    const float a10 = quad_bcast<0>(a[1]), a20 = quad_bcast<0>(a[2]), a30 = quad_bcast<0>(a[3]);
    const float a21 = quad_bcast<1>(a[2]), a31 = quad_bcast<1>(a[3]);
    const float a32 = quad_bcast<2>(a[3]);
    // column c of the block inverse: x = e_c, then eliminate column by column
    float x0 = c == 0 ? 1.f : 0.f, x1 = c == 1 ? 1.f : 0.f, x2 = c == 2 ? 1.f : 0.f, x3 = c == 3 ? 1.f : 0.f;
    x1 -= a10 * x0;
    x2 -= a20 * x0 + a21 * x1;
    x3 -= a30 * x0 + a31 * x1 + a32 * x2;
    // row c of the block inverse: y = e_c^T, then eliminate from the right
    float y0 = c == 0 ? 1.f : 0.f, y1 = c == 1 ? 1.f : 0.f, y2 = c == 2 ? 1.f : 0.f, y3 = c == 3 ? 1.f : 0.f;
    y2 -= y3 * a32;
    y1 -= y2 * a21 + y3 * a31;
    y0 -= y1 * a10 + y2 * a20 + y3 * a30;
    // "c" = accumulator layout of a matrix, "r" = accumulator layout of its transpose
    // (lane (g, n) holds M[n][4g+e]), which is its row-operand form
    const f4 Dc = diag ? f4{x0, x1, x2, x3} : f4{0.f, 0.f, 0.f, 0.f};
    const f4 Dr = diag ? f4{y0, y1, y2, y3} : f4{0.f, 0.f, 0.f, 0.f};
    f4 Aoc;
#pragma unroll
    for (int e = 0; e < 4; ++e) Aoc[e] = (n >> 2) < g ? a[e] : 0.f;
    // P = X Y: Pc = mma(Xr, Yc) and Pr = mma(Yc, Xr)
    const f4 Nc = mma16_reg<T>(Dr, Aoc);
    const f4 Nr = mma16_reg<T>(Aoc, Dr);
    const f4 N2c = mma16_reg<T>(Nr, Nc);
    const f4 N2r = mma16_reg<T>(Nc, Nr);
    const f4 N3r = mma16_reg<T>(N2c, Nr);
    f4 Mr;
#pragma unroll
    for (int e = 0; e < 4; ++e) Mr[e] = (4 * g + e == n ? 1.f : 0.f) - Nr[e] + N2r[e] - N3r[e];
    return mma16_reg<T>(Mr, Dc);
}

// One step of a recursive-halving sum over lanes: lanes with bit M set keep the upper
// HALF of their 2*HALF partial sums, the others the lower half, and each adds what the
// partner (lane ^ M) sends of the same half.  Compile-time sizes keep every array index
// static (a select between two indices would become a dynamic index into the array).
template <int HALF, bool ON, int M, int N>
__device__ __forceinline__ void halve_sums(float (&x)[N], int lane, int &base) {
    if constexpr (ON) {
        const bool up = (lane & M) != 0;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const float lo = x[i], hi = x[i + HALF];
            const float keep = up ? hi : lo;
            const float send = up ? lo : hi;
            x[i] = keep + __shfl_xor(send, M);
        }
        base += up ? HALF : 0;
    }
}

// The A-matrix work of one chunk, shared out over NW waves (w = 0..NW-1).  Wave p % NW
// computes A_kk's diagonal tile p and inverts I + A_pp, giving T's diagonal block p; the off-diagonal A_kk tiles (kept in fp32 for T's off-diagonal
// blocks) and the lower A_qk tiles are dealt round-robin after them.  Reads the operand
// staging of the chunk; writes Akk, Tf and the Tm / Aqk tiles of package `pk`.
// With NORM the staged operands carry the raw q and k; the tiles are scaled by the
// reciprocal row norms (A_kk[i,j] by 1/(|k_i||k_j|), A_qk[i,j] by 1/(|q_i||k_j|)),
// which the prep waves left in LDS as per-wave partial sums of squares.
// INVN: the reciprocal row norms are already in the row-norm buffer after buffer nb, as
// [q rows, k rows] (the pre-pass forms them once per item).
template <class P, int K, int V, int C, int BV, bool NORM, int NW = 4, bool INVN = false>
__device__ __forceinline__ void a_matrix_work(unsigned char *smem, unsigned char *pk, int nb, int w, int lane) {
    using L = Layout<P, K, V, C, BV>;
    static_assert(L::KS == K, "the whole key width is staged (else a_matrix_work_blocks)");
    using TA = typename P::TA;
    using TM = typename P::TM;
    constexpr int NP = L::NP;
    const int g = lane >> 4;
    const TA *Lk = reinterpret_cast<const TA *>(smem + L::oLk);
    const TA *St = reinterpret_cast<const TA *>(smem + L::oSt);
    float *Akk = reinterpret_cast<float *>(smem + L::oAkk);
    float *Tf = reinterpret_cast<float *>(smem + L::oTf);
    TM *Tm = reinterpret_cast<TM *>(pk + L::pTm);
    TM *Aqk = reinterpret_cast<TM *>(pk + L::pAqk);
    TM *Aql = reinterpret_cast<TM *>(pk + L::pAql);
    const float *Nrm = reinterpret_cast<const float *>(smem + L::oNrm) + nb * L::NNRM;
    // 1 / max(|x_r|, 1e-6) of chunk row r, for x = q (qk = 0) or k (qk = 1)
    auto inv_norm = [&](int qk, int r) -> float {
        if constexpr (INVN) return Nrm[L::NNRM + qk * C + r];
        float n = 0.f;
#pragma unroll
        for (int pt = 0; pt < L::NPART; ++pt) n += Nrm[(((r >> 4) * 2 + qk) * 16 + (r & 15)) * L::NPART + pt];
        return __builtin_amdgcn_rsqf(fmaxf(n, 1e-12f));
    };
    // right operand of tile (p, qt)
    auto right_of = [&](int p, int qt) -> const TA * {
        if (qt == p) return St + L::sRd + qt * 16 * L::LKS;
        if (qt == p - 1) return St + L::sRo + qt * 16 * L::LKS;
        int xi = 0;
        for (int pp = 2; pp < p; ++pp) xi += pp - 1;
        return St + L::sX + (xi + qt) * 16 * L::LKS;
    };
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if ((p % NW) != w) continue;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        mma_stage<P, false, K>(acc, Lk + p * 16 * L::LKA, L::LKA, right_of(p, p), L::LKS, 0, lane);
        if constexpr (NORM) {
            const float cj = inv_norm(1, p * 16 + (lane & 15));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= cj * inv_norm(1, p * 16 + 4 * g + e);
        }
        const f4 t = unit_lower_inverse16<TM>(acc, lane);
        const int j = lane & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            const float x = (j <= i) ? t[e] : 0.f;
            Tf[(p * 16 + i) * L::LCF + p * 16 + j] = x;
            Tm[(p * 16 + i) * L::LCM + p * 16 + j] = from_f32<TM>(x);
        }
    }
    constexpr int NOFF = NP * (NP - 1) / 2;
    int t = 0;
#pragma unroll
    for (int p = 1; p < NP; ++p)
#pragma unroll
        for (int qt = 0; qt < p; ++qt, ++t) {
            if (((t + NP) % NW) != w) continue;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_stage<P, false, K>(acc, Lk + p * 16 * L::LKA, L::LKA, right_of(p, qt), L::LKS, 0, lane);
            const int i0 = p * 16 + 4 * g, j = qt * 16 + (lane & 15);
            if constexpr (NORM) {
                const float cj = inv_norm(1, j);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= cj * inv_norm(1, i0 + e);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Akk[(i0 + e) * L::LCF + j] = acc[e];
        }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int qt = 0; qt <= p; ++qt) {
            const int tq = NOFF + p * (p + 1) / 2 + qt;
            if (((tq + NP) % NW) != w) continue;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_stage<P, P::kSplit, K>(acc, St + L::sLq + p * 16 * L::LKS, L::LKS, right_of(p, qt), L::LKS, L::NST, lane);
            const int i0 = p * 16 + 4 * g, j = qt * 16 + (lane & 15);
            if constexpr (NORM) {
                const float cj = inv_norm(1, j);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= cj * inv_norm(0, i0 + e);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = (j <= i0 + e) ? acc[e] : 0.f;
                const TM hi = from_f32<TM>(x);
                Aqk[(i0 + e) * L::LCM + j] = hi;
                if constexpr (P::kAqParts == 2) Aql[(i0 + e) * L::LCM + j] = from_f32<TM>(x - to_f32(hi));
            }
        }
}

// a_matrix_work for a staging area that holds KS < K key columns at a time (the pre-pass of
// 64-token chunks at K = 128).  Every tile's product is a sum over the key index, so each
// tile accumulates over the K / KS column blocks in registers: block 0 is staged by the
// caller before the call, restage(b) stages block b >= 1 (barriers included).  The tiles are
// a_matrix_work's, in its order (diagonal A_kk tiles, lower A_kk tiles, lower A_qk tiles),
// tile i on wave i % NW; the products are finished as there.  The reciprocal row norms
// (NORM) are read from the table after the first row-norm buffer.
template <class P, int K, int C, bool NORM, int NW, class Restage>
__device__ __forceinline__ void a_matrix_work_blocks(unsigned char *smem, unsigned char *pk, int w, int lane,
                                                     Restage &&restage) {
    using L = Layout<P, K, 16, C, 16>;
    using TA = typename P::TA;
    using TM = typename P::TM;
    constexpr int NP = L::NP;
    constexpr int NOFF = NP * (NP - 1) / 2;
    constexpr int NT = NP + NOFF + NP * (NP + 1) / 2;
    constexpr int MS = (NT + NW - 1) / NW;  // tiles per wave, at most
    constexpr int NB = K / L::KS;
    static_assert(NB * L::KS == K, "the column blocks cover the key width");
    const int g = lane >> 4;
    const TA *Lk = reinterpret_cast<const TA *>(smem + L::oLk);
    const TA *St = reinterpret_cast<const TA *>(smem + L::oSt);
    float *Akk = reinterpret_cast<float *>(smem + L::oAkk);
    float *Tf = reinterpret_cast<float *>(smem + L::oTf);
    TM *Tm = reinterpret_cast<TM *>(pk + L::pTm);
    TM *Aqk = reinterpret_cast<TM *>(pk + L::pAqk);
    TM *Aql = reinterpret_cast<TM *>(pk + L::pAql);
    const float *InvN = reinterpret_cast<const float *>(smem + L::oNrm) + L::NNRM;  // [q rows, k rows]
    // tile i: kind 0 (diagonal A_kk tile p), 1 (A_kk tile (p, qt), qt < p), 2 (A_qk tile (p, qt), qt <= p)
    auto decode = [&](int i, int &kind, int &p, int &qt) {
        if (i < NP) {
            kind = 0;
            p = qt = i;
        } else if (i < NP + NOFF) {
            kind = 1;
            int t = i - NP;
            p = 1;
            while (t >= p) { t -= p; ++p; }
            qt = t;
        } else {
            kind = 2;
            int t = i - NP - NOFF;
            p = 0;
            while (t > p) { t -= p + 1; ++p; }
            qt = t;
        }
    };
    auto right_of = [&](int p, int qt) -> const TA * {
        if (qt == p) return St + L::sRd + qt * 16 * L::LKS;
        if (qt == p - 1) return St + L::sRo + qt * 16 * L::LKS;
        int xi = 0;
        for (int pp = 2; pp < p; ++pp) xi += pp - 1;
        return St + L::sX + (xi + qt) * 16 * L::LKS;
    };
    f4 acc[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < NB; ++b) {
        if (b > 0) restage(b);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int i = w + NW * m;
            if (i >= NT) continue;  // wave-uniform
            int kind, p, qt;
            decode(i, kind, p, qt);
            if (kind == 2)
                mma_stage<P, P::kSplit, L::KS>(acc[m], St + L::sLq + p * 16 * L::LKS, L::LKS, right_of(p, qt), L::LKS,
                                               L::NST, lane);
            else
                mma_stage<P, false, L::KS>(acc[m], Lk + p * 16 * L::LKA, L::LKA, right_of(p, qt), L::LKS, 0, lane);
        }
    }
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        const int i = w + NW * m;
        if (i >= NT) continue;
        int kind, p, qt;
        decode(i, kind, p, qt);
        f4 x = acc[m];
        const int i0 = p * 16 + 4 * g, j = qt * 16 + (lane & 15);
        if constexpr (NORM) {
            const float cj = InvN[C + j];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] *= cj * InvN[(kind == 2 ? 0 : C) + i0 + e];
        }
        if (kind == 0) {
            const f4 t = unit_lower_inverse16<TM>(x, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float y = (j <= i0 + e) ? t[e] : 0.f;
                Tf[(i0 + e) * L::LCF + j] = y;
                Tm[(i0 + e) * L::LCM + j] = from_f32<TM>(y);
            }
        } else if (kind == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Akk[(i0 + e) * L::LCF + j] = x[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float y = (j <= i0 + e) ? x[e] : 0.f;
                const TM hi = from_f32<TM>(y);
                Aqk[(i0 + e) * L::LCM + j] = hi;
                if constexpr (P::kAqParts == 2) Aql[(i0 + e) * L::LCM + j] = from_f32<TM>(y - to_f32(hi));
            }
        }
    }
}

// 2^e as a float (e clamped to the normal range)
__device__ __forceinline__ float pow2f(int e) {
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    return __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
}

// largest magnitude over this lane's accumulator tiles (a pairwise tree: short dependences)
template <int N>
__device__ __forceinline__ float maxabs(const f4 (&x)[N]) {
    float m[N];
#pragma unroll
    for (int i = 0; i < N; ++i) m[i] = fmaxf(fmaxf(fabsf(x[i][0]), fabsf(x[i][1])), fmaxf(fabsf(x[i][2]), fabsf(x[i][3])));
#pragma unroll
    for (int w = 1; w < N; w *= 2)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) m[i] = fmaxf(m[i], m[i + w]);
    return m[0];
}

// The exponent s >= 0 of the power-of-two scale that brings the wave's largest magnitude
// m below 2^15, inside the 16-bit float range (0 whenever m < 2^15).
__device__ __forceinline__ int wave_scale_exp(float m) {
    m = fmaxf(m, row_ror<8>(m));
    m = fmaxf(m, row_ror<4>(m));
    m = fmaxf(m, row_ror<2>(m));
    m = fmaxf(m, row_ror<1>(m));
    const int b = __builtin_bit_cast(int, m);
    const int r = max(max(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16)),
                      max(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48)));
    const int e = (r >> 23) & 0xff;  // biased exponent of the wave's maximum
    return e > 141 ? e - 141 : 0;
}

// hi + lo 16-bit operand parts of accumulator tiles (lo = the rounded remainder x - hi):
// with both parts a product keeps about 22 mantissa bits of x
template <int NKT>
__device__ __forceinline__ void set_split(BFrag<_Float16, NKT> &hi, BFrag<_Float16, NKT> &lo, const f4 (&t)[NKT]) {
    hi.set(t);
    f4 r[NKT];
#pragma unroll
    for (int i = 0; i < NKT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[i][e] = t[i][e] - (float)(_Float16)t[i][e];
    lo.set(r);
}
template <int NKT>
__device__ __forceinline__ void set_split(BFrag<float, NKT> &hi, BFrag<float, NKT> &, const f4 (&t)[NKT]) {
    hi.set(t);  // float32 operands: no low part
}

// Sh = the 16-bit operand form of the state S 2^-sS, with sS from the state's magnitude on
// the 16-bit path (always 0 on the float32 path).
template <bool P16, typename TM, int NKT>
__device__ __forceinline__ void set_state_frag(BFrag<TM, NKT> &Sh, int &sS, const f4 (&S)[NKT]) {
    sS = 0;
    if constexpr (P16) {
        sS = wave_scale_exp(maxabs(S));
        if (sS) {
            const float d = pow2f(-sS);
            f4 x[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) x[t] = S[t] * d;
            Sh.set(x);
            return;
        }
    }
    Sh.set(S);
}

// The state waves (w = 0..NSW-1): the float32 state of this workgroup's value columns in
// registers, advanced chunk by chunk through the serial part.  The packages sit at pkg0 in
// two buffers, by chunk parity.  Without PK the state waves also do the A-matrix work of
// the chunk staged in the previous period (two barriers a period); with PK each package
// arrives complete from the pre-pass (one barrier a period), its matrix operands stored
// with the row swizzle of mma_bfrag.
template <class P, int K, int V, int C, int BV, bool NORM, bool PK, bool FEW_REGS = false>
__device__ __forceinline__ void state_waves(const ChunkArgs &a, unsigned char *smem, unsigned char *pkg0, int s,
                                            int h, int vb, int64_t bos, int64_t eos, int nchunks, int wave,
                                            int lane) {
    using L = Layout<P, K, V, C, BV>;
    using TM = typename P::TM;
    using TIn = typename std::conditional<std::is_same<P, PrecF32>::value, float, __bf16>::type;
    constexpr bool P16 = !std::is_same<TM, float>::value;  // 16-bit matrix-core operands
    // Lean order (fewer fragments live at once): the single kernel, whose twelve waves have
    // fewer registers each, float32 fragments of 64-token chunks, and 16-bit fragments of
    // 64-token chunks at K = 128.
    constexpr bool LEAN = FEW_REGS || !PK || (!P16 && C >= 64) || L::kWide;
    constexpr int NP = L::NP;
    constexpr int NKT_K = K / 16;
    const int g = lane >> 4;
    const int H = a.H;
    auto pkg = [&](int buf) { return pkg0 + (size_t)buf * L::szPkg; };
    f4 S[L::MJ][NKT_K];
    const float *s0 = a.initial_state ? a.initial_state + ((int64_t)s * H + h) * K * V : nullptr;
#pragma unroll
    for (int mj = 0; mj < L::MJ; ++mj) {
        const int jt = wave + NSW * mj;
#pragma unroll
        for (int t = 0; t < NKT_K; ++t) {
            f4 x = {0.f, 0.f, 0.f, 0.f};
            if (jt < L::NJT && s0) {
                const int vc = vb * BV + jt * 16 + (lane & 15);
                if (a.state_vk) {
                    const float4 y = *reinterpret_cast<const float4 *>(s0 + (int64_t)vc * K + 16 * t + 4 * g);
                    x[0] = y.x; x[1] = y.y; x[2] = y.z; x[3] = y.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = s0[(int64_t)(16 * t + 4 * g + e) * V + vc];
                }
            }
            S[mj][t] = x;
        }
    }
    BFrag<TM, NKT_K> Sh[L::MJ];  // the state as a 16-bit operand: S 2^-sS
    int sS[L::MJ];
#pragma unroll
    for (int mj = 0; mj < L::MJ; ++mj) set_state_frag<P16>(Sh[mj], sS[mj], S[mj]);

    for (int it = 0; it <= nchunks; ++it) {
        if constexpr (!PK) {
            float *Akk = reinterpret_cast<float *>(smem + L::oAkk);
            float *Tf = reinterpret_cast<float *>(smem + L::oTf);
            // the A-matrix tiles and T's diagonal blocks of the chunk staged in the previous
            // period, whose package the serial part consumes after the next barrier
            if (it >= 1) a_matrix_work<P, K, V, C, BV, NORM>(smem, pkg((it - 1) & 1), (it - 1) & 1, wave, lane);
            lds_barrier();  // B1: chunk it-1's A-matrix tiles are done; chunk it's decay products are in LDS
            if (NP > 1 && it >= 1) {
                // T's off-diagonal blocks of the chunk about to be consumed, one block
                // distance at a time on fp32 matrix cores:
                //   M = sum_{r=q}^{p-1} A_pr T_rq,   T_pq = -T_pp M
                // Every state wave computes all of them: it reads back only what it wrote
                // itself, and the other waves write the same values to the same places, so
                // no barrier is needed before the serial part uses them.
                TM *Tm = reinterpret_cast<TM *>(pkg((it - 1) & 1) + L::pTm);
                for (int d = 1; d < NP; ++d) {
                    for (int qb = 0; qb + d < NP; ++qb) {
                        const int p = qb + d;
                        f4 m = {0.f, 0.f, 0.f, 0.f};
                        for (int r = qb; r < p; ++r)
#pragma unroll
                            for (int s4 = 0; s4 < 4; ++s4)
                                m = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    Akk[(p * 16 + (lane & 15)) * L::LCF + r * 16 + 4 * s4 + g],
                                    Tf[(r * 16 + 4 * s4 + g) * L::LCF + qb * 16 + (lane & 15)], m, 0, 0, 0);
                        // M's accumulator layout is the B operand with k = 4g + s4
                        f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4)
                            t = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                Tf[(p * 16 + (lane & 15)) * L::LCF + p * 16 + 4 * g + s4], m[s4], t, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = p * 16 + 4 * g + e, j = qb * 16 + (lane & 15);
                            Tf[i * L::LCF + j] = -t[e];
                            Tm[i * L::LCM + j] = from_f32<TM>(-t[e]);
                        }
                    }
                    lds_fence();
                }
            }
        }
        const int cn = it - 1;  // chunk handled by the state waves in this iteration
        if (cn >= 0) {
            // The package of chunk cn is complete in LDS.  Its operand fragments are read in
            // three groups, each issued before the products of the phase ahead of it, so their
            // LDS latency overlaps the previous phase instead of stalling every product.
            const unsigned char *pk = pkg(cn & 1);
            const TM *Qt = reinterpret_cast<const TM *>(pk + L::pQt);
            const TM *Bw = reinterpret_cast<const TM *>(pk + L::pBw);
            const TM *Kt = reinterpret_cast<const TM *>(pk + L::pKt);
            const TM *Tm = reinterpret_cast<const TM *>(pk + L::pTm);
            const TM *Aqk = reinterpret_cast<const TM *>(pk + L::pAqk);
            const TM *Aql = reinterpret_cast<const TM *>(pk + L::pAql);
            const TIn *vL = reinterpret_cast<const TIn *>(pk + L::pbV);
            const float *eGC = reinterpret_cast<const float *>(pk + L::pGC);
            const float *bL = reinterpret_cast<const float *>(pk + L::pBt);
            const int r16 = lane & 15;
            // group 1: -Bw and T (Y and Vt), beta V in float32
            AFrag<TM, NKT_K> fb[NP];
            AFrag<TM, NP> ft[NP];
            f4 bv[L::MJ][NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                fb[p].template load<PK>(Bw + (16 * p + r16) * L::LKM, NKT_K, lane);
                ft[p].template load<PK>(Tm + (16 * p + r16) * L::LCM, p + 1, lane);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float4 b4 = *reinterpret_cast<const float4 *>(bL + 16 * p + 4 * g);
#pragma unroll
                for (int mj = 0; mj < L::MJ; ++mj) {
                    const int jt = wave + NSW * mj < L::NJT ? wave + NSW * mj : 0;
                    const TIn *vr = vL + (jt * 16 + r16) * L::LCM + 16 * p + 4 * g;
                    bv[mj][p] = f4{b4.x * to_f32(vr[0]), b4.y * to_f32(vr[1]), b4.z * to_f32(vr[2]),
                                   b4.w * to_f32(vr[3])};
                }
            }
            sched_fence();
            // group 2: Qt and A_qk (the output); in the lean order after Y and Vt
            AFrag<TM, NKT_K> fq[NP];
            AFrag<TM, NP> fa[NP], fl[NP];  // A_qk, and its low part on the 16-bit path
            auto load_group2 = [&]() {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    fq[p].template load<PK>(Qt + (16 * p + r16) * L::LKM, NKT_K, lane);
                    fa[p].template load<PK>(Aqk + (16 * p + r16) * L::LCM, p + 1, lane);
                    if constexpr (P16) fl[p].template load<PK>(Aql + (16 * p + r16) * L::LCM, p + 1, lane);
                }
                sched_fence();
            };
            if constexpr (!LEAN) load_group2();
            // With 16-bit operands every product input goes through an exact power-of-two
            // scale 2^-x chosen per wave so its largest magnitude stays below 2^15 (x = 0
            // unless a value reaches that): sS for the state, sY for Y, sV for Vt, each
            // relative to the one before.  The float32 quantities are rescaled by the same
            // powers of two, so any finite state or value magnitude stays in range.
            // On the 16-bit path Y and Vt enter their products as hi + lo parts: the
            // products that carry a token's own value into its output and into the state
            // need more than fp16's 11 bits for the workload's largest outputs.
            BFrag<TM, NP> Vh[L::MJ], Vl[L::MJ];
            int sV[L::MJ];  // Vh (+ Vl) holds Vt 2^-(sS + sY + sV)
#pragma unroll
            for (int mj = 0; mj < L::MJ; ++mj) {
                sV[mj] = 0;
                if (wave + NSW * mj >= L::NJT) continue;
                // Y = beta V - Bw S   (rows: tokens; this wave's 16 columns), kept as Y 2^-sS
                const float dS = pow2f(-sS[mj]);
                f4 Y[NP];
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    Y[p] = bv[mj][p] * dS;
                    mma_frag<false>(Y[p], fb[p], Sh[mj], NKT_K);
                }
                int sY = 0;
                if constexpr (P16) {
                    sY = wave_scale_exp(maxabs(Y));
                    if (sY) {
                        const float d = pow2f(-sY);
#pragma unroll
                        for (int p = 0; p < NP; ++p) Y[p] *= d;
                    }
                }
                BFrag<TM, NP> Yh, Yl;
                set_split(Yh, Yl, Y);
                // Vt = T Y (T lower triangular: row tile p needs token tiles 0..p)
                f4 Vt[NP];
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    Vt[p] = f4{0.f, 0.f, 0.f, 0.f};
                    mma_frag<false>(Vt[p], ft[p], Yh, p + 1);
                    if constexpr (P16) mma_frag<false>(Vt[p], ft[p], Yl, p + 1);
                }
                int sv = 0;
                if constexpr (P16) {
                    sv = wave_scale_exp(maxabs(Vt));
                    if (sv) {
                        const float d = pow2f(-sv);
#pragma unroll
                        for (int p = 0; p < NP; ++p) Vt[p] *= d;
                    }
                }
                set_split(Vh[mj], Vl[mj], Vt);
                sV[mj] = sY + sv;
            }
            if constexpr (LEAN) load_group2();
            // group 3: Kt and gamma_C (the state update); in the lean order after the output
            AFrag<TM, NP> fk[NKT_K];
            f4 gc[NKT_K];
            auto load_group3 = [&]() {
#pragma unroll
                for (int t = 0; t < NKT_K; ++t) {
                    fk[t].template load<PK>(Kt + (16 * t + r16) * L::LCM, NP, lane);
                    const float4 d = *reinterpret_cast<const float4 *>(eGC + 16 * t + 4 * g);
                    gc[t] = f4{d.x, d.y, d.z, d.w};
                }
                sched_fence();
            };
            if constexpr (!LEAN) load_group3();
            const int64_t t0 = bos + (int64_t)cn * C;
            const int n = (int)((eos - t0) < C ? (eos - t0) : C);
            unsigned char *ob = static_cast<unsigned char *>(a.out) + (t0 * H + h) * V * (a.out_bf16 ? 2 : 4);
#pragma unroll
            for (int mj = 0; mj < L::MJ; ++mj) {
                const int jt = wave + NSW * mj;
                if (jt >= L::NJT) continue;
                // O^T = S^T Qt^T + Vt^T A_qk^T: lane (g, r16) holds value columns 4g..4g+3 of
                // token r16 of the tile, one 8- or 16-byte store per tile
                const int j0 = vb * BV + jt * 16 + 4 * g;
                const float dV = pow2f(-sV[mj]);                       // S-scaled -> Vt-scaled
                const float uO = a.scale * pow2f(sS[mj] + sV[mj]);     // Vt-scaled -> output
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    f4 o = {0.f, 0.f, 0.f, 0.f};
                    mma_frag<true>(o, fq[p], Sh[mj], NKT_K);
                    o *= dV;
                    mma_frag<true>(o, fa[p], Vh[mj], p + 1);
                    if constexpr (P16) {
                        mma_frag<true>(o, fa[p], Vl[mj], p + 1);
                        mma_frag<true>(o, fl[p], Vh[mj], p + 1);
                    }
                    o *= uO;
                    const int i = 16 * p + r16;
                    const uint32_t off = (uint32_t)(i * H * V + j0);
                    if (i < n) {
                        if (a.out_bf16) {
                            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                            *reinterpret_cast<bf16x4 *>(ob + 2u * off) =
                                bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                        } else {
                            *reinterpret_cast<float4 *>(ob + 4u * off) = float4{o[0], o[1], o[2], o[3]};
                        }
                    }
                }
                if (LEAN && mj == 0) load_group3();
                // S = gamma_C S + Kt^T Vt, accumulated as S 2^-w with w the scale of Vh
                const int w = sS[mj] + sV[mj];
                const float dW = pow2f(-w), uW = pow2f(w);
#pragma unroll
                for (int t = 0; t < NKT_K; ++t) {
                    f4 x = S[mj][t];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] *= gc[t][e] * dW;
                    mma_frag<false>(x, fk[t], Vh[mj], NP);
                    if constexpr (P16) mma_frag<false>(x, fk[t], Vl[mj], NP);
                    S[mj][t] = x * uW;
                }
                set_state_frag<P16>(Sh[mj], sS[mj], S[mj]);
            }
        }
        // B2 (with the package built in the workgroup: chunk it is staged and its package
        // operands are stored); with PK the one barrier of the period: the next package is in LDS
        lds_barrier();
    }
    if (a.final_state) {
        float *sf = a.final_state + ((int64_t)s * H + h) * K * V;
#pragma unroll
        for (int mj = 0; mj < L::MJ; ++mj) {
            const int jt = wave + NSW * mj;
            if (jt >= L::NJT) continue;
            const int vc = vb * BV + jt * 16 + (lane & 15);
#pragma unroll
            for (int t = 0; t < NKT_K; ++t) {
                if (a.state_vk) {
                    *reinterpret_cast<float4 *>(sf + (int64_t)vc * K + 16 * t + 4 * g) =
                        float4{S[mj][t][0], S[mj][t][1], S[mj][t][2], S[mj][t][3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sf[(int64_t)(16 * t + 4 * g + e) * V + vc] = S[mj][t][e];
                }
            }
        }
    }
}

// GM = 0: the gate is a float32 tensor of alpha or ln alpha (a.gate.mode); GM = 1: it
// arrives as logits (GATE_LOGITS) and is evaluated in the prep waves; GM = 2: as 1, and q
// and k are also divided by their L2 norms over K in the prep waves.
template <class P, int K, int V, int C, int BV, int GM>
__global__ __launch_bounds__(NT) void chunk_fwd_kernel(ChunkArgs a) {
    constexpr bool ZG = GM >= 1;
    constexpr bool NORM = GM == 2;
    using L = Layout<P, K, V, C, BV>;
    using TA = typename P::TA;
    using TM = typename P::TM;
    using TIn = typename std::conditional<std::is_same<P, PrecF32>::value, float, __bf16>::type;
    constexpr int NP = L::NP;
    constexpr int NKT_K = K / 16;  // 16-channel tiles

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;

    // ---- which (sequence, head, value block) this workgroup owns ----------------------
    constexpr int NVB = V / BV;
    const int G = gridDim.x;
    int lin = blockIdx.x;
    if ((G & 7) == 0) lin = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);  // a head's value blocks
    const int vb = lin % NVB;                                                   // share one XCD
    const int pair = lin / NVB;
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
    const int nchunks = (int)((eos - bos + C - 1) / C);
    const TIn *q = static_cast<const TIn *>(a.q);
    const TIn *k = static_cast<const TIn *>(a.k);
    const TIn *v = static_cast<const TIn *>(a.v);

    auto pkg = [&](int buf) { return smem + L::oPkg + (size_t)buf * L::szPkg; };

    if (wave < NSW) {
        state_waves<P, K, V, C, BV, NORM, false>(a, smem, smem + L::oPkg, s, h, vb, bos, eos, nchunks, wave,
                                                 lane);
        return;
    }

    // ====================================== prep waves =======================================
    const int tp = tid - NSW * 64;  // 0 .. NPT-1
    const int pw = wave - NSW;      // prep wave 0..NPW-1
    TA *Lk = reinterpret_cast<TA *>(smem + L::oLk);         // [C][LKA]
    TA *St = reinterpret_cast<TA *>(smem + L::oSt);         // Lq, Rd, Ro, X (+ low parts)
    float *TPv = reinterpret_cast<float *>(smem + L::oTP);  // [NP][K] tile decay products
    float *Btv = reinterpret_cast<float *>(smem + L::oBt);  // [C] beta of the chunk
    float *Nrm = reinterpret_cast<float *>(smem + L::oNrm); // row-norm partials

    // The strictly upper 16x16 blocks of T and A_qk are zero in every chunk: write them
    // once, in both package buffers.  (The state waves first read a package after the
    // first iteration's last barrier.)
    for (int buf = 0; buf < 2; ++buf) {
        TM *Tm = reinterpret_cast<TM *>(pkg(buf) + L::pTm);
        TM *Aq = reinterpret_cast<TM *>(pkg(buf) + L::pAqk);
        TM *Al = reinterpret_cast<TM *>(pkg(buf) + L::pAql);
        for (int e = tp; e < C * C; e += NPT) {
            const int i = e / C, j = e % C;
            if ((j >> 4) > (i >> 4)) {
                Tm[i * L::LCM + j] = from_f32<TM>(0.f);
                Aq[i * L::LCM + j] = from_f32<TM>(0.f);
                if constexpr (P::kAqParts == 2) Al[i * L::LCM + j] = from_f32<TM>(0.f);
            }
        }
    }

    // Prep mapping: a "combo" is a (channel pair, 16-row tile); each combo is handled by
    // four lanes of one wave, lanes l, l + 16, l + 32 and l + 48 (l < 16) taking rows
    // 0..3, 4..7, 8..11 and 12..15 of the tile, so in-tile prefix and suffix decay
    // products need one exchange among the four.
    constexpr int NCP = K / 2;                   // channel pairs
    constexpr int NCOMBO = NCP * NP;
    constexpr int CPR = 16 * NPW;                // combos per round (16 lane quadruples per wave)
    constexpr int CPT = (NCOMBO + CPR - 1) / CPR;  // combos per lane quadruple
    const int qd = lane >> 4;                    // which quarter of the tile
    auto combo_of = [&](int u) { return CPR * u + 16 * pw + (lane & 15); };

    // Raw inputs of one chunk: for each combo, 4 rows x 2 channels of the gate, q and k;
    // beta of row tp; this thread's share of the value block.  The loads are
    // unconditional (rows past the sequence end read its last row) and nothing is
    // computed from them until they are used in the next iteration, so they stay in
    // flight while the current chunk is processed; the padding rows are masked at use.
    using RawIn = typename std::conditional<std::is_same<TIn, float>::value, float, unsigned short>::type;
    using RawPair = typename std::conditional<std::is_same<TIn, float>::value, float2, uint32_t>::type;
    float2 ral[CPT][4];
    RawPair rq[CPT][4], rk[CPT][4];
    float rbeta = 0.f;
    constexpr int NVE = (BV * C / 2 + NPT - 1) / NPT;  // (column, token pair) items per prep thread
    RawIn rv[NVE][2];
    // a gate given as logits: the per-head scale and this thread's channel biases
    const bool glog = a.gate.mode == GATE_LOG;
    float gs2 = 0.f, gl2 = 0.f;
    float2 zbias[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) zbias[u] = float2{0.f, 0.f};
    if constexpr (ZG) {
        gs2 = expf(a.gate.log_scale[h]) * 1.44269504088896341f;  // e^A log2(e)
        gl2 = a.gate.lower_bound * 1.44269504088896341f;
        if (a.gate.bias) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u) < NCOMBO ? combo_of(u) : 0;
                const float *bp = a.gate.bias + h * K + 2 * (cm % NCP);
                zbias[u] = float2{bp[0], bp[1]};
            }
        }
    }
    auto load_raw = [&](int cn) {
        const int64_t t0 = bos + (int64_t)cn * C;
        const int last = (int)((eos - t0) < C ? (eos - t0) : C) - 1;  // last valid row (>= 0)
        const int rs = H * K;                                        // row stride of q, k, gate
        const int64_t cb = (t0 * H + h) * K;                         // chunk base (uniform)
        const float *gb = a.gate.gate + cb;
        const RawIn *zb = reinterpret_cast<const RawIn *>(a.gate.logits) + cb;
        const RawIn *qb = reinterpret_cast<const RawIn *>(q) + cb;
        const RawIn *kb = reinterpret_cast<const RawIn *>(k) + cb;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int cm = combo_of(u) < NCOMBO ? combo_of(u) : 0;
            const int c0 = 2 * (cm % NCP);
            int p = cm / NCP;
            if constexpr (NCP % 16 == 0) p = __builtin_amdgcn_readfirstlane(p);  // one tile per wave
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * p + 4 * qd + i;
                const uint32_t o = (uint32_t)((r < last ? r : last) * rs + c0);
                const uint32_t ob = o * (uint32_t)sizeof(RawIn);  // byte offsets from uniform bases
                if constexpr (!ZG) {
                    ral[u][i] = ld_at<float2>(gb, 4u * o);
                } else if constexpr (std::is_same<RawPair, float2>::value) {
                    ral[u][i] = ld_at<float2>(zb, ob);
                } else {
                    ral[u][i].x = __builtin_bit_cast(float, ld_at<RawPair>(zb, ob));
                }
                rq[u][i] = ld_at<RawPair>(qb, ob);
                rk[u][i] = ld_at<RawPair>(kb, ob);
            }
        }
        rbeta = ld_at<float>(a.beta + t0 * H + h, 4u * (uint32_t)((tp < last ? tp : last) * H));
        const RawIn *vbp = reinterpret_cast<const RawIn *>(v) + (t0 * H + h) * V + vb * BV;
#pragma unroll
        for (int w = 0; w < NVE; ++w) {
            const int e = (tp + NPT * w) % (BV * C / 2);
            const int j = e % BV, r = 2 * (e / BV);
            rv[w][0] = ld_at<RawIn>(vbp, (uint32_t)sizeof(RawIn) * (uint32_t)((r < last ? r : last) * H * V + j));
            rv[w][1] = ld_at<RawIn>(vbp, (uint32_t)sizeof(RawIn) * (uint32_t)((r + 1 < last ? r + 1 : last) * H * V + j));
        }
    };
    auto raw_f32 = [&](RawIn x) -> float {
        if constexpr (std::is_same<RawIn, float>::value) return x;
        else return __builtin_bit_cast(float, (uint32_t)x << 16);
    };
    auto pair_f32 = [&](RawPair x, float &lo, float &hi) {
        if constexpr (std::is_same<RawPair, float2>::value) {
            lo = x.x;
            hi = x.y;
        } else {
            lo = __builtin_bit_cast(float, x << 16);
            hi = __builtin_bit_cast(float, x & 0xffff0000u);
        }
    };
    if (nchunks > 0) load_raw(0);

    // per combo: decay factors entering this quarter from the others (prefix: product of the
    // tile's rows before it; suffix: product of the rows after it)
    float2 pin[CPT], sin[CPT];
    for (int it = 0; it <= nchunks; ++it) {
        const bool work = it < nchunks;
        const int n_it = work ? (int)((eos - (bos + (int64_t)it * C)) < C ? (eos - (bos + (int64_t)it * C)) : C) : 0;
        // ---- phase 1a: retention factors (1 on padding rows), tile totals, beta --------
        if (work) {
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u);
                const int p = cm / NCP;
                float2 run = {1.f, 1.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float2 al = ral[u][i];
                    if constexpr (!ZG) {
                        if (glog) {
                            al.x = __expf(al.x);
                            al.y = __expf(al.y);
                        }
                    } else {
                        float z0, z1;
                        if constexpr (std::is_same<RawPair, float2>::value) {
                            z0 = al.x;
                            z1 = al.y;
                        } else {
                            pair_f32(__builtin_bit_cast(RawPair, al.x), z0, z1);
                        }
                        al.x = fast_bounded_alpha(z0 + zbias[u].x, gs2, gl2);
                        al.y = fast_bounded_alpha(z1 + zbias[u].y, gs2, gl2);
                    }
                    if (16 * p + 4 * qd + i >= n_it) al = float2{1.f, 1.f};
                    ral[u][i] = al;
                    run.x *= al.x;
                    run.y *= al.y;
                }
                // the four quarters' products: lane quarter qd ^ d sends its own
                float2 xq[4];
                xq[0] = run;
                xq[1] = float2{__shfl_xor(run.x, 16), __shfl_xor(run.y, 16)};
                xq[2] = float2{__shfl_xor(run.x, 32), __shfl_xor(run.y, 32)};
                xq[3] = float2{__shfl_xor(run.x, 48), __shfl_xor(run.y, 48)};
                float2 qp[4];  // product of quarter j
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = qd ^ j;
                    qp[j] = d == 0 ? xq[0] : d == 1 ? xq[1] : d == 2 ? xq[2] : xq[3];
                }
                float2 pi = {1.f, 1.f}, si = {1.f, 1.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j < qd) { pi.x *= qp[j].x; pi.y *= qp[j].y; }
                    if (j > qd) { si.x *= qp[j].x; si.y *= qp[j].y; }
                }
                pin[u] = pi;
                sin[u] = si;
                if (qd == 0 && cm < NCOMBO) {
                    const int c0 = 2 * (cm % NCP);
                    *reinterpret_cast<float2 *>(TPv + p * K + c0) =
                        float2{(qp[0].x * qp[1].x) * (qp[2].x * qp[3].x), (qp[0].y * qp[1].y) * (qp[2].y * qp[3].y)};
                }
                if constexpr (NORM) {
                    // this thread's share of the row sums of q^2 (0..3) and k^2 (4..7)
                    float x2[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float q0, q1, k0, k1;
                        pair_f32(rq[u][i], q0, q1);
                        pair_f32(rk[u][i], k0, k1);
                        const bool ok = 16 * p + 4 * qd + i < n_it;
                        x2[i] = ok ? q0 * q0 + q1 * q1 : 0.f;
                        x2[4 + i] = ok ? k0 * k0 + k1 * k1 : 0.f;
                    }
                    // sum the row shares over the NG lanes of this tile in this quarter-wave
                    // by recursive halving (each exchange keeps half of the remaining sums
                    // and adds the partner's half: 8 sums over 16 lanes in 7 exchanges); the
                    // waves' partial sums meet in LDS
                    constexpr int NG = NCP < 16 ? NCP : 16;
                    static_assert(NG == 8 || NG == 16, "8 or 16 lanes share a tile row");
                    int base = 0;  // index of x2[0] among the 8 sums
                    halve_sums<4, true, NG / 2>(x2, lane, base);
                    halve_sums<2, true, NG / 4>(x2, lane, base);
                    halve_sums<1, true, NG / 8>(x2, lane, base);
                    if constexpr (NG == 16) x2[0] += __shfl_xor(x2[0], 1);  // one sum on two lanes
                    if (cm < NCOMBO && (NG != 16 || (lane & 1) == 0)) {
                        const int part = (cm % NCP) / 16;  // which wave's share of the row
                        Nrm[(it & 1) * L::NNRM + ((p * 2 + (base >> 2)) * 16 + 4 * qd + (base & 3)) * L::NPART + part] = x2[0];
                    }
                }
            }
            if (tp < C) {
                const float b = a.beta_logits ? __builtin_amdgcn_rcpf(1.f + __expf(-rbeta)) : rbeta;
                Btv[tp] = tp < n_it ? b : 0.f;
            }
        }
        lds_barrier();  // B1
        // ---- phase 1b: A-matrix operand staging of chunk `it` ---------------------------
        // The package operands are computed here too but kept in registers and stored in
        // phase 2, after the prefetch has gone out.
        float2 kq[CPT][4], kk[CPT][4], kr[CPT][4];  // q gamma/R, beta k gamma/R, k E/gamma per row
        float2 keR[CPT], keCE[CPT];                 // R_p and E_C / E_p of the combo's tile
        float2 bvv[NVE];                            // beta v pairs of this thread's value items
        if (work) {
            unsigned char *pk = pkg(it & 1);
            float *eGC = reinterpret_cast<float *>(pk + L::pGC);
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u);
                if (cm >= NCOMBO) continue;
                const int c0 = 2 * (cm % NCP), p = cm / NCP;
                float2 tpr[NP];
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) tpr[pp] = *reinterpret_cast<const float2 *>(TPv + pp * K + c0);
                float2 eR = {1.f, 1.f}, eCE = {1.f, 1.f}, eAll = {1.f, 1.f}, own = {1.f, 1.f};
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    if (pp < p) { eR.x *= tpr[pp].x; eR.y *= tpr[pp].y; }
                    if (pp > p) { eCE.x *= tpr[pp].x; eCE.y *= tpr[pp].y; }
                    if (pp == p) own = tpr[pp];
                    eAll.x *= tpr[pp].x;
                    eAll.y *= tpr[pp].y;
                }
                if (p == 0 && qd == 0) *reinterpret_cast<float2 *>(eGC + c0) = eAll;
                const float2 rT = {__builtin_amdgcn_rcpf(own.x), __builtin_amdgcn_rcpf(own.y)};
                // extra right-operand versions for tiles (pp, p) with pp >= p + 2
                float2 xf[NP];
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    float2 f = {1.f, 1.f};
#pragma unroll
                    for (int r2 = 0; r2 < NP; ++r2)
                        if (r2 > p && r2 < pp) { f.x *= tpr[r2].x; f.y *= tpr[r2].y; }
                    xf[pp] = f;
                }
                float bet[4];
                {
                    const float4 b4 = *reinterpret_cast<const float4 *>(Btv + 16 * p + 4 * qd);
                    bet[0] = b4.x; bet[1] = b4.y; bet[2] = b4.z; bet[3] = b4.w;
                }
                float2 suf[4];  // E_p / gamma_i: product of the tile's later factors
                {
                    float2 run = sin[u];
#pragma unroll
                    for (int i = 3; i >= 0; --i) {
                        suf[i] = run;
                        run.x *= ral[u][i].x;
                        run.y *= ral[u][i].y;
                    }
                }
                float2 pre = pin[u];  // gamma_i / R_p
                keR[u] = eR;
                keCE[u] = eCE;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * p + 4 * qd + i;
                    pre.x *= ral[u][i].x;
                    pre.y *= ral[u][i].y;
                    const bool ok = r < n_it;
                    float q0, q1, k0, k1;
                    pair_f32(rq[u][i], q0, q1);
                    pair_f32(rk[u][i], k0, k1);
                    if (!ok) q0 = q1 = k0 = k1 = 0.f;
                    const float2 lq = {q0 * pre.x, q1 * pre.y};
                    const float2 lk = {bet[i] * k0 * pre.x, bet[i] * k1 * pre.y};
                    const float2 ro = {k0 * suf[i].x, k1 * suf[i].y};  // k E_p / gamma <= |k|
                    const float2 rd = {ro.x * rT.x, ro.y * rT.y};        // k R_p / gamma <= e^80 |k|
                    st2<TA>(Lk + r * L::LKA + c0, lk.x, lk.y);
                    st2_stage<P>(St + L::sLq + r * L::LKS + c0, L::NST, lq.x, lq.y);
                    st2_stage<P>(St + L::sRd + r * L::LKS + c0, L::NST, rd.x, rd.y);
                    if (p < NP - 1) st2_stage<P>(St + L::sRo + r * L::LKS + c0, L::NST, ro.x, ro.y);
                    if constexpr (L::NX > 0) {
                        int xi = 0;
#pragma unroll
                        for (int pp = 2; pp < NP; ++pp)
#pragma unroll
                            for (int qq = 0; qq + 2 <= pp; ++qq, ++xi)
                                if (qq == p)
                                    st2_stage<P>(St + L::sX + (xi * 16 + 4 * qd + i) * L::LKS + c0, L::NST,
                                                 ro.x * xf[pp].x, ro.y * xf[pp].y);
                    }
                    kq[u][i] = lq;
                    kk[u][i] = lk;
                    kr[u][i] = ro;
                }
            }
#pragma unroll
            for (int w = 0; w < NVE; ++w) {
                const int e = tp + NPT * w;
                if (e < BV * C / 2) {
                    bvv[w] = float2{raw_f32(rv[w][0]), raw_f32(rv[w][1])};  // raw values (exact)
                }
            }
        }
        // ---- phase 2: send the prefetch of the next chunk, then store the package operands
        // of this one (the state waves run the serial part of the previous chunk meanwhile)
        if (work) {
            if (it + 1 < nchunks) load_raw(it + 1);  // consumed next iteration
            unsigned char *pk = pkg(it & 1);
            TM *Qt = reinterpret_cast<TM *>(pk + L::pQt);
            TM *Bw = reinterpret_cast<TM *>(pk + L::pBw);
            TM *Kt = reinterpret_cast<TM *>(pk + L::pKt);
            TIn *vL = reinterpret_cast<TIn *>(pk + L::pbV);
            if (tp < C) reinterpret_cast<float *>(pk + L::pBt)[tp] = Btv[tp];
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u);
                if (cm >= NCOMBO) continue;
                const int c0 = 2 * (cm % NCP), p = cm / NCP;
                const float2 eR = keR[u], eCE = keCE[u];
                float iq[4], ik[4];  // reciprocal row norms (1 without normalisation)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    iq[i] = 1.f;
                    ik[i] = 1.f;
                    if constexpr (NORM) {
                        float nq = 0.f, nk = 0.f;
#pragma unroll
                        for (int pt = 0; pt < L::NPART; ++pt) {
                            nq += Nrm[(it & 1) * L::NNRM + ((p * 2 + 0) * 16 + 4 * qd + i) * L::NPART + pt];
                            nk += Nrm[(it & 1) * L::NNRM + ((p * 2 + 1) * 16 + 4 * qd + i) * L::NPART + pt];
                        }
                        iq[i] = __builtin_amdgcn_rsqf(fmaxf(nq, 1e-12f));
                        ik[i] = __builtin_amdgcn_rsqf(fmaxf(nk, 1e-12f));
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * p + 4 * qd + i;
                    st2<TM>(Qt + r * L::LKM + c0, kq[u][i].x * eR.x * iq[i], kq[u][i].y * eR.y * iq[i]);
                    st2<TM>(Bw + r * L::LKM + c0, -kk[u][i].x * eR.x * ik[i], -kk[u][i].y * eR.y * ik[i]);
                    if (i & 1) {
                        // two consecutive tokens per channel row of Kt
                        st2<TM>(Kt + c0 * L::LCM + r - 1, kr[u][i - 1].x * eCE.x * ik[i - 1], kr[u][i].x * eCE.x * ik[i]);
                        st2<TM>(Kt + (c0 + 1) * L::LCM + r - 1, kr[u][i - 1].y * eCE.y * ik[i - 1],
                                kr[u][i].y * eCE.y * ik[i]);
                    }
                }
            }
#pragma unroll
            for (int w = 0; w < NVE; ++w) {
                const int e = tp + NPT * w;
                if (e < BV * C / 2) {
                    const int j = e % BV, r = 2 * (e / BV);
                    st2<TIn>(vL + j * L::LCM + r, bvv[w].x, bvv[w].y);
                }
            }
        }
        lds_barrier();  // B2
    }
}

// Largest value block (64, 32, 16; not above V) whose LDS layout fits; 0 if none does.
template <class P, int K, int V, int C>
constexpr int pick_bv() {
    if constexpr (V >= 64 && Layout<P, K, V, C, 64>::fits) return 64;
    else if constexpr (V >= 32 && Layout<P, K, V, C, 32>::fits) return 32;
    else if constexpr (Layout<P, K, V, C, 16>::fits) return 16;
    else return 0;
}

template <class P, int GM, int K, int V, int C>
hipError_t launch_kvc(const ChunkArgs &a, int num_pairs, hipStream_t stream, int *bv_out) {
    constexpr int BV = pick_bv<P, K, V, C>();
    if constexpr (BV == 0) {
        return hipErrorNotSupported;
    } else {
        using L = Layout<P, K, V, C, BV>;
        auto kern = chunk_fwd_kernel<P, K, V, C, BV, GM>;
        static std::atomic<bool> attr_set{false};  // per instantiation, once per process
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::total);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        if (bv_out) *bv_out = BV;
        const int grid = num_pairs * (V / BV);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), L::total, stream, a);
        return hipGetLastError();
    }
}

template <class P, int GM, int K, int V>
hipError_t launch_kv(const ChunkArgs &a, int C, int num_pairs, hipStream_t stream, int *bv) {
    if (!a.q) {  // query only: report the value block, launch nothing
        const int b = C == 16 ? pick_bv<P, K, V, 16>() : C == 32 ? pick_bv<P, K, V, 32>()
                    : C == 64 ? pick_bv<P, K, V, 64>() : 0;
        if (bv) *bv = b;
        return b ? hipSuccess : hipErrorNotSupported;
    }
    switch (C) {
        case 16: return launch_kvc<P, GM, K, V, 16>(a, num_pairs, stream, bv);
        case 32: return launch_kvc<P, GM, K, V, 32>(a, num_pairs, stream, bv);
        case 64: return launch_kvc<P, GM, K, V, 64>(a, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

template <class P, int GM, int K>
hipError_t launch_k(const ChunkArgs &a, int V, int C, int num_pairs, hipStream_t stream, int *bv) {
    switch (V) {
        case 16: return launch_kv<P, GM, K, 16>(a, C, num_pairs, stream, bv);
        case 32: return launch_kv<P, GM, K, 32>(a, C, num_pairs, stream, bv);
        case 64: return launch_kv<P, GM, K, 64>(a, C, num_pairs, stream, bv);
        case 128: return launch_kv<P, GM, K, 128>(a, C, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

template <class P, int GM>
hipError_t launch_p(const ChunkArgs &a, int K, int V, int C, int num_pairs, hipStream_t stream, int *bv) {
    switch (K) {
        case 16: return launch_k<P, GM, 16>(a, V, C, num_pairs, stream, bv);
        case 32: return launch_k<P, GM, 32>(a, V, C, num_pairs, stream, bv);
        case 64: return launch_k<P, GM, 64>(a, V, C, num_pairs, stream, bv);
        case 128: return launch_k<P, GM, 128>(a, V, C, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

}  // namespace kda
