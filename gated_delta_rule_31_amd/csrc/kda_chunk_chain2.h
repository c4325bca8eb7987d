// kda_chunk_chain2.h -- the serial part of the two-kernel chunkwise prefill (KDA cheat
// sheet, "Chunkwise parallel form": recurrent across chunks, parallel within each), for
// 16-bit operands, fed by direct global-to-LDS copies instead of copy waves.
//
// One workgroup of four waves per (sequence, head, 64 value columns); wave w owns the
// 16-column tile w and holds its float32 state S[K x 16] in registers.  Per chunk:
//   Y = beta V - Bw S,  Vt = T Y,  O = Qt S + A_qk Vt,  S = gamma_C S + Kt^T Vt
// with the package (Qt, -Bw, Kt, T, A_qk hi/lo, gamma_C, beta) written by the pre-pass in
// the "paired" column order (below) and the chunk's value rows copied from the input.
//
// Pipeline, per chunk c (one barrier per chunk; four LDS chunk buffers, chunk c in c % 4):
//   the output of chunk c-1 is stored; the copies of chunk c+4 into chunk c's buffer (its
//   fragments are already in registers) go out in four groups spread over the step; the
//   step of chunk c runs from registers, and each part of the register set is refilled
//   with chunk c+1's fragments as soon as its last product has issued; then the wave waits
//   until chunk c+2 has landed (the copies of chunks c+3 and c+4 may still be in flight)
//   and all its LDS reads are done, and the workgroup meets at the barrier.  So a copy has
//   three chunk steps to arrive, and the LDS reads run under the products.
//
// Paired column order: a matrix-core step over k tiles 2m, 2m+1 takes, in lane group g,
// k = 32m + 4g + 0..3 and 32m + 16 + 4g + 0..3 (the order the accumulator tiles give the
// B operand).  The pre-pass stores column k = 32m + 16h + 4g + e at 32m + 8g + 4h + e, so a
// lane's eight k values are one 16-byte piece.  In LDS every row's 16-byte pieces are
// XOR-swizzled by the row index (chosen by the copy's source addresses; the copy itself
// writes 1 KB blocks in lane order), which makes the 16-byte fragment reads of sixteen
// consecutive rows conflict-free without padding.
#pragma once

#include "kda_chunk_pack.h"

namespace kda {

namespace {

// XOR swizzle of the 16-byte pieces of a row of R pieces (R = 4, 8 or 16).  16 / R rows
// share one 256-byte span of the LDS banks; the swizzle of row r is its span index mod R,
// so the reads of one piece index by sixteen consecutive rows (one LDS cycle of a 16-byte
// read) fall on sixteen distinct 16-byte bank groups.
__device__ __forceinline__ constexpr int swz_of(int R, int r) { return (r * R / 16) & (R - 1); }
template <int R>
__device__ __forceinline__ int row_swz(int r) {
    static_assert(R == 4 || R == 8 || R == 16, "rows of 64, 128 or 256 bytes");
    return swz_of(R, r);
}

template <int K, int V, int C, int NW>
struct Chain2Layout {
    using PL = PackLayout<PrecMixed, K, C>;
    static constexpr int BV = 16 * NW;     // value columns of a workgroup: 16 per wave
    static constexpr int RK = K * 2 / 16;  // pieces per row of Qt / Bw
    static constexpr int RC = C * 2 / 16;  // pieces per row of Kt, T, A_qk
    // A copy instruction moves 64 NW pieces of 16 bytes (NW waves x 64 lanes).  The package
    // takes JV whole instructions (padded), the chunk's values [C][BV] bf16 exactly one more.
    static constexpr size_t IB = 1024 * NW;
    static constexpr int JV = (int)((PL::bytes + IB - 1) / IB);
    static constexpr size_t oV = (size_t)JV * IB;
    static constexpr int J = JV + 1;                         // copy instructions per wave per chunk
    static constexpr size_t buf = (size_t)J * IB;            // one chunk buffer
    // buffers: with four waves four (copies run three chunks ahead), with eight three (two)
    static constexpr int NB = NW == 4 ? 4 : 3;
    static constexpr size_t total = NB * buf;
    // 32-token chunks: C * BV * 2 == IB, and a 64-token chunk's fragments do not fit
    static constexpr bool ok = (NW == 4 || NW == 8) && K % 32 == 0 && C == 32 && V % BV == 0 &&
                               total <= 160 * 1024 - 2048 && (NB - 2) * J <= 63 &&
                               (RK == 4 || RK == 8 || RK == 16) && (RC == 4 || RC == 8);
};

// A 16-bit A-operand fragment of row r, k pair m, from a swizzled paired-order row of R pieces
template <int R>
__device__ __forceinline__ f16x8 ld_pair(const unsigned char *rowbase, int r, int m, int g) {
    const int p = (4 * m + g) ^ row_swz<R>(r);
    return *reinterpret_cast<const f16x8 *>(rowbase + 16 * p);
}

template <int K, int V, int C>
struct Chain2Frags {
    static constexpr int NP = C / 16, NKT = K / 16;
    f16x8 fb[NP][NKT / 2];   // -Bw rows (Y)
    f16x8 ft[NP][NP / 2];    // T rows (Vt)
    f16x8 fq[NP][NKT / 2];   // Qt rows (O)
    f16x8 fa[NP][NP / 2];    // A_qk rows, hi and lo (O)
    f16x8 fl[NP][NP / 2];
    f16x8 fk[NKT][NP / 2];   // Kt rows (S)
    f4 gc[NKT];              // gamma_C of this lane's key rows
    f4 bt[NP];               // beta of this lane's rows
    unsigned short vr[NP][4];  // v of this lane's rows and column, bf16 bits
};

template <int I>
using IC = std::integral_constant<int, I>;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// x - (float)h for the low / high half h of a packed 16-bit pair, in one mixed-precision fma
// (exact: x minus its own 16-bit rounding needs no more than float32's mantissa)
__device__ __forceinline__ float rem16_lo(uint32_t h, float x) {
    float r;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
    return r;
}
__device__ __forceinline__ float rem16_hi(uint32_t h, float x) {
    float r;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
    return r;
}

// hi + lo 16-bit operand parts of accumulator tiles (lo = the rounded remainder x - hi); a
// pair m of BFrag holds tile 2m's four values, then tile 2m+1's
template <int N>
__device__ __forceinline__ void split16(BFrag<_Float16, N> &hi, BFrag<_Float16, N> &lo, const f4 (&t)[N]) {
    static_assert(N % 2 == 0, "whole k pairs");
    hi.set(t);
    f4 r[N];
#pragma unroll
    for (int m = 0; m < N / 2; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // halves 2q, 2q + 1 of pair m
            const uint32_t h2 = __builtin_bit_cast(uint32_t, f16x2{hi.pair[m][2 * q], hi.pair[m][2 * q + 1]});
            const int i0 = 2 * q, i1 = 2 * q + 1;  // element i of the pair: tile 2m + i / 4, value i % 4
            r[2 * m + i0 / 4][i0 % 4] = rem16_lo(h2, t[2 * m + i0 / 4][i0 % 4]);
            r[2 * m + i1 / 4][i1 % 4] = rem16_hi(h2, t[2 * m + i1 / 4][i1 % 4]);
        }
    lo.set(r);
}

// Largest magnitude over this lane's tiles.  IEEE maximum (NaN-propagating) needs no
// canonicalisation of its inputs, so with the absolute-value modifiers it is one
// three-input instruction per two values.
template <int N>
__device__ __forceinline__ float amax(const f4 (&x)[N]) {
    float m = __builtin_fabsf(x[0][0]);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int e = (i == 0 ? 1 : 0); e < 4; ++e) m = __builtin_elementwise_maximum(m, __builtin_fabsf(x[i][e]));
    return m;
}

// The exponent s >= 0 of the power-of-two scale that brings the wave's largest magnitude m
// below 2^15: 0 when no lane reaches 2^15 (one vote, the usual case); else a
// rotate-and-maximum within each row of 16 lanes, then the row broadcasts of lanes 15 and
// 31, so lane 63 holds the wave's maximum.
__device__ __forceinline__ int wave_exp(float m) {
    if (__builtin_amdgcn_ballot_w64(m >= 32768.f) == 0) return 0;
    auto step = [&](auto ctrl, auto rows) {
        const int b = __builtin_bit_cast(int, m);
        const int t = __builtin_amdgcn_update_dpp(b, b, decltype(ctrl)::value, decltype(rows)::value, 0xf, false);
        m = __builtin_elementwise_maximum(m, __builtin_bit_cast(float, t));
    };
    step(IC<0x128>{}, IC<0xf>{});  // row_ror:8
    step(IC<0x124>{}, IC<0xf>{});  // row_ror:4
    step(IC<0x122>{}, IC<0xf>{});  // row_ror:2
    step(IC<0x121>{}, IC<0xf>{});  // row_ror:1
    step(IC<0x142>{}, IC<0xa>{});  // row_bcast:15 into rows 1 and 3
    step(IC<0x143>{}, IC<0xc>{});  // row_bcast:31 into rows 2 and 3
    const int e = (__builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 63) >> 23) & 0xff;
    return e > 141 ? e - 141 : 0;
}

template <int K, int V, int C, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_chain2_kernel(ChunkArgs a) {
    using L2 = Chain2Layout<K, V, C, NW>;
    constexpr int NB = L2::NB;
    using PL = PackLayout<PrecMixed, K, C>;
    using F = Chain2Frags<K, V, C>;
    static_assert(L2::ok, "layout");
    // eight waves (two per SIMD): each part of a chunk's fragments is read from LDS right
    // before its products, the other wave of the SIMD covering the latency; four waves: the
    // next chunk's fragments are read into registers during the step
    constexpr bool JIT = NW == 8;
    constexpr int NP = C / 16, NKT = K / 16, BV = L2::BV, J = L2::J;
    constexpr int RK = L2::RK, RC = L2::RC;

    // Separate arrays, not one: a copy into one buffer and the reads of another are then
    // distinct objects, so the compiler need not wait for the copies before every LDS read.
    __shared__ __align__(16) unsigned char lds0[L2::buf], lds1[L2::buf], lds2[L2::buf], lds3[NB > 3 ? L2::buf : 16];
    auto bufp = [&](auto I) -> unsigned char * {
        constexpr int i = decltype(I)::value % NB;
        if constexpr (i == 0) return lds0;
        else if constexpr (i == 1) return lds1;
        else if constexpr (i == 2) return lds2;
        else return lds3;
    };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;

    // Which (sequence, head, value block).  Workgroups go out in blockIdx order, round-robin
    // over the 8 XCDs: block b = 8 (NVB q + v) + x takes pair 8q + x and value block v, so
    // a head's value blocks share an XCD (and its L2) while consecutive pairs spread over
    // all XCDs.  With packed sequences (up to 256) the pairs are numbered longest sequence
    // first, so the longest chains start first.
    constexpr int NVB = V / BV;
    const int G = gridDim.x;
    int vb, pair;
    if (G % (8 * NVB) == 0) {
        const int x = blockIdx.x & 7, rest = blockIdx.x >> 3;
        vb = rest % NVB;
        pair = (rest / NVB) * 8 + x;
    } else {
        vb = blockIdx.x % NVB;
        pair = blockIdx.x / NVB;
    }
    const int H = a.H, h = pair % H;
    int s = pair / H;
    if (a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= 256) {  // workgroup-uniform
        __shared__ int slen[256], sorder[256];
        const int N = a.num_seqs;
        if (tid < N) slen[tid] = a.cu_seqlens[tid + 1] - a.cu_seqlens[tid];
        __syncthreads();
        if (tid < N) {
            const int lj = slen[tid];
            int rank = 0;  // sequences before this one: longer, or as long with a lower index
            for (int i = 0; i < N; ++i) rank += (slen[i] > lj) || (slen[i] == lj && i < tid);
            sorder[rank] = tid;
        }
        __syncthreads();
        s = sorder[s];
    }
    int64_t bos, eos;
    int base;  // first chunk slot of the sequence
    if (a.cu_seqlens) {
        bos = a.cu_seqlens[s];
        eos = a.cu_seqlens[s + 1];
        base = (int)(bos / C) + s;
    } else {
        bos = (int64_t)s * a.T;
        eos = bos + a.T;
        base = s * (int)((a.T + C - 1) / C);
    }
    // this launch's chunks of the sequence: [c_begin, c_end) clipped to it; the state comes
    // from initial_state and goes to final_state at the ends of the range
    const int nall = (int)((eos - bos + C - 1) / C);
    const int cfirst = a.c_begin < nall ? a.c_begin : nall;
    const int nchunks = (a.c_end < nall ? a.c_end : nall) - cfirst;

    // ---- the copy: piece x of a chunk buffer <- 16 source bytes ------------------------------
    // Package pieces (instructions j < JV) map to package bytes (rows of Qt, Bw, Kt, T, A_qk
    // swizzled; gamma_C and beta as they are); the padding pieces past the package copy its
    // first 16 bytes again.  Instruction JV copies the chunk's values: piece y = row * 8 + p.
    // Every lane issues the same J copies, which the partial waits below count on.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t srcoff[L2::JV];  // byte offset in the package
#pragma unroll
    for (int j = 0; j < L2::JV; ++j) {
        const int x = 64 * (wave + NW * j) + lane;
        const size_t b = (size_t)x * 16;
        uint32_t off = 0;
        if (b < PL::bytes) {
            auto mat = [&](size_t o0, int R) {  // a swizzled matrix region starting at o0
                const int rel = (int)((b - o0) / 16), r = rel / R, ps = rel % R;
                const int swz = swz_of(R, r);
                return (uint32_t)(o0 + 16 * (size_t)(r * R + (ps ^ swz)));
            };
            if (b < PL::gBw) off = mat(PL::gQt, RK);
            else if (b < PL::gKt) off = mat(PL::gBw, RK);
            else if (b < PL::gTm) off = mat(PL::gKt, RC);
            else if (b < PL::gAqk) off = mat(PL::gTm, RC);
            else if (b < PL::gAqk + (size_t)C * C * 2) off = mat(PL::gAqk, RC);
            else if (b < PL::gGC) off = mat(PL::gAqk + (size_t)C * C * 2, RC);
            else off = (uint32_t)b;  // gamma_C, beta
        }
        srcoff[j] = off;
    }
    constexpr int PV = BV * 2 / 16;                            // 16-byte pieces per value row
    const int vrow = (64 * wave + lane) / PV;                  // value piece: row and 16 bytes
    const uint32_t vcol = (uint32_t)((64 * wave + lane) % PV) * 16;
    const uint32_t vstride = (uint32_t)H * V * 2;              // bytes between token rows of v
    // The copies of one chunk go out in four groups spread over the serial step, so the
    // vector-memory path of the compute unit works beside the arithmetic instead of stalling
    // the waves at the start of the period.  Group k takes package instructions
    // [k JV / 4, (k + 1) JV / 4); group 0 also the value instruction.
    // The copies are buffer loads into LDS: the chunk's package and its value rows each get a
    // raw buffer resource (a scalar base, no stride), and each lane's byte offset in it is a
    // 32-bit vector operand (the package offsets are fixed for the whole kernel), so a copy
    // instruction needs no per-lane address arithmetic.
    // (the resources are made where they are used: a lambda returning one, or a struct
    // holding one, fails in the host-side pass of hipcc, which then drops the launch stub)
    struct CopySrc {
        const unsigned char *pk;  // the chunk's package
        const unsigned char *vr;  // the chunk's value rows
        uint32_t voff;            // this lane's value piece
    };
    // The chunks are copied in order: the sources of the next one advance by fixed steps.
    const unsigned char *pk_next = a.pack + ((size_t)(base + cfirst) * H + h) * PL::bytes;
    const unsigned char *v_next =
        static_cast<const unsigned char *>(a.v) + (((bos + (int64_t)cfirst * C) * H + h) * V + vb * BV) * 2;
    // This lane's value piece in a whole chunk, and in the sequence's partial last chunk (rows
    // past its end read its last row): chosen per chunk by one scalar comparison.
    const int64_t t_first = bos + (int64_t)cfirst * C;
    const int nfull = (int)((eos - t_first) / C);                 // whole chunks from t_first on
    const int tail_last = (int)((eos - t_first) - (int64_t)nfull * C) - 1;  // -1: no partial chunk
    const uint32_t voff_full = (uint32_t)vrow * vstride + vcol;
    const uint32_t voff_tail = (uint32_t)(vrow < tail_last ? vrow : (tail_last > 0 ? tail_last : 0)) * vstride + vcol;
    int ci_next = 0;  // index of the next chunk in the range
    auto next_src = [&]() {  // the next chunk's sources (past the range: not used)
        const CopySrc cs{pk_next, v_next, ci_next < nfull ? voff_full : voff_tail};
        pk_next += (size_t)H * PL::bytes;
        v_next += (size_t)C * vstride;
        ++ci_next;
        return cs;
    };
    auto copy_group = [&](const CopySrc &cs, unsigned char *lb, auto G) {
        constexpr int k = decltype(G)::value;
        if constexpr (k == 0) {
            __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(cs.vr), (short)0, (int)(C * vstride), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void *)(lb + L2::oV + 1024 * wv),
                                                     16, (int)cs.voff, 0, 0, 0);
        }
        __amdgpu_buffer_rsrc_t rp =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(cs.pk), (short)0, (int)PL::bytes, 0x00020000);
#pragma unroll
        for (int j = k * L2::JV / 4; j < (k + 1) * L2::JV / 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (__attribute__((address_space(3))) void *)(lb + 1024 * (wv + NW * j)),
                                                     16, (int)srcoff[j], 0, 0, 0);
    };
    auto copy_chunk = [&](bool go, unsigned char *lb) {
        const CopySrc cs = next_src();
        if (!go) return;
        copy_group(cs, lb, IC<0>{});
        copy_group(cs, lb, IC<1>{});
        copy_group(cs, lb, IC<2>{});
        copy_group(cs, lb, IC<3>{});
    };

    // ---- fragments of one chunk into registers, in the parts the serial step consumes -------
    auto read_y = [&](const unsigned char *lb, F &f) {  // -Bw, beta, v
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = 16 * p + r16;
#pragma unroll
            for (int m = 0; m < NKT / 2; ++m) f.fb[p][m] = ld_pair<RK>(lb + PL::gBw + (size_t)r * RK * 16, r, m, g);
            const float4 b4 = *reinterpret_cast<const float4 *>(lb + PL::gBt + 4 * (16 * p + 4 * g));
            f.bt[p] = f4{b4.x, b4.y, b4.z, b4.w};
            const unsigned short *vr = reinterpret_cast<const unsigned short *>(lb + L2::oV) + (16 * p + 4 * g) * BV + wave * 16 + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) f.vr[p][e] = vr[e * BV];
        }
    };
    auto read_t = [&](const unsigned char *lb, F &f) {  // T
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int m = 0; m < NP / 2; ++m)
                if (2 * m <= p)  // T and A_qk are lower triangular: row tile p needs k tiles <= p
                    f.ft[p][m] = ld_pair<RC>(lb + PL::gTm + (size_t)(16 * p + r16) * RC * 16, 16 * p + r16, m, g);
    };
    auto read_o = [&](const unsigned char *lb, F &f) {  // Qt, A_qk hi and lo
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = 16 * p + r16;
#pragma unroll
            for (int m = 0; m < NKT / 2; ++m) f.fq[p][m] = ld_pair<RK>(lb + PL::gQt + (size_t)r * RK * 16, r, m, g);
#pragma unroll
            for (int m = 0; m < NP / 2; ++m) {
                if (2 * m <= p) {
                    f.fa[p][m] = ld_pair<RC>(lb + PL::gAqk + (size_t)r * RC * 16, r, m, g);
                    f.fl[p][m] = ld_pair<RC>(lb + PL::gAqk + (size_t)C * C * 2 + (size_t)r * RC * 16, r, m, g);
                }
            }
        }
    };
    auto read_s = [&](const unsigned char *lb, F &f) {  // Kt, gamma_C
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            const int r = 16 * t + r16;
#pragma unroll
            for (int m = 0; m < NP / 2; ++m) f.fk[t][m] = ld_pair<RC>(lb + PL::gKt + (size_t)r * RC * 16, r, m, g);
            const float4 d = *reinterpret_cast<const float4 *>(lb + PL::gGC + 4 * (16 * t + 4 * g));
            f.gc[t] = f4{d.x, d.y, d.z, d.w};
        }
    };

    // ---- state -------------------------------------------------------------------------------
    f4 S[NKT];
    const int vc = vb * BV + wave * 16 + r16;  // this lane's value column
    const float *s0 = a.initial_state ? a.initial_state + ((int64_t)s * H + h) * K * V : nullptr;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        f4 x = {0.f, 0.f, 0.f, 0.f};
        if (s0) {
            if (a.state_vk) {
                const float4 y = *reinterpret_cast<const float4 *>(s0 + (int64_t)vc * K + 16 * t + 4 * g);
                x = f4{y.x, y.y, y.z, y.w};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = s0[(int64_t)(16 * t + 4 * g + e) * V + vc];
            }
        }
        S[t] = x;
    }
    BFrag<_Float16, NKT> Sh;  // S 2^-sS
    int sS;
    // Sh from S: the unscaled conversion first (the usual case), redone scaled when the
    // state's magnitude leaves the 16-bit range (S itself stays live, so a scaled copy on
    // every path would cost a move per element)
    auto state_operand = [&]() {
        Sh.set(S);
        sS = wave_exp(amax(S));
        if (sS) {
            const float d = pow2f(-sS);
            f4 x[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) x[t] = S[t] * d;
            Sh.set(x);
        }
    };
    state_operand();

    // output of the previous chunk, stored at the start of the next period
    // The stores go through a buffer resource over the chunk's output rows: a lane's row past
    // the sequence's end lies past the resource's bound, and the hardware drops that store.
    f4 opend[NP];
    bool pend = false;
    const unsigned char *o_pend = nullptr;
    uint32_t nb_pend = 0;
    const int esz = a.out_bf16 ? 2 : 4;
    const int j0 = vb * BV + wave * 16 + 4 * g;  // first of this lane's four output columns
    unsigned char *o_run = static_cast<unsigned char *>(a.out) + ((bos + (int64_t)cfirst * C) * H + h) * V * esz;
    int64_t t_run = bos + (int64_t)cfirst * C;   // first token of the chunk being computed
    auto store_pending = [&]() {
        if (!pend) return;
        __amdgpu_buffer_rsrc_t ro =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(o_pend), (short)0, (int)nb_pend, 0x00020000);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int off = ((16 * p + r16) * H * V + j0) * esz;
            if (a.out_bf16) {
                typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
                typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
                const u32x2 x = {__builtin_bit_cast(unsigned int, bf16x2{(__bf16)opend[p][0], (__bf16)opend[p][1]}),
                                 __builtin_bit_cast(unsigned int, bf16x2{(__bf16)opend[p][2], (__bf16)opend[p][3]})};
                __builtin_amdgcn_raw_buffer_store_b64(x, ro, off, 0, 0);
            } else {
                typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, opend[p]), ro, off, 0, 0);
            }
        }
        pend = false;
    };

    // One chunk's serial step from the fragments in f (the math of state_waves); each part of
    // f is refilled from the next chunk's buffer nb as soon as its last product has issued, so
    // the LDS reads run under the rest of the step.  The power-of-two range scales are
    // wave-uniform and almost always 0: the unscaled forms skip their multiplies.
    auto compute = [&](F &f, const unsigned char *cb, const unsigned char *nb, int cn, auto &&issue)
                       __attribute__((always_inline)) {
        issue(IC<0>{});
        if constexpr (JIT) read_y(cb, f);
        f4 Y[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) Y[p][e] = f.bt[p][e] * __builtin_bit_cast(float, (uint32_t)f.vr[p][e] << 16);
        if (sS) {
            const float dS = pow2f(-sS);
#pragma unroll
            for (int p = 0; p < NP; ++p) Y[p] *= dS;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int m = 0; m < NKT / 2; ++m)
                Y[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.fb[p][m], Sh.pair[m], Y[p], 0, 0, 0);
        issue(IC<1>{});
        if constexpr (!JIT) read_y(nb, f);
        const int sY = wave_exp(amax(Y));
        if (sY) {
            const float d = pow2f(-sY);
#pragma unroll
            for (int p = 0; p < NP; ++p) Y[p] *= d;
        }
        BFrag<_Float16, NP> Yh, Yl;
        split16(Yh, Yl, Y);
        if constexpr (JIT) read_t(cb, f);
        f4 Vt[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            Vt[p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NP / 2; ++m) {
                if (2 * m <= p) {
                    Vt[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.ft[p][m], Yh.pair[m], Vt[p], 0, 0, 0);
                    Vt[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.ft[p][m], Yl.pair[m], Vt[p], 0, 0, 0);
                }
            }
        }
        issue(IC<2>{});
        if constexpr (!JIT) read_t(nb, f);
        const int sv = wave_exp(amax(Vt));
        if (sv) {
            const float d = pow2f(-sv);
#pragma unroll
            for (int p = 0; p < NP; ++p) Vt[p] *= d;
        }
        BFrag<_Float16, NP> Vh, Vl;
        split16(Vh, Vl, Vt);
        if constexpr (JIT) read_o(cb, f);
        const int sV = sY + sv;  // Vh (+ Vl) holds Vt 2^-(sS + sV)
        // O^T = S^T Qt^T + Vt^T A_qk^T: lane (g, r16) holds value columns 4g..4g+3 of token r16
        // (two accumulators: the state part is at scale 2^-sS, the intra-chunk part at
        // 2^-(sS + sV); each takes its own factor, with the output scale, at the end)
        const float uQ = a.scale * pow2f(sS), uA = a.scale * pow2f(sS + sV);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            f4 o = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NKT / 2; ++m) o = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sh.pair[m], f.fq[p][m], o, 0, 0, 0);
#pragma unroll
            for (int m = 0; m < NP / 2; ++m) {
                if (2 * m <= p) {
                    oa = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vh.pair[m], f.fa[p][m], oa, 0, 0, 0);
                    oa = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vl.pair[m], f.fa[p][m], oa, 0, 0, 0);
                    oa = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vh.pair[m], f.fl[p][m], oa, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) opend[p][e] = __builtin_fmaf(o[e], uQ, oa[e] * uA);
        }
        issue(IC<3>{});
        if constexpr (!JIT) read_o(nb, f);
        if constexpr (JIT) read_s(cb, f);
        pend = true;
        o_pend = o_run;
        nb_pend = (uint32_t)((eos - t_run) < C ? (eos - t_run) : C) * (uint32_t)(H * V * esz);
        o_run += (size_t)C * H * V * esz;
        t_run += C;
        // S = gamma_C S + Kt^T Vt, accumulated as S 2^-w with w the scale of Vh (the rare
        // rescales in place, so the state keeps its registers from chunk to chunk)
        const int w = sS + sV;
        f4 X[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) X[t] = S[t] * f.gc[t];
        if (w) {
            const float dW = pow2f(-w);
#pragma unroll
            for (int t = 0; t < NKT; ++t) X[t] *= dW;
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int m = 0; m < NP / 2; ++m) {
                X[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.fk[t][m], Vh.pair[m], X[t], 0, 0, 0);
                X[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.fk[t][m], Vl.pair[m], X[t], 0, 0, 0);
            }
        if (w) {
            const float uW = pow2f(w);
#pragma unroll
            for (int t = 0; t < NKT; ++t) X[t] *= uW;
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t) S[t] = X[t];
        if constexpr (!JIT) read_s(nb, f);
        state_operand();
    };

    // Wait until at most N vector-memory operations of this wave are in flight and all its LDS
    // reads are done, then the workgroup barrier.  The wait is the compiler's own instruction
    // (vmcnt N, lgkmcnt 0, expcnt any), so it knows these loads have landed and adds no
    // waits of its own for them later; the empty asm statements keep every memory access on
    // its side of the wait.
    auto wait_barrier = [&](auto N) {
        constexpr int n = decltype(N)::value;
        static_assert(n >= 0 && n <= 63, "vmcnt holds 6 bits");
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
        asm volatile("s_barrier" ::: "memory");
    };

    // ---- prologue: the range's first NB chunks copied, chunk 0's fragments read ----------------
    F f;
    copy_chunk(nchunks > 0, bufp(IC<0>{}));
    copy_chunk(nchunks > 1, bufp(IC<1>{}));
    if constexpr (!JIT) {
        copy_chunk(nchunks > 2, bufp(IC<2>{}));
        if constexpr (NB > 3) copy_chunk(nchunks > 3, bufp(IC<3>{}));
    }
    wait_barrier(IC<0>{});
    if constexpr (!JIT) {
        read_y(bufp(IC<0>{}), f);
        read_t(bufp(IC<0>{}), f);
        read_o(bufp(IC<0>{}), f);
        read_s(bufp(IC<0>{}), f);
        // every wave's reads of buffer 0 are done before period 0 copies into it
        wait_barrier(IC<0>{});
    }

    // Period c (chunk c of the range in buffer c % 4): store chunk c-1's output; copy chunk
    // c+4 into chunk c's buffer (its fragments are in registers); compute chunk c while
    // reading chunk c+1's fragments (past the last chunk they are read and not used); then
    // wait until chunk c+2 is in LDS and every wave's LDS reads are done, and barrier.  The
    // vector-memory counter retires in issue order, so "at most n in flight" with the copies
    // of chunks c+3 and c+4 (J each, issued after chunk c+2's) the last ones means chunk c+2
    // has landed.
    auto period = [&](auto I, int c) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        store_pending();
        if constexpr (JIT) {
            // chunk c is read from its own buffer during the step; chunk c+2 is copied into
            // the buffer chunk c-1 left (read before the last barrier)
            const bool cp = c + 2 < nchunks;
            const CopySrc cs = next_src();  // chunk c+2
            compute(f, bufp(IC<i>{}), bufp(IC<i + 1>{}), c, [&](auto G) {
                if (cp) copy_group(cs, bufp(IC<i + 2>{}), G);
            });
            if (cp) wait_barrier(IC<J>{});  // chunk c+1 has landed
            else wait_barrier(IC<0>{});
        } else {
            const bool cp = c + NB < nchunks;
            const CopySrc cs = next_src();  // chunk c+NB
            compute(f, bufp(IC<i>{}), bufp(IC<i + 1>{}), c, [&](auto G) {
                if (cp) copy_group(cs, bufp(I), G);
            });
            if (NB > 3 && c + 4 < nchunks) wait_barrier(IC<(NB - 2) * J>{});
            else if (c + 3 < nchunks) wait_barrier(IC<J>{});
            else wait_barrier(IC<0>{});
        }
    };
    for (int c = 0; c < nchunks; c += NB) {  // workgroup-uniform
        period(IC<0>{}, c);
        if (c + 1 < nchunks) period(IC<1>{}, c + 1);
        if (c + 2 < nchunks) period(IC<2>{}, c + 2);
        if constexpr (NB > 3)
            if (c + 3 < nchunks) period(IC<3>{}, c + 3);
    }
    store_pending();

    if (a.final_state) {
        float *sf = a.final_state + ((int64_t)s * H + h) * K * V;
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            if (a.state_vk) {
                *reinterpret_cast<float4 *>(sf + (int64_t)vc * K + 16 * t + 4 * g) = float4{S[t][0], S[t][1], S[t][2], S[t][3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) sf[(int64_t)(16 * t + 4 * g + e) * V + vc] = S[t][e];
            }
        }
    }
}

}  // namespace

}  // namespace kda
