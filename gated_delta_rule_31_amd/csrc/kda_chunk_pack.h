// kda_chunk_pack.h -- the two-kernel form of the chunkwise prefill (KDA cheat sheet,
// "Chunkwise parallel form"): the same arithmetic as chunk_fwd_kernel, split where the
// work stops depending on the state.
//
//  * chunk_pack_kernel, a persistent grid over the (chunk, head) items, all chunks at
//    once: per item the decay products, the A-matrix tiles, T = (I + A_kk)^-1 and A_qk
//    of one chunk, written as a dense package (Qt, -Bw, Kt, T, A_qk, gamma_C, beta) into
//    a caller-owned workspace.  Nothing in it depends on the state or on the value
//    columns, so it runs once per (chunk, head) instead of once per value block, on every
//    compute unit.
//  * chunk_chain_kernel, one workgroup per (sequence, head, value block): the state waves
//    of chunk_fwd_kernel (the serial part), fed by four copy waves that move each package
//    from the workspace into a double-buffered LDS area and form beta V; one barrier per
//    chunk.
//  * chunk_segment_kernel: one launch holding the chain over one segment of chunks in its
//    first workgroups and the pre-pass of the next segment in the rest, so the two
//    overlap on one stream (the host's schedule is in kda_chunk_chain.hip).
//
// Chunk slots: without cu_seqlens slot b * NC + j (NC = ceil(T / C)) is chunk j of batch
// row b; with them, sequence s owns slots floor(cu[s] / C) + s + j for j < ceil(len_s / C)
// (disjoint, fewer than T / C + N in all); a slot no sequence owns is left unwritten.
#pragma once

#include "kda_chunk_kernel.h"

namespace kda {

namespace {

constexpr int PPW = 8;          // waves of a pre-pass workgroup
constexpr int PPT = 64 * PPW;
constexpr int NCW = 4;          // copy waves of the chain kernel
constexpr int NTC = 64 * (NSW + NCW);

// One package in the workspace, dense, byte offsets: Qt and -Bw [C][K], Kt [K][C] (token
// index contiguous, the LDS operand order), T and A_qk [C][C] (upper blocks zero; A_qk as
// hi and lo parts on the 16-bit path), all in the matrix-operand type; gamma_C [K] and
// beta [C] (0 on padding rows) in float32.
template <class P, int K, int C>
struct PackLayout {
    using TM = typename P::TM;
    static constexpr size_t gQt = 0;
    static constexpr size_t gBw = gQt + (size_t)C * K * sizeof(TM);
    static constexpr size_t gKt = gBw + (size_t)C * K * sizeof(TM);
    static constexpr size_t gTm = gKt + (size_t)K * C * sizeof(TM);
    static constexpr size_t gAqk = gTm + (size_t)C * C * sizeof(TM);
    static constexpr size_t gGC = gAqk + (size_t)P::kAqParts * C * C * sizeof(TM);
    static constexpr size_t gBt = gGC + (size_t)K * 4;
    static constexpr size_t bytes = gBt + (size_t)C * 4;
    static_assert(bytes % 16 == 0, "packages stay 16-byte aligned");
};

// LDS of the pre-pass: the chunk kernel's staging area, then T and A_qk (row stride LCM)
// where a package's Tm and Aqk would sit, so a_matrix_work writes them unchanged.
template <class P, int K, int C>
struct PrepassLds {
    using L = Layout<P, K, 16, C, 16>;
    static constexpr size_t oTA = L::oPkg;
    static constexpr size_t total = oTA + (L::pbV - L::pTm);
    static_assert(L::oPkg >= L::pTm, "the package base lies inside the workgroup's LDS");
    static constexpr bool fits = total <= 160 * 1024;
};

template <class P, int K, int V, int C, int BV>
struct ChainLds {
    static constexpr size_t total = 2 * Layout<P, K, V, C, BV>::szPkg;
    static constexpr bool fits = total <= 160 * 1024;
};

// Column k = 32m + 16h + 4g + e of a matrix stored in the paired order sits at
// 32m + 8g + 4h + e: the eight k values one lane group takes in a 16x16x32 step over k tiles
// 2m, 2m+1 (in the permuted order the accumulator tiles give) become one 16-byte piece.
__device__ __forceinline__ int paired_col(int k) {
    return (k & ~31) | (k & 3) | (((k >> 4) & 1) << 2) | (((k >> 2) & 3) << 3);
}

// GM as in chunk_fwd_kernel.  Persistent: workgroup b takes items b, b + G, ... of the
// slots * H (chunk slot, head) items (slot-major, heads adjacent), skipping slots no
// sequence owns, and has the raw inputs of its next item in flight while it works on the
// current one.  PERM: the matrices go out in the paired column order (the reduction index
// of every product: Qt, Bw by key column; Kt, T, A_qk by token), for the chain kernel that
// reads 16-byte fragments.
template <class P, int K, int C, int GM, bool PERM = false>
__device__ __forceinline__ void pack_body(const ChunkArgs &a, int bid, int G) {
    static_assert(!PERM || (K % 32 == 0 && C % 32 == 0), "the paired order works on 32-wide blocks");
    constexpr bool ZG = GM >= 1;
    constexpr bool NORM = GM == 2;
    using L = Layout<P, K, 16, C, 16>;
    using PL = PackLayout<P, K, C>;
    using TA = typename P::TA;
    using TM = typename P::TM;
    using TIn = typename std::conditional<std::is_same<P, PrecF32>::value, float, __bf16>::type;
    constexpr int NP = L::NP;

    extern __shared__ __align__(16) unsigned char smem[];
    const int H = a.H;
    // items: without cu_seqlens, chunks [c0, c1) of every batch row (b, c, h order); with
    // them, every chunk slot (slot-major).  Fewer than 2^31 (checked by the host).
    const int NC = (int)((a.T + C - 1) / C);
    const int c0 = a.c_begin < NC ? a.c_begin : NC;
    const int W = (a.c_end < NC ? a.c_end : NC) - c0;
    const int nitems = a.cu_seqlens ? a.pack_slots * H : (a.pack_slots / NC) * W * H;

    TA *Lk = reinterpret_cast<TA *>(smem + L::oLk);
    TA *St = reinterpret_cast<TA *>(smem + L::oSt);
    float *TPv = reinterpret_cast<float *>(smem + L::oTP);
    float *Btv = reinterpret_cast<float *>(smem + L::oBt);
    float *Nrm = reinterpret_cast<float *>(smem + L::oNrm);
    float *Akk = reinterpret_cast<float *>(smem + L::oAkk);
    float *Tf = reinterpret_cast<float *>(smem + L::oTf);
    using PXL = PrepassLds<P, K, C>;
    TM *TmL = reinterpret_cast<TM *>(smem + PXL::oTA);
    TM *AqL = reinterpret_cast<TM *>(smem + PXL::oTA + (L::pAqk - L::pTm));
    TM *AlL = reinterpret_cast<TM *>(smem + PXL::oTA + (L::pAql - L::pTm));

    // the strictly upper 16x16 blocks of T and A_qk are zero in every item (nothing else
    // writes them); the first barrier below orders this before any read
    for (int e = threadIdx.x; e < C * C; e += PPT) {
        const int i = e / C, j = e % C;
        if ((j >> 4) > (i >> 4)) {
            TmL[i * L::LCM + j] = from_f32<TM>(0.f);
            AqL[i * L::LCM + j] = from_f32<TM>(0.f);
            if constexpr (P::kAqParts == 2) AlL[i * L::LCM + j] = from_f32<TM>(0.f);
        }
    }

    // the next item at or after `from` whose slot some sequence owns (nitems if none)
    struct Item {
        int n, h, len;
        int64_t t0;
    };
    // Fixed-length items it = (b W + c) H + h come in the order bid, bid + G, bid + 2G, ...
    // (every one owns tokens): a cursor holds the decomposition of the next one and
    // advances by G with carries, so the loop divides nothing.
    int cb_ = 0, cc_ = 0, ch_ = 0, dB = 0, dC = 0, dH = 0;
    // Packed sequences: items it = n H + h (slot n) come in the same order; the cursor holds
    // (n, h) of the next one and the sequence sq_ whose slots start at or before n (slots
    // only grow, so it moves forward; fs_, fsn_: first slots of sq_ and sq_ + 1).
    // sa0_, slen_: start and length of sequence sq_, read when the cursor moves (not per item:
    // a load per item would also make the item wait for every store still in flight)
    int sq_ = 0, fs_ = 0, fsn_ = 0;
    int64_t sa0_ = 0, slen_ = 0;
    if (a.cu_seqlens) {
        dH = G % H;
        dC = G / H;
        ch_ = bid % H;
        cc_ = bid / H;
        fs_ = a.cu_seqlens[0] / C;
        fsn_ = a.num_seqs > 1 ? a.cu_seqlens[1] / C + 1 : INT_MAX;
        if (a.num_seqs > 0) {
            sa0_ = a.cu_seqlens[0];
            slen_ = (int64_t)a.cu_seqlens[1] - sa0_;
        }
    }
    if (!a.cu_seqlens && W > 0) {
        dH = G % H;
        dC = (G / H) % W;
        dB = G / (W * H);
        ch_ = bid % H;
        cc_ = (bid / H) % W;
        cb_ = bid / (W * H);
    }
    auto find = [&](int from, Item &x) -> int {
        if (!a.cu_seqlens) {  // `from` is the cursor's item
            if (from >= nitems) return nitems;
            const int c = c0 + cc_;
            x.h = ch_;
            x.n = cb_ * NC + c;
            x.t0 = (int64_t)cb_ * a.T + (int64_t)c * C;
            x.len = (int)min((int64_t)C, a.T - (int64_t)c * C);
            ch_ += dH;
            const int k1 = ch_ >= H ? 1 : 0;
            ch_ -= k1 * H;
            cc_ += dC + k1;
            const int k2 = cc_ >= W ? 1 : 0;
            cc_ -= k2 * W;
            cb_ += dB + k2;
            return from;
        }
        for (int it = from; it < nitems; it += G) {  // `from` is the cursor's item
            const int n = cc_, hh = ch_;
            ch_ += dH;
            const int k1 = ch_ >= H ? 1 : 0;
            ch_ -= k1 * H;
            cc_ += dC + k1;
            while (n >= fsn_) {
                ++sq_;
                fs_ = fsn_;
                fsn_ = sq_ + 1 < a.num_seqs ? a.cu_seqlens[sq_ + 1] / C + sq_ + 1 : INT_MAX;
                sa0_ = a.cu_seqlens[sq_];
                slen_ = (int64_t)a.cu_seqlens[sq_ + 1] - sa0_;
            }
            const int64_t a0 = sa0_, l = slen_;
            const int64_t off = (int64_t)(n - fs_) * C;
            if (off < l) {
                x.n = n;
                x.h = hh;
                x.t0 = a0 + off;
                x.len = (int)min((int64_t)C, l - off);
                return it;
            }
        }
        return nitems;
    };

    // Mapping as in the chunk kernel's prep waves: a combo is a (channel pair, 16-row
    // tile), handled by lanes l, l + 16, l + 32, l + 48 of one wave (rows 0..3, 4..7,
    // 8..11, 12..15 of the tile).
    constexpr int NCP = K / 2;
    constexpr int NCOMBO = NCP * NP;
    constexpr int CPR = 16 * PPW;
    constexpr int CPT = (NCOMBO + CPR - 1) / CPR;
    using RawPair = typename std::conditional<std::is_same<TIn, float>::value, float2, uint32_t>::type;
    using RawGate = typename std::conditional<ZG, RawPair, float2>::type;
    auto pair_f32 = [&](RawPair x, float &lo, float &hi) {
        if constexpr (std::is_same<RawPair, float2>::value) {
            lo = x.x;
            hi = x.y;
        } else {
            lo = __builtin_bit_cast(float, x << 16);
            hi = __builtin_bit_cast(float, x & 0xffff0000u);
        }
    };
    // raw inputs of one item, loaded unconditionally (rows past the end read the last row)
    RawGate rg[CPT][4];
    RawPair rq[CPT][4], rk[CPT][4];
    float2 rzb[CPT];
    float rbeta, rls;
    auto fetch = [&](const Item &x) {
        // the thread index, hidden from loop-invariant code motion: the per-combo offsets
        // are recomputed per item instead of being held in registers across the loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = tid >> 6, qd = lane >> 4;
        const int last = x.len - 1;
        const int rs = H * K;
        const int64_t cb = (x.t0 * H + x.h) * K;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            int cm = CPR * u + 16 * wave + (lane & 15);
            cm = cm < NCOMBO ? cm : 0;
            const int c0 = 2 * (cm % NCP), p = cm / NCP;
            rzb[u] = float2{0.f, 0.f};
            if constexpr (ZG) {
                if (a.gate.bias) rzb[u] = *reinterpret_cast<const float2 *>(a.gate.bias + x.h * K + c0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * p + 4 * qd + i;
                const uint32_t o = (uint32_t)((r < last ? r : last) * rs + c0);
                if constexpr (ZG)
                    rg[u][i] = ld_at<RawGate>(static_cast<const TIn *>(a.gate.logits) + cb, o * (uint32_t)sizeof(TIn));
                else
                    rg[u][i] = ld_at<RawGate>(a.gate.gate + cb, 4u * o);
                rq[u][i] = ld_at<RawPair>(static_cast<const TIn *>(a.q) + cb, o * (uint32_t)sizeof(TIn));
                rk[u][i] = ld_at<RawPair>(static_cast<const TIn *>(a.k) + cb, o * (uint32_t)sizeof(TIn));
            }
        }
        rbeta = ld_at<float>(a.beta + x.t0 * H + x.h, 4u * (uint32_t)((tid < last ? tid : last) * H));
        if constexpr (ZG) rls = a.gate.log_scale[x.h];
    };

    Item cur;
    int item = find(bid, cur);
    if (item < nitems) fetch(cur);
    while (item < nitems) {  // workgroup-uniform
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, qd = lane >> 4;
        const int h = cur.h, last = cur.len - 1;
        unsigned char *gp = a.pack + ((size_t)cur.n * H + h) * PL::bytes;
        auto combo_of = [&](int u) { return CPR * u + 16 * wave + (lane & 15); };
        // The 16-row tile of combo cm.  When NCP is a multiple of 16 the sixteen combos of a
        // wave (and their validity) share one tile, so the tile index is wave-uniform: in a
        // scalar register its comparisons select without vector instructions.
        auto tile_of = [&](int cm) -> int {
            if constexpr (NCP % 16 == 0) return __builtin_amdgcn_readfirstlane(cm / NCP);
            else return cm / NCP;
        };

        // ---- phase 1: retention factors (1 on padding rows), tile totals, beta --------
        const bool glog = a.gate.mode == GATE_LOG;
        float gs2 = 0.f, gl2 = 0.f;
        if constexpr (ZG) {
            gs2 = __builtin_amdgcn_exp2f(rls * 1.44269504088896341f) * 1.44269504088896341f;  // e^A log2(e)
            gl2 = a.gate.lower_bound * 1.44269504088896341f;
        }
        float2 ral[CPT][4], fq[CPT][4], fk[CPT][4];
        float2 pin[CPT], sin[CPT];
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float2 al;
                if constexpr (ZG) {
                    float z0, z1;
                    if constexpr (std::is_same<RawGate, float2>::value) {
                        z0 = rg[u][i].x;
                        z1 = rg[u][i].y;
                    } else {
                        pair_f32(rg[u][i], z0, z1);
                    }
                    al = float2{fast_bounded_alpha(z0 + rzb[u].x, gs2, gl2), fast_bounded_alpha(z1 + rzb[u].y, gs2, gl2)};
                } else {
                    al = rg[u][i];
                    if (glog) al = float2{__expf(al.x), __expf(al.y)};
                }
                float q0, q1, k0, k1;
                pair_f32(rq[u][i], q0, q1);
                pair_f32(rk[u][i], k0, k1);
                ral[u][i] = al;
                fq[u][i] = float2{q0, q1};
                fk[u][i] = float2{k0, k1};
            }
        }
        if (last < C - 1) {  // a partial chunk (workgroup-uniform): padding rows get alpha 1, q = k = 0
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u);
                const int p = tile_of(cm < NCOMBO ? cm : 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (16 * p + 4 * qd + i > last) {
                        ral[u][i] = float2{1.f, 1.f};
                        fq[u][i] = float2{0.f, 0.f};
                        fk[u][i] = float2{0.f, 0.f};
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int cm = combo_of(u);
            const bool valid = cm < NCOMBO;
            const int cmc = valid ? cm : 0;
            const int c0 = 2 * (cmc % NCP), p = tile_of(cmc);
            float2 run = {1.f, 1.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                run.x *= ral[u][i].x;
                run.y *= ral[u][i].y;
            }
            // the four quarters' products: lane quarter qd ^ d sends its own
            float2 xq[4];
            xq[0] = run;
            xq[1] = float2{__shfl_xor(run.x, 16), __shfl_xor(run.y, 16)};
            xq[2] = float2{__shfl_xor(run.x, 32), __shfl_xor(run.y, 32)};
            xq[3] = float2{__shfl_xor(run.x, 48), __shfl_xor(run.y, 48)};
            float2 qp[4];
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
            if (qd == 0 && valid)
                *reinterpret_cast<float2 *>(TPv + p * K + c0) =
                    float2{(qp[0].x * qp[1].x) * (qp[2].x * qp[3].x), (qp[0].y * qp[1].y) * (qp[2].y * qp[3].y)};
            if constexpr (NORM) {
                // row sums of q^2 (0..3) and k^2 (4..7) over this tile's channel pairs
                float x2[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x2[i] = fq[u][i].x * fq[u][i].x + fq[u][i].y * fq[u][i].y;
                    x2[4 + i] = fk[u][i].x * fk[u][i].x + fk[u][i].y * fk[u][i].y;
                }
                constexpr int NG = NCP < 16 ? NCP : 16;
                static_assert(NG == 8 || NG == 16, "8 or 16 lanes share a tile row");
                int base = 0;
                halve_sums<4, true, NG / 2>(x2, lane, base);
                halve_sums<2, true, NG / 4>(x2, lane, base);
                halve_sums<1, true, NG / 8>(x2, lane, base);
                if constexpr (NG == 16) x2[0] += __shfl_xor(x2[0], 1);
                if (valid && (NG != 16 || (lane & 1) == 0)) {
                    const int part = (cm % NCP) / 16;
                    Nrm[((p * 2 + (base >> 2)) * 16 + 4 * qd + (base & 3)) * L::NPART + part] = x2[0];
                }
            }
        }
        if (tid < C) {
            const float b = a.beta_logits ? __builtin_amdgcn_rcpf(1.f + __expf(-rbeta)) : rbeta;
            const float bt = tid <= last ? b : 0.f;
            Btv[tid] = bt;
            reinterpret_cast<float *>(gp + PL::gBt)[tid] = bt;
        }
        // the raw inputs are consumed: send the next item's loads
        Item nx;
        const int nxt = find(item + G, nx);
        fetch(nxt < nitems ? nx : cur);
        lds_barrier();
        // The item's 2 C reciprocal row norms, once (wave 0 sums each row's per-wave partials),
        // into the second row-norm buffer, which the pre-pass does not otherwise use: the
        // staging and the A-matrix tiles then read one value per row instead of summing the
        // partials and taking the reciprocal square root per lane.
        float *InvN = Nrm + L::NNRM;
        if constexpr (NORM) {
            if (wave == 0) {  // wave-uniform
                for (int e = lane; e < 2 * C; e += 64) {
                    const int qk = e / C, r = e % C;
                    float n = 0.f;
#pragma unroll
                    for (int pt = 0; pt < L::NPART; ++pt) n += Nrm[(((r >> 4) * 2 + qk) * 16 + (r & 15)) * L::NPART + pt];
                    InvN[e] = __builtin_amdgcn_rsqf(fmaxf(n, 1e-12f));
                }
            }
            lds_barrier();
        }

        // ---- phase 2: A-matrix operand staging and the package's Qt, -Bw, gamma_C; Kt is
        // kept in registers and goes out through LDS after phase 3 (16-byte stores)
        float2 ktk[CPT][4];
        // (paired order, 16-bit: Qt and -Bw wait in registers as packed pairs and leave
        // through LDS with the copy-out's 16-byte stores, a quarter of the store instructions)
        constexpr bool STQ = PERM && !std::is_same<TM, float>::value;
        uint32_t qtp[CPT][4], bwp[CPT][4];
        // Phase 2 for key-column block BLK of the staging (the only block unless the staging
        // holds fewer than K columns); OUTS: also the package's Qt, -Bw, gamma_C and Kt
        auto phase2 = [&](auto blk_c, auto outs_c) {
            constexpr int BLK = decltype(blk_c)::value;
            constexpr bool OUTS = decltype(outs_c)::value;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                const int cm = combo_of(u);
                if (cm >= NCOMBO) continue;
                const int c0 = 2 * (cm % NCP), p = tile_of(cm);
                // this combo's columns in the staged block (c0, c0 + 1 stay in one block)
                const bool stg = L::KS == K || c0 / L::KS == BLK;
                if (!OUTS && !stg) continue;
                const int cs = L::KS == K ? c0 : c0 - BLK * L::KS;
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
                if (OUTS && p == 0 && qd == 0) st2_at<float>(gp, (uint32_t)(PL::gGC + 4 * c0), eAll.x, eAll.y);
                const float2 rT = {__builtin_amdgcn_rcpf(own.x), __builtin_amdgcn_rcpf(own.y)};
                float2 xf[NP];  // extra right-operand factors for tiles (pp, p), pp >= p + 2
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
                float2 suf[4];  // E_p / gamma_i
                {
                    float2 run = sin[u];
#pragma unroll
                    for (int i = 3; i >= 0; --i) {
                        suf[i] = run;
                        run.x *= ral[u][i].x;
                        run.y *= ral[u][i].y;
                    }
                }
                float iq[4], ik[4];  // reciprocal row norms (1 without normalisation)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    iq[i] = 1.f;
                    ik[i] = 1.f;
                    if constexpr (NORM) {
                        iq[i] = InvN[16 * p + 4 * qd + i];
                        ik[i] = InvN[C + 16 * p + 4 * qd + i];
                    }
                }
                float2 pre = pin[u];  // gamma_i / R_p
                float2 kro[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * p + 4 * qd + i;
                    pre.x *= ral[u][i].x;
                    pre.y *= ral[u][i].y;
                    const float2 q2 = fq[u][i], k2 = fk[u][i];
                    const float2 lq = {q2.x * pre.x, q2.y * pre.y};
                    const float2 lk = {bet[i] * k2.x * pre.x, bet[i] * k2.y * pre.y};
                    const float2 ro = {k2.x * suf[i].x, k2.y * suf[i].y};  // k E_p / gamma <= |k|
                    const float2 rd = {ro.x * rT.x, ro.y * rT.y};        // k R_p / gamma <= e^80 |k|
                    if (stg) {
                        st2<TA>(Lk + r * L::LKA + cs, lk.x, lk.y);
                        st2_stage<P>(St + L::sLq + r * L::LKS + cs, L::NST, lq.x, lq.y);
                        st2_stage<P>(St + L::sRd + r * L::LKS + cs, L::NST, rd.x, rd.y);
                        if (p < NP - 1) st2_stage<P>(St + L::sRo + r * L::LKS + cs, L::NST, ro.x, ro.y);
                        if constexpr (L::NX > 0) {
                            int xi = 0;
#pragma unroll
                            for (int pp = 2; pp < NP; ++pp)
#pragma unroll
                                for (int qq = 0; qq + 2 <= pp; ++qq, ++xi)
                                    if (qq == p)
                                        st2_stage<P>(St + L::sX + (xi * 16 + 4 * qd + i) * L::LKS + cs, L::NST,
                                                     ro.x * xf[pp].x, ro.y * xf[pp].y);
                        }
                    }
                    if constexpr (!OUTS) continue;
                    constexpr uint32_t E = sizeof(TM);
                    const int cq = PERM ? paired_col(c0) : c0;  // (c0 even: c0, c0 + 1 stay adjacent)
                    if constexpr (STQ) {
                        typedef __attribute__((ext_vector_type(2))) _Float16 h2;
                        qtp[u][i] = __builtin_bit_cast(uint32_t, h2{(_Float16)(lq.x * eR.x * iq[i]), (_Float16)(lq.y * eR.y * iq[i])});
                        bwp[u][i] = __builtin_bit_cast(uint32_t, h2{(_Float16)(-lk.x * eR.x * ik[i]), (_Float16)(-lk.y * eR.y * ik[i])});
                    } else {
                        st2_at<TM>(gp, (uint32_t)PL::gQt + E * (uint32_t)(r * K + cq), lq.x * eR.x * iq[i], lq.y * eR.y * iq[i]);
                        st2_at<TM>(gp, (uint32_t)PL::gBw + E * (uint32_t)(r * K + cq), -lk.x * eR.x * ik[i], -lk.y * eR.y * ik[i]);
                    }
                    kro[i] = float2{ro.x * eCE.x * ik[i], ro.y * eCE.y * ik[i]};
                    ktk[u][i] = kro[i];
                }
            }
        };
        phase2(std::integral_constant<int, 0>{}, std::true_type{});
        lds_barrier();

        // ---- phase 3: A-matrix tiles, T's diagonal blocks, A_qk ------------------------
        if constexpr (L::KS == K) {
            a_matrix_work<P, K, 16, C, 16, NORM, PPW, true>(smem, smem + PXL::oTA - L::pTm, 0, wave, lane);
        } else {
            // the second half of the key columns is staged once every wave is done with the first
            static_assert(2 * L::KS == K, "two column blocks");
            a_matrix_work_blocks<P, K, C, NORM, PPW>(smem, smem + PXL::oTA - L::pTm, wave, lane, [&](int) {
                lds_barrier();
                phase2(std::integral_constant<int, 1>{}, std::false_type{});
                lds_barrier();
            });
        }
        lds_barrier();

        // Kt [K][C] into the staging area, free now (row stride LCT), two tokens per store
        constexpr int LCT = C + 16 / (int)sizeof(TM);
        static_assert((size_t)K * LCT * sizeof(TM) <= (size_t)L::NST * sizeof(TA) * (P::kSplit ? 2 : 1),
                      "the Kt tile fits in the operand staging area");
        TM *KtL = reinterpret_cast<TM *>(St);
        // Qt and -Bw [C][K] (paired columns) after Kt, row stride LQT
        constexpr int LQT = K + 16 / (int)sizeof(TM);
        constexpr size_t oQtL = ((size_t)K * LCT * sizeof(TM) + 15) & ~size_t(15);
        constexpr size_t oBwL = oQtL + (size_t)C * LQT * sizeof(TM);
        static_assert(!STQ || oBwL + (size_t)C * LQT * sizeof(TM) <= (size_t)L::NST * sizeof(TA) * (P::kSplit ? 2 : 1),
                      "Kt, Qt and -Bw fit in the operand staging area");
        unsigned char *StB = reinterpret_cast<unsigned char *>(St);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int cm = combo_of(u);
            if (cm >= NCOMBO) continue;
            const int c0 = 2 * (cm % NCP), p = tile_of(cm);
#pragma unroll
            for (int i = 1; i < 4; i += 2) {
                const int r = 16 * p + 4 * qd + i;
                st2<TM>(KtL + c0 * LCT + r - 1, ktk[u][i - 1].x, ktk[u][i].x);
                st2<TM>(KtL + (c0 + 1) * LCT + r - 1, ktk[u][i - 1].y, ktk[u][i].y);
            }
            if constexpr (STQ) {
                const int cq = paired_col(c0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * p + 4 * qd + i;
                    *reinterpret_cast<uint32_t *>(StB + oQtL + ((size_t)r * LQT + cq) * sizeof(TM)) = qtp[u][i];
                    *reinterpret_cast<uint32_t *>(StB + oBwL + ((size_t)r * LQT + cq) * sizeof(TM)) = bwp[u][i];
                }
            }
        }

        // ---- phase 4: T's off-diagonal blocks.  Block column qb depends only on itself
        // (T_pq = -T_pp sum_{r=q}^{p-1} A_pr T_rq), so wave qb fills column qb top down.
        if constexpr (NP == 2) {
            // one off-diagonal block: T_10 = -T_11 (A_10 T_00), every operand read first
            if (wave == 0) {
                const int l15 = lane & 15;
                float av[4], tv[4], tt[4];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    av[s4] = Akk[(16 + l15) * L::LCF + 4 * s4 + g];
                    tv[s4] = Tf[(4 * s4 + g) * L::LCF + l15];
                    tt[s4] = Tf[(16 + l15) * L::LCF + 16 + 4 * g + s4];
                }
                f4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) m = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s4], tv[s4], m, 0, 0, 0);
                f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) t = __builtin_amdgcn_mfma_f32_16x16x4f32(tt[s4], m[s4], t, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 + 4 * g + e, j = l15;
                    Tf[i * L::LCF + j] = -t[e];
                    TmL[i * L::LCM + j] = from_f32<TM>(-t[e]);
                }
            }
        } else if (NP > 1 && wave < NP - 1) {
            const int qb = wave;
            for (int p = qb + 1; p < NP; ++p) {
                f4 m = {0.f, 0.f, 0.f, 0.f};
                for (int r = qb; r < p; ++r)
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        m = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            Akk[(p * 16 + (lane & 15)) * L::LCF + r * 16 + 4 * s4 + g],
                            Tf[(r * 16 + 4 * s4 + g) * L::LCF + qb * 16 + (lane & 15)], m, 0, 0, 0);
                f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(Tf[(p * 16 + (lane & 15)) * L::LCF + p * 16 + 4 * g + s4],
                                                             m[s4], t, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = p * 16 + 4 * g + e, j = qb * 16 + (lane & 15);
                    Tf[i * L::LCF + j] = -t[e];
                    TmL[i * L::LCM + j] = from_f32<TM>(-t[e]);
                }
                lds_fence();
            }
        }
        lds_barrier();

        // ---- Qt and -Bw (paired order), Kt, T and A_qk to the package, 16 bytes per lane ---
        // (the next item's phase 1 touches neither these nor the staging area, and its
        // first barrier comes before anything here is written again).  A lane reads all its
        // pieces from LDS before it stores any, so it waits for LDS once; piece e of the lane
        // is tid + j PPT, and with tid < PPT known the region of most pieces is fixed at
        // compile time.
        {
            constexpr int RC = C * (int)sizeof(TM) / 16;            // 16-byte pieces per row
            constexpr int RQ = K * (int)sizeof(TM) / 16;
            constexpr int NQP = STQ ? 2 * C * RQ : 0;                // Qt's C rows, then -Bw's C
            constexpr int NKP = (K + (1 + P::kAqParts) * C) * RC;   // Kt's K, T's C, A_qk's C per part
            constexpr int NJ = (NQP + NKP + PPT - 1) / PPT;
            __builtin_assume(tid >= 0 && tid < PPT);
            uint4 x[NJ];
            uint32_t dst[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e = tid + j * PPT;
                dst[j] = 0xffffffffu;  // no piece
                if (e < NQP) {
                    const int row = e / RQ, pc = e % RQ;
                    const size_t src = (row < C ? oQtL : oBwL) + ((size_t)(row % C) * LQT) * sizeof(TM) + 16 * pc;
                    dst[j] = (uint32_t)((row < C ? PL::gQt : PL::gBw) + (size_t)(row % C) * K * sizeof(TM) + 16 * pc);
                    x[j] = *reinterpret_cast<const uint4 *>(StB + src);
                } else if (e < NQP + NKP) {
                    const int f = e - NQP;
                    const int row = f / RC, pc = f % RC;
                    const TM *src;
                    size_t d;
                    if (row < K) {
                        src = KtL + row * LCT;
                        d = PL::gKt + (size_t)row * C * sizeof(TM);
                    } else if (row < K + C) {
                        src = TmL + (row - K) * L::LCM;
                        d = PL::gTm + (size_t)(row - K) * C * sizeof(TM);
                    } else if (row < K + 2 * C) {
                        src = AqL + (row - K - C) * L::LCM;
                        d = PL::gAqk + (size_t)(row - K - C) * C * sizeof(TM);
                    } else {
                        src = AlL + (row - K - 2 * C) * L::LCM;
                        d = PL::gAqk + (size_t)(row - K - C) * C * sizeof(TM);  // the lo part follows
                    }
                    dst[j] = (uint32_t)(d + 16 * pc);
                    if constexpr (PERM && !std::is_same<TM, float>::value) {
                        // piece pc of the paired row: tokens 32m + 4g + 0..3 and 32m + 16 + 4g + 0..3
                        const int k0 = 32 * (pc >> 2) + 4 * (pc & 3);
                        const uint2 lo = *reinterpret_cast<const uint2 *>(src + k0);
                        const uint2 hi = *reinterpret_cast<const uint2 *>(src + k0 + 16);
                        x[j] = uint4{lo.x, lo.y, hi.x, hi.y};
                    } else {
                        x[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const unsigned char *>(src) + 16 * pc);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (dst[j] != 0xffffffffu) *reinterpret_cast<uint4 *>(gp + dst[j]) = x[j];
        }
        item = nxt;
        cur = nx;
    }
}

template <class P, int K, int C, int GM, bool PERM>
__global__ __launch_bounds__(PPT) void chunk_pack_kernel(ChunkArgs a) {
    pack_body<P, K, C, GM, PERM>(a, (int)blockIdx.x, (int)gridDim.x);
}

// The chain kernel: state waves as in chunk_fwd_kernel, copy waves for the packages.
// Workgroup bid of G (G a multiple of 8: a head's value blocks share one XCD).
// FEW_REGS: the state waves keep fewer operand fragments live (the chain beside the pre-pass
// in one launch, at four waves per SIMD).
template <class P, int K, int V, int C, int BV, bool FEW_REGS = false>
__device__ __forceinline__ void chain_body(const ChunkArgs &a, int bid, int G) {
    using L = Layout<P, K, V, C, BV>;
    using PL = PackLayout<P, K, C>;
    using TM = typename P::TM;
    using TIn = typename std::conditional<std::is_same<P, PrecF32>::value, float, __bf16>::type;

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    constexpr int NVB = V / BV;
    int lin = bid;
    if ((G & 7) == 0) lin = (bid & 7) * (G >> 3) + (bid >> 3);  // a head's value blocks
    const int vb = lin % NVB;                                                   // share one XCD
    const int pair = lin / NVB;
    const int H = a.H;
    const int h = pair % H;
    const int s = pair / H;
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
    // this launch's chunks of the sequence: [c_begin, c_end) clipped to it (the state
    // comes in through a.initial_state and leaves through a.final_state)
    const int nall = (int)((eos - bos + C - 1) / C);
    const int cfirst = a.c_begin < nall ? a.c_begin : nall;
    const int nchunks = (a.c_end < nall ? a.c_end : nall) - cfirst;
    bos += (int64_t)cfirst * C;
    base += cfirst;

    // The pre-pass of the next chunk segment may share these compute units: the serial part
    // issues first, then the copy waves that feed it.
    if (wave < NSW) {
        __builtin_amdgcn_s_setprio(3);
        state_waves<P, K, V, C, BV, false, true, FEW_REGS>(a, smem, smem, s, h, vb, bos, eos, nchunks, wave, lane);
        return;
    }
    __builtin_amdgcn_s_setprio(2);

    // ====================================== copy waves =======================================
    constexpr int NCT = 64 * NCW;
    const int tp = tid - NSW * 64;
    // 16-byte pieces of a package in workspace order (Qt, Bw, Kt, T, A_qk, then gamma_C and
    // beta, adjacent in both places), each with its LDS destination
    constexpr int RQ = K * (int)sizeof(TM) / 16, RC = C * (int)sizeof(TM) / 16;
    constexpr int NQ = C * RQ, NKT = K * RC, NCC = C * RC, NGC = (K + C) * 4 / 16;
    constexpr int NAQ = P::kAqParts * NCC;  // A_qk's pieces (hi, then lo)
    constexpr int NPC = 2 * NQ + NKT + NCC + NAQ + NGC;
    static_assert(PL::gGC + 16 * NGC == PL::bytes, "the pieces cover the whole package");
    static_assert(L::pBt == L::pGC + (size_t)K * 4, "gamma_C and beta adjacent in LDS");
    constexpr int CPT = (NPC + NCT - 1) / NCT;
    // The matrix operands go into LDS with the row swizzle the state waves read them with
    // (mma_bfrag): in rows whose index has bit 3 set the two 8-byte halves of each piece
    // trade places.
    uint32_t src[CPT], dst[CPT];
    bool swp[CPT];
#pragma unroll
    for (int w = 0; w < CPT; ++w) {
        int e = tp + NCT * w;
        e = e < NPC ? e : NPC - 1;  // surplus lanes repeat the last piece (same value, same place)
        src[w] = 16u * (uint32_t)e;
        uint32_t d;
        int row = 0;
        if (e < NQ) {
            row = e / RQ;
            d = (uint32_t)(L::pQt + row * L::LKM * sizeof(TM) + 16 * (e % RQ));
        } else if (e < 2 * NQ) {
            const int x = e - NQ;
            row = x / RQ;
            d = (uint32_t)(L::pBw + row * L::LKM * sizeof(TM) + 16 * (x % RQ));
        } else if (e < 2 * NQ + NKT) {
            const int x = e - 2 * NQ;
            row = x / RC;
            d = (uint32_t)(L::pKt + row * L::LCM * sizeof(TM) + 16 * (x % RC));
        } else if (e < 2 * NQ + NKT + NCC) {
            const int x = e - 2 * NQ - NKT;
            row = x / RC;
            d = (uint32_t)(L::pTm + row * L::LCM * sizeof(TM) + 16 * (x % RC));
        } else if (e < 2 * NQ + NKT + NCC + NAQ) {
            const int x = e - 2 * NQ - NKT - NCC;  // A_qk rows 0..C-1, then its lo part's
            row = (x / RC) % C;
            d = (uint32_t)((x < NCC ? L::pAqk : L::pAql) + row * L::LCM * sizeof(TM) + 16 * (x % RC));
        } else {
            d = (uint32_t)(L::pGC + 16 * (e - 2 * NQ - NKT - NCC - NAQ));  // gamma_C, beta: no matrix
        }
        dst[w] = d;
        swp[w] = (row & 8) != 0;
    }
    // value items: four value columns of two consecutive tokens, the token pairs on
    // consecutive lanes (the transposed LDS writes then fall in distinct banks)
    using RawV = typename std::conditional<std::is_same<TIn, float>::value, float4, uint2>::type;
    constexpr int NVI = BV / 4 * (C / 2);
    constexpr int VPT = (NVI + NCT - 1) / NCT;
    // Inputs of DP chunks in flight at once (register sets, by chunk index mod DP).
    constexpr int DP = 1;
    uint4 buf[DP][CPT];
    RawV rv[DP][VPT][2];
    auto load = [&](int cn, uint4 (&buf)[CPT], RawV (&rv)[VPT][2]) {
        const int64_t t0 = bos + (int64_t)cn * C;
        const int last = (int)((eos - t0) < C ? (eos - t0) : C) - 1;
        const unsigned char *gp = a.pack + ((size_t)(base + cn) * H + h) * PL::bytes;
#pragma unroll
        for (int w = 0; w < CPT; ++w) buf[w] = ld_at<uint4>(gp, src[w]);
        const unsigned char *vbp = static_cast<const unsigned char *>(a.v) + ((t0 * H + h) * V + vb * BV) * sizeof(TIn);
#pragma unroll
        for (int w = 0; w < VPT; ++w) {
            int e = tp + NCT * w;
            e = e < NVI ? e : NVI - 1;
            const int j = 4 * (e / (C / 2)), r = 2 * (e % (C / 2));
            const int r0 = r < last ? r : last, r1 = r + 1 < last ? r + 1 : last;
            rv[w][0] = ld_at<RawV>(vbp, (uint32_t)sizeof(TIn) * (uint32_t)(r0 * H * V + j));
            rv[w][1] = ld_at<RawV>(vbp, (uint32_t)sizeof(TIn) * (uint32_t)(r1 * H * V + j));
        }
    };
    auto raw4 = [](RawV x, float (&f)[4]) {
        if constexpr (std::is_same<TIn, float>::value) {
            f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
        } else {
            f[0] = __builtin_bit_cast(float, x.x << 16);
            f[1] = __builtin_bit_cast(float, x.x & 0xffff0000u);
            f[2] = __builtin_bit_cast(float, x.y << 16);
            f[3] = __builtin_bit_cast(float, x.y & 0xffff0000u);
        }
    };
#pragma unroll
    for (int d = 0; d < DP; ++d)
        if (d < nchunks) load(d, buf[d], rv[d]);
    for (int it0 = 0; it0 <= nchunks; it0 += DP) {
#pragma unroll
        for (int d = 0; d < DP; ++d) {  // register set d holds chunk it = it0 + d
            const int it = it0 + d;
            if (it > nchunks) break;  // workgroup-uniform
            if (it < nchunks) {
                unsigned char *pk = smem + (size_t)(it & 1) * L::szPkg;
#pragma unroll
                for (int w = 0; w < CPT; ++w) {
                    const uint4 x = buf[d][w];
                    *reinterpret_cast<uint4 *>(pk + dst[w]) = swp[w] ? uint4{x.z, x.w, x.x, x.y} : x;
                }
                TIn *vL = reinterpret_cast<TIn *>(pk + L::pbV);
#pragma unroll
                for (int w = 0; w < VPT; ++w) {
                    int e = tp + NCT * w;
                    e = e < NVI ? e : NVI - 1;
                    const int j = 4 * (e / (C / 2)), r = 2 * (e % (C / 2));
                    float f0[4], f1[4];
                    raw4(rv[d][w][0], f0);
                    raw4(rv[d][w][1], f1);
#pragma unroll
                    for (int x = 0; x < 4; ++x) st2<TIn>(vL + (j + x) * L::LCM + r, f0[x], f1[x]);
                }
                if (it + DP < nchunks) load(it + DP, buf[d], rv[d]);  // consumed DP periods on
            }
            lds_barrier();  // the one barrier of the period: package it is in LDS
        }
    }
}

template <class P, int K, int V, int C, int BV>
__global__ __launch_bounds__(NTC) void chunk_chain_kernel(ChunkArgs a) {
    chain_body<P, K, V, C, BV>(a, (int)blockIdx.x, (int)gridDim.x);
}

// Waves per SIMD the segment kernel is compiled for: the precision's choice for chunks of
// up to 32 tokens, two for 64-token chunks (too many live fragments for four).
template <class P, int C>
constexpr int seg_waves() {
    return C <= 32 ? P::kSegWaves : 2;
}

// One launch of a chunk segment: workgroups [0, nchain) run the chain over segment s
// (arguments ca), the rest the pre-pass of segment s + 1 (arguments pa).  The chain's
// workgroups come first in dispatch order, so they are placed before the pre-pass fills
// the remaining room; nothing in one launch waits for another workgroup of it.
template <class P, int K, int V, int C, int BV, int GM>
__global__ __launch_bounds__(NTC) __attribute__((amdgpu_waves_per_eu(seg_waves<P, C>()))) void chunk_segment_kernel(
    ChunkArgs ca, ChunkArgs pa, int nchain) {
    static_assert(NTC == PPT, "both roles run with the same workgroup size");
    if ((int)blockIdx.x < nchain)
        chain_body<P, K, V, C, BV, (seg_waves<P, C>() > 2)>(ca, (int)blockIdx.x, nchain);
    else
        pack_body<P, K, C, GM>(pa, (int)blockIdx.x - nchain, (int)gridDim.x - nchain);
}

template <class P, int K, int V, int C>
constexpr int pick_chain_bv() {
    if constexpr (V >= 64 && ChainLds<P, K, V, C, 64>::fits) return 64;
    else if constexpr (V >= 32 && ChainLds<P, K, V, C, 32>::fits) return 32;
    else if constexpr (ChainLds<P, K, V, C, 16>::fits) return 16;
    else return 0;
}

template <class P, int GM, int K, int C, bool PERM>
hipError_t launch_pack_kcp(const ChunkArgs &a, int64_t items, int max_wgs, hipStream_t stream) {
    using X = PrepassLds<P, K, C>;
    if constexpr (!X::fits || (PERM && (K % 32 != 0 || C % 32 != 0))) {
        return hipErrorNotSupported;
    } else {
        auto kern = chunk_pack_kernel<P, K, C, GM, PERM>;
        static std::atomic<bool> attr_set{false};
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)X::total);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        // persistent: at most as many workgroups as fit at once (LDS-bound), max_wgs and items
        const int per_cu = (int)(160 * 1024 / X::total) < 4 ? (int)(160 * 1024 / X::total) : 4;
        int64_t grid = (int64_t)device_cu_count() * per_cu;
        if (max_wgs > 0 && grid > max_wgs) grid = max_wgs;
        if (grid > items) grid = items;
        if (grid <= 0) return hipSuccess;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(PPT), X::total, stream, a);
        return hipGetLastError();
    }
}

// the pre-pass in the plain order, or in the paired order when a.pack_paired is set
template <class P, int GM, int K, int C>
hipError_t launch_pack_kc(const ChunkArgs &a, int64_t items, int max_wgs, hipStream_t stream) {
    if (a.pack_paired) {
        if constexpr (std::is_same<P, PrecMixed>::value) return launch_pack_kcp<P, GM, K, C, true>(a, items, max_wgs, stream);
        return hipErrorNotSupported;
    }
    return launch_pack_kcp<P, GM, K, C, false>(a, items, max_wgs, stream);
}

template <class P, int GM>
hipError_t launch_pack_p(const ChunkArgs &a, int K, int C, int64_t items, int max_wgs, hipStream_t stream) {
#define KDA_PACK_C(KK)                                                         \
    switch (C) {                                                               \
        case 16: return launch_pack_kc<P, GM, KK, 16>(a, items, max_wgs, stream);     \
        case 32: return launch_pack_kc<P, GM, KK, 32>(a, items, max_wgs, stream);     \
        case 64: return launch_pack_kc<P, GM, KK, 64>(a, items, max_wgs, stream);     \
        default: return hipErrorNotSupported;                                  \
    }
    switch (K) {
        case 16: KDA_PACK_C(16)
        case 32: KDA_PACK_C(32)
        case 64: KDA_PACK_C(64)
        case 128: KDA_PACK_C(128)
        default: return hipErrorNotSupported;
    }
#undef KDA_PACK_C
}

template <class P, int K, int V, int C>
hipError_t launch_chain_kvc(const ChunkArgs &a, int num_pairs, hipStream_t stream, int *bv_out) {
    constexpr int BV = pick_chain_bv<P, K, V, C>();
    if constexpr (BV == 0 || !PrepassLds<P, K, C>::fits) {
        return hipErrorNotSupported;
    } else {
        using X = ChainLds<P, K, V, C, BV>;
        if (bv_out) *bv_out = BV;
        if (!a.q) return hipSuccess;  // query only
        auto kern = chunk_chain_kernel<P, K, V, C, BV>;
        static std::atomic<bool> attr_set{false};
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)X::total);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL(kern, dim3(num_pairs * (V / BV)), dim3(NTC), X::total, stream, a);
        return hipGetLastError();
    }
}

template <class P>
hipError_t launch_chain_p(const ChunkArgs &a, int K, int V, int C, int num_pairs, hipStream_t stream, int *bv) {
#define KDA_CHAIN_C(KK, VV)                                                          \
    switch (C) {                                                                     \
        case 16: return launch_chain_kvc<P, KK, VV, 16>(a, num_pairs, stream, bv);   \
        case 32: return launch_chain_kvc<P, KK, VV, 32>(a, num_pairs, stream, bv);   \
        case 64: return launch_chain_kvc<P, KK, VV, 64>(a, num_pairs, stream, bv);   \
        default: return hipErrorNotSupported;                                        \
    }
#define KDA_CHAIN_V(KK)                        \
    switch (V) {                               \
        case 16: KDA_CHAIN_C(KK, 16)           \
        case 32: KDA_CHAIN_C(KK, 32)           \
        case 64: KDA_CHAIN_C(KK, 64)           \
        case 128: KDA_CHAIN_C(KK, 128)         \
        default: return hipErrorNotSupported;  \
    }
    switch (K) {
        case 16: KDA_CHAIN_V(16)
        case 32: KDA_CHAIN_V(32)
        case 64: KDA_CHAIN_V(64)
        case 128: KDA_CHAIN_V(128)
        default: return hipErrorNotSupported;
    }
#undef KDA_CHAIN_V
#undef KDA_CHAIN_C
}

template <class P, int GM, int K, int V, int C>
hipError_t launch_segment_kvc(const ChunkArgs &ca, const ChunkArgs &pa, int num_pairs, int64_t items, int pack_wgs,
                              hipStream_t stream) {
    constexpr int BV = pick_chain_bv<P, K, V, C>();
    if constexpr (BV == 0 || !PrepassLds<P, K, C>::fits) {
        return hipErrorNotSupported;
    } else {
        constexpr size_t lds = ChainLds<P, K, V, C, BV>::total > PrepassLds<P, K, C>::total
                                   ? ChainLds<P, K, V, C, BV>::total : PrepassLds<P, K, C>::total;
        auto kern = chunk_segment_kernel<P, K, V, C, BV, GM>;
        static std::atomic<bool> attr_set{false};
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        const int nchain = num_pairs * (V / BV);
        const int np = (int)(items < pack_wgs ? items : pack_wgs);
        hipLaunchKernelGGL(kern, dim3(nchain + np), dim3(NTC), lds, stream, ca, pa, nchain);
        return hipGetLastError();
    }
}

template <class P, int GM>
hipError_t launch_segment_p(const ChunkArgs &ca, const ChunkArgs &pa, int K, int V, int C, int num_pairs,
                            int64_t items, int pack_wgs, hipStream_t stream) {
#define KDA_SEG_C(KK, VV)                                                                                \
    switch (C) {                                                                                         \
        case 16: return launch_segment_kvc<P, GM, KK, VV, 16>(ca, pa, num_pairs, items, pack_wgs, stream); \
        case 32: return launch_segment_kvc<P, GM, KK, VV, 32>(ca, pa, num_pairs, items, pack_wgs, stream); \
        case 64: return launch_segment_kvc<P, GM, KK, VV, 64>(ca, pa, num_pairs, items, pack_wgs, stream); \
        default: return hipErrorNotSupported;                                                            \
    }
#define KDA_SEG_V(KK)                          \
    switch (V) {                               \
        case 16: KDA_SEG_C(KK, 16)             \
        case 32: KDA_SEG_C(KK, 32)             \
        case 64: KDA_SEG_C(KK, 64)             \
        case 128: KDA_SEG_C(KK, 128)           \
        default: return hipErrorNotSupported;  \
    }
    switch (K) {
        case 16: KDA_SEG_V(16)
        case 32: KDA_SEG_V(32)
        case 64: KDA_SEG_V(64)
        case 128: KDA_SEG_V(128)
        default: return hipErrorNotSupported;
    }
#undef KDA_SEG_V
#undef KDA_SEG_C
}

}  // namespace

}  // namespace kda
