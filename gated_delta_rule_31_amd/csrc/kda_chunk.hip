// kda_chunk.hip -- chunkwise-parallel KDA prefill on gfx950 matrix cores.
//
// Method (KDA cheat sheet, "Chunkwise parallel form", with the UT transform the
// page names written out): for a chunk of C tokens with start state S and
// in-chunk inclusive cumulative log-decay Gamma_i = sum_{r<=i} g_r (per key
// channel),
//   A_kk[i,j] = beta_i sum_c k_ic k_jc e^{Gamma_ic - Gamma_jc}  (j < i),  T = (I + A_kk)^-1
//   W = T (beta e^Gamma K),  U = T (beta V),  Vt = U - W S          (pseudo-values)
//   A_qk[i,j] = sum_c q_ic k_jc e^{Gamma_ic - Gamma_jc}           (j <= i: the read
//               follows the write, so the diagonal is kept)
//   O  = (e^Gamma Q) S + A_qk Vt                                    (inter + intra chunk)
//   S' = e^{Gamma_C} S + (K e^{Gamma_C - Gamma})^T Vt
// This equals the token recurrence exactly in real arithmetic.
//
// Rescaling (cheat sheet gate table): with every g >= -5 the log-decay across a
// 16-token tile stays above -80, so the split e^{Gamma_i - Gamma_j} =
// e^{Gamma_i - R} e^{R - Gamma_j} with a per-tile reference R keeps both factors
// within [e^-80, e^80] -- inside float and bf16 range -- and every tile of A_kk
// and A_qk is a dense matrix-core product:
//   diagonal tile p:      R = Gamma at the row before tile p,
//   off-diagonal (p, q):  left e^{Gamma_i - R_p} (<= 1), right e^{R_p - Gamma_j} (<= 1),
//                         built as k_j e^{E_q - Gamma_j} times e^{R_p - E_q} (E_q = Gamma at
//                         the last row of tile q) so that nothing underflows early.
// Gamma is carried in log2 units so each factor is one exp2.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, block of BV
// value columns).  Value columns of the state evolve independently, so the
// split is exact; the key-side work of a chunk is recomputed per value block.
// The float32 master state lives in the accumulator registers across chunks; an
// operand copy sits in LDS.
//
// Precision (bf16 inputs): the A-matrix operands carry factors up to e^80 and
// use bf16; A_qk, which feeds each token's own value straight to its output, is
// formed from hi+lo bf16 splits of both operands.  Every other product has
// operands bounded by ~1 or by the state/value magnitude and uses fp16, which
// has 3 more mantissa bits than bf16.  fp32 inputs use fp32 matrix cores
// throughout.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int NT = 256;  // threads per workgroup
constexpr int NW = NT / 64;

constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

struct PrecMixed {
    using TA = __bf16;    // operands of the decay-rescaled key/query products
    using TM = _Float16;  // every other matrix-core operand
    static constexpr bool kSplit = true;
};
struct PrecF32 {
    using TA = float;
    using TM = float;
    static constexpr bool kSplit = false;
};

template <class P, int K, int V, int C, int BV>
struct Layout {
    using TA = typename P::TA;
    using TM = typename P::TM;
    static constexpr int NP = C / 16;                                  // 16-row tiles per chunk
    static constexpr int NX = NP >= 3 ? (NP - 1) * (NP - 2) / 2 : 0;  // tiles (p,q) with q <= p-2
    static constexpr int NSPL = P::kSplit ? 2 : 1;
    static constexpr int LKA = K + 16 / (int)sizeof(TA);  // padded row strides (elements)
    static constexpr int LKM = K + 16 / (int)sizeof(TM);
    static constexpr int LCM = C + 16 / (int)sizeof(TM);
    static constexpr int LCF = C + 4;
    static constexpr int NSEG = NT / K;      // threads sharing one key channel in the prep
    static constexpr int RPS = C / NSEG;     // rows per prep thread
    static_assert(NSEG >= 1 && RPS >= 1 && C % NSEG == 0, "prep mapping");

    static constexpr size_t szA = al16((size_t)C * LKA * sizeof(TA));
    // region 1: A-phase operands; after the A phase it holds Tm, W and Vt
    static constexpr size_t oLk = 0;
    static constexpr size_t oLq = oLk + szA;
    static constexpr size_t oRd = oLq + NSPL * szA;
    static constexpr size_t oRo = oRd + NSPL * szA;
    static constexpr size_t szRo = al16((size_t)(C - 16) * LKA * sizeof(TA));
    static constexpr size_t oX = oRo + NSPL * szRo;
    static constexpr size_t szX = al16((size_t)16 * LKA * sizeof(TA));
    static constexpr size_t r1a = oX + (size_t)NSPL * NX * szX;
    static constexpr size_t oTm = 0;
    static constexpr size_t oW = oTm + al16((size_t)C * LCM * sizeof(TM));
    static constexpr size_t oVt = oW + al16((size_t)C * LKM * sizeof(TM));
    static constexpr size_t r1b = oVt + al16((size_t)BV * LCM * sizeof(TM));
    static constexpr size_t r1 = cmax(r1a, r1b);
    // region 2: the other per-chunk operands
    static constexpr size_t oQt = r1;
    static constexpr size_t oBw = oQt + al16((size_t)C * LKM * sizeof(TM));
    static constexpr size_t oKt = oBw + al16((size_t)K * LCM * sizeof(TM));
    static constexpr size_t obV = oKt + al16((size_t)K * LCM * sizeof(TM));
    // region 3: A_kk, T (fp32 while it is built), A_qk, scratch for T's off-diagonal blocks
    static constexpr size_t oAkk = obV + al16((size_t)BV * LCM * sizeof(TM));
    static constexpr size_t oTf = oAkk + al16((size_t)C * LCF * 4);
    static constexpr size_t oAqk = oTf + al16((size_t)C * LCF * 4);
    static constexpr size_t oM = oAqk + al16((size_t)C * LCM * sizeof(TM));
    // persistent: operand copy of the state (S^T: value rows, key contiguous)
    static constexpr size_t oSt = oM + al16((size_t)3 * 256 * 4);
    // per-chunk vectors (float): references R[NP][K], E[NP][K], e^{Gamma_C}[K],
    // segment totals [NSEG][K], beta [C]
    static constexpr size_t oR = oSt + al16((size_t)BV * LKM * sizeof(TM));
    static constexpr size_t oE = oR + (size_t)NP * K * 4;
    static constexpr size_t oGC = oE + (size_t)NP * K * 4;
    static constexpr size_t oEGC = oGC + (size_t)K * 4;
    static constexpr size_t oSeg = oEGC + (size_t)K * 4;
    static constexpr size_t oBeta = oSeg + (size_t)NSEG * K * 4;
    static constexpr size_t total = al16(oBeta + (size_t)C * 4);
    static constexpr bool fits = total <= 160 * 1024;

    static constexpr int NTO = NP * (BV / 16);         // [C x BV] output / pseudo-value tiles
    static constexpr int NTS = (K / 16) * (BV / 16);   // [K x BV] state tiles
    static constexpr int MO = (NTO + NW - 1) / NW;     // tiles owned per wave
    static constexpr int MS = (NTS + NW - 1) / NW;
};

template <class P, int K, int V, int C, int BV>
__global__ __launch_bounds__(NT) void chunk_fwd_kernel(ChunkArgs a) {
    using L = Layout<P, K, V, C, BV>;
    using TA = typename P::TA;
    using TM = typename P::TM;
    using TIn = typename std::conditional<std::is_same<P, PrecF32>::value, float, __bf16>::type;
    constexpr int NP = L::NP;
    constexpr float LOG2E = 1.4426950408889634f;

    extern __shared__ __align__(16) unsigned char smem[];
    TA *Lk = reinterpret_cast<TA *>(smem + L::oLk);
    TA *Lq = reinterpret_cast<TA *>(smem + L::oLq);  // [NSPL][C][LKA]
    TA *Rd = reinterpret_cast<TA *>(smem + L::oRd);
    TA *Ro = reinterpret_cast<TA *>(smem + L::oRo);  // [NSPL][C-16][LKA]
    TA *Xv = reinterpret_cast<TA *>(smem + L::oX);   // [NSPL][NX][16][LKA]
    TM *Tm = reinterpret_cast<TM *>(smem + L::oTm);
    TM *Wn = reinterpret_cast<TM *>(smem + L::oW);   // holds -W
    TM *Vt = reinterpret_cast<TM *>(smem + L::oVt);  // [BV][LCM]
    TM *Qt = reinterpret_cast<TM *>(smem + L::oQt);
    TM *Bw = reinterpret_cast<TM *>(smem + L::oBw);  // [K][LCM]
    TM *Kt = reinterpret_cast<TM *>(smem + L::oKt);  // [K][LCM]
    TM *bV = reinterpret_cast<TM *>(smem + L::obV);  // [BV][LCM]
    float *Akk = reinterpret_cast<float *>(smem + L::oAkk);
    float *Tf = reinterpret_cast<float *>(smem + L::oTf);
    TM *Aqk = reinterpret_cast<TM *>(smem + L::oAqk);
    float *Msc = reinterpret_cast<float *>(smem + L::oM);
    TM *St = reinterpret_cast<TM *>(smem + L::oSt);  // [BV][LKM]
    float *Rv = reinterpret_cast<float *>(smem + L::oR);
    float *Ev = reinterpret_cast<float *>(smem + L::oE);
    float *GCv = reinterpret_cast<float *>(smem + L::oGC);
    float *eGC = reinterpret_cast<float *>(smem + L::oEGC);
    float *Seg = reinterpret_cast<float *>(smem + L::oSeg);
    float *Bt = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- which (sequence, head, value block) this workgroup owns -------------------
    constexpr int NVB = V / BV;
    const int G = gridDim.x;
    int lin = blockIdx.x;
    if ((G & 7) == 0) lin = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);  // keep a head's value
    const int vb = lin % NVB;                                                   // blocks on one XCD
    const int pair = lin / NVB;
    const int h = pair % a.H;
    const int s = pair / a.H;
    int64_t bos, eos;
    if (a.cu_seqlens) {
        bos = a.cu_seqlens[s];
        eos = a.cu_seqlens[s + 1];
    } else {
        bos = (int64_t)s * a.T;
        eos = bos + a.T;
    }
    const int H = a.H;
    const TIn *q = static_cast<const TIn *>(a.q);
    const TIn *k = static_cast<const TIn *>(a.k);
    const TIn *v = static_cast<const TIn *>(a.v);

    // ---- master state in registers (wave-owned [16 x 16] tiles of S[K x BV]) -------
    f4 accS[L::MS];
    const float *s0 = a.initial_state ? a.initial_state + ((int64_t)s * H + h) * K * V : nullptr;
#pragma unroll
    for (int m = 0; m < L::MS; ++m) {
        const int ts = wave + NW * m;
        f4 x = {0.f, 0.f, 0.f, 0.f};
        if (ts < L::NTS && s0) {
            const int kr = (ts / (BV / 16)) * 16 + 4 * (lane >> 4);
            const int vc = vb * BV + (ts % (BV / 16)) * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = s0[(int64_t)(kr + e) * V + vc];
        }
        accS[m] = x;
    }
    auto write_state_copy = [&]() {
#pragma unroll
        for (int m = 0; m < L::MS; ++m) {
            const int ts = wave + NW * m;
            if (ts < L::NTS) {
                const int kr = (ts / (BV / 16)) * 16 + 4 * (lane >> 4);
                const int vc = (ts % (BV / 16)) * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) St[vc * L::LKM + kr + e] = from_f32<TM>(accS[m][e]);
            }
        }
    };
    write_state_copy();

    // prep mapping: thread -> (key channel c, segment of RPS consecutive rows)
    const int pc = tid % K;
    const int pseg = tid / K;

    for (int64_t t0 = bos; t0 < eos; t0 += C) {
        const int n = (int)((eos - t0) < C ? (eos - t0) : C);

        // ---- 1. cumulative log2-decay Gamma of the chunk ----------------------------
        if (tid < C) Bt[tid] = tid < n ? a.beta[(t0 + tid) * H + h] : 0.f;
        float G2[L::RPS];
        {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < L::RPS; ++i) {
                const int r = pseg * L::RPS + i;
                float g = 0.f;
                if (r < n) {
                    const float x = a.gate[((t0 + r) * H + h) * K + pc];
                    g = a.gate_is_log ? x * LOG2E : __log2f(x);
                }
                run += g;
                G2[i] = run;
            }
            Seg[pseg * K + pc] = run;
        }
        __syncthreads();
        {
            float off = 0.f;
            for (int sg = 0; sg < pseg; ++sg) off += Seg[sg * K + pc];
#pragma unroll
            for (int i = 0; i < L::RPS; ++i) {
                G2[i] += off;
                const int r = pseg * L::RPS + i;
                if ((r & 15) == 15) {
                    Ev[(r >> 4) * K + pc] = G2[i];
                    if ((r >> 4) + 1 < NP) Rv[((r >> 4) + 1) * K + pc] = G2[i];
                }
                if (r == C - 1) {
                    GCv[pc] = G2[i];
                    eGC[pc] = exp2f(G2[i]);
                }
            }
            if (pseg == 0) Rv[pc] = 0.f;
        }
        __syncthreads();

        // ---- 2. rescaled operands ----------------------------------------------------
        {
            const float gC = GCv[pc];
#pragma unroll
            for (int i = 0; i < L::RPS; ++i) {
                const int r = pseg * L::RPS + i;
                const int p = r >> 4;
                const float Rp = Rv[p * K + pc];
                const float Ep = Ev[p * K + pc];
                float qv = 0.f, kv = 0.f;
                if (r < n) {
                    qv = ld_f32(q, ((t0 + r) * H + h) * K + pc);
                    kv = ld_f32(k, ((t0 + r) * H + h) * K + pc);
                }
                const float be = Bt[r];
                const float ea = exp2f(G2[i] - Rp);  // <= 1
                const float eb = exp2f(Rp - G2[i]);  // in [1, e^80]
                const float lq = qv * ea;
                const float lk = be * kv * ea;
                const float rd = kv * eb;
                const float ro = rd * exp2f(Ep - Rp);  // k e^{E_p - Gamma} <= 1
                const float eR = exp2f(Rp);
                Lk[r * L::LKA + pc] = from_f32<TA>(lk);
                {
                    const TA hq = from_f32<TA>(lq), hr = from_f32<TA>(rd);
                    Lq[r * L::LKA + pc] = hq;
                    Rd[r * L::LKA + pc] = hr;
                    if constexpr (P::kSplit) {
                        Lq[C * L::LKA + r * L::LKA + pc] = from_f32<TA>(lq - to_f32(hq));
                        Rd[C * L::LKA + r * L::LKA + pc] = from_f32<TA>(rd - to_f32(hr));
                    }
                }
                if (p < NP - 1) {
                    const TA ho = from_f32<TA>(ro);
                    Ro[r * L::LKA + pc] = ho;
                    if constexpr (P::kSplit)
                        Ro[(C - 16) * L::LKA + r * L::LKA + pc] = from_f32<TA>(ro - to_f32(ho));
                }
                if constexpr (L::NX > 0) {
                    // versions of tile q = p for row tiles pp >= p + 2
                    int xi = 0;
                    for (int pp = 2; pp < NP; ++pp)
                        for (int qq = 0; qq + 2 <= pp; ++qq, ++xi) {
                            if (qq != p) continue;
                            const float xv = ro * exp2f(Rv[pp * K + pc] - Ep);
                            const TA hx = from_f32<TA>(xv);
                            const int row = r - 16 * p;
                            Xv[(size_t)xi * 16 * L::LKA + row * L::LKA + pc] = hx;
                            if constexpr (P::kSplit)
                                Xv[(size_t)(L::NX + xi) * 16 * L::LKA + row * L::LKA + pc] =
                                    from_f32<TA>(xv - to_f32(hx));
                        }
                }
                Qt[r * L::LKM + pc] = from_f32<TM>(lq * eR);
                Bw[pc * L::LCM + r] = from_f32<TM>(lk * eR);
                Kt[pc * L::LCM + r] = from_f32<TM>(ro * exp2f(gC - Ep));
            }
            // beta * V for this value block, transposed (token contiguous)
            for (int e = tid; e < BV * C; e += NT) {
                const int j = e % BV, r = e / BV;
                float x = 0.f;
                if (r < n) x = Bt[r] * ld_f32(v, ((t0 + r) * H + h) * V + vb * BV + j);
                bV[j * L::LCM + r] = from_f32<TM>(x);
            }
        }
        __syncthreads();

        // ---- 3. A_kk (strictly lower, fp32), A_qk (lower incl. diagonal), O = Qt S ----
        {
            constexpr int NTA = NP * NP;  // all tiles; the upper ones are zero
            for (int task = wave; task < 2 * NTA; task += NW) {
                const bool isq = task >= NTA;
                const int tt = isq ? task - NTA : task;
                const int p = tt / NP, qt = tt % NP;
                f4 acc = {0.f, 0.f, 0.f, 0.f};
                if (qt <= p) {
                    const TA *right;
                    int rstride_lo;  // offset of the lo copy of `right`
                    if (qt == p) {
                        right = Rd + qt * 16 * L::LKA;
                        rstride_lo = C * L::LKA;
                    } else if (qt == p - 1) {
                        right = Ro + qt * 16 * L::LKA;
                        rstride_lo = (C - 16) * L::LKA;
                    } else {
                        int xi = 0;
                        for (int pp = 2; pp < p; ++pp) xi += pp - 1;
                        xi += qt;
                        right = Xv + (size_t)xi * 16 * L::LKA;
                        rstride_lo = L::NX * 16 * L::LKA;
                    }
                    if (!isq) {
                        mma_tile<TA>(acc, Lk + p * 16 * L::LKA, L::LKA, right, L::LKA, K, lane);
                    } else {
                        const TA *left = Lq + p * 16 * L::LKA;
                        mma_tile<TA>(acc, left, L::LKA, right, L::LKA, K, lane);
                        if constexpr (P::kSplit) {
                            mma_tile<TA>(acc, left, L::LKA, right + rstride_lo, L::LKA, K, lane);
                            mma_tile<TA>(acc, left + C * L::LKA, L::LKA, right, L::LKA, K, lane);
                        }
                    }
                }
                const int i0 = p * 16 + 4 * (lane >> 4), j = qt * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = i0 + e;
                    if (!isq)
                        Akk[i * L::LCF + j] = (j < i) ? acc[e] : 0.f;
                    else
                        Aqk[i * L::LCM + j] = from_f32<TM>((j <= i) ? acc[e] : 0.f);
                }
            }
        }
        f4 accO[L::MO];
#pragma unroll
        for (int m = 0; m < L::MO; ++m) {
            accO[m] = f4{0.f, 0.f, 0.f, 0.f};
            const int to = wave + NW * m;
            if (to < L::NTO) {
                const int p = to / (BV / 16), jt = to % (BV / 16);
                mma_tile<TM>(accO[m], Qt + p * 16 * L::LKM, L::LKM, St + jt * 16 * L::LKM, L::LKM, K,
                             lane);
            }
        }
        __syncthreads();

        // ---- 4. T = (I + A_kk)^-1 -------------------------------------------------------
        if (tid < 16 * NP) {
            // diagonal 16x16 blocks by forward substitution, one column per thread
            const int p = tid >> 4, c = tid & 15;
            const float *A = Akk + (p * 16) * L::LCF + p * 16;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
                for (int jj = 0; jj < i; ++jj) acc -= A[i * L::LCF + jj] * x[jj];
                x[i] = (i < c) ? 0.f : acc;
            }
            float *Td = Tf + (p * 16) * L::LCF + p * 16;
#pragma unroll
            for (int i = 0; i < 16; ++i) Td[i * L::LCF + c] = x[i];
        }
        __syncthreads();
        for (int d = 1; d < NP; ++d) {
            // blocks (p, p-d): M = sum_{r=q}^{p-1} A_pr T_rq ; T_pq = -T_pp M
            for (int e = tid; e < (NP - d) * 256; e += NT) {
                const int b = e >> 8, i = (e >> 4) & 15, jj = e & 15;
                const int p = d + b, qb = b;
                float acc = 0.f;
                for (int r = qb; r < p; ++r)
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        acc += Akk[(p * 16 + i) * L::LCF + r * 16 + m] * Tf[(r * 16 + m) * L::LCF + qb * 16 + jj];
                Msc[b * 256 + i * 16 + jj] = acc;
            }
            __syncthreads();
            for (int e = tid; e < (NP - d) * 256; e += NT) {
                const int b = e >> 8, i = (e >> 4) & 15, jj = e & 15;
                const int p = d + b, qb = b;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += Tf[(p * 16 + i) * L::LCF + p * 16 + m] * Msc[b * 256 + m * 16 + jj];
                Tf[(p * 16 + i) * L::LCF + qb * 16 + jj] = -acc;
            }
            __syncthreads();
        }
        // operand copy of T with an explicit zero upper triangle (region 1 is free now)
        for (int e = tid; e < C * C; e += NT) {
            const int i = e / C, jj = e % C;
            Tm[i * L::LCM + jj] = from_f32<TM>(jj <= i ? Tf[i * L::LCF + jj] : 0.f);
        }
        __syncthreads();

        // ---- 5. -W = -T (beta e^Gamma K) into LDS, U = T (beta V) into registers -------
        for (int task = wave; task < NP * (K / 16); task += NW) {
            const int p = task / (K / 16), ct = task % (K / 16);
            f4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_tile<TM>(acc, Tm + p * 16 * L::LCM, L::LCM, Bw + ct * 16 * L::LCM, L::LCM, 16 * (p + 1),
                         lane);
            const int i0 = p * 16 + 4 * (lane >> 4), c = ct * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) Wn[(i0 + e) * L::LKM + c] = from_f32<TM>(-acc[e]);
        }
        f4 accU[L::MO];
#pragma unroll
        for (int m = 0; m < L::MO; ++m) {
            accU[m] = f4{0.f, 0.f, 0.f, 0.f};
            const int to = wave + NW * m;
            if (to < L::NTO) {
                const int p = to / (BV / 16), jt = to % (BV / 16);
                mma_tile<TM>(accU[m], Tm + p * 16 * L::LCM, L::LCM, bV + jt * 16 * L::LCM, L::LCM,
                             16 * (p + 1), lane);
            }
        }
        __syncthreads();

        // ---- 6. Vt = U - W S  (stored transposed: value rows, token contiguous) ----------
#pragma unroll
        for (int m = 0; m < L::MO; ++m) {
            const int to = wave + NW * m;
            if (to < L::NTO) {
                const int p = to / (BV / 16), jt = to % (BV / 16);
                mma_tile<TM>(accU[m], Wn + p * 16 * L::LKM, L::LKM, St + jt * 16 * L::LKM, L::LKM, K, lane);
                const int i0 = p * 16 + 4 * (lane >> 4), j = jt * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) Vt[j * L::LCM + i0 + e] = from_f32<TM>(accU[m][e]);
            }
        }
        __syncthreads();

        // ---- 7. O += A_qk Vt -> out ;  S = e^{Gamma_C} S + K~^T Vt ----------------------
#pragma unroll
        for (int m = 0; m < L::MO; ++m) {
            const int to = wave + NW * m;
            if (to < L::NTO) {
                const int p = to / (BV / 16), jt = to % (BV / 16);
                mma_tile<TM>(accO[m], Aqk + p * 16 * L::LCM, L::LCM, Vt + jt * 16 * L::LCM, L::LCM,
                             16 * (p + 1), lane);
                const int i0 = p * 16 + 4 * (lane >> 4);
                const int j = vb * BV + jt * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (i0 + e < n) st_out(a.out, a.out_bf16, ((t0 + i0 + e) * H + h) * V + j, a.scale * accO[m][e]);
            }
        }
#pragma unroll
        for (int m = 0; m < L::MS; ++m) {
            const int ts = wave + NW * m;
            if (ts < L::NTS) {
                const int kt = ts / (BV / 16), jt = ts % (BV / 16);
                const int kr = kt * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[m][e] *= eGC[kr + e];
                mma_tile<TM>(accS[m], Kt + kt * 16 * L::LCM, L::LCM, Vt + jt * 16 * L::LCM, L::LCM, C, lane);
            }
        }
        write_state_copy();
        __syncthreads();
    }

    // ---- final state ------------------------------------------------------------------
    if (a.final_state) {
        float *sf = a.final_state + ((int64_t)s * H + h) * K * V;
#pragma unroll
        for (int m = 0; m < L::MS; ++m) {
            const int ts = wave + NW * m;
            if (ts < L::NTS) {
                const int kr = (ts / (BV / 16)) * 16 + 4 * (lane >> 4);
                const int vc = vb * BV + (ts % (BV / 16)) * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) sf[(int64_t)(kr + e) * V + vc] = accS[m][e];
            }
        }
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

template <class P, int K, int V, int C>
hipError_t launch_kvc(const ChunkArgs &a, int num_pairs, hipStream_t stream, int *bv_out) {
    constexpr int BV = pick_bv<P, K, V, C>();
    if constexpr (BV == 0) {
        return hipErrorNotSupported;
    } else {
        using L = Layout<P, K, V, C, BV>;
        auto kern = chunk_fwd_kernel<P, K, V, C, BV>;
        static bool attr_set = false;  // per-instantiation, set once per process
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

template <class P, int K, int V>
hipError_t launch_kv(const ChunkArgs &a, int C, int num_pairs, hipStream_t stream, int *bv) {
    switch (C) {
        case 16: return launch_kvc<P, K, V, 16>(a, num_pairs, stream, bv);
        case 32: return launch_kvc<P, K, V, 32>(a, num_pairs, stream, bv);
        case 64: return launch_kvc<P, K, V, 64>(a, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

template <class P, int K>
hipError_t launch_k(const ChunkArgs &a, int V, int C, int num_pairs, hipStream_t stream, int *bv) {
    switch (V) {
        case 16: return launch_kv<P, K, 16>(a, C, num_pairs, stream, bv);
        case 32: return launch_kv<P, K, 32>(a, C, num_pairs, stream, bv);
        case 64: return launch_kv<P, K, 64>(a, C, num_pairs, stream, bv);
        case 128: return launch_kv<P, K, 128>(a, C, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

template <class P>
hipError_t launch_p(const ChunkArgs &a, int K, int V, int C, int num_pairs, hipStream_t stream, int *bv) {
    switch (K) {
        case 16: return launch_k<P, 16>(a, V, C, num_pairs, stream, bv);
        case 32: return launch_k<P, 32>(a, V, C, num_pairs, stream, bv);
        case 64: return launch_k<P, 64>(a, V, C, num_pairs, stream, bv);
        case 128: return launch_k<P, 128>(a, V, C, num_pairs, stream, bv);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_chunk_fwd(const ChunkArgs &a, bool fp32_inputs, int K, int V, int C, int num_pairs,
                            hipStream_t stream, int *bv) {
    return fp32_inputs ? launch_p<PrecF32>(a, K, V, C, num_pairs, stream, bv)
                       : launch_p<PrecMixed>(a, K, V, C, num_pairs, stream, bv);
}

}  // namespace kda
