// kda_prefill_impl.h -- chunkwise-parallel KDA prefill kernel (gfx950).
//
// What is computed: the token recurrence S_t = (I - b_t k_t k_t^T)
// Diag(exp g_t) S_{t-1} + b_t k_t v_t^T, o_t = scale S_t^T q_t ("Understanding
// Kimi K3's attention", state-update and readout equations), evaluated a chunk
// of C = 16 * NS tokens at a time with the state passed from chunk to chunk
// ("Inside Kimi K3", section "Sequence mixing"; "Hybrid Attention", section
// "But isn't a recurrent update sequential?").
//
// Chunk algebra (S0 = state entering the chunk, rows r, s = tokens of the
// chunk, G_r = inclusive per-channel cumulative log-decay from the chunk start):
//   u_r = b_r (v_r - (D_r S_{r-1})^T k_r) makes every step S_r = D_r S_{r-1} + k_r u_r^T.
//   Unrolled over the chunk this gives
//     (I + A) U = diag(b) (V - Kt S0),   A_rs = b_r sum_c k_rc k_sc e^{G_rc - G_sc}, s < r
//     O = Qt S0 + P U,                   P_rs = sum_c q_rc k_sc e^{G_rc - G_sc},    s <= r
//     S_C = Diag(e^{G_C}) S0 + Kbar^T U
//   with Kt = k * e^{G_r}, Qt = q * e^{G_r}, Kbar = k * e^{G_C - G_s}.  P keeps
//   its diagonal because each token reads the state after its own write
//   ("Inside Kimi K3", section "Sequence mixing"); the solve of I + A is the
//   triangular solve of "Hybrid Attention".
//
// Numerics of e^{G_r - G_s} as a matrix product.  The chunk is split into
// 16-token sub-tiles; the log-decay is at least -5 per token ("Understanding
// Kimi K3's attention", g_min equation), so one sub-tile decays by at least
// -80 ("Inside Kimi K3": 16-token tiles stay above -80; "Kimi K3.1 and the
// Road ...", section 5: the chunked form divides by the cumulative decay).
// For a pair of sub-tiles (i >= j) the factor is split at the END of sub-tile
// j:  e^{G_r - G_s} = [e^{L_r} e^{b_i - b_{j+1}}] * [e^{tot_j - L_s}]
// (L = cumulative decay inside the own sub-tile, b_i = decay before sub-tile i,
// tot_j = decay over sub-tile j).  The right factor lies in [e^-80, 1].  The
// left factor is <= 1 for i > j and lies in [1, e^80] for i == j, so neither
// overflows fp32/bf16 (8-bit exponent, max ~3.4e38 > 128 * e^80) and an
// underflow only drops terms far below every tolerance.
//
// Work split (one workgroup per (sequence, head, d_v slab)):
//   - each of the NWC waves owns 16 value columns.  Its fp32 state slice
//     S[:, cols], the intermediates X = Kt S0, Qt S0, Y, U and O stay in its
//     registers for the whole chunk: the MFMA accumulator layout doubles as
//     the next product's B operand (see kda_device.h), so the S-dependent
//     chain needs no LDS round trip and no barrier.
//   - all waves share the S-independent, d_k-side work through LDS: the
//     cumulative decay, the scaled operand tiles, the Gram tiles A and P
//     (bf16 MFMA), and the 16x16 diagonal blocks T_ii = (I + A_ii)^{-1}
//     (fp32 forward substitution).  Off-diagonal blocks of (I + A)^{-1} are
//     never formed: U is found by block forward substitution,
//     U_i = T_ii (Y_i - sum_{j<i} A_ij U_j), in registers.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename TIn, int D, int NS, int NWC>
struct PrefillCfg {
    static constexpr int C = 16 * NS;        // chunk tokens
    static constexpr int NT = 64 * NWC;      // threads
    static constexpr int DVW = 16 * NWC;     // value columns per workgroup
    static constexpr int PAD = Elem<TIn>::pad;
    static constexpr int PD = D + PAD;       // pitch of [C][D] tiles
    static constexpr int PC = C + PAD;       // pitch of [*][C] tiles
    static constexpr int PV = DVW;           // pitch of the V tile
    static constexpr int PT = 16 + PAD;      // pitch of a T_ii block
    static constexpr int PA = 20;            // pitch (floats) of an fp32 A_ii block
    static constexpr int NP = NS * (NS + 1) / 2;  // sub-tile pairs i >= j
    static constexpr int KSTEP = sizeof(TIn) == 2 ? 2 : 1;  // K blocks per product step

    static constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_TILE = al16(sizeof(TIn) * C * PD);
    static constexpr size_t OFF_V = 0;                       // [C][DVW], unpadded
    static constexpr size_t OFF_QB = OFF_V + al16(sizeof(TIn) * C * DVW);
    static constexpr size_t OFF_KB = OFF_QB + SZ_TILE;
    static constexpr size_t OFF_KR = OFF_KB + SZ_TILE;
    static constexpr size_t OFF_QT = OFF_KR + SZ_TILE;
    static constexpr size_t OFF_KT = OFF_QT + SZ_TILE;
    static constexpr size_t OFF_KBT = OFF_KT + SZ_TILE;
    static constexpr size_t OFF_P = OFF_KBT + al16(sizeof(TIn) * D * PC);
    static constexpr size_t OFF_AO = OFF_P + al16(sizeof(TIn) * C * PC);
    static constexpr size_t OFF_T = OFF_AO + al16(sizeof(TIn) * C * PC);
    static constexpr size_t OFF_AD = OFF_T + al16(sizeof(TIn) * NS * 16 * PT);
    static constexpr size_t OFF_F = OFF_AD + al16(sizeof(float) * NS * 16 * PA);
    static constexpr size_t OFF_GAM = OFF_F + al16(sizeof(float) * NP * D);
    static constexpr size_t OFF_TOT = OFF_GAM + al16(sizeof(float) * D);
    static constexpr size_t OFF_BETA = OFF_TOT + al16(sizeof(float) * NS * D);
    static constexpr size_t LDS = OFF_BETA + al16(sizeof(float) * C);

    static_assert(D % 16 == 0 && D >= 16, "head dim");
    static_assert(DVW <= D && D % DVW == 0, "value slab");
    static_assert(D % (16 * KSTEP) == 0, "K steps");
    static_assert(LDS <= 160 * 1024, "LDS budget (160 KiB per CU on gfx950)");
};

// acc += A(16 x 16*nb) * B(16*nb x 16), A rows read from LDS at a[kb*16]
// (row pitch handled by the caller), B fragments from registers, pairing K
// blocks into 32-deep products where the element type allows it.
template <typename TIn, int NB>
__device__ __forceinline__ void mma_rowblocks(f32x4& acc, const TIn* a_row, const typename Elem<TIn>::frag* b) {
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int j = 0; j + 1 < NB; j += 2)
            mma32(acc, ld_frag(a_row + 16 * j), ld_frag(a_row + 16 * (j + 1)), b[j], b[j + 1]);
        if constexpr (NB & 1) mma16(acc, ld_frag(a_row + 16 * (NB - 1)), b[NB - 1]);
    } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) mma16(acc, ld_frag(a_row + 16 * j), b[j]);
    }
}

// Same with a runtime block count (nb <= NBMAX).
template <typename TIn, int NBMAX>
__device__ __forceinline__ void mma_rowblocks_n(f32x4& acc, const TIn* a_row, const typename Elem<TIn>::frag* b,
                                                int nb) {
#pragma unroll
    for (int j = 0; j < NBMAX; ++j)
        if (j < nb) mma16(acc, ld_frag(a_row + 16 * j), b[j]);
}

template <typename TIn, int D, int NS, int NWC>
__global__ __launch_bounds__(64 * NWC) void kda_prefill_kernel(PrefillParams p) {
    typedef PrefillCfg<TIn, D, NS, NWC> Cfg;
    typedef Elem<TIn> E;
    typedef typename E::frag Frag;
    constexpr int C = Cfg::C, NT = Cfg::NT, DVW = Cfg::DVW;
    constexpr int PD = Cfg::PD, PC = Cfg::PC, PV = Cfg::PV, PT = Cfg::PT, PA = Cfg::PA;
    constexpr int NP = Cfg::NP, KSTEP = Cfg::KSTEP;
    constexpr int NKB = D / 16;  // K blocks over d_k

    __shared__ __align__(16) char smem[Cfg::LDS];
    TIn* sV = reinterpret_cast<TIn*>(smem + Cfg::OFF_V);
    TIn* sQB = reinterpret_cast<TIn*>(smem + Cfg::OFF_QB);
    TIn* sKB = reinterpret_cast<TIn*>(smem + Cfg::OFF_KB);
    TIn* sKR = reinterpret_cast<TIn*>(smem + Cfg::OFF_KR);
    TIn* sQT = reinterpret_cast<TIn*>(smem + Cfg::OFF_QT);
    TIn* sKT = reinterpret_cast<TIn*>(smem + Cfg::OFF_KT);
    TIn* sKbT = reinterpret_cast<TIn*>(smem + Cfg::OFF_KBT);
    TIn* sP = reinterpret_cast<TIn*>(smem + Cfg::OFF_P);
    TIn* sAo = reinterpret_cast<TIn*>(smem + Cfg::OFF_AO);
    TIn* sT = reinterpret_cast<TIn*>(smem + Cfg::OFF_T);
    float* sAd = reinterpret_cast<float*>(smem + Cfg::OFF_AD);
    float* sF = reinterpret_cast<float*>(smem + Cfg::OFF_F);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::OFF_GAM);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::OFF_TOT);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int g4 = lane >> 4;
    const int l16 = lane & 15;

    // ---- which (sequence, head, slab) this workgroup owns ----
    const int bid = blockIdx.x;
    const int z = bid % p.nslab;
    const int uh = bid / p.nslab;
    const int h = uh % p.H;
    const int n = uh / p.H;
    const int H = p.H;
    int64_t t_begin, t_end;
    seq_bounds(p, n, &t_begin, &t_end);
    const int col0 = z * DVW + w * 16;  // first value column of this wave
    const int64_t sbase = ((int64_t)n * H + h) * D * D;

    const TIn* gq = static_cast<const TIn*>(p.q);
    const TIn* gk = static_cast<const TIn*>(p.k);
    const TIn* gv = static_cast<const TIn*>(p.v);
    TIn* go = static_cast<TIn*>(p.o);

    // ---- fp32 master state slice: Sm[ct][pp] = S[16ct + 4g4 + pp][col0 + l16] ----
    // Buffer accesses: one per-lane offset, rows as wave-uniform offsets;
    // without an initial state the range is empty and the loads read 0.
    const uint32_t s_voff = (uint32_t)(4 * g4 * D + col0 + l16) * 4u;
    f32x4 Sm[NKB];
    {
        const auto rs = p.S0 ? buffer_rsrc(p.S0 + sbase, D * D * 4) : buffer_rsrc(p.g, 0);
#pragma unroll
        for (int ct = 0; ct < NKB; ++ct) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
                Sm[ct][pp] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rs, s_voff, (16 * ct + pp) * D * 4, 0));
        }
    }

    // Prologue items: wave-item wi = (sub-tile i, 16-channel block cb); lane
    // (g4, l16) holds token 16 i + l16 and channels 16 cb + 4 g4 .. + 3 -- the
    // MFMA operand layout -- so the 16 tokens of a sub-tile sit in one 16-lane
    // DPP row and the per-channel cumulative decay is a row prefix scan.
    constexpr int NCB = D / 16;
    constexpr int NWI = NS * NCB;
    constexpr int IPT = (NWI + NWC - 1) / NWC;     // wave-items per wave
    constexpr int VE = 16 / sizeof(TIn);           // V elements per 16-byte load
    constexpr int VCPR = DVW / VE;                 // 16-byte chunks per V row
    constexpr int VPT = (C * VCPR + NT - 1) / NT;  // V chunks per thread

    // Next-chunk inputs, loaded while the current chunk computes.
    float4 pg[IPT];
    Frag pq[IPT], pk[IPT];
    uint4 pv[VPT];
    float pb = 0.f;
    auto prefetch = [&](int64_t tn, int nvn) {
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int wi = w + NWC * it;
            const int i = wi / NCB, cb = wi % NCB;
            const int row = 16 * i + l16;
            pg[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            pq[it] = E::zero();
            pk[it] = E::zero();
            if (wi < NWI && row < nvn) {
                const int64_t off = ((tn + row) * H + h) * D + 16 * cb + 4 * g4;
                pg[it] = *reinterpret_cast<const float4*>(p.g + off);
                pq[it] = ld_frag(gq + off);
                pk[it] = ld_frag(gk + off);
            }
        }
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int idx = tid + it * NT;
            const int row = idx / VCPR, ch = idx % VCPR;
            pv[it] = make_uint4(0u, 0u, 0u, 0u);
            if (idx < C * VCPR && row < nvn)
                pv[it] = *reinterpret_cast<const uint4*>(gv + ((tn + row) * H + h) * D + z * DVW + ch * VE);
        }
        pb = 0.f;
        if (tid < C && tid < nvn) pb = p.beta[(tn + tid) * H + h];
    };
    if (t_begin < t_end) prefetch(t_begin, (t_end - t_begin) < C ? (int)(t_end - t_begin) : C);

    const int ck0 = p.ckpt ? __builtin_amdgcn_readfirstlane((int)ckpt_first_slot(p, n, lane)) : 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += C) {
        const int nv = (t_end - t0) < C ? (int)(t_end - t0) : C;

        // ================= stage 1: decay, scaled operand tiles =================
        // 1a: inclusive cumulative log-decay inside each 16-token sub-tile.
        float4 cum[IPT];
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int wi = w + NWC * it;
            float x[4] = {pg[it].x, pg[it].y, pg[it].z, pg[it].w};
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) x[ch] = row_inclusive_sum16(x[ch]);
            cum[it] = make_float4(x[0], x[1], x[2], x[3]);
            if (wi < NWI && l16 == 15) {
                const int i = wi / NCB, cb = wi % NCB;
                *reinterpret_cast<float4*>(sTot + i * D + 16 * cb + 4 * g4) = cum[it];
            }
        }
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int idx = tid + it * NT;
            const int row = idx / VCPR, ch = idx % VCPR;
            if (idx < C * VCPR) *reinterpret_cast<uint4*>(sV + row * PV + ch * VE) = pv[it];
        }
        if (tid < C) sBeta[tid] = pb;
        __syncthreads();

        // 1b: scaled tiles from the registers, pair factors, chunk decay.
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int wi = w + NWC * it;
            if (wi < NWI) {
                const int i = wi / NCB, cb = wi % NCB;
                const int c0 = 16 * cb + 4 * g4;
                const int row = 16 * i + l16;
                float L[4] = {cum[it].x, cum[it].y, cum[it].z, cum[it].w};
                float qv[4], kv[4], qb[4], kb[4], kr[4], qt[4], kt[4], kbar[4];
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    qv[ch] = E::get(pq[it], ch);
                    kv[ch] = E::get(pk[it], ch);
                    float b_i = 0.f, b_all = 0.f, tot_i = 0.f;
#pragma unroll
                    for (int ii = 0; ii < NS; ++ii) {
                        const float t = sTot[ii * D + c0 + ch];
                        if (ii < i) b_i += t;
                        if (ii == i) tot_i = t;
                        b_all += t;
                    }
                    const float e1 = __expf(L[ch]);          // e^{L_r}, in [e^-80, 1]
                    const float e2 = __expf(tot_i - L[ch]);  // e^{tot_i - L_r}, in [e^-80, 1]
                    qb[ch] = qv[ch] * e1;
                    kb[ch] = kv[ch] * e1;
                    kr[ch] = kv[ch] * e2;
                    const float e_bi = __expf(b_i);            // chunk start -> sub-tile start
                    const float e_kbar = __expf(b_all - b_i - tot_i);  // sub-tile end -> chunk end
                    qt[ch] = qb[ch] * e_bi;
                    kt[ch] = kb[ch] * e_bi;
                    kbar[ch] = kr[ch] * e_kbar;
                    if (l16 == 0) {
                        // Gram scale factors of pairs (i, j <= i), applied to the left operand.
                        float b_j1 = 0.f;  // decay before sub-tile j + 1
#pragma unroll
                        for (int j = 0; j < NS; ++j) {
                            if (j <= i) {
                                b_j1 += sTot[j * D + c0 + ch];
                                sF[(i * (i + 1) / 2 + j) * D + c0 + ch] = (j == i) ? __expf(-tot_i) : __expf(b_i - b_j1);
                            }
                        }
                        if (i == NS - 1) sGam[c0 + ch] = __expf(b_all);
                    }
                }
                st_frag(sQB + row * PD + c0, E::make(qb[0], qb[1], qb[2], qb[3]));
                st_frag(sKB + row * PD + c0, E::make(kb[0], kb[1], kb[2], kb[3]));
                st_frag(sKR + row * PD + c0, E::make(kr[0], kr[1], kr[2], kr[3]));
                st_frag(sQT + row * PD + c0, E::make(qt[0], qt[1], qt[2], qt[3]));
                st_frag(sKT + row * PD + c0, E::make(kt[0], kt[1], kt[2], kt[3]));
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) sKbT[(c0 + ch) * PC + row] = E::from_f32(kbar[ch]);
            }
        }
        // The registers are free again: start loading the next chunk.
        if (t0 + C < t_end) prefetch(t0 + C, (t_end - t0 - C) < C ? (int)(t_end - t0 - C) : C);
        __syncthreads();

        // ================= stage 2: Gram tiles A and P (MFMA) =================
        for (int tile = w; tile < 2 * NP; tile += NWC) {
            const int which = tile & 1;  // 0: A (keys), 1: P (queries)
            int pp = tile >> 1, i = 0;
            while (pp > i) { pp -= i + 1; ++i; }
            const int j = pp;
            const TIn* xrow = (which ? sQB : sKB) + (16 * i + l16) * PD + 4 * g4;
            const TIn* krow = sKR + (16 * j + l16) * PD + 4 * g4;
            const float* frow = sF + (i * (i + 1) / 2 + j) * D + 4 * g4;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; kb += KSTEP) {
                Frag bx[KSTEP], ak[KSTEP];
#pragma unroll
                for (int u = 0; u < KSTEP; ++u) {
                    const Frag x = ld_frag(xrow + 16 * (kb + u));
                    const float4 f = *reinterpret_cast<const float4*>(frow + 16 * (kb + u));
                    bx[u] = E::make(E::get(x, 0) * f.x, E::get(x, 1) * f.y, E::get(x, 2) * f.z, E::get(x, 3) * f.w);
                    ak[u] = ld_frag(krow + 16 * (kb + u));
                }
                if constexpr (KSTEP == 2) mma32(acc, ak[0], ak[1], bx[0], bx[1]);
                else mma16(acc, ak[0], bx[0]);
            }
            // acc[pp] = M[r = l16][s = 4 g4 + pp] for rows r of sub-tile i, columns s of sub-tile j.
            const int r = l16;
            if (which) {
                f32x4 v4;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) v4[q4] = (i == j && 4 * g4 + q4 > r) ? 0.f : acc[q4];
                st_frag(sP + (16 * i + r) * PC + 16 * j + 4 * g4, E::make(v4));
            } else {
                const float br = sBeta[16 * i + r];
                if (i == j) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int s = 4 * g4 + q4;
                        sAd[(16 * i + r) * PA + s] = s < r ? br * acc[q4] : 0.f;
                    }
                } else {
                    st_frag(sAo + (16 * i + r) * PC + 16 * j + 4 * g4,
                            E::make(-br * acc[0], -br * acc[1], -br * acc[2], -br * acc[3]));
                }
            }
        }
        __syncthreads();

        // ================= stage 3: V tile, T_ii solve, X = Kt S0, Qt S0 =================
        if (w == 0 && lane < 16 * NS) {
            // T_ii = (I + A_ii)^{-1} by forward substitution, one column per lane.
            const int i = lane >> 4, col = l16;
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == col) ? 1.f : 0.f;
                const float* arow = sAd + (16 * i + r) * PA;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= arow[s] * tc[s];
                tc[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * i + r) * PT + col] = E::from_f32(tc[r]);
        }
        Frag Sop[NKB];
#pragma unroll
        for (int ct = 0; ct < NKB; ++ct) Sop[ct] = E::make(Sm[ct]);
        f32x4 X[NS], QS[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            X[i] = zero4();
            QS[i] = zero4();
            mma_rowblocks<TIn, NKB>(X[i], sKT + (16 * i + l16) * PD + 4 * g4, Sop);
            mma_rowblocks<TIn, NKB>(QS[i], sQT + (16 * i + l16) * PD + 4 * g4, Sop);
        }
        __syncthreads();

        // ================= stage 4: U, O and the state pass (per wave) =================
        Frag Uf[NS];
        const int cl = w * 16 + l16;  // column inside the slab's V tile
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            f32x4 Z;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int row = 16 * i + 4 * g4 + q4;
                Z[q4] = sBeta[row] * (E::to_f32(sV[row * PV + cl]) - X[i][q4]);
            }
            // Z -= sum_{j<i} A_ij U_j   (sAo holds -A)
            mma_rowblocks_n<TIn, NS>(Z, sAo + (16 * i + l16) * PC + 4 * g4, Uf, i);
            f32x4 U = zero4();
            mma16(U, ld_frag(sT + (16 * i + l16) * PT + 4 * g4), E::make(Z));
            Uf[i] = E::make(U);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            // P U gets its own accumulator: QS comes from 32-deep products,
            // and an MFMA of another shape does not take it as its
            // accumulator input straight after it (see kda_device.h).
            f32x4 PU = zero4();
            mma_rowblocks_n<TIn, NS>(PU, sP + (16 * i + l16) * PC + 4 * g4, Uf, i + 1);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int row = 16 * i + 4 * g4 + q4;
                if (row < nv) go[((t0 + row) * H + h) * D + col0 + l16] = E::from_f32(p.scale * (QS[i][q4] + PU[q4]));
            }
        }
#pragma unroll
        for (int ct = 0; ct < NKB; ++ct) {
            f32x4 acc;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) acc[q4] = sGam[16 * ct + 4 * g4 + q4] * Sm[ct][q4];
            mma_rowblocks<TIn, NS>(acc, sKbT + (16 * ct + l16) * PC + 4 * g4, Uf);
            Sm[ct] = acc;
        }
        // State checkpoint when the tokens done so far are a whole number of
        // intervals (the interval is a multiple of C, so only at chunk ends).
        if (p.ckpt && t0 + C <= t_end && (t0 + C - t_begin) % p.ckpt_interval == 0) {
            const int64_t slot = (int64_t)ck0 + (t0 + C - t_begin) / p.ckpt_interval - 1;
            if (slot < p.ckpt_cap) {
                // one per-lane offset; rows as wave-uniform offsets
                const auto rc = buffer_rsrc(p.ckpt + (slot * H + h) * D * D, D * D * 4);
#pragma unroll
                for (int ct = 0; ct < NKB; ++ct)
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sm[ct][pp]), rc, s_voff,
                                                              (16 * ct + pp) * D * 4, 0);
            }
        }
        __syncthreads();
    }

    if (p.Sout) {
        const auto rs = buffer_rsrc(p.Sout + sbase, D * D * 4);
#pragma unroll
        for (int ct = 0; ct < NKB; ++ct) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sm[ct][pp]), rs, s_voff,
                                                      (16 * ct + pp) * D * 4, 0);
        }
    }
}

template <typename TIn, int D, int NS, int NWC>
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.N * p.H * p.nslab;
    hipLaunchKernelGGL((kda_prefill_kernel<TIn, D, NS, NWC>), dim3((unsigned)blocks), dim3(64 * NWC), 0, s, p);
    return hipGetLastError();
}

#define KDA_PREFILL_VARIANT(DT, TIN, D, NS, NWC) \
    { 0, DT, D, 16 * NS, NWC, PrefillCfg<TIN, D, NS, NWC>::LDS, &launch_prefill<TIN, D, NS, NWC> }

}  // namespace kda
