// kda_prefill_ws.h -- wave-specialised, software-pipelined KDA prefill for
// bf16 q/k/v, d_k = d_v = 128, 16-token chunks (gfx950).
//
// Same chunk algebra as kda_prefill_impl.h with one 16-token sub-tile per
// chunk (so Kt = k e^G, Qt = q e^G and Kbar = k e^{G_C - G} need no extra
// factors), but the work of a chunk is split over waves with different jobs
// that run concurrently on consecutive chunks:
//
//   stage A   (NSA waves)  chunk c = m + 3: cumulative log-decay L (DPP row
//                          scan), scaled tiles QB = q e^L, KB = k e^L,
//                          KL = k e^{-L} and its transpose, gamma = e^{L_15},
//                          beta; requests the raw inputs of chunk c + 3.
//   Gram      (1 wave)     chunk m + 2: P = scale incl-lower(QB KL^T) and
//                          A = strict-lower(diag(beta) KB KL^T) on MFMA
//                          (and parks V of chunk m + 1, as beta V in fp32
//                          for slabs of up to 64 columns):
//                          e^{L_r - L_s} = e^{L_r} e^{-L_s} with
//                          e^{L_r} in [e^-80, 1] and e^{-L_s} in [1, e^80]
//                          (a 16-token tile decays by at least -80), so no
//                          factor leaves the bf16/fp32 exponent range.
//   solve     (1 wave)     chunk m + 1: T = (I + A)^{-1} by a column sweep
//                          (fp32; four lanes per column, four rows each).
//   consumers (NCW waves)  chunk m: X = Kt S, Qt S, U = T diag(beta)(V - X),
//                          O = scale Qt S + P U, S <- Diag(gamma)(S + KL^T U)
//                          (= Diag(gamma) S + Kbar^T U, Kbar = k e^{tot-L}:
//                          the decay of each contribution is applied to the
//                          sum, which is also exact up to relative rounding
//                          because e^{-L_s} <= 1/gamma); each
//                          wave owns TPW x 16 value columns of the fp32 state
//                          in registers (see kda_device.h for the MFMA
//                          layout that chains the products in registers).
//
// Iteration m ends with the only barrier.  LDS slots rotate with the chunk
// index: QB/KB/KL^T/gamma/beta live 4 iterations, P 3, KL, A, T and V 2, so no
// slot is written while another wave still reads it.  Raw q/k/g/beta are
// requested three iterations ahead by the stage-A waves, each wave loading
// whole cache lines of its share of the chunk; the pieces are assembled
// row-major in LDS and read back in the compute layout one iteration ahead.
// The V tile travels through the Gram wave's registers into a 2-deep LDS
// slot.  The load loops are unrolled twice so both register sets have fixed
// names, and every load is issued unconditionally (buffer loads, rows past
// the end of the tensor read as 0) so the compiler's counted waits never
// collapse to a full drain.  The consumers write each 16-token output tile
// with one 16-byte store per lane.  Rows past
// the end of a sequence read q = k = g = beta = 0 (the load ranges end with
// the sequence): then their A rows, Y rows and hence U rows are zero, they
// change neither the state nor the earlier rows, and their outputs are not
// stored.
//
// Sources for what is computed: as in kda_prefill_impl.h ("Understanding Kimi
// K3's attention" state-update / readout / g_min equations; "Inside Kimi K3",
// section "Sequence mixing"; "Hybrid Attention", section "But isn't a
// recurrent update sequential?").
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int NCW, int TPW, int NSA, bool FUSED = false, bool GATE = false>
struct WsCfg {
    static constexpr int D = 128;
    static constexpr int C = 16;
    static constexpr int NCB = D / 16;               // 16-channel blocks
    static constexpr int NWAVES = NCW + 2 + NSA;
    static constexpr int NT = 64 * NWAVES;
    // Eight consumer waves make the segment scan's map pair (waves 0-3 the map
    // M, waves 4-7 the map B of the same segment, sharing stage A, Gram and
    // solve): two parts of four waves over the same value columns.
    static constexpr int NCWP = NCW == 8 ? 4 : NCW;  // consumer waves per part
    static constexpr int DVW = NCWP * TPW * 16;      // value columns per workgroup (per part)
    // Wave w runs on SIMD w mod 4.  With 14 waves, SIMDs 0 and 1 hold four
    // waves and SIMDs 2 and 3 three: the solve and Gram waves go to the
    // latter (waves 6 and 7), the stage-A waves are 4, 5 and 8-13.
    static constexpr int W_SOLVE = NCW == 4 ? 6 : NCW;
    static constexpr int W_GRAM = NCW == 4 ? 7 : NCW + 1;
    static constexpr int W_A0 = NCW + 2;             // first stage-A wave (NCW < 4)
    static constexpr int IPW = NCB / NSA;            // stage-A items (16-channel blocks) per wave

    // Row pitches chosen so that the 8-byte fragment accesses of 16 lanes (16
    // rows, one fragment each) hit 32 distinct banks: 66 and 10 dwords.
    static constexpr int PD = D + 4;                 // bf16 pitch of [16][D] tiles
    static constexpr int PK = C + 4;                 // bf16 pitch of KL^T [D][16] and of 16x16 tiles
    static constexpr int PA = 20;                    // fp32 pitch of A^T

    static constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
    // 4-deep slot: QB, KB, KL^T, gamma, beta
    static constexpr size_t S4_QB = 0;
    static constexpr size_t S4_KB = S4_QB + al16(2 * C * PD);
    static constexpr size_t S4_KT = S4_KB + al16(2 * C * PD);
    static constexpr size_t S4_GAM = S4_KT + al16(2 * D * PK);
    static constexpr size_t S4_BETA = S4_GAM + al16(4 * D);
    static constexpr size_t S4 = S4_BETA + al16(4 * C);
    // 2-deep slot: KL (row-major, the Gram right operand)
    static constexpr size_t S2_KL = 0;
    static constexpr size_t S2 = S2_KL + al16(2 * C * PD);
    static constexpr size_t SP = al16(2 * C * PK);   // P (3-deep) and T (2-deep)
    static constexpr size_t SA = al16(4 * C * PA);   // A^T (2-deep)
    // V tile (2-deep): for slabs of up to 64 columns the Gram wave parks
    // beta V in fp32 (VF), taking that multiply off the consumers; the
    // 128-column kernel, whose Gram wave shares a SIMD with a consumer, keeps
    // the bf16 tile and its consumers form beta v (the same arithmetic).
    static constexpr bool VF = DVW <= 64;
    static constexpr int PV = VF ? DVW + 4 : DVW + 8;  // fp32 / bf16 pitch of the V tile
    static constexpr size_t SV = al16((VF ? 4 : 2) * C * PV);
    static constexpr int VLB = C * DVW * 2 / 64;     // V tile bytes per Gram-wave lane
    static constexpr int VCB = VLB >= 16 ? 16 : 8;   // bytes per V chunk (one load)
    static constexpr int VCH = VLB / VCB;            // V chunks per Gram-wave lane: 4, 2 or 1

    static constexpr size_t OFF4 = 0;
    static constexpr size_t OFF2 = OFF4 + 4 * S4;
    static constexpr size_t OFFP = OFF2 + 2 * S2;
    static constexpr size_t OFFT = OFFP + 3 * SP;
    static constexpr size_t OFFA = OFFT + 2 * SP;
    // Raw q, k, g (or, fused, the gate input z), beta of one chunk, row-major,
    // assembled in LDS by the stage-A waves (2-deep).  A q, k or z load covers
    // 4 token rows (1056 B of the tile at pitch PD), a g load 2 rows (1056 B
    // at pitch PG): the same step, so every parking store has a constant
    // offset.
    static constexpr int PG = D + 4;                 // fp32 pitch of the raw g tile
    static constexpr size_t R_Q = 0;
    static constexpr size_t R_K = R_Q + al16(2 * C * PD);
    static constexpr size_t R_G = R_K + al16(2 * C * PD);
    static constexpr size_t R_B = R_G + (FUSED ? al16(2 * C * PD) : al16(4 * C * PG));
    static constexpr size_t R_X = R_B + 4 * 64 * NSA;  // beta: 64 floats per stage-A wave; then the
                                                       // parking area of waves without a raw load
    static constexpr size_t SR = R_X + (FUSED ? (size_t)(16 / NSA - 1) * 4 * 2 * PD + 64 * 16 : 0);
    static constexpr int NUNITS = FUSED ? 12 : 16;     // raw loads per chunk
    static constexpr int RAW_STEP = 4 * 2 * PD;      // LDS bytes per raw load
    static constexpr size_t OFFV = OFFA + 2 * SA;
    static constexpr size_t OFFR = OFFV + 2 * SV;
    // Output gate (GATE): per chunk slot the consumer waves' bf16 o tiles (64
    // lanes x 16 B per wave), 2-deep; the RMSNorm weight of the slab's
    // columns.  The gate factors Sigmoid(gate) * weight reach a 2-deep
    // [C][PGT] fp32 tile from the stage-A waves.
    static constexpr size_t G_OST = OFFR + 2 * SR;
    static constexpr size_t G_W = G_OST + (GATE ? 2 * 1024 * NCW : 0);
    static constexpr int PGT = DVW + 4;              // fp32 pitch of the gate factor tile
    static constexpr size_t SGT = al16(4 * C * PGT);
    static constexpr size_t G_GT = G_W + (GATE ? 4 * DVW : 0);
    // Fused kernel: per chunk the row factors of the L2 norms (8-deep ring):
    // r_k, |k| = 1 / r_k (0 for the zero vector) and scale r_q (from the Gram
    // wave one chunk ahead), beta r_k and beta r_k^2 (from the Gram wave with
    // the chunk's Gram tiles).
    static constexpr size_t NR_RK = 0, NR_NK = 4 * C, NR_SQ = 8 * C, NR_BK = 12 * C, NR_B2 = 16 * C;
    static constexpr size_t SNR = 20 * C;
    static constexpr size_t OFFN = G_GT + (GATE ? 2 * SGT : 0);
    static constexpr size_t LDS = OFFN + (FUSED ? 8 * SNR : 0);

    static_assert(DVW <= D && D % DVW == 0, "value slab");
    static constexpr int LPW = 16 / NSA;             // raw loads per stage-A wave and chunk
    static_assert(NSA == 4 || NSA == 8, "a stage-A wave's raw loads stay within one of q, k, g");
    static_assert(!FUSED || NSA == 8, "the fused loads are laid out for eight stage-A waves");
    static_assert(2 * 4 * PG == RAW_STEP, "q/k and g raw loads step equally through LDS");
    static_assert(TPW == 1 || TPW == 2, "a consumer lane stores 4 TPW adjacent outputs");
    static_assert(NCB % NSA == 0, "stage-A waves split the channel blocks evenly");
    static_assert(VLB == VCB * VCH && (VCH == 1 || VCH == 2 || VCH == 4), "V tile split over the Gram wave");
    static_assert(PA % 4 == 0, "rows of A^T are read as float4");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(!GATE || (DVW == D && TPW == 2 && !FUSED), "the fused gate needs whole heads");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache policy (the nt bit of the buffer instructions' policy operand) of the
// loads whose lines no other workgroup reads: the V tile of a slab and, where
// a workgroup holds a whole head, also q, k, g and beta (the slabs of a split
// head share those through the L2).  Marked non-temporal they do not displace
// lines that are still wanted (16-sequence varlen pack: 1-3.5% faster,
// depending on the device; the dense launch unchanged).  The o stores keep the
// default policy: non-temporal, the halves of a line that two consumer waves
// write reached memory separately (35-45% more bytes written, no faster).
constexpr int kStream = 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One stage-A wave's share of a chunk's raw inputs, as loaded: LPW 16-byte
// pieces of whole token rows per lane (plus beta in wave 0).
template <int LPW>
struct LoadSet {
    u32x4 x[LPW];
    float beta;
};

// Raw inputs of one chunk as a stage-A wave computes on them: per item
// (16-channel block) one token x 4 channels of g, q, k per lane, plus beta.
template <int IPW>
struct RawSet {
    f32x4 g[IPW];   // 4 channels of g (fused: of the gate input z)
    u32x4 qk[IPW];  // 4 bf16 channels of q (words 0, 1) and of k (words 2, 3)
    float beta;
};

// V tile of one chunk held by the Gram wave between its load and its copy
// into LDS: up to four chunks of 16 (or 8) bytes per lane, in named
// registers (no array, so the compiler keeps them in VGPRs), written out
// untouched.  Only the first VCH members are used.
template <typename T>
struct VRegs {
    T a, b, c, d;
};

// Broadcast lane 15 of each 16-lane row to the whole row.
__device__ __forceinline__ float row_bcast15(float x) {
    // ds_swizzle bit mode inside 32-lane halves: lane' = (lane & 0x10) | 0x0f
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F0));
}

// A wave-uniform 64-bit value moved into scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E - 1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Lane K of each quad (4 adjacent lanes) broadcast to the quad (DPP
// quad_perm [K, K, K, K]).
template <int K>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), K * 0x55, 0xf, 0xf, false));
}

// What one workgroup of a pipelined launch works on: the token range of its
// sequence or segment, the head, the value slab, where its state starts and
// ends, and whether it stores outputs and reads v.
struct WsWork {
    int64_t t_begin, t_end;
    int n, h, z;
    const float* s_in;  // start state [D][D] of the (sequence, head), or nullptr (zeros)
    float* s_out;       // end state [D][D], or nullptr
    float* s_out_m;     // map pair: the end state of the part run from the identity with v = 0 (M)
};

// Block -> work.  The dispatcher deals consecutive workgroups to the 8 XCDs
// in turn, so block b runs on XCD b % 8.  All slabs of one item get the same
// b % 8 and neighbouring b / 8, so they run on one XCD at the same pace and
// the q, k, g and beta they all read come from that XCD's L2 after the first
// slab's miss.  Items are padded to whole groups of 8; padding blocks get no
// work.  Segment-scan launches list their items the same way: phase 1 (the
// map-pair kernel, whole heads) the map pairs of segments 1 .. seg_G - 2 of
// every (sequence, head), then segment 0 of each, run with its outputs from
// the initial state (it needs no map: its start is known), on the compute
// units the pairs leave free; phase 3 segments 1 .. seg_G - 1 with their
// slabs.
// Sequence of descending-length rank r (ties in sequence order), for a packed
// batch of at most 64 sequences: lane m holds the length of sequence m and
// counts the sequences that go before it.  Called by every lane of a wave;
// returns the same value in all lanes.
__device__ inline int ws_seq_of_rank(const PrefillParams& p, int r) {
    const int lane = threadIdx.x & 63;
    int64_t a = 0, b = 0;
    if (lane < p.N) seq_bounds(p, lane, &a, &b);
    const int len = lane < p.N ? (int)(b - a) : -1;  // token counts are below 2^31
    int before = 0;
    for (int m = 0; m < p.N; ++m) {
        const int lm = __builtin_amdgcn_readlane(len, m);
        before += (lm > len || (lm == len && m < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < p.N && before == r);
    return hit ? (int)__builtin_ctzll(hit) : r;  // one lane for every r < N
}

template <int D, bool SEG, bool PAIR>
__device__ inline bool ws_resolve(const PrefillParams& p, int bid, WsWork& w) {
    const int units = p.N * p.H;
    const int xcd = bid & 7;
    const int64_t sdd = (int64_t)D * D;
    auto map_slot = [&](int uh, int g, int part) {
        return p.seg_ws + (((int64_t)uh * (p.seg_G - 1) + g) * 2 + part) * sdd;
    };
    // segment g: tokens [g seg_len, (g + 1) seg_len) of its sequence, the last
    // one running to the end of the sequence
    auto seg_range = [&](int n, int g) {
        const int64_t s0 = (int64_t)n * p.seq_len;
        w.t_begin = s0 + (int64_t)g * p.seg_len;
        w.t_end = g == p.seg_G - 1 ? s0 + p.seq_len : w.t_begin + p.seg_len;
    };
    w.s_out_m = nullptr;
    if constexpr (PAIR) {
        // phase 1: the maps of segment 1 <= g <= seg_G - 2 (M into slot (g, 0),
        // B into slot (g, 1)); then segment 0, run from the initial state with
        // its outputs: its end state, the start of segment 1, into slot (0, 1)
        // (s_out_m = nullptr marks the run)
        const int item = (bid >> 3) * 8 + xcd;
        const int npair = units * (p.seg_G - 2);
        if (item >= npair + units) return false;
        w.z = 0;
        if (item < npair) {
            const int uh = item / (p.seg_G - 2), g = 1 + item % (p.seg_G - 2);
            w.h = uh % p.H;
            w.n = uh / p.H;
            seg_range(w.n, g);
            w.s_in = nullptr;
            w.s_out = map_slot(uh, g, 1);
            w.s_out_m = map_slot(uh, g, 0);
        } else {
            const int uh = item - npair;
            w.h = uh % p.H;
            w.n = uh / p.H;
            seg_range(w.n, 0);
            w.s_in = p.S0 ? p.S0 + (int64_t)uh * sdd : nullptr;
            w.s_out = map_slot(uh, 0, 1);
        }
        return true;
    }
    const int rest = bid >> 3;
    w.z = rest % p.nslab;
    if (!SEG || p.seg_phase == 0) {
        // Dispatch position k -> (sequence, head).  The workgroups of a launch
        // start in block order as compute units free up, so the sequences of a
        // packed batch (up to 64 of them) go out longest first: the long ones
        // then do not run on alone at the end (a 16-sequence, 96-head pack:
        // -6% against sequence order).  Every unit is independent, so the
        // order changes no result.
        const int k = (rest / p.nslab) * 8 + xcd;
        if (k >= units) return false;
        w.h = k % p.H;
        w.n = (p.cu && p.N > 1 && p.N <= 64) ? ws_seq_of_rank(p, k / p.H) : k / p.H;
        const int uh = w.n * p.H + w.h;
        seq_bounds(p, w.n, &w.t_begin, &w.t_end);
        w.s_in = p.S0 ? p.S0 + (int64_t)uh * sdd : nullptr;
        w.s_out = p.Sout ? p.Sout + (int64_t)uh * sdd : nullptr;
        return true;
    }
    // phase 3: segment g >= 1 from the start state the combine (or, for
    // g = 1, phase 1's run of segment 0) left in slot (g - 1, 1)
    const int item = (rest / p.nslab) * 8 + xcd;
    if (item >= units * (p.seg_G - 1)) return false;
    const int uh = item / (p.seg_G - 1), g = 1 + item % (p.seg_G - 1);
    w.h = uh % p.H;
    w.n = uh / p.H;
    seg_range(w.n, g);
    w.s_in = map_slot(uh, g - 1, 1);
    w.s_out = (g == p.seg_G - 1 && p.Sout) ? p.Sout + (int64_t)uh * sdd : nullptr;
    return true;
}

// CKB: the backward's forward run.  Checkpoints as bf16 in the blocked layout
// the backward kernel reads ([row / 4][column][row % 4] per state: the 4 rows
// a lane holds of one column are 8 adjacent bytes) instead of the fp32
// row-major states of the public checkpoint call, and no output o (p.o is not
// read): the readout products Q~ S and P U and the P tile are skipped.
//
// SEG: the variants that run the segment-scan phases (PrefillParams::
// seg_phase 1: the map-pair kernel, NCW = 8; seg_phase 3: the runs of the
// segments); the plain kernels are compiled without that code.
//
// MAP: the body of the map-pair kernel (segment scan, phase 1): only the end
// states are wanted, so, as with CKB, no readout and no o; q is not read
// either (its loads use an empty range: no memory request).  Consumer waves
// 0-3 start from the identity with v read as zero (the map M), waves 4-7 from
// the start state (zero, or the initial state for segment 0) with v (the map
// B); stage A, Gram and solve serve both.
template <int NCW, int TPW, int NSA, bool FUSED, bool CKB, bool SEG, bool MAP, bool GATE>
__device__ __forceinline__ void ws_body(const PrefillParams& p, const WsWork& wk, char* smem) {
    typedef WsCfg<NCW, TPW, NSA, FUSED, GATE> Cfg;
    typedef Elem<bf16_t> E;
    typedef uint2 Frag;
    constexpr int D = Cfg::D, C = Cfg::C, NCB = Cfg::NCB, DVW = Cfg::DVW, IPW = Cfg::IPW;
    constexpr int PD = Cfg::PD, PK = Cfg::PK, PA = Cfg::PA;
    constexpr bool NOOUT = CKB || MAP;  // no readout, no o

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform by construction
    const int g4 = lane >> 4;
    const int l16 = lane & 15;

    // Segment-map pair (MAP: eight consumer waves): waves 0-3 run the map M
    // (from the identity, v read as zero), waves 4-7 the map B.  Compile-time
    // false outside the map body.
    static_assert(!MAP || (NCW == 8 && SEG), "the map body is the pair kernel's");
    const bool w_identity = MAP && w < Cfg::NCWP;
    const bool w_v_zero = w_identity;
    float* const s_dst = w_identity ? wk.s_out_m : wk.s_out;  // this wave's end state
    const int z = wk.z;
    const int h = wk.h;
    const int n = wk.n;
    const int H = p.H;
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int64_t ntok = t_end - t_begin;
    // fused gate: e^{A_h} log2(e) for this head (A_h = a_log[h], a per-head log-scale)
    const float gate_ea_l2e =
        (FUSED && ntok > 0) ? __builtin_amdgcn_exp2f(p.a_log[h] * 1.4426950408889634f) * 1.4426950408889634f : 0.f;
    const int nch = (int)((ntok + C - 1) / C);

    const bf16_t* gq = static_cast<const bf16_t*>(p.q);
    const bf16_t* gk = static_cast<const bf16_t*>(p.k);
    const bf16_t* gv = static_cast<const bf16_t*>(p.v);
    bf16_t* go = static_cast<bf16_t*>(p.o);

    auto slot4 = [&](int c) { return smem + Cfg::OFF4 + (size_t)(c & 3) * Cfg::S4; };
    auto slot2 = [&](int c) { return smem + Cfg::OFF2 + (size_t)(c & 1) * Cfg::S2; };
    auto slotP = [&](int c) { return smem + Cfg::OFFP + (size_t)(c % 3) * Cfg::SP; };
    auto slotT = [&](int c) { return smem + Cfg::OFFT + (size_t)(c & 1) * Cfg::SP; };
    auto slotA = [&](int c) { return smem + Cfg::OFFA + (size_t)(c & 1) * Cfg::SA; };
    auto slotV = [&](int c) { return smem + Cfg::OFFV + (size_t)(c & 1) * Cfg::SV; };
    auto slotN = [&](int c) { return reinterpret_cast<float*>(smem + Cfg::OFFN + (size_t)(c & 7) * Cfg::SNR); };
    // Element offset of token row 0 of chunk c for head h (uniform per wave).
    auto chunk_base = [&](int c) -> int64_t { return ((t_begin + (int64_t)c * C) * H + h) * D; };
    // Byte address of row 0 of chunk c in a [T, H, D] tensor of es-byte
    // elements: the workgroup's first chunk plus c strides of 16 token rows.
    // A stride is below 2^31 bytes (the host checks H D 64 < 2^31), so each
    // chunk costs one 32 x 32 -> 64-bit scalar multiply-add instead of the
    // 64-bit index arithmetic of chunk_base.
    const int64_t e_first = chunk_base(0);
    auto chunk_ptr = [&](const void* base, int es, int c) -> const char* {
        return static_cast<const char*>(base) + e_first * es +
               (uint64_t)(uint32_t)c * (uint32_t)(C * H * D * es);
    };
    auto rows_valid = [&](int c) -> int {
        // (32-bit: token counts are below 2^31, so this stays in scalar registers)
        const int left = (int)ntok - c * C;
        return left >= C ? C : left;
    };

    // ------------------------------------------------------------ role setup
    const bool is_cons = w < NCW;
    const bool is_stageA = w >= NCW && w != Cfg::W_SOLVE && w != Cfg::W_GRAM;
    const int sa = NCW == 4 ? (w < 6 ? w - 4 : w - 6) : w - Cfg::W_A0;  // stage-A wave index
    const int col_base = z * DVW + (is_cons ? (w % Cfg::NCWP) * TPW * 16 : 0);
    // Value column of MFMA column j of consumer tile t, relative to col_base:
    // the 4 TPW columns a lane's outputs fall on (see consume) are adjacent.
    auto vcol = [&](int t, int j) { return 4 * TPW * (j >> 2) + 4 * t + (j & 3); };


    // Global reads of the per-chunk inputs are buffer loads: a wave-uniform
    // resource per chunk (base = the chunk's first token row for this head)
    // and a per-lane byte offset that is the same for every chunk.  For q, k,
    // g (or z) and beta the resource ends with the chunk's last row in the
    // sequence (or segment), so rows past it read zeros without a memory
    // request: g = beta = 0 there, which makes them identity transitions
    // (fused: z = 0 is not g = 0, so g is zeroed there explicitly); their
    // outputs are not stored.  V reads end with the tensor (their rows past
    // the sequence meet beta = 0).  No per-lane address is recomputed per
    // chunk, so issuing the next chunk's loads never waits on the registers
    // of loads in flight.
    const int64_t n_tok_elems = p.T_total * H * D;  // elements of q, k, g (and v)
    auto rsrc = [](const void* base, int64_t bytes_left) {
        const int num = bytes_left > 0x7fffffff ? 0x7fffffff : (int)bytes_left;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num, 0x00020000);
    };
    // The same for ranges inside one chunk (at most 16 token rows of H heads:
    // below 2^31 bytes, which the host checks), in 32-bit scalar arithmetic.
    auto rsrc_chunk = [](const void* base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
    };
    // Raw q, k, g, beta of chunk c.  A chunk is 16 loads of 16 B per lane
    // over whole token rows: units 0-3 the q tile and 4-7 the k tile (4 rows
    // of 256 B each), units 8-15 the g tile (2 rows of 512 B each); fused,
    // units 8-11 the bf16 gate input z (4 rows each) and no more.  Stage-A
    // wave sa issues the LPW units of its group, LPW ld_grp .. LPW ld_grp +
    // LPW - 1 (all of one tensor; ld_grp = sa except as below), and wave 0
    // also beta, so every cache line is requested by exactly one load
    // instruction.  The pieces are parked row-major in LDS and read back
    // after a barrier in the layout stage A computes on.  A wave past the
    // last unit still issues its loads, at an out-of-range offset (zeros, no
    // memory request), and parks them in its own corner of LDS, so that no
    // load or its use depends on the wave.
    constexpr int LPW = Cfg::LPW;
    constexpr int kRawPolicy = DVW == D ? kStream : 0;  // whole heads: no other workgroup reads these lines
    // Fused, the 12 units leave two stage-A waves without a raw load.  With
    // two consumer waves (SIMDs 0 and 1, stage-A wave sa on SIMD sa mod 4) the
    // q and k units go to the stage-A waves on SIMDs 2 and 3, the z units to
    // the older and no load to the younger stage-A wave of SIMDs 0 and 1 (the
    // parking stores stay off the consumers' SIMDs where they can): unit
    // groups 4 5 0 1 6 7 2 3.
    const int ld_grp = (FUSED && NCW == 2) ? (int)((0x32761054u >> (4 * sa)) & 15u) : sa;
    const int ld_u0 = ld_grp * LPW;
    const bool ld_none = ld_u0 >= Cfg::NUNITS;
    const bool ld_bf16 = FUSED || ld_u0 < 8;
    const int ld_lpr = ld_bf16 ? 16 : 32;  // lanes per token row
    const int ld_row = (ld_bf16 ? 4 * (ld_u0 & 3) : 2 * (ld_u0 - 8)) + lane / ld_lpr;
    const int ld_es = ld_bf16 ? 2 : 4;    // element bytes
    const char* ld_base = ld_u0 < 4 ? reinterpret_cast<const char*>(gq)
                        : ld_u0 < 8 ? reinterpret_cast<const char*>(gk)
                        : FUSED     ? reinterpret_cast<const char*>(p.z)
                                    : reinterpret_cast<const char*>(p.g);
    const uint32_t ld_step = 8u * (uint32_t)(H * D);  // global bytes per load (4 bf16 or 2 fp32 rows)
    // (a map workgroup's q loads also take the out-of-range offset: q is not needed)
    const uint32_t ld_voff = (ld_none || (MAP && ld_u0 < 4))
                                 ? 0x80000000u
                                 : (uint32_t)ld_row * (uint32_t)(H * D) * (uint32_t)ld_es + 16u * (uint32_t)(lane % ld_lpr);
    // beta bytes; the other waves read out of range (zeros, no memory request)
    // so that the load and its use stay unconditional
    const uint32_t lb = sa == 0 ? (uint32_t)l16 * (uint32_t)H * 4u : 0x80000000u;
    const char* const beta_first = reinterpret_cast<const char*>(p.beta + (t_begin * H + h));
    auto load_raw = [&](int c, LoadSet<LPW>& R) {
        const int cc = c < nch ? c : nch - 1;
        // the ranges end with the chunk's last row in the sequence: later rows read 0
        const int nv = rows_valid(cc);
        const auto r = rsrc_chunk(chunk_ptr(ld_base, ld_es, cc), ((nv - 1) * H * D + D) * ld_es);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            R.x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ld_voff + i * ld_step, 0, kRawPolicy));
        const auto rb = rsrc_chunk(beta_first + (uint64_t)(uint32_t)cc * (uint32_t)(C * H * 4), ((nv - 1) * H + 1) * 4);
        R.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lb, 0, 0));
    };
    // Gate logits (GATE): stage-A waves carry a chunk's [C][DVW] bf16 gate
    // tile from HBM into gate slot (c & 1), as two row pairs (8 bytes per lane
    // each, 4 columns per lane): loaded in iteration c + 2, parked in c + 3,
    // read by the gated store (Gram and solve waves) in c + 4; the slot is
    // next written (chunk c + 2) in c + 5.  The older stage-A waves of SIMDs 0
    // and 1 (0 and 1), which have the slack, take rows 0-3 and 4-7; waves 2-5
    // rows 8-15, two each; the youngest, 6 and 7, none (a timing copy of the
    // gated launch: 2.6% shorter than with two rows on every stage-A wave).
    // A wave's unused pair, and chunks outside the sequence, read
    // zeros without a memory request and are not parked, so every wave issues
    // the same two loads.
    const int gt_col = 4 * (lane & 31);
    const bool gt_a = sa < 6, gt_b = sa < 2;
    const int gt_row_a = (sa < 2 ? 4 * sa : 8 + 2 * (sa - 2)) + (lane >> 5);
    const int gt_row_b = 4 * sa + 2 + (lane >> 5);
    struct GtSet {
        u32x2 a, b;
    };
    auto load_gt = [&](int c) -> GtSet {
        const bool in = c >= 0 && c < nch;
        const int cc = in ? c : 0;
        const int64_t base = chunk_base(cc) + z * DVW;
        const auto rg = rsrc(static_cast<const bf16_t*>(p.gate) + base, (n_tok_elems - base) * 2);
        const uint32_t oa = in && gt_a ? ((uint32_t)gt_row_a * (uint32_t)(H * D) + (uint32_t)gt_col) * 2u : 0x80000000u;
        const uint32_t ob = in && gt_b ? ((uint32_t)gt_row_b * (uint32_t)(H * D) + (uint32_t)gt_col) * 2u : 0x80000000u;
        return GtSet{__builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, oa, 0, 0)),
                     __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, ob, 0, 0))};
    };
    auto park_one = [&](int c, u32x2 x, int row) {
        const float* wt = reinterpret_cast<const float*>(smem + Cfg::G_W) + gt_col;
        f32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t wd = x[e >> 1];
            const float gl = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
            f[e] = wt[e] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gl));
        }
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(smem + Cfg::G_GT + (size_t)(c & 1) * Cfg::SGT) +
                                  row * Cfg::PGT + gt_col) = f;
    };
    auto park_gt = [&](int c, const GtSet& x) {
        if (c >= 0 && c < nch) {
            if (gt_a) park_one(c, x.a, gt_row_a);
            if (gt_b) park_one(c, x.b, gt_row_b);
        }
    };
    // Raw tile of chunk c (two slots in rotation).
    auto raw_slot = [&](int c) { return smem + Cfg::OFFR + (size_t)(c & 1) * Cfg::SR; };
    const uint32_t park_off =
        ld_none ? (uint32_t)Cfg::R_X + 16u * (uint32_t)lane
                : (uint32_t)(ld_u0 < 4 ? Cfg::R_Q : ld_u0 < 8 ? Cfg::R_K : Cfg::R_G) +
                      (uint32_t)ld_row * (uint32_t)(ld_bf16 ? 2 * PD : 4 * Cfg::PG) + 16u * (uint32_t)(lane % ld_lpr);
    auto park_raw = [&](int c, const LoadSet<LPW>& R) {
        char* b = raw_slot(c) + park_off;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            // q/k rows are only 8-byte aligned (pitch PD): two 8-byte halves
            *reinterpret_cast<u32x2*>(b + i * Cfg::RAW_STEP) = R.x[i].xy;
            *reinterpret_cast<u32x2*>(b + i * Cfg::RAW_STEP + 8) = R.x[i].zw;
        }
        reinterpret_cast<float*>(raw_slot(c) + Cfg::R_B)[64 * sa + lane] = R.beta;  // wave 0's rows 0-15 are used
    };
    // Stage-A layout: token row l16, channels c0..c0+3 of each item.
    auto fetch_raw = [&](int c, RawSet<IPW>& R) {
        const char* b = raw_slot(c);
#pragma unroll
        for (int it = 0; it < IPW; ++it) {
            const int c0 = 16 * (IPW * sa + it) + 4 * g4;
            if constexpr (FUSED) {
                const u32x2 zv = *reinterpret_cast<const u32x2*>(b + Cfg::R_G + (l16 * PD + c0) * 2);
                R.g[it] = f32x4{__uint_as_float(zv.x << 16), __uint_as_float(zv.x & 0xffff0000u),
                                __uint_as_float(zv.y << 16), __uint_as_float(zv.y & 0xffff0000u)};
            } else {
                R.g[it] = *reinterpret_cast<const f32x4*>(b + Cfg::R_G + (l16 * Cfg::PG + c0) * 4);
            }
            const u32x2 qv = *reinterpret_cast<const u32x2*>(b + Cfg::R_Q + (l16 * PD + c0) * 2);
            const u32x2 kv = *reinterpret_cast<const u32x2*>(b + Cfg::R_K + (l16 * PD + c0) * 2);
            R.qk[it] = u32x4{qv.x, qv.y, kv.x, kv.y};
        }
        R.beta = reinterpret_cast<const float*>(b + Cfg::R_B)[l16];
    };

    // V tile [C][DVW] of chunk c: lane chunk i covers row (lane + 64 i) / VCPR,
    // VCB / 2 bf16 columns (buffer loads as above, the range ending with the
    // chunk's last row in the sequence).  Slabs of up to 64 columns park it
    // as beta_r v_r in fp32, the form the consumers' Z = beta v - beta X takes
    // it in; the 128-column kernel parks the bf16 tile.
    typedef typename std::conditional<Cfg::VCB == 16, u32x4, u32x2>::type VChunk;
    constexpr int VCOL = Cfg::VCB / 2;  // bf16 columns per chunk
    constexpr int VCPR = DVW / VCOL;    // chunks per row
    auto v_off = [&](int i) -> uint32_t {
        const int idx = lane + 64 * i;
        return (uint32_t)(idx / VCPR) * (uint32_t)(H * D) * 2u + (uint32_t)(VCOL * (idx % VCPR)) * 2u;
    };
    auto v_load = [&](int c, int i) -> VChunk {
        const int cc = c < 0 ? 0 : (c < nch ? c : nch - 1);
        const auto rv = rsrc_chunk(chunk_ptr(gv, 2, cc) + z * DVW * 2, w_v_zero ? 0 : ((rows_valid(cc) - 1) * H * D + DVW) * 2);
        if constexpr (Cfg::VCB == 16)
            return __builtin_bit_cast(VChunk, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off(i), 0, kStream));
        else
            return __builtin_bit_cast(VChunk, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off(i), 0, kStream));
    };
    auto v_park = [&](int c, int i, VChunk x) {
        const int idx = lane + 64 * i;
        const int r = idx / VCPR, ch = idx % VCPR;
        if constexpr (!Cfg::VF) {
            *reinterpret_cast<VChunk*>(reinterpret_cast<bf16_t*>(slotV(c)) + r * Cfg::PV + VCOL * ch) = x;
            return;
        }
        // (fused: beta r_k, which the Gram wave stored with chunk c's tiles)
        const float br = FUSED ? slotN(c)[Cfg::NR_BK / 4 + r]
                               : reinterpret_cast<const float*>(slot4(c) + Cfg::S4_BETA)[r];
        float* dst = reinterpret_cast<float*>(slotV(c)) + r * Cfg::PV + VCOL * ch;
#pragma unroll
        for (int q4 = 0; q4 < VCOL / 4; ++q4) {
            const uint32_t lo = x[2 * q4], hi = x[2 * q4 + 1];
            *reinterpret_cast<f32x4*>(dst + 4 * q4) =
                f32x4{br * __uint_as_float(lo << 16), br * __uint_as_float(lo & 0xffff0000u),
                      br * __uint_as_float(hi << 16), br * __uint_as_float(hi & 0xffff0000u)};
        }
    };
    auto load_v = [&](int c, VRegs<VChunk>& V) {
        V.a = v_load(c, 0);
        if constexpr (Cfg::VCH > 1) V.b = v_load(c, 1);
        if constexpr (Cfg::VCH > 2) {
            V.c = v_load(c, 2);
            V.d = v_load(c, 3);
        }
    };
    auto store_v = [&](int c, const VRegs<VChunk>& V) {
        v_park(c, 0, V.a);
        if constexpr (Cfg::VCH > 1) v_park(c, 1, V.b);
        if constexpr (Cfg::VCH > 2) {
            v_park(c, 2, V.c);
            v_park(c, 3, V.d);
        }
    };

    // ------------------------------------------------------------ stage A
    auto stage_a = [&](int c, const RawSet<IPW>& R, int u) __attribute__((always_inline)) {  // u = c & 3
        // No multiply-add contraction here: contracting the scaling of g
        // into the first scan step gives a move, a DPP move and an FMA per
        // value where one DPP add does.
#pragma clang fp contract(off)
        char* s4 = smem + Cfg::OFF4 + (size_t)u * Cfg::S4;  // slot4(c)
        bf16_t* QB = reinterpret_cast<bf16_t*>(s4 + Cfg::S4_QB);
        bf16_t* KB = reinterpret_cast<bf16_t*>(s4 + Cfg::S4_KB);
        bf16_t* KLT = reinterpret_cast<bf16_t*>(s4 + Cfg::S4_KT);
        float* GAM = reinterpret_cast<float*>(s4 + Cfg::S4_GAM);
        float* BETA = reinterpret_cast<float*>(s4 + Cfg::S4_BETA);
        bf16_t* KL = reinterpret_cast<bf16_t*>(slot2(c) + Cfg::S2_KL);
        constexpr float LOG2E = 1.4426950408889634f;
        // Cumulative log-decay in base-2 units, all items and channels
        // interleaved so the dependent DPP steps of one scan overlap the others.
        // Rows past the end of the sequence read g = 0.
        float L[IPW][4];
        if constexpr (FUSED) {
            // g = g_min Sigmoid(e^{A_h} z), g_min = -5 ("Understanding Kimi
            // K3's attention", gate equation), in base-2 units:
            // log2(e) g = -5 log2(e) / (1 + 2^{-log2(e) e^{A_h} z}).
            // Rows past the end read z = 0, which is not g = 0: zeroed here.
            const float gscale = l16 < rows_valid(c) ? -5.f * LOG2E : 0.f;
#pragma unroll
            for (int it = 0; it < IPW; ++it)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const float t = __builtin_amdgcn_exp2f(-gate_ea_l2e * R.g[it][ch]);
                    L[it][ch] = gscale * __builtin_amdgcn_rcpf(1.f + t);
                }
        } else {
#pragma unroll
            for (int it = 0; it < IPW; ++it) {
                L[it][0] = R.g[it][0] * LOG2E;
                L[it][1] = R.g[it][1] * LOG2E;
                L[it][2] = R.g[it][2] * LOG2E;
                L[it][3] = R.g[it][3] * LOG2E;
            }
        }
#pragma unroll
        for (int it = 0; it < IPW; ++it)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) L[it][ch] += dpp_row_shr<0x111>(L[it][ch]);
#pragma unroll
        for (int it = 0; it < IPW; ++it)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) L[it][ch] += dpp_row_shr<0x112>(L[it][ch]);
#pragma unroll
        for (int it = 0; it < IPW; ++it)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) L[it][ch] += dpp_row_shr<0x114>(L[it][ch]);
#pragma unroll
        for (int it = 0; it < IPW; ++it)
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) L[it][ch] += dpp_row_shr<0x118>(L[it][ch]);
#pragma unroll
        for (int it = 0; it < IPW; ++it) {
            const int c0 = 16 * (IPW * sa + it) + 4 * g4;
            float e1[4], qb[4], kb[4], kl[4];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                e1[ch] = __builtin_amdgcn_exp2f(L[it][ch]);         // e^{L_r}  in [e^-80, 1]
                const float e2 = __builtin_amdgcn_exp2f(-L[it][ch]);  // e^{-L_r} in [1, e^80]
                const uint32_t qw = R.qk[it][ch >> 1], kw = R.qk[it][2 + (ch >> 1)];
                float qv = __uint_as_float((ch & 1) ? (qw & 0xffff0000u) : (qw << 16));
                float kv = __uint_as_float((ch & 1) ? (kw & 0xffff0000u) : (kw << 16));
                qb[ch] = qv * e1[ch];
                kb[ch] = kv * e1[ch];
                kl[ch] = kv * e2;
            }
            const Frag klf = E::make(kl[0], kl[1], kl[2], kl[3]);
            if constexpr (!NOOUT) st_frag(QB + l16 * PD + c0, E::make(qb[0], qb[1], qb[2], qb[3]));
            st_frag(KB + l16 * PD + c0, E::make(kb[0], kb[1], kb[2], kb[3]));
            st_frag(KL + l16 * PD + c0, klf);
            uint16_t* klt = reinterpret_cast<uint16_t*>(KLT) + l16;
            klt[(c0 + 0) * PK] = (uint16_t)(klf.x & 0xffffu);
            klt[(c0 + 1) * PK] = (uint16_t)(klf.x >> 16);
            klt[(c0 + 2) * PK] = (uint16_t)(klf.y & 0xffffu);
            klt[(c0 + 3) * PK] = (uint16_t)(klf.y >> 16);
            if (l16 == 15)  // e^{L_15} is the decay of the whole chunk
                *reinterpret_cast<float4*>(GAM + c0) = make_float4(e1[0], e1[1], e1[2], e1[3]);
        }
        if (sa == 0 && lane < C) BETA[lane] = R.beta;
    };

    // ------------------------------------------------------------ Gram tiles
    auto gram = [&](int c) {
        char* s4 = slot4(c);
        const bf16_t* QB = reinterpret_cast<const bf16_t*>(s4 + Cfg::S4_QB);
        const bf16_t* KB = reinterpret_cast<const bf16_t*>(s4 + Cfg::S4_KB);
        const float* BETA = reinterpret_cast<const float*>(s4 + Cfg::S4_BETA);
        const bf16_t* KL = reinterpret_cast<const bf16_t*>(slot2(c) + Cfg::S2_KL);
        f32x4 accA = zero4(), accP = zero4();
#pragma unroll
        for (int kb = 0; kb < NCB; kb += 2) {
            const int c0 = 16 * kb + 4 * g4;
            const Frag a0 = ld_frag(KL + l16 * PD + c0), a1 = ld_frag(KL + l16 * PD + c0 + 16);
            const Frag k0 = ld_frag(KB + l16 * PD + c0), k1 = ld_frag(KB + l16 * PD + c0 + 16);
            mma32(accA, a0, a1, k0, k1);
            if constexpr (!NOOUT) {
                const Frag q0 = ld_frag(QB + l16 * PD + c0), q1 = ld_frag(QB + l16 * PD + c0 + 16);
                mma32(accP, a0, a1, q0, q1);
            }
        }
        // acc[pp] = M[s = 4 g4 + pp][r = l16] = sum_c KL[s][c] X[r][c]
        bf16_t* P = reinterpret_cast<bf16_t*>(slotP(c));
        float* AT = reinterpret_cast<float*>(slotA(c));
        const int r = l16;
        if constexpr (FUSED) {
            static_assert(!NOOUT, "the fused kernels read out");
            // Raw q and k: the norms enter as row and column factors of the
            // 16 x 16 tiles.  A = Diag(beta r_k) A_raw Diag(r_k); P keeps only
            // its row factor scale r_q, the column factor r_k travels with
            // U' = Diag(r_k) U = (Diag(r_k) T Diag(1 / r_k)) (Diag(r_k) Z):
            // the solve wave scales T that way (its unit diagonal stays
            // exact) and the consumers form Diag(r_k) Z = (beta r_k) v -
            // (beta r_k^2) X_raw from the row factors stored here.
            const float* nr = slotN(c);
            const float sqr = nr[Cfg::NR_SQ / 4 + r];
            const float bkr = BETA[r] * nr[Cfg::NR_RK / 4 + r];
            const float4 rks = *reinterpret_cast<const float4*>(nr + Cfg::NR_RK / 4 + 4 * g4);
            const float rk4[4] = {rks.x, rks.y, rks.z, rks.w};
            f32x4 pv;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) pv[pp] = (4 * g4 + pp <= r) ? sqr * accP[pp] : 0.f;
            st_frag(P + r * PK + 4 * g4, E::make(pv));
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const int s = 4 * g4 + pp;
                AT[s * PA + r] = (r > s) ? bkr * rk4[pp] * accA[pp] : 0.f;  // AT[s][r] = A[r][s]
            }
            if (g4 == 0) {
                slotN(c)[Cfg::NR_BK / 4 + r] = bkr;
                slotN(c)[Cfg::NR_B2 / 4 + r] = bkr * nr[Cfg::NR_RK / 4 + r];
            }
        } else {
            if constexpr (!NOOUT) {
                f32x4 pv;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) pv[pp] = (4 * g4 + pp <= r) ? p.scale * accP[pp] : 0.f;  // scale P
                st_frag(P + r * PK + 4 * g4, E::make(pv));
            }
            const float br = BETA[r];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const int s = 4 * g4 + pp;
                AT[s * PA + r] = (r > s) ? br * accA[pp] : 0.f;  // AT[s][r] = A[r][s]
            }
        }
    };

    // ------------------------------------------------------------ row norms (fused)
    // Inverse L2 norms of the 16 raw q and k rows of chunk c (L2Norm of the
    // query and key, "Understanding Kimi K3's attention", symbol table), from
    // the raw tile while it is parked: the diagonals of q q^T and k k^T on
    // MFMA (bf16 products exact, fp32 sums).  The zero vector gets factor 0.
    // Stored for the Gram, solve and consumer waves of that chunk: r_k, |k|
    // and scale r_q.
    auto row_norms = [&](int c) {
        const char* b = raw_slot(c);
        const bf16_t* Qr = reinterpret_cast<const bf16_t*>(b + Cfg::R_Q);
        const bf16_t* Kr = reinterpret_cast<const bf16_t*>(b + Cfg::R_K);
        f32x4 aq = zero4(), ak = zero4();
#pragma unroll
        for (int kb = 0; kb < NCB; kb += 2) {
            const int c0 = 16 * kb + 4 * g4;
            const Frag q0 = ld_frag(Qr + l16 * PD + c0), q1 = ld_frag(Qr + l16 * PD + c0 + 16);
            const Frag k0 = ld_frag(Kr + l16 * PD + c0), k1 = ld_frag(Kr + l16 * PD + c0 + 16);
            mma32(aq, q0, q1, q0, q1);
            mma32(ak, k0, k1, k0, k1);
        }
        // acc[pp] = G[4 g4 + pp][l16]: the diagonal entry of row l16 is in
        // the lane with g4 = l16 / 4, register l16 % 4
        const int pd = l16 & 3;
        const float sq = pd == 0 ? aq[0] : pd == 1 ? aq[1] : pd == 2 ? aq[2] : aq[3];
        const float sk = pd == 0 ? ak[0] : pd == 1 ? ak[1] : pd == 2 ? ak[2] : ak[3];
        if ((l16 >> 2) == g4) {
            float* nr = slotN(c);
            const float rk = sk > 0.f ? __builtin_amdgcn_rsqf(sk) : 0.f;
            nr[Cfg::NR_RK / 4 + l16] = rk;
            nr[Cfg::NR_NK / 4 + l16] = sk * rk;  // |k|, 0 for the zero vector
            nr[Cfg::NR_SQ / 4 + l16] = sq > 0.f ? p.scale * __builtin_amdgcn_rsqf(sq) : 0.f;
        }
    };

    // ------------------------------------------------------------ solve
    auto solve = [&](int c) {
        // Column sweep of the unit lower-triangular system: once T[s][col] is
        // final, remove its contribution A[r][s] T[s][col] from every later row
        // r (all independent).  Lane (col, q) = 4 col + q holds rows
        // 4q .. 4q + 3 of column col; at step s the lane of the quad owning row
        // s hands T[s][col] to the other three (a DPP quad broadcast) and every
        // lane updates its four rows (A^T is stored with zeros at r <= s, so
        // rows that are already final subtract exactly 0).  Each element sees
        // the same multiply-adds in the same order as a one-lane-per-column
        // sweep, with a quarter of the instructions.  The lanes of one quad
        // row read the same 16 bytes of A^T row s (broadcast), requested W
        // steps ahead through one VGPR base and immediate offsets.
        const int col = lane >> 2, q = lane & 3;
        const float4* AT4 = reinterpret_cast<const float4*>(slotA(c)) + opaque_zero() + q;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (4 * q + j == col) ? 1.f : 0.f;
        constexpr int W = 4;
        f32x4 row[15];  // A[4q .. 4q + 3][s], named registers
#pragma unroll
        for (int st = 0; st < W; ++st) row[st] = *reinterpret_cast<const f32x4*>(AT4 + st * (PA / 4));
        static_for<0, 15>([&](auto sc) __attribute__((always_inline)) {
            constexpr int st = decltype(sc)::value;
            if constexpr (st + W < 15) row[st + W] = *reinterpret_cast<const f32x4*>(AT4 + (st + W) * (PA / 4));
            asm volatile("" ::"v"(row[st]));  // the whole quad: no narrowing into 4-byte reads
            const float ts = quad_bcast<st / 4>(x[st % 4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] -= row[st][j] * ts;
        });
        if constexpr (FUSED) {
            // Diag(r_k) T Diag(1 / r_k): row factor r_k of the row, column
            // factor |k| of the column (a zero key row or column gets 0 off
            // the diagonal; its Z' row is 0 too); the unit diagonal is kept.
            const float4 rk = *reinterpret_cast<const float4*>(slotN(c) + Cfg::NR_RK / 4 + 4 * q);
            const float nk = slotN(c)[Cfg::NR_NK / 4 + col];
            const float rr[4] = {rk.x, rk.y, rk.z, rk.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * q + j != col) x[j] *= rr[j] * nk;
        }
        uint16_t* tq = reinterpret_cast<uint16_t*>(slotT(c)) + (4 * q) * PK + col;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const uint32_t pr = pack_bf16x2(x[j], x[j + 1]);
            tq[j * PK] = (uint16_t)(pr & 0xffffu);
            tq[(j + 1) * PK] = (uint16_t)(pr >> 16);
        }
    };

    // ------------------------------------------------------------ consumers
    const uint32_t o_voff = (uint32_t)l16 * (uint32_t)(H * D) * 2u + (uint32_t)(col_base + 4 * TPW * g4) * 2u;
    // Output gate (GATE), applied one iteration after the consumers park
    // chunk c's o tiles (the gate factors are in LDS by then too, brought by
    // the stage-A waves): the consumers, the critical chain, only park their
    // tiles; the Gram wave (part 0) and the solve wave (part 1), which have
    // the slack, each form every row's sum of squares and scale and store
    // half of the tiles.
    auto finish_gate = [&](int c, auto partc) {
        constexpr int part = decltype(partc)::value;
        // y = Sigmoid(gate) * o / sqrt(mean over the head's d_v of o^2 + eps)
        // * weight ("Understanding Kimi K3's attention", output equation), o
        // as rounded to the output dtype (the value a separate pass would read).
        // Lane (g4, l16) takes token row l16 and, from each consumer wave's
        // tile, the piece that wave's lane `lane` parked: columns
        // 32 w2 + 8 g4 .. + 7.  The row's sum of squares adds the lane's 32
        // columns, then the 4 lanes of the row; the lane then stores its
        // pieces of tiles w2 = part NCW/2 .. part NCW/2 + NCW/2 - 1.
        const int nv = rows_valid(c);
        const char* ost = smem + Cfg::G_OST + (size_t)(c & 1) * NCW * 1024 + lane * 16;
        u32x4 ov[NCW];
        float ss = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NCW; ++w2) {
            ov[w2] = *reinterpret_cast<const u32x4*>(ost + w2 * 1024);
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) ss = dot2_bf16(ov[w2][wd], ov[w2][wd], ss);
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float rinv = __builtin_amdgcn_rsqf(ss * (1.f / D) + p.gate_eps);
        const float* gf = reinterpret_cast<const float*>(smem + Cfg::G_GT + (size_t)(c & 1) * Cfg::SGT) + l16 * Cfg::PGT;
        const auto ro = rsrc_chunk(chunk_ptr(go, 2, c), ((nv - 1) * H * D + D) * 2);
#pragma unroll
        for (int w2 = part * (NCW / 2); w2 < (part + 1) * (NCW / 2); ++w2) {
            const int col = w2 * TPW * 16 + 4 * TPW * g4;  // first of the piece's columns in the slab
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(gf + col), f1 = *reinterpret_cast<const f32x4*>(gf + col + 4);
            const float fv[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
            u32x4 yv;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const float lo = __uint_as_float(ov[w2][wd] << 16), hi = __uint_as_float(ov[w2][wd] & 0xffff0000u);
                yv[wd] = pack_bf16x2(lo * rinv * fv[2 * wd], hi * rinv * fv[2 * wd + 1]);
            }
            // one 16-byte store; rows past the chunk's last row in the sequence are dropped
            __builtin_amdgcn_raw_buffer_store_b128(
                yv, ro, (uint32_t)l16 * (uint32_t)(H * D) * 2u + (uint32_t)(z * DVW + col) * 2u, 0, 0);
        }
    };
    auto consume = [&](int c, f32x4 (&Sm)[TPW][NCB]) {
        [[maybe_unused]] const int nv = rows_valid(c);
        char* s4 = slot4(c);
        const bf16_t* QB = reinterpret_cast<const bf16_t*>(s4 + Cfg::S4_QB);
        const bf16_t* KB = reinterpret_cast<const bf16_t*>(s4 + Cfg::S4_KB);
        const bf16_t* KT = reinterpret_cast<const bf16_t*>(s4 + Cfg::S4_KT);
        const float* GAM = reinterpret_cast<const float*>(s4 + Cfg::S4_GAM);
        const float* BETA = reinterpret_cast<const float*>(s4 + Cfg::S4_BETA);
        const bf16_t* P = reinterpret_cast<const bf16_t*>(slotP(c));
        const bf16_t* T = reinterpret_cast<const bf16_t*>(slotT(c));
        const int sv0 = (col_base - z * DVW) + vcol(0, l16);

        // Every LDS operand of this step is requested up front, so their
        // latency overlaps the state conversion and the X / QS products.
        // (CKB: the backward's run needs only the states, not o: no Q~ S, P U)
        Frag kf[NCB], qf[NCB];
#pragma unroll
        for (int kb = 0; kb < NCB; ++kb) {
            kf[kb] = ld_frag(KB + l16 * PD + 16 * kb + 4 * g4);
            if constexpr (!NOOUT) qf[kb] = ld_frag(QB + l16 * PD + 16 * kb + 4 * g4);
        }
        const Frag Tf = ld_frag(T + l16 * PK + 4 * g4);
        Frag Pf;
        if constexpr (!NOOUT) Pf = ld_frag(P + l16 * PK + 4 * g4);
        // Row factors of Z = (beta v) - (beta) X; fused, of Diag(r_k) Z =
        // (beta r_k) v - (beta r_k^2) X_raw (from the Gram wave, which also
        // parks beta r_k v for the slabs that take V in fp32), and O = scale
        // r_q (Q_raw S) + P' U'.
        const float4 b4 = *reinterpret_cast<const float4*>((FUSED ? slotN(c) + Cfg::NR_BK / 4 : BETA) + 4 * g4);
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
        float bx[4] = {b4.x, b4.y, b4.z, b4.w};
        if constexpr (FUSED) {
            const float4 b24 = *reinterpret_cast<const float4*>(slotN(c) + Cfg::NR_B2 / 4 + 4 * g4);
            bx[0] = b24.x;
            bx[1] = b24.y;
            bx[2] = b24.z;
            bx[3] = b24.w;
        }
        float vv[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const int e = sv0 + (4 * g4 + pp) * Cfg::PV + 4 * t;
                if constexpr (Cfg::VF)
                    vv[t][pp] = reinterpret_cast<const float*>(slotV(c))[e];  // beta v, parked
                else
                    vv[t][pp] = w_v_zero ? 0.f : bb[pp] * bf16_to_f32(reinterpret_cast<const uint16_t*>(slotV(c))[e]);
            }
        Frag ktf[NCB];
        float4 gm[NCB];
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct) {
            ktf[ct] = ld_frag(KT + (16 * ct + l16) * PK + 4 * g4);
            gm[ct] = *reinterpret_cast<const float4*>(GAM + 16 * ct + 4 * g4);
        }

        Frag Sop[TPW][NCB];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int ct = 0; ct < NCB; ++ct) Sop[t][ct] = E::make(Sm[t][ct]);
        // X = Kt S as is (its rows feed U); Qt S transposed, by swapping the
        // operands, so that the output ends up token-major in the lanes.
        f32x4 X[TPW], QS[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            X[t] = zero4();
            QS[t] = zero4();
        }
#pragma unroll
        for (int kb = 0; kb < NCB; kb += 2)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                mma32(X[t], kf[kb], kf[kb + 1], Sop[t][kb], Sop[t][kb + 1]);
                if constexpr (!NOOUT) mma32(QS[t], Sop[t][kb], Sop[t][kb + 1], qf[kb], qf[kb + 1]);
            }
        // U = T diag(beta) (V - X) = T (beta V - diag(beta) X), all tiles side by side.
        Frag Uf[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 Z;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) Z[pp] = fmaf(-bx[pp], X[t][pp], vv[t][pp]);
            f32x4 U = zero4();
            mma16(U, Tf, E::make(Z));
            Uf[t] = E::make(U);
        }
        // The state update (the chain into the next step) is issued before the
        // output path, whose work then fills the products' latency.
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
            for (int t = 0; t < TPW; ++t) mma16(Sm[t][ct], ktf[ct], Uf[t]);  // S + KL^T U
        // O^T = (Qt S)^T + U^T P^T: lane (g4, l16) holds token l16 at the
        // value columns vcol(t, 4 g4 + pp) = 4 TPW g4 + 4 t + pp, adjacent.
        [[maybe_unused]] uint32_t ov[TPW][2];
        if constexpr (!NOOUT) {
            const float o_scale = FUSED ? slotN(c)[Cfg::NR_SQ / 4 + l16] : p.scale;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                // (P U)^T in its own accumulator, added to the 32-deep QS
                // product by VALU (kda_device.h: no SrcC chain across shapes)
                f32x4 PU = zero4();
                mma16(PU, Uf[t], Pf);
                // O = scale Qt S + (scale P) U (P is stored scaled)
                ov[t][0] = pack_bf16x2(fmaf(o_scale, QS[t][0], PU[0]), fmaf(o_scale, QS[t][1], PU[1]));
                ov[t][1] = pack_bf16x2(fmaf(o_scale, QS[t][2], PU[2]), fmaf(o_scale, QS[t][3], PU[3]));
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                Sm[t][ct][0] *= gm[ct].x;  // then the chunk decay, per key channel
                Sm[t][ct][1] *= gm[ct].y;
                Sm[t][ct][2] *= gm[ct].z;
                Sm[t][ct][3] *= gm[ct].w;
            }
        // One store per lane; the range ends with the chunk's last row in the
        // sequence, and buffer stores out of range are dropped.
        if constexpr (!NOOUT && !GATE) {
            const auto ro = rsrc_chunk(chunk_ptr(go, 2, c), ((nv - 1) * H * D + D) * 2);
            const uint32_t oo = o_voff;
            if constexpr (TPW == 2)
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{ov[0][0], ov[0][1], ov[1][0], ov[1][1]}, ro, oo, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{ov[0][0], ov[0][1]}, ro, oo, 0, 0);
        }
        if constexpr (GATE) {
            // the o tile, parked for the gated store of the Gram and solve
            // waves in the next iteration
            const u32x4 o4 = {ov[0][0], ov[0][1], ov[1][0], ov[1][1]};
            *reinterpret_cast<u32x4*>(smem + Cfg::G_OST + ((c & 1) * NCW + w) * 1024 + lane * 16) = o4;
        }
    };

    // ------------------------------------------------------------ pipeline
    // Iteration j works on: stage A chunk j, Gram chunk j-1, solve chunk j-2,
    // consumers chunk j-3, and ends with the workgroup barrier.  Each role
    // runs its own copy of the loop (the role is uniform per wave and every
    // copy passes the same number of barriers), so the register live ranges
    // of different roles never overlap.  The stage-A and Gram loops are
    // unrolled twice so their two prefetch register sets have fixed names.
    if (nch > 0) {
        // (GATE: one more iteration, for the gated store of the last chunk)
        const int iters = nch + 3 + (GATE ? 1 : 0);
        if (is_stageA) {
            // Iteration j requests chunk j + 3, works on chunk j (already in
            // registers), parks chunk j + 2 (requested one iteration earlier)
            // and reads back its part of chunk j + 1 (parked one iteration
            // earlier by all stage-A waves) just before the barrier, so the
            // LDS latency of that read overlaps the barrier wait.  Chunk c
            // uses raw slot c & 1 from its parking (iteration c - 2) to its
            // read (iteration c - 1); chunk c + 2 is parked after the barrier
            // that ends iteration c - 1.
            LoadSet<LPW> rawA, rawB;
            RawSet<IPW> cur;
            [[maybe_unused]] GtSet gtA = {}, gtB = {};
            load_raw(0, rawA);
            load_raw(1, rawB);
            park_raw(0, rawA);
            __syncthreads();  // prologue 1: chunk 0 parked
            load_raw(2, rawA);
            park_raw(1, rawB);
            fetch_raw(0, cur);
            __syncthreads();  // prologue 2: chunk 1 parked, chunk 0 read
            // Unrolled four times, so that the 4-deep slot of the chunk that
            // stage A works on (c & 3 = u) is an immediate offset.  Even steps
            // load into set B and park set A, odd steps the other way round.
            auto step = [&](int jj, auto uc, LoadSet<LPW>& into, const LoadSet<LPW>& from, GtSet& gt_into,
                            const GtSet& gt_from) __attribute__((always_inline)) {
                load_raw(jj + 3, into);
                if constexpr (GATE) gt_into = load_gt(jj - 2);
                if (jj < nch) stage_a(jj, cur, decltype(uc)::value);
                park_raw(jj + 2, from);
                if constexpr (GATE) park_gt(jj - 3, gt_from);
                fetch_raw(jj + 1, cur);
                __syncthreads();
            };
            for (int j = 0; j < iters; j += 4) {
                step(j, std::integral_constant<int, 0>{}, rawB, rawA, gtB, gtA);
                if (j + 1 < iters) step(j + 1, std::integral_constant<int, 1>{}, rawA, rawB, gtA, gtB);
                if (j + 2 < iters) step(j + 2, std::integral_constant<int, 2>{}, rawB, rawA, gtB, gtA);
                if (j + 3 < iters) step(j + 3, std::integral_constant<int, 3>{}, rawA, rawB, gtA, gtB);
            }
        } else if (w == Cfg::W_GRAM) {
            // This wave also moves V: chunk c is loaded into registers in
            // iteration c + 1, copied verbatim into V slot (c & 1) in
            // iteration c + 2 and read by the consumers in iteration c + 3;
            // the slot is next written (chunk c + 2) in iteration c + 4.
            // Only a memory instruction touches the loaded registers, so the
            // copy cannot be hoisted above the barrier that follows the load.
            VRegs<VChunk> va, vb;
            __syncthreads();  // the two prologue barriers of the stage-A waves
            if constexpr (FUSED) row_norms(0);  // chunk 0 parked
            __syncthreads();
            // (GATE: it also finishes chunk j - 4, whose o tiles the consumers
            // parked in iteration j - 1, with the gated store of half the
            // tiles; the solve wave stores the other half.)
            for (int j = 0; j < iters; j += 2) {
                load_v(j - 1, vb);
                if (j - 2 >= 0 && j - 2 < nch) store_v(j - 2, va);
                if (j - 1 >= 0 && j - 1 < nch) gram(j - 1);
                if constexpr (FUSED) {
                    if (j + 1 < nch) row_norms(j + 1);  // parked in iteration j - 1, read by stage A at the end of j
                }
                if constexpr (GATE) {
                    if (j - 4 >= 0 && j - 4 < nch) finish_gate(j - 4, std::integral_constant<int, 0>{});
                }
                __syncthreads();
                if (j + 1 < iters) {
                    load_v(j, va);
                    if (j - 1 >= 0 && j - 1 < nch) store_v(j - 1, vb);
                    if (j < nch) gram(j);
                    if constexpr (FUSED) {
                        if (j + 2 < nch) row_norms(j + 2);
                    }
                    if constexpr (GATE) {
                        if (j - 3 >= 0 && j - 3 < nch) finish_gate(j - 3, std::integral_constant<int, 0>{});
                    }
                    __syncthreads();
                }
            }
        } else if (w == Cfg::W_SOLVE) {
            __syncthreads();
            __syncthreads();
            for (int j = 0; j < iters; ++j) {
                if (j - 2 >= 0 && j - 2 < nch) solve(j - 2);
                if constexpr (GATE) {
                    if (j - 4 >= 0 && j - 4 < nch) finish_gate(j - 4, std::integral_constant<int, 1>{});
                }
                __syncthreads();
            }
        } else {
            // Consumer state: Sm[t][ct][pp] = S[16 ct + 4 g4 + pp][col_base + vcol(t, l16)]
            // The state slice moves through buffer accesses: one per-lane
            // offset (row 4 g4, the lane's column), rows as wave-uniform offsets.
            // Without an initial state the range is empty and the loads read 0.
            const uint32_t s_voff = (uint32_t)(4 * g4 * D + col_base + vcol(0, l16)) * 4u;
            f32x4 Sm[TPW][NCB];
            if (w_identity) {
                // segment map M: the run from the identity (row == column)
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp)
                            Sm[t][ct][pp] = (16 * ct + 4 * g4 + pp == col_base + vcol(t, l16)) ? 1.f : 0.f;
            } else {
                const auto rs = wk.s_in ? buffer_rsrc(wk.s_in, D * D * 4) : buffer_rsrc(p.g, 0);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp)
                            Sm[t][ct][pp] = __builtin_bit_cast(
                                float, __builtin_amdgcn_raw_buffer_load_b32(rs, s_voff + 16 * t, (16 * ct + pp) * D * 4, 0));
            }
            // State checkpoints: after chunk c when (c + 1) C tokens of the
            // sequence are done and that count is a multiple of the interval.
            // (uniform values kept in scalar registers: the consumer is at its
            // vector-register limit in the 14-wave workgroup)
            const int ck0 = p.ckpt ? __builtin_amdgcn_readfirstlane((int)ckpt_first_slot(p, n, lane)) : 0;
            const int ck_chunks = p.ckpt ? p.ckpt_interval / C : 1;
            // the next checkpoint's chunk and how many came before it (no
            // division per chunk: (c + 1) % ck_chunks == 0 exactly when c
            // reaches ck_next, the chunks being visited in order)
            int ck_next = ck_chunks - 1, ck_k = 0;
            if constexpr (GATE) {
                // the slab's RMSNorm weights, read before the first gated store
                // (two barriers away)
                if (w == 0)
                    for (int i = lane; i < DVW; i += 64)
                        reinterpret_cast<float*>(smem + Cfg::G_W)[i] = p.gate_weight[z * DVW + i];
            }
            __syncthreads();
            __syncthreads();
            for (int j = 0; j < iters; ++j) {
                if (j - 3 >= 0 && j - 3 < nch) {
                    consume(j - 3, Sm);
                    const int c = j - 3;
                    if (p.ckpt && c == ck_next) {
                        const int64_t slot = (int64_t)ck0 + ck_k;
                        ck_next += ck_chunks;
                        ++ck_k;
                        if ((c + 1) * C <= (int)ntok && slot < p.ckpt_cap) {
                            if constexpr (CKB) {
                                // rows 16ct + 4g4 .. + 3 of a column: one 8-byte store
                                const auto rc = buffer_rsrc(reinterpret_cast<uint16_t*>(p.ckpt) + (slot * H + h) * D * D,
                                                            D * D * 2);
                                const uint32_t b_voff = (uint32_t)(g4 * D + col_base + vcol(0, l16)) * 8u;
#pragma unroll
                                for (int t = 0; t < TPW; ++t)
#pragma unroll
                                    for (int ct = 0; ct < NCB; ++ct) {
                                        u32x2 pk;
                                        pk[0] = pack_bf16x2(Sm[t][ct][0], Sm[t][ct][1]);
                                        pk[1] = pack_bf16x2(Sm[t][ct][2], Sm[t][ct][3]);
                                        __builtin_amdgcn_raw_buffer_store_b64(pk, rc, b_voff + 32 * t, ct * 4 * D * 8, 0);
                                    }
                            } else {
                                // one per-lane offset; rows as wave-uniform offsets
                                const auto rc = buffer_rsrc(p.ckpt + (slot * H + h) * D * D, D * D * 4);
#pragma unroll
                                for (int t = 0; t < TPW; ++t)
#pragma unroll
                                    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                                        for (int pp = 0; pp < 4; ++pp)
                                            __builtin_amdgcn_raw_buffer_store_b32(
                                                __float_as_uint(Sm[t][ct][pp]), rc, s_voff + 16 * t,
                                                (16 * ct + pp) * D * 4, 0);
                            }
                        }
                    }
                }
                __syncthreads();
            }
            if (s_dst) {
                const auto rs = buffer_rsrc(s_dst, D * D * 4);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                        for (int pp = 0; pp < 4; ++pp)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sm[t][ct][pp]), rs,
                                                                  s_voff + 16 * t, (16 * ct + pp) * D * 4, 0);
            }
        }
    } else if (is_cons && s_dst) {
        // empty sequence: the final state is the initial state.  Buffer
        // accesses, as everywhere in this kernel: a generic (flat) access
        // would make the compiler's waits on every wave's loads in flight
        // collapse to full drains.
        const auto ro = buffer_rsrc(s_dst, D * D * 4);
        const auto ri = wk.s_in ? buffer_rsrc(wk.s_in, D * D * 4) : buffer_rsrc(p.g, 0);
        for (int t = 0; t < TPW; ++t)
            for (int ct = 0; ct < NCB; ++ct)
                for (int pp = 0; pp < 4; ++pp) {
                    const int row = 16 * ct + 4 * g4 + pp, col = col_base + 16 * t + l16;
                    const int off = (row * D + col) * 4;
                    const float x = w_identity ? (row == col ? 1.f : 0.f)
                                               : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, 0));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), ro, off, 0, 0);
                }
    }
}

template <int NCW, int TPW, int NSA, bool FUSED, bool CKB, bool SEG, bool GATE>
__global__ __launch_bounds__(64 * (NCW + 2 + NSA)) void kda_prefill_ws_kernel(PrefillParams p) {
    typedef WsCfg<NCW, TPW, NSA, FUSED, GATE> Cfg;
    // (the map-pair kernel also runs segment 0 with the whole-head layout)
    typedef WsCfg<4, 2, 8, FUSED, false> RunCfg;
    constexpr size_t kLds = NCW == 8 && RunCfg::LDS > Cfg::LDS ? RunCfg::LDS : Cfg::LDS;
    __shared__ __align__(16) char smem[kLds];
    // XCD-aware block order (ws_resolve); padding blocks exit at once.  The
    // work description is uniform: pinned to scalar registers (integer
    // divisions by run-time values leave their results in vector registers).
    constexpr bool PAIR = NCW == 8;  // the segment scan's map-pair kernel (phase 1)
    static_assert(!PAIR || SEG, "map pairs belong to the segment scan");
    WsWork wk;
    if (!ws_resolve<Cfg::D, SEG, PAIR>(p, blockIdx.x, wk)) return;
    wk.t_begin = uniform_i64(wk.t_begin);
    wk.t_end = uniform_i64(wk.t_end);
    wk.n = __builtin_amdgcn_readfirstlane(wk.n);
    wk.h = __builtin_amdgcn_readfirstlane(wk.h);
    wk.z = __builtin_amdgcn_readfirstlane(wk.z);
    wk.s_in = reinterpret_cast<const float*>(uniform_i64(reinterpret_cast<int64_t>(wk.s_in)));
    wk.s_out = reinterpret_cast<float*>(uniform_i64(reinterpret_cast<int64_t>(wk.s_out)));
    wk.s_out_m = reinterpret_cast<float*>(uniform_i64(reinterpret_cast<int64_t>(wk.s_out_m)));
    if constexpr (PAIR) {
        if (wk.s_out_m)
            ws_body<NCW, TPW, NSA, FUSED, CKB, SEG, true, false>(p, wk, smem);
        else  // segment 0 with its outputs, whole heads, 14 waves as the pair
            ws_body<4, 2, 8, FUSED, CKB, SEG, false, false>(p, wk, smem);
    } else
        ws_body<NCW, TPW, NSA, FUSED, CKB, SEG, false, GATE>(p, wk, smem);
}

template <int NCW, int TPW, int NSA, bool FUSED = false, bool CKB = false, bool SEG = false, bool GATE = false>
hipError_t launch_prefill_ws(const PrefillParams& p, hipStream_t s) {
    if (!SEG && p.seg_phase != 0) return hipErrorInvalidValue;
    if (SEG && p.seg_phase != (NCW == 8 ? 1 : 3)) return hipErrorInvalidValue;  // pairs: phase 1, runs: phase 3
    const int64_t blocks = ws_grid_blocks(p);  // whole groups of 8 items
    hipLaunchKernelGGL((kda_prefill_ws_kernel<NCW, TPW, NSA, FUSED, CKB, SEG, GATE>), dim3((unsigned)blocks),
                       dim3(64 * (NCW + 2 + NSA)), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
