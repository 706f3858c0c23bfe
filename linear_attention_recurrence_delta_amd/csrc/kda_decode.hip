// kda_decode.hip -- one KDA decode step per (sequence, head), state in place.
//
// Per (n, h), with S the d_k x d_v fp32 state (rows = key channels):
//   D = Diag(exp g);  a = (D S)^T k;  b = (D S)^T q;  kappa = k . q
//   u = beta (v - a);  S <- D S + k u^T;  o = scale (b + kappa u)
// The last line is S_new^T q expanded, so the state is read once and written
// once.  This is the recurrence of "Understanding Kimi K3's attention"
// (state-update and readout equations) in the fade / predict / correct order
// of "Hybrid Attention" (section "KDA: don't write the same information
// twice"), with the readout after the write ("KDA: the memory matrix").
//
// Work split: one workgroup per (n, h).  Thread (rg, cg) owns the 4 value
// columns 4cg..4cg+3 (16-byte coalesced row segments) of rows rg, rg + RG, ...
// (four rows per thread where the state allows).
// Column partial sums over rows are combined through LDS in a fixed order,
// so results are bitwise reproducible.  State traffic uses non-temporal
// loads and stores: each state is touched once per step.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int D>
struct DecodeCfg {
    // Four 16-byte row segments per thread (1024 threads for a 128 x 128
    // state): measured on MI355X, more threads per state keep more of the
    // read stream in flight while other workgroups write (256 threads:
    // 5.2 TB/s, 512: 5.3, 1024: 5.7 at 256 x 96 states).
    static constexpr int NT = D * D / 16 < 64 ? 64 : (D * D / 16 > 1024 ? 1024 : D * D / 16);
    static constexpr int CG = D / 4;                 // float4 column groups
    static constexpr int RG = NT / CG;               // row groups
    static constexpr int RPT = D / RG;               // rows per thread
    static_assert(RG * CG == NT && RPT * RG == D, "decode tiling");
};

template <typename TIn, int D>
__global__ __launch_bounds__(DecodeCfg<D>::NT) void kda_decode_kernel(DecodeParams p) {
    typedef DecodeCfg<D> Cfg;
    constexpr int NT = Cfg::NT, CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT;
    __shared__ float sK[D], sQ[D], sAl[D];
    __shared__ __align__(16) float sPa[RG][D];
    __shared__ __align__(16) float sPb[RG][D];
    __shared__ float sKap[RG];

    const int64_t unit = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    float* S = p.S + unit * (int64_t)D * D;
    const TIn* q = static_cast<const TIn*>(p.q) + unit * D;
    const TIn* k = static_cast<const TIn*>(p.k) + unit * D;
    const TIn* v = static_cast<const TIn*>(p.v) + unit * D;
    const float* g = p.g + unit * D;

    // Issue the state loads first: they are the whole cost of the step.
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (int64_t)r * D + 4 * cg));
    }
    for (int i = tid; i < D; i += NT) {
        sK[i] = Elem<TIn>::load(k + i);
        sQ[i] = Elem<TIn>::load(q + i);
        sAl[i] = __expf(g[i]);
    }
    __syncthreads();

    f32x4 a = zero4(), b = zero4();
    float kap = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        const float al = sAl[r], kr = sK[r], qr = sQ[r];
        s[m] *= al;  // fade: Diag(alpha) scales key-channel row r
        a += s[m] * kr;
        b += s[m] * qr;
        kap += kr * qr;
    }
    *reinterpret_cast<f32x4*>(&sPa[rg][4 * cg]) = a;
    *reinterpret_cast<f32x4*>(&sPb[rg][4 * cg]) = b;
    if (cg == 0) sKap[rg] = kap;
    __syncthreads();

    f32x4 A = zero4(), B = zero4();
    float kappa = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        A += *reinterpret_cast<const f32x4*>(&sPa[j][4 * cg]);
        B += *reinterpret_cast<const f32x4*>(&sPb[j][4 * cg]);
        kappa += sKap[j];
    }
    const float bet = p.beta[unit];
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bet * (Elem<TIn>::load(v + 4 * cg + c) - A[c]);

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        const f32x4 out = s[m] + sK[r] * u;  // correct: S += k u^T
        __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(S + (int64_t)r * D + 4 * cg));
    }
    if (rg == 0) {
        TIn* o = static_cast<TIn*>(p.o) + unit * D + 4 * cg;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = Elem<TIn>::from_f32(p.scale * (B[c] + kappa * u[c]));
    }
}

template <typename TIn>
static hipError_t launch_decode(int D, const DecodeParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.units));
    switch (D) {
#define KDA_DECODE_CASE(DD)                                                                   \
    case DD:                                                                                  \
        hipLaunchKernelGGL((kda_decode_kernel<TIn, DD>), grid, dim3(DecodeCfg<DD>::NT), 0, s, p); \
        return hipGetLastError();
        KDA_DECODE_CASE(16)
        KDA_DECODE_CASE(32)
        KDA_DECODE_CASE(64)
        KDA_DECODE_CASE(128)
#undef KDA_DECODE_CASE
        default:
            return hipErrorInvalidValue;
    }
}

bool decode_d_supported(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }
hipError_t launch_decode_bf16(int D, const DecodeParams& p, hipStream_t s) { return launch_decode<bf16_t>(D, p, s); }
hipError_t launch_decode_f32(int D, const DecodeParams& p, hipStream_t s) { return launch_decode<float>(D, p, s); }

}  // namespace kda
