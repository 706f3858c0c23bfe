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
// Work split: thread (rg, cg) of a workgroup owns the 4 value columns
// 4cg..4cg+3 (16-byte coalesced row segments) of rows rg, rg + RG, ... (four
// rows per thread where the state allows).  Column partial sums over rows go
// through LDS and are summed in a fixed order (row group 0 first), so results
// are bitwise reproducible and independent of the grid size.
//
// Persistent, double-buffered: a fixed grid of workgroups walks the
// (sequence, head) units with stride gridDim.x, and each workgroup issues the
// loads of its next unit (state, q, k, v, g, beta) before it reduces, updates
// and writes back the current one, so one unit's reads are in flight during
// another's arithmetic and stores.  State traffic is non-temporal (each state
// is touched once per step) and goes through buffer loads and stores whose
// row offsets are scalar constants.  Measured on MI355X at 256 x 96 states of
// 128 x 128: one workgroup per unit 5.8-5.9 TB/s, this scheme 6.4-6.5 TB/s.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kDecodeWavesPerCU = 64;  // grid = CUs x this / waves per workgroup

template <int D>
struct DecodeCfg {
    static constexpr int NT = D * D / 16 < 64 ? 64 : (D * D / 16 > 1024 ? 1024 : D * D / 16);
    static constexpr int CG = D / 4;                 // float4 column groups
    static constexpr int RG = NT / CG;               // row groups
    static constexpr int RPT = D / RG;               // rows per thread
    static_assert(RG * CG == NT && RPT * RG == D, "decode tiling");
    static_assert(NT >= 2 * D, "one thread per column sum and per q/k/v/g element");
};

template <typename TIn> struct DecodeElem;
template <> struct DecodeElem<bf16_t> {
    static constexpr int bytes = 2;
    __device__ __forceinline__ static float load(__amdgpu_buffer_rsrc_t r, int off) {
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
    }
};
template <> struct DecodeElem<float> {
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float load(__amdgpu_buffer_rsrc_t r, int off) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
};

// The loads of one unit, held in registers until its turn.
template <int RPT>
struct DecodeUnit {
    f32x4 s[RPT];
    float k, q, v, g, beta;
};

constexpr int kNonTemporal = 2;  // buffer instruction cache policy: nt

template <typename TIn, int D>
__global__ __launch_bounds__(DecodeCfg<D>::NT) void kda_decode_kernel(DecodeParams p) {
    typedef DecodeCfg<D> Cfg;
    typedef DecodeElem<TIn> E;
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    constexpr int NT = Cfg::NT, CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT;
    constexpr int ROW_STRIDE = RG * D * 4;  // bytes between a thread's rows

    // Vectors of two consecutive units (a fast thread may write unit i+1's
    // while a slow one still reads unit i's).  The partial sums need one set:
    // three barriers per unit separate their writes and reads.
    __shared__ float sK[2][D], sQ[2][D], sV[2][D], sAl[2][D];
    __shared__ f32x4 sPa[RG][CG], sPb[RG][CG];
    __shared__ float sKap[RG];
    __shared__ __align__(16) float sAB[2 * D + 4];  // column sums of a, b; kappa

    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int voff = (rg * D + 4 * cg) * 4;
    const int eoff = tid < D ? tid * E::bytes : 0x20000000;  // past every range: loads 0
    const int64_t units = p.units;
    const int64_t G = gridDim.x;

    // Issue every load of one unit.  A unit past the end gets empty ranges:
    // its loads return zeros without touching memory.
    auto fetch = [&](int64_t unit, DecodeUnit<RPT>& b) {
        const bool live = unit < units;
        const int64_t uu = live ? unit : 0;
        const auto rs = buffer_rsrc(p.S + uu * D * D, live ? D * D * 4 : 0);
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            b.s[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, m * ROW_STRIDE,
                                                                                     kNonTemporal));
        const int vb = live ? D * E::bytes : 0;
        b.k = E::load(buffer_rsrc(static_cast<const TIn*>(p.k) + uu * D, vb), eoff);
        b.q = E::load(buffer_rsrc(static_cast<const TIn*>(p.q) + uu * D, vb), eoff);
        b.v = E::load(buffer_rsrc(static_cast<const TIn*>(p.v) + uu * D, vb), eoff);
        b.g = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.g + uu * D, live ? D * 4 : 0),
                                                                   tid < D ? 4 * tid : 0x20000000, 0, 0));
        b.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.beta + uu, live ? 4 : 0), 0, 0, 0));
    };

    auto step = [&](int64_t unit, DecodeUnit<RPT>& b, int par) {
        if (tid < D) {
            sK[par][tid] = b.k;
            sQ[par][tid] = b.q;
            sV[par][tid] = b.v;
            sAl[par][tid] = __expf(b.g);
        }
        __syncthreads();
        f32x4 a = zero4(), bq = zero4();
        float kap = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + RG * m;
            const float kr = sK[par][r], qr = sQ[par][r];
            b.s[m] *= sAl[par][r];  // fade: Diag(alpha) scales key-channel row r
            a += b.s[m] * kr;
            bq += b.s[m] * qr;
            kap += kr * qr;
        }
        sPa[rg][cg] = a;
        sPb[rg][cg] = bq;
        if (cg == 0) sKap[rg] = kap;
        __syncthreads();
        // One thread per column sum (a for tid < D, b for D <= tid < 2D).
        if (tid < 2 * D) {
            const float* src = reinterpret_cast<const float*>(tid < D ? &sPa[0][0] : &sPb[0][0]);
            const int col = tid % D;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < RG; ++j) acc += src[j * D + col];
            sAB[tid] = acc;
        }
        if (tid == (2 * D) % NT) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < RG; ++j) acc += sKap[j];
            sAB[2 * D] = acc;
        }
        __syncthreads();
        const f32x4 A = *reinterpret_cast<const f32x4*>(&sAB[4 * cg]);
        const f32x4 B = *reinterpret_cast<const f32x4*>(&sAB[D + 4 * cg]);
        const float kappa = sAB[2 * D];
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = b.beta * (sV[par][4 * cg + c] - A[c]);
        const auto rs = buffer_rsrc(p.S + unit * D * D, D * D * 4);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + RG * m;
            const f32x4 out = b.s[m] + sK[par][r] * u;  // correct: S += k u^T
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, out), rs, voff, m * ROW_STRIDE,
                                                   kNonTemporal);
        }
        if (rg == 0) {
            TIn* o = static_cast<TIn*>(p.o) + unit * D + 4 * cg;
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = Elem<TIn>::from_f32(p.scale * (B[c] + kappa * u[c]));
        }
    };

    int64_t unit = blockIdx.x;
    if (unit >= units) return;
    DecodeUnit<RPT> b0, b1;
    int par = 0;
    fetch(unit, b0);
    for (;;) {
        fetch(unit + G, b1);
        step(unit, b0, par);
        par ^= 1;
        unit += G;
        if (unit >= units) break;
        fetch(unit + G, b0);
        step(unit, b1, par);
        par ^= 1;
        unit += G;
        if (unit >= units) break;
    }
}

template <typename TIn, int D>
hipError_t launch_decode_d(const DecodeParams& p, int cus, hipStream_t s) {
    constexpr int NT = DecodeCfg<D>::NT;
    int64_t blocks = (int64_t)cus * kDecodeWavesPerCU / (NT / 64);
    if (blocks > p.units) blocks = p.units;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((kda_decode_kernel<TIn, D>), dim3((unsigned)blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_decode(int D, const DecodeParams& p, int cus, hipStream_t s) {
    switch (D) {
        case 16: return launch_decode_d<TIn, 16>(p, cus, s);
        case 32: return launch_decode_d<TIn, 32>(p, cus, s);
        case 64: return launch_decode_d<TIn, 64>(p, cus, s);
        case 128: return launch_decode_d<TIn, 128>(p, cus, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_d_supported(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }
hipError_t launch_decode_bf16(int D, const DecodeParams& p, int cus, hipStream_t s) {
    return launch_decode<bf16_t>(D, p, cus, s);
}
hipError_t launch_decode_f32(int D, const DecodeParams& p, int cus, hipStream_t s) {
    return launch_decode<float>(D, p, cus, s);
}

}  // namespace kda
