// kda_output_gate.hip -- the gated output of a KDA layer before its output
// projection: per (token, head) row o of d_v channels,
//
//   y = Sigmoid(gate) * o / sqrt(mean(o^2) + eps) * weight
//
// i.e. Sigmoid(W_g x_t) (the gate logits, computed upstream) times
// RMSNorm(o~_t) ("Understanding Kimi K3's attention", output equation; W_g
// and W_o are outside this operation).  One pass over HBM: o and the gate
// logits are read once, y written once.
//
// Layout: each lane owns 16 bytes of a row (8 bf16 or 4 fp32 values); the
// lanes of a row are consecutive and sum their squares with an xor butterfly
// (fixed order: the result is the same for every lane and every run).  A wave
// covers 64 * 16 / (d_v * element size) rows; workgroups of 4 waves stride
// over the rows, four row groups per step with all their loads issued first.
// Loads and stores are non-temporal (each byte is touched once): measured on
// MI355X at 32768 x 96 rows of 128 bf16, 5.4 TB/s with ordinary accesses,
// 6.0 TB/s with these.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kGateThreads = 256;
constexpr int kGateUnroll = 4;     // row groups in flight per step
constexpr int kGateBlocksPerCU = 4;

template <typename TIn, int DV>
struct GateCfg {
    static constexpr int EPL = 16 / (int)sizeof(TIn);  // elements per lane
    static constexpr int LPR = DV / EPL;               // lanes per row
    static constexpr int RPW = 64 / LPR;               // rows per wave
    static constexpr int RPB = RPW * (kGateThreads / 64);
    static_assert(DV % EPL == 0 && LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row split");
};

__device__ __forceinline__ float sigmoidf_fast(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

template <typename TIn, int DV>
__global__ __launch_bounds__(kGateThreads) void kda_output_gate_kernel(OutputGateParams p) {
    typedef GateCfg<TIn, DV> Cfg;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPB = Cfg::RPB;
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x;
    const int sub = tid % LPR;              // lane within the row
    const int rloc = tid / LPR;             // row within the workgroup's group
    float w[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) w[e] = p.weight[sub * EPL + e];
    const float inv_dv = 1.f / (float)DV;

    constexpr int UN = kGateUnroll;
    const TIn* po = static_cast<const TIn*>(p.o);
    const TIn* pg = static_cast<const TIn*>(p.gate);
    TIn* py = static_cast<TIn*>(p.y);
    for (int64_t r0 = (int64_t)blockIdx.x * RPB * UN; r0 < p.rows; r0 += (int64_t)gridDim.x * RPB * UN) {
        u32x4v ov[UN], gv[UN];
        int64_t off[UN];
        bool ok[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t row = r0 + (int64_t)u * RPB + rloc;
            ok[u] = row < p.rows;
            off[u] = (ok[u] ? row : 0) * DV + (int64_t)sub * EPL;  // element offset (row 0 stands in)
            ov[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(po + off[u]));
            gv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(pg + off[u]));
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            float x[EPL], gl[EPL];
            if constexpr (sizeof(TIn) == 2) {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    x[2 * wd] = __uint_as_float(ov[u][wd] << 16);
                    x[2 * wd + 1] = __uint_as_float(ov[u][wd] & 0xffff0000u);
                    gl[2 * wd] = __uint_as_float(gv[u][wd] << 16);
                    gl[2 * wd + 1] = __uint_as_float(gv[u][wd] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = __uint_as_float(ov[u][e]);
                    gl[e] = __uint_as_float(gv[u][e]);
                }
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
            const float rinv = __builtin_amdgcn_rsqf(ss * inv_dv + p.eps);
            u32x4v yv;
            if constexpr (sizeof(TIn) == 2) {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd)
                    yv[wd] = pack_bf16x2(x[2 * wd] * rinv * w[2 * wd] * sigmoidf_fast(gl[2 * wd]),
                                         x[2 * wd + 1] * rinv * w[2 * wd + 1] * sigmoidf_fast(gl[2 * wd + 1]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) yv[e] = __float_as_uint(x[e] * rinv * w[e] * sigmoidf_fast(gl[e]));
            }
            if (ok[u]) __builtin_nontemporal_store(yv, reinterpret_cast<u32x4v*>(py + off[u]));
        }
    }
}

template <typename TIn, int DV>
hipError_t launch_gate(const OutputGateParams& p, int cus, hipStream_t s) {
    typedef GateCfg<TIn, DV> Cfg;
    const int64_t groups = (p.rows + Cfg::RPB * kGateUnroll - 1) / (Cfg::RPB * kGateUnroll);
    int64_t blocks = (int64_t)cus * kGateBlocksPerCU;
    if (blocks > groups) blocks = groups;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((kda_output_gate_kernel<TIn, DV>), dim3((unsigned)blocks), dim3(kGateThreads), 0, s, p);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_gate_d(int DV, const OutputGateParams& p, int cus, hipStream_t s) {
    switch (DV) {
        case 16: return launch_gate<TIn, 16>(p, cus, s);
        case 32: return launch_gate<TIn, 32>(p, cus, s);
        case 64: return launch_gate<TIn, 64>(p, cus, s);
        case 128: return launch_gate<TIn, 128>(p, cus, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool output_gate_d_supported(int DV) { return DV == 16 || DV == 32 || DV == 64 || DV == 128; }

hipError_t launch_output_gate_bf16(int DV, const OutputGateParams& p, int cus, hipStream_t s) {
    return launch_gate_d<bf16_t>(DV, p, cus, s);
}
hipError_t launch_output_gate_f32(int DV, const OutputGateParams& p, int cus, hipStream_t s) {
    return launch_gate_d<float>(DV, p, cus, s);
}

}  // namespace kda
