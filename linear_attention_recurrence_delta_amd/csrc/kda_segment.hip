// kda_segment.hip -- the combine step of the sequence-segment scan (gfx950).
//
// The state update is affine in the state ("Understanding Kimi K3's
// attention", state-update equation: S_t = (I - beta_t k_t k_t^T)
// Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T), so a whole segment of tokens is
// one affine map S_end = M S_start + B, with M (d_k x d_k) the segment run
// from the identity with v = 0 and B (d_k x d_v) the run from zero.  The
// pipelined prefill computes those maps for every segment in parallel; this
// kernel chains them, start(g + 1) = M_g start(g) + B_g, which is the state
// passed between segments as the pages pass it between chunks ("Inside Kimi
// K3", section "Sequence mixing"), so that every segment can then be re-run
// in parallel from its true start state.  Segment 0 needs no map: the
// map-pair launch runs it outright from the initial state and leaves its end
// state, start(1), in the B slot of segment 0.
//
// Work: one workgroup per (sequence, head, 16 value columns); value columns
// never mix (the map acts on the key side), so the 8 column groups of a head
// run independently.  fp32 FMA in a fixed order: deterministic.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int SD = 128;        // d_k = d_v
constexpr int SPM = SD + 4;    // fp32 pitch of M rows in LDS (rows 4 apart land 16 banks apart)
constexpr int SNT = 256;

__global__ __launch_bounds__(SNT) void kda_segment_combine_kernel(PrefillParams p) {
    __shared__ __align__(16) float sM[2][SD * SPM];
    __shared__ __align__(16) float sS[SD * 16];  // start(g) columns: [row][16]

    const int tid = threadIdx.x;
    const int units = p.N * p.H;
    const int uh = blockIdx.x / (SD / 16);
    const int c0 = (blockIdx.x % (SD / 16)) * 16;
    if (uh >= units) return;
    const int j = tid & 15;   // column within the group
    const int rg = tid >> 4;  // rows rg + 16 r, r = 0..7
    const int64_t sdd = (int64_t)SD * SD;
    auto slot = [&](int g, int part) { return p.seg_ws + (((int64_t)uh * (p.seg_G - 1) + g) * 2 + part) * sdd; };

    // M_g rows as 16-byte pieces: piece i of 4096 -> row i / 32, columns 4 (i % 32)
    auto load_m = [&](int g, f32x4 (&r)[16]) {
        const f32x4* src = reinterpret_cast<const f32x4*>(slot(g, 0));
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = src[tid + SNT * i];
    };
    auto park_m = [&](int buf, const f32x4 (&r)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int pc = tid + SNT * i;
            *reinterpret_cast<f32x4*>(&sM[buf][(pc >> 5) * SPM + 4 * (pc & 31)]) = r[i];
        }
    };

    // start(1) = the end state of segment 0, kept in slot (0, B)
    {
        const float* s1 = slot(0, 1);
#pragma unroll
        for (int r = 0; r < 8; ++r) sS[(rg + 16 * r) * 16 + j] = s1[(int64_t)(rg + 16 * r) * SD + c0 + j];
    }
    f32x4 pre[16];
    if (p.seg_G > 2) {
        load_m(1, pre);
        park_m(1 & 1, pre);
    }
    __syncthreads();
    for (int g = 1; g <= p.seg_G - 2; ++g) {
        const bool more = g + 1 <= p.seg_G - 2;
        if (more) load_m(g + 1, pre);  // in flight during this step
        float* bg = slot(g, 1);
        float acc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = bg[(int64_t)(rg + 16 * r) * SD + c0 + j];
        const float* M = sM[g & 1];
        for (int k = 0; k < SD; k += 4) {
            const float s0 = sS[(k + 0) * 16 + j], s1 = sS[(k + 1) * 16 + j];
            const float s2 = sS[(k + 2) * 16 + j], s3 = sS[(k + 3) * 16 + j];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const f32x4 m = *reinterpret_cast<const f32x4*>(&M[(rg + 16 * r) * SPM + k]);
                acc[r] = fmaf(m[0], s0, acc[r]);
                acc[r] = fmaf(m[1], s1, acc[r]);
                acc[r] = fmaf(m[2], s2, acc[r]);
                acc[r] = fmaf(m[3], s3, acc[r]);
            }
        }
        __syncthreads();  // every thread has read start(g) and M_g
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            sS[(rg + 16 * r) * 16 + j] = acc[r];
            bg[(int64_t)(rg + 16 * r) * SD + c0 + j] = acc[r];  // start(g + 1) in place of B_g
        }
        if (more) park_m((g + 1) & 1, pre);
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_segment_combine(const PrefillParams& p, hipStream_t s) {
    const int64_t units = (int64_t)p.N * p.H;
    if (units <= 0 || p.seg_G <= 2) return hipSuccess;
    hipLaunchKernelGGL(kda_segment_combine_kernel, dim3((unsigned)(units * (SD / 16))), dim3(SNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
