// kda_validate.hip -- opt-in device-side check of the inputs the kernels take
// on trust (environment KDA_VALIDATE=1).
//
// The kernels assume g in [g_min, 0] with g_min = -5 (the bound that keeps a
// 16-token tile's cumulative log-decay above -80, "Understanding Kimi K3's
// attention", g_min equation; "Inside Kimi K3", section "Sequence mixing"),
// beta in [0, 1] (the symbol table of the same page), and, for packed
// batches, cu_seqlens with cu[0] = 0, non-decreasing entries and cu[N] equal
// to the token count.  Out-of-range values are not clamped by the compute
// kernels; they lose precision or overflow.  This check reads those arrays
// once and reports any violation before the compute kernel is launched.
//
// The violation mask lives in one __device__ word per GPU (no allocation).
// The check waits for the stream, so it cannot run under graph capture, and
// two threads validating on one GPU at the same time share the word.
#include "kda_internal.h"

namespace kda {
namespace {

__device__ unsigned int g_violation;

constexpr float kGMin = -5.0f;

__global__ void __launch_bounds__(256) check_inputs_kernel(const float4* g4, int64_t n_g4, const float* beta,
                                                           int64_t n_beta, const int32_t* cu, int32_t n_seqs,
                                                           int64_t total_tokens) {
    unsigned int bits = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = first; i < n_g4; i += stride) {
        const float4 x = g4[i];
        // written so that NaN fails the test
        const bool ok = (x.x >= kGMin && x.x <= 0.f) && (x.y >= kGMin && x.y <= 0.f) &&
                        (x.z >= kGMin && x.z <= 0.f) && (x.w >= kGMin && x.w <= 0.f);
        if (!ok) bits |= KDA_VIOLATION_G;
    }
    for (int64_t i = first; i < n_beta; i += stride) {
        const float b = beta[i];
        if (!(b >= 0.f && b <= 1.f)) bits |= KDA_VIOLATION_BETA;
    }
    if (cu) {
        for (int64_t i = first; i <= n_seqs; i += stride) {
            const int32_t c = cu[i];
            if (i == 0 && c != 0) bits |= KDA_VIOLATION_CU;
            if (i > 0 && c < cu[i - 1]) bits |= KDA_VIOLATION_CU;
            if (i == n_seqs && (int64_t)c != total_tokens) bits |= KDA_VIOLATION_CU;
        }
    }
    if (bits) atomicOr(&g_violation, bits);
}

}  // namespace

hipError_t check_inputs(const float* g, int64_t n_g, const float* beta, int64_t n_beta, const int32_t* cu,
                        int32_t n_seqs, int64_t total_tokens, hipStream_t s, unsigned int* violation) {
    static const unsigned int kZero = 0;
    *violation = 0;
    hipError_t err = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_violation), &kZero, sizeof(kZero), 0,
                                            hipMemcpyHostToDevice, s);
    if (err != hipSuccess) return err;
    // n_g is a multiple of 16 (d_k is), so g is read as float4.
    const int64_t n_g4 = n_g / 4;
    int64_t work = n_g4 > n_beta ? n_g4 : n_beta;
    if (work < (int64_t)n_seqs + 1) work = (int64_t)n_seqs + 1;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(check_inputs_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(g), n_g4, beta, n_beta, cu, n_seqs, total_tokens);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    unsigned int out = 0;
    err = hipMemcpyFromSymbolAsync(&out, HIP_SYMBOL(g_violation), sizeof(out), 0, hipMemcpyDeviceToHost, s);
    if (err != hipSuccess) return err;
    err = hipStreamSynchronize(s);
    if (err != hipSuccess) return err;
    *violation = out;
    return hipSuccess;
}

}  // namespace kda
