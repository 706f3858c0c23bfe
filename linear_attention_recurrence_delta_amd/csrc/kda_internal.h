// kda_internal.h -- host-side declarations shared by the C-ABI layer and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Everything a prefill launch needs; pointers are device pointers.
struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* S0;        // [N,H,D,D] or nullptr (zeros)
    const int32_t* cu;      // [N+1] or nullptr (dense)
    void* o;
    float* Sout;            // [N,H,D,D] or nullptr
    int64_t T_total;
    int32_t N;
    int32_t H;
    int32_t seq_len;        // dense sequences: tokens per sequence
    int32_t nslab;          // d_v column slabs per (sequence, head)
    float scale;
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* S;
    void* o;
    int64_t units;          // N * H
    float scale;
};

// One entry per built prefill kernel.
struct PrefillVariant {
    int kind;               // 0: chunk-staged kernel, 1: wave-specialised pipeline
    int dtype;              // kda_dtype
    int D;                  // d_k = d_v
    int C;                  // chunk size
    int nwc;                // column waves per workgroup (16 d_v columns each)
    size_t lds_bytes;
    hipError_t (*launch)(const PrefillParams&, hipStream_t);
};

// Tables defined in the kernel translation units.
const PrefillVariant* prefill_variants_bf16(int* count);
const PrefillVariant* prefill_variants_f32(int* count);

// Opt-in input check (KDA_VALIDATE=1): violation bits reported by check_inputs.
enum : unsigned int {
    KDA_VIOLATION_G = 1u,     // g outside [-5, 0] or NaN
    KDA_VIOLATION_BETA = 2u,  // beta outside [0, 1] or NaN
    KDA_VIOLATION_CU = 4u,    // cu_seqlens not 0 = cu[0] <= ... <= cu[N] = total_tokens
};
// Reads g [n_g], beta [n_beta] and cu [n_seqs + 1] (cu may be nullptr) on
// stream s, waits for it, and stores the violation bits in *violation.
hipError_t check_inputs(const float* g, int64_t n_g, const float* beta, int64_t n_beta, const int32_t* cu,
                        int32_t n_seqs, int64_t total_tokens, hipStream_t s, unsigned int* violation);

// Decode launchers; return hipErrorInvalidValue for an unsupported D.
hipError_t launch_decode_bf16(int D, const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_f32(int D, const DecodeParams& p, hipStream_t s);
bool decode_d_supported(int D);

}  // namespace kda
