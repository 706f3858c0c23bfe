// kda_internal.h -- declarations shared by the C-ABI layer and the kernel
// translation units (plus two small device helpers over the launch
// parameters).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_bounds.h"

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
    // State checkpoints (ckpt == nullptr: none).  Checkpoint j of sequence n
    // is the state after its first (j + 1) * ckpt_interval tokens, stored at
    // slot ckpt_first_slot(n) + j of [ckpt_cap, H, D, D]; ckpt_interval is a
    // multiple of the kernel's chunk.
    float* ckpt;
    int64_t ckpt_cap;
    int32_t ckpt_interval;
    // Fused gate and q/k norm (the kernels built for it): q and k arrive
    // unnormalised, g is not read; z [T_total, H, d_k] (qkv dtype) and
    // a_log [H] give g = -5 Sigmoid(exp(a_log[h]) z).
    const void* z;
    const float* a_log;
    // Sequence-segment scan (dense batches, pipelined kernel).  seg_phase 0:
    // off, one workgroup chain per (sequence, head, slab) walks the whole
    // sequence.  Otherwise each sequence is cut into seg_G segments of
    // seg_len tokens, the last one running to the end of the sequence.
    // Phase 1 (the map-pair kernel) computes, for g = 1 .. seg_G - 2, the
    // affine map of segment g: S_end = M_g S_start + B_g, with M_g the run
    // from the identity with v = 0 and B_g the run from zero with the real v,
    // and runs segment 0 from the initial state with its outputs (its end
    // state into the B slot of segment 0; the M slot stays unused).  A
    // combine kernel turns the maps into every segment's start state; phase 3
    // runs segments 1 .. seg_G - 1 from those states with outputs.  seg_ws
    // holds [N H][seg_G - 1][2][D][D] fp32: (M_g, B_g), the B slot replaced
    // by the start state of segment g + 1.
    // Output gate fused into the o store (kernels built with it): o is not
    // stored; y = Sigmoid(gate) o / sqrt(mean(o^2) + gate_eps) * gate_weight
    // goes to the o buffer instead (gate [T_total, H, D] in the qkv dtype,
    // gate_weight [D] fp32).
    const void* gate = nullptr;
    const float* gate_weight = nullptr;
    float gate_eps = 0.f;
    int32_t seg_phase = 0;  // 0, 1 or 3
    int32_t seg_G = 1;
    int32_t seg_len = 0;
    float* seg_ws = nullptr;
};

// Workgroups of a pipelined-kernel launch: units are padded to whole groups
// of 8 (one per XCD), each unit or segment item with nslab slabs; the
// map-pair kernel (segment scan, phase 1) takes whole heads, one workgroup per
// (sequence, head, segment 0 .. seg_G - 2); phase 3 one per (sequence, head,
// segment 1 .. seg_G - 1, slab).
inline int64_t ws_pad8(int64_t x) { return (x + 7) / 8 * 8; }
inline int64_t ws_grid_blocks(const PrefillParams& p) {
    const int64_t units = (int64_t)p.N * p.H;
    if (p.seg_phase == 1) return ws_pad8(units * (p.seg_G - 1));
    if (p.seg_phase == 3) return ws_pad8(units * (p.seg_G - 1)) * p.nslab;
    return ws_pad8(units) * p.nslab;
}

// Token range [*a, *b) of sequence n, with the bounds read from cu clamped to
// [0, T_total] and b >= a (malformed offsets change the numbers, never the
// memory touched).  Every prefill kernel uses these bounds.
__device__ inline void seq_bounds(const PrefillParams& p, int n, int64_t* a, int64_t* b) {
    if (p.cu) {
        const SeqRange r = clamp_seq(p.cu[n], p.cu[n + 1], p.T_total);
        *a = r.a;
        *b = r.b;
    } else {
        *a = (int64_t)n * p.seq_len;
        *b = *a + p.seq_len;
    }
}

// First checkpoint slot of sequence n: the checkpoints of the sequences before
// it, floor(length / interval) each.  Called by every lane of a wave (the
// lanes split the sequences, then a butterfly sum); returns the same value in
// all lanes.
__device__ inline int64_t ckpt_first_slot(const PrefillParams& p, int n, int lane) {
    if (!p.cu) return (int64_t)n * (p.seq_len / p.ckpt_interval);
    int part = 0;  // at most T_total / interval < 2^31
    for (int m = lane; m < n; m += 64) {
        int64_t a, b;
        seq_bounds(p, m, &a, &b);
        part += (int)((b - a) / p.ckpt_interval);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    return part;
}

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

struct OutputGateParams {
    const void* o;          // [rows, d_v] dtype
    const void* gate;       // [rows, d_v] dtype
    const float* weight;    // [d_v]
    void* y;                // [rows, d_v] dtype
    int64_t rows;           // T_total * H
    float eps;
};

// The static device buffer of kda_prefill_ex_noalloc (kda_scratch.hip): its
// size, and its device address on the current device (taken once per device
// with hipGetSymbolAddress).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// Phase 2 of the segment scan: for g = 1 .. seg_G - 2, start(g + 1) =
// M_g start(g) + B_g in fp32, in place of B_g, per (sequence, head) and
// 16-column group.
hipError_t launch_segment_combine(const PrefillParams& p, hipStream_t s);

// One entry per built prefill kernel.
struct PrefillVariant {
    int kind;               // 0: chunk-staged kernel, 1: wave-specialised pipeline, 2: the same, fused gate/norm
    int dtype;              // kda_dtype
    int D;                  // d_k = d_v
    int C;                  // chunk size
    int nwc;                // column waves per workgroup (16 d_v columns each)
    size_t lds_bytes;
    hipError_t (*launch)(const PrefillParams&, hipStream_t);
    // the same kernel built for the segment scan's runs (phase 3), or nullptr
    hipError_t (*launch_seg)(const PrefillParams&, hipStream_t) = nullptr;
    // the same kernel with the output gate fused into the o store, or nullptr
    hipError_t (*launch_gate)(const PrefillParams&, hipStream_t) = nullptr;
    // the segment scan's map-pair kernel (phase 1), where launch_seg is built
    hipError_t (*launch_pair)(const PrefillParams&, hipStream_t) = nullptr;
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
hipError_t launch_decode_bf16(int D, const DecodeParams& p, int cus, hipStream_t s);
hipError_t launch_decode_f32(int D, const DecodeParams& p, int cus, hipStream_t s);
bool decode_d_supported(int D);

// Output gate launchers (cus = compute units of the device); return
// hipErrorInvalidValue for an unsupported d_v.
hipError_t launch_output_gate_bf16(int DV, const OutputGateParams& p, int cus, hipStream_t s);
hipError_t launch_output_gate_f32(int DV, const OutputGateParams& p, int cus, hipStream_t s);
bool output_gate_d_supported(int DV);

}  // namespace kda
