// kda_backward.h -- parameters and launcher of the prefill backward kernel
// (kda_backward.hip), used by the C ABI in kda_abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Backward of the prefill (bf16 q/k/v/dO, d_k = d_v = 128, chunk 16): two
// workgroups per (sequence, head), one per half of the value columns, walk
// the chunks last to first; a second kernel adds their key-side partials.
struct BackwardParams {
    const void* q;          // [T, H, 128] bf16
    const void* k;
    const void* v;
    const float* g;         // [T, H, 128]
    const float* beta;      // [T, H]
    const float* S0;        // [N, H, 128, 128] or nullptr (zeros)
    const int32_t* cu;      // [N + 1] or nullptr (dense, seq_len each)
    const void* dO;         // [T, H, 128] bf16: gradient with respect to o
    const float* dST;       // [N, H, 128, 128] or nullptr: gradient with respect to the final state
    const void* ckpt;       // state after every 16 tokens of each sequence, bf16 blocked (below)
    void* S0b;              // bf16 blocked copy of S0 (written by the first launch) or nullptr
    void* dq;               // [T, H, 128] bf16
    void* dk;
    void* dv;
    float* dg;              // [T, H, 128]
    float* dbeta;           // [T, H]
    float* dS0;             // [N, H, 128, 128] or nullptr
    float* part;            // per value half: dq, dk, dg [2][T, H, 128], then dbeta [2][T, H] (fp32)
    int64_t T_total;
    int32_t N, H, seq_len;
    float scale;
};

// Blocked state layout of ckpt and S0b (bf16, 32 KB per state): element
// (row, col) at ((row / 4) * 128 + col) * 4 + row % 4, so the 4 rows of one
// column that an MFMA fragment holds are 8 adjacent bytes.  The prefill
// kernels of kind 3 write checkpoints this way.
//
// Bytes of the partial buffer `part` for T_total tokens and H heads.
size_t backward_partial_bytes(int64_t T_total, int32_t H);
// The S0 conversion (when S0 and S0b are set), the reverse kernel and the
// sum of the halves, in order, on stream s.
hipError_t launch_backward_bf16_d128(const BackwardParams& p, hipStream_t s);

}  // namespace kda
