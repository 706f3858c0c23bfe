// kda_prefill_ws_ilp.hip -- the narrower slabs of the wave-specialised bf16
// prefill (kda_prefill_ws.h): 64, 32 and 16 value columns per workgroup (12,
// 11 and 11 waves, at most three per SIMD), plain, fused, with the backward's
// checkpoints, and (64 columns) with the segment-scan phases.  This file is compiled with LLVM's instruction-
// level-parallelism scheduler (build_lib.py): these kernels have registers
// to spare at their occupancy, and a schedule that interleaves independent
// products and loads shortened the dense K3 launch (64 columns) by about 4%.
// The 128-column slab (14 waves) would spill under it and stays in
// kda_prefill_bf16.hip with the default scheduler.
#include "kda_prefill_ws.h"

namespace kda {

template hipError_t launch_prefill_ws<2, 2, 8, false, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 2, 8, false, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 1, 8, false, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<2, 2, 8, true, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 2, 8, true, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 1, 8, true, false>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<2, 2, 8, false, true>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 2, 8, false, true>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<1, 1, 8, false, true>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_ws<2, 2, 8, false, false, true>(const PrefillParams&, hipStream_t);

}  // namespace kda
