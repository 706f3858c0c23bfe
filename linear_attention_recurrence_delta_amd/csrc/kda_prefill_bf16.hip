// kda_prefill_bf16.hip -- bf16 q/k/v instantiations of the chunked prefill
// (bf16 MFMA products, fp32 accumulation, fp32 state).
#include "kda_prefill_impl.h"
#include "kda_prefill_ws.h"

namespace kda {

// instantiated in kda_prefill_ws_ilp.hip (built with another scheduler)
extern template hipError_t launch_prefill_ws<2, 2, 8, false, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 2, 8, false, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 1, 8, false, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<2, 2, 8, true, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 2, 8, true, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 1, 8, true, false>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<2, 2, 8, false, true>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 2, 8, false, true>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<1, 1, 8, false, true>(const PrefillParams&, hipStream_t);
extern template hipError_t launch_prefill_ws<2, 2, 8, false, false, true>(const PrefillParams&, hipStream_t);

static const PrefillVariant kBf16Variants[] = {
    // wave-specialised pipeline: NCW consumer waves x TPW 16 columns, 8 stage-A waves
    // (whole-head and 64-column slabs also built for the segment scan's runs,
    // with the map-pair kernel <8, 2, 4, ..., SEG> for its maps)
    // (whole heads also with the output gate fused into the o store)
    {1, 1, 128, 16, 8, WsCfg<4, 2, 8>::LDS, &launch_prefill_ws<4, 2, 8>, &launch_prefill_ws<4, 2, 8, false, false, true>,
     &launch_prefill_ws<4, 2, 8, false, false, false, true>, &launch_prefill_ws<8, 2, 4, false, false, true>},
    {1, 1, 128, 16, 4, WsCfg<2, 2, 8>::LDS, &launch_prefill_ws<2, 2, 8>, &launch_prefill_ws<2, 2, 8, false, false, true>,
     nullptr, &launch_prefill_ws<8, 2, 4, false, false, true>},
    {1, 1, 128, 16, 2, WsCfg<1, 2, 8>::LDS, &launch_prefill_ws<1, 2, 8>},
    {1, 1, 128, 16, 1, WsCfg<1, 1, 8>::LDS, &launch_prefill_ws<1, 1, 8>},
    // the same with the gate and the q/k L2 norm computed in the kernel
    {2, 1, 128, 16, 8, WsCfg<4, 2, 8, true>::LDS, &launch_prefill_ws<4, 2, 8, true>},
    {2, 1, 128, 16, 4, WsCfg<2, 2, 8, true>::LDS, &launch_prefill_ws<2, 2, 8, true>},
    {2, 1, 128, 16, 2, WsCfg<1, 2, 8, true>::LDS, &launch_prefill_ws<1, 2, 8, true>},
    {2, 1, 128, 16, 1, WsCfg<1, 1, 8, true>::LDS, &launch_prefill_ws<1, 1, 8, true>},
    // kind 3: the plain pipeline writing its checkpoints as bf16 in the blocked
    // layout of the backward kernel (only the backward launches these)
    {3, 1, 128, 16, 8, WsCfg<4, 2, 8>::LDS, &launch_prefill_ws<4, 2, 8, false, true>},
    {3, 1, 128, 16, 4, WsCfg<2, 2, 8>::LDS, &launch_prefill_ws<2, 2, 8, false, true>},
    {3, 1, 128, 16, 2, WsCfg<1, 2, 8>::LDS, &launch_prefill_ws<1, 2, 8, false, true>},
    {3, 1, 128, 16, 1, WsCfg<1, 1, 8>::LDS, &launch_prefill_ws<1, 1, 8, false, true>},
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 4, 8),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 4, 4),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 4, 2),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 2, 8),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 2, 4),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 2, 2),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 1, 8),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 1, 4),
    KDA_PREFILL_VARIANT(1, bf16_t, 128, 1, 2),
};

const PrefillVariant* prefill_variants_bf16(int* count) {
    *count = static_cast<int>(sizeof(kBf16Variants) / sizeof(kBf16Variants[0]));
    return kBf16Variants;
}

}  // namespace kda
