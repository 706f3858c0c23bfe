// kda_prefill_f32.hip -- fp32 q/k/v instantiations of the chunked prefill
// (fp32 MFMA products, fp32 everywhere).  One workgroup per (sequence, head).
#include "kda_prefill_impl.h"

namespace kda {

static const PrefillVariant kF32Variants[] = {
    KDA_PREFILL_VARIANT(0, float, 16, 1, 1),
    KDA_PREFILL_VARIANT(0, float, 16, 2, 1),
    KDA_PREFILL_VARIANT(0, float, 16, 4, 1),
    KDA_PREFILL_VARIANT(0, float, 32, 1, 2),
    KDA_PREFILL_VARIANT(0, float, 32, 2, 2),
    KDA_PREFILL_VARIANT(0, float, 32, 4, 2),
    KDA_PREFILL_VARIANT(0, float, 64, 1, 4),
    KDA_PREFILL_VARIANT(0, float, 64, 2, 4),
    KDA_PREFILL_VARIANT(0, float, 128, 1, 8),
    KDA_PREFILL_VARIANT(0, float, 128, 2, 8),
};

const PrefillVariant* prefill_variants_f32(int* count) {
    *count = static_cast<int>(sizeof(kF32Variants) / sizeof(kF32Variants[0]));
    return kF32Variants;
}

}  // namespace kda
