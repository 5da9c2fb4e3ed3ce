// f16-input kernel variants: v_mfma_f32_32x32x16_f16, fp32 accumulate, 64-element K-slabs.
#include "variants.hpp"

namespace mgemm {

const Variant *f16_variants(int *count)
{
    // Preference order: the first variant that gives at least one workgroup
    // per CU is taken (see the selection in mgemm_api.cpp).
    static const Variant table[] = {
        MGEMM_VARIANT_D(_Float16, 1, 256, 256, 64, 2, 4, true, 2, "mgemm_f16_256x256x64_w2x4_d2"),
        MGEMM_VARIANT(_Float16, 1, 256, 256, 64, 2, 4, true, "mgemm_f16_256x256x64_w2x4"),
        MGEMM_VARIANT(_Float16, 1, 256, 256, 64, 4, 2, true, "mgemm_f16_256x256x64_w4x2"),
        MGEMM_VARIANT(_Float16, 1, 256, 256, 64, 2, 2, true, "mgemm_f16_256x256x64_w2x2"),
        MGEMM_VARIANT_D(_Float16, 1, 256, 256, 64, 2, 2, true, 2, "mgemm_f16_256x256x64_w2x2_d2"),
        MGEMM_VARIANT(_Float16, 1, 128, 128, 64, 2, 2, true, "mgemm_f16_128x128x64_w2x2"),
        // rows 4-byte aligned (and K even): 4-byte copies into LDS, every tile
        MGEMM_VARIANT_D(_Float16, 1, 128, 128, 64, 2, 2, false, 4, "mgemm_f16_128x128x64_w2x2_d4_u"),
        MGEMM_VARIANT(_Float16, 1, 128, 128, 64, 2, 2, false, "mgemm_f16_128x128x64_w2x2_u"),
        MGEMM_VARIANT(_Float16, 1, 64, 64, 64, 2, 2, true, "mgemm_f16_64x64x64_w2x2"),
        MGEMM_VARIANT_D(_Float16, 1, 64, 64, 64, 2, 2, false, 4, "mgemm_f16_64x64x64_w2x2_d4_u"),
        MGEMM_VARIANT(_Float16, 1, 64, 64, 64, 2, 2, false, "mgemm_f16_64x64x64_w2x2_u"),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
