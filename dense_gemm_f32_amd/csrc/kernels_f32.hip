// fp32 (SGEMM) kernel variants: v_mfma_f32_32x32x2_f32, 32-float K-slabs.
#include "variants.hpp"

namespace mgemm {

const Variant *f32_variants(int *count)
{
    // Preference order: the first variant that gives at least one workgroup
    // per CU is taken (see the selection in mgemm_api.cpp).
    static const Variant table[] = {
        MGEMM_VARIANT_F32(256, 256, 32, 4, 2, true, "mgemm_f32_256x256x32_w4x2"),
        MGEMM_VARIANT_F32(256, 256, 32, 2, 2, true, "mgemm_f32_256x256x32_w2x2"),
        MGEMM_VARIANT_F32(128, 128, 32, 2, 2, true, "mgemm_f32_128x128x32_w2x2"),
        MGEMM_VARIANT_F32_D(128, 128, 32, 2, 2, false, 4, "mgemm_f32_128x128x32_w2x2_d4_u"),
        MGEMM_VARIANT_F32(128, 128, 32, 2, 2, false, "mgemm_f32_128x128x32_w2x2_u"),
        // 64x64: two stages of 32 (one barrier per 16 MFMAs) measured 9-14%
        // faster than four of 16 at 512^3 to 2048^3 (deeper rings of 8 or 16
        // stages gained nothing)
        MGEMM_VARIANT_F32_D(64, 64, 32, 2, 2, true, 2, "mgemm_f32_64x64x32_w2x2_d2"),
        MGEMM_VARIANT_F32_D(64, 64, 32, 2, 2, false, 4, "mgemm_f32_64x64x32_w2x2_d4_u"),
        MGEMM_VARIANT_F32(64, 64, 32, 2, 2, false, "mgemm_f32_64x64x32_w2x2_u"),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
