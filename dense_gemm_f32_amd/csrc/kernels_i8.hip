// int8-input kernel variants: v_mfma_i32_32x32x32_i8, int32 accumulate and int32 C,
// 128-element K-slabs; A K-contiguous and B K-contiguous (the only layout built).
#include "variants.hpp"

namespace mgemm {

const Variant *i8_variants(int *count)
{
    // Preference order: the first variant that gives at least one workgroup
    // per CU is taken (see the selection in mgemm_api.cpp).
    static const Variant table[] = {
        MGEMM_VARIANT_I8(256, 256, 128, 2, 4, true, 2, "mgemm_i8_256x256x128_w2x4_d2"),
        MGEMM_VARIANT_I8(256, 256, 128, 2, 4, true, 1, "mgemm_i8_256x256x128_w2x4"),
        MGEMM_VARIANT_I8(256, 256, 128, 4, 2, true, 1, "mgemm_i8_256x256x128_w4x2"),
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, true, 1, "mgemm_i8_128x128x128_w2x2"),
        // rows 4-byte aligned (and K a multiple of 4): 4-byte copies into LDS, every tile
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, false, 4, "mgemm_i8_128x128x128_w2x2_d4_u"),
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, false, 1, "mgemm_i8_128x128x128_w2x2_u"),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, true, 1, "mgemm_i8_64x64x128_w2x2"),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 4, "mgemm_i8_64x64x128_w2x2_d4_u"),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 1, "mgemm_i8_64x64x128_w2x2_u"),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
