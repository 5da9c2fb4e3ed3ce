// fp64 kernel variants: v_mfma_f64_16x16x4_f64, double accumulate and double C,
// 16- or 32-element K-slabs, every transpose combination.
#include "variants.hpp"

namespace mgemm {

const Variant *f64_variants(int *count)
{
    // Preference order: the first variant that gives at least one workgroup
    // per CU is taken (see the selection in mgemm_api.cpp).  Measured on
    // DGEMM 4096^3 NN: 128x128 with eight waves 63.8 TFLOP/s, with four waves
    // (64x64 per wave: 280 registers, one wave per SIMD) 46.5, 128x64 54.8,
    // 64x64 54.5, 32-deep slabs 43-54.
    static const Variant table[] = {
        MGEMM_VARIANT_F64(128, 128, 16, 4, 2, true, "mgemm_f64_128x128x16_w4x2"),
        MGEMM_VARIANT_F64(128, 128, 16, 2, 4, true, "mgemm_f64_128x128x16_w2x4"),
        MGEMM_VARIANT_F64(128, 64, 16, 2, 2, true, "mgemm_f64_128x64x16_w2x2"),
        MGEMM_VARIANT_F64(128, 128, 16, 4, 2, false, "mgemm_f64_128x128x16_w4x2_u"),
        MGEMM_VARIANT_F64(64, 64, 16, 2, 2, true, "mgemm_f64_64x64x16_w2x2"),
        MGEMM_VARIANT_F64(64, 64, 16, 2, 2, false, "mgemm_f64_64x64x16_w2x2_u"),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
