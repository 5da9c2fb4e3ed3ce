// int8-input kernel variants: v_mfma_i32_32x32x32_i8, int32 accumulate and int32 C,
// 128-element K-slabs; A K-contiguous and B K-contiguous (the only layout built).
#include "variants.hpp"

namespace mgemm {

const Variant *i8_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp): the 256x256
    // two-stage tile 0.0131 us per K per round (0.51 of the matrix peak per
    // CU), 128x128 0.0045 (0.37), 64x64 0.0021 (0.20); the register-path
    // factor (16-byte rows, K no multiple of 16) is a round estimate.  Builds
    // without an estimate run when forced, or by preference order when no
    // estimated build fits (unaligned rows: 4-byte copies first).
    static const Variant table[] = {
        MGEMM_VARIANT_I8(256, 256, 128, 2, 4, true, 2, "mgemm_i8_256x256x128_w2x4_d2", {0.0f, 0.01308f, 1.5f, 1.18f}),
        MGEMM_VARIANT_I8(256, 256, 128, 2, 4, true, 1, "mgemm_i8_256x256x128_w2x4", {}),
        MGEMM_VARIANT_I8(256, 256, 128, 4, 2, true, 1, "mgemm_i8_256x256x128_w4x2", {}),
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, true, 1, "mgemm_i8_128x128x128_w2x2", {3.83f, 0.00448f, 1.5f, 1.13f}),
        // rows 4-byte aligned (and K a multiple of 4): 4-byte copies into LDS, every tile
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, false, 4, "mgemm_i8_128x128x128_w2x2_d4_u", {}),
        MGEMM_VARIANT_I8(128, 128, 128, 2, 2, false, 1, "mgemm_i8_128x128x128_w2x2_u", {}),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, true, 1, "mgemm_i8_64x64x128_w2x2", {0.59f, 0.00207f, 1.5f, 3.51f}),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 4, "mgemm_i8_64x64x128_w2x2_d4_u", {}),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 1, "mgemm_i8_64x64x128_w2x2_u", {}),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
