// int8-input kernel variants: v_mfma_i32_32x32x32_i8, int32 accumulate and int32 C,
// 128-element K-slabs.  The 256x256 and 128x128 tiles take every transpose
// (MN-contiguous operands through transposing LDS reads); the 64x64 ones take A
// K-contiguous and B K-contiguous only.
#include "variants.hpp"

namespace mgemm {

const Variant *i8_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp): the 256x256
    // two-stage tile 0.0121 us per K per round (0.55 of the matrix peak per
    // CU; its t0 is set from a K = 256 launch, the fit over whole-K rounds
    // having too few points), 128x128 with eight waves 0.0034 (two stages of
    // 128, several workgroups per CU) or 0.0044 (four of 64, better for one
    // round), 64x64 0.0014 to 0.0020.  The register-path factor (16-byte
    // rows, K no multiple of 16) is a round estimate.  Builds without an
    // estimate run when forced, or by preference order when no estimated
    // build fits (rows not 4-byte aligned, or offsets past 32 bits: the
    // register-path builds).
    static const Variant table[] = {
        MGEMM_VARIANT_I8_ALL(256, 256, 128, 2, 4, true, 2, "mgemm_i8_256x256x128_w2x4_d2", {8.0f, 0.0121f, 1.5f, 1.15f}),
        MGEMM_VARIANT_I8_ALL(256, 256, 128, 2, 4, true, 1, "mgemm_i8_256x256x128_w2x4", {}),
        MGEMM_VARIANT_I8_ALL(256, 256, 128, 4, 2, true, 1, "mgemm_i8_256x256x128_w4x2", {}),
        // 128x128 with eight waves (four waves measured 3-20% slower)
        MGEMM_VARIANT_I8_ALL(128, 128, 128, 2, 4, true, 1, "mgemm_i8_128x128x128_w2x4", {3.39f, 0.00441f, 1.5f, 1.15f},
                         MGEMM_SK_I8_ALL(128, 128, 128, 2, 4, true, 1)),
        MGEMM_VARIANT_I8_ALL(128, 128, 128, 2, 4, true, 2, "mgemm_i8_128x128x128_w2x4_d2", {3.59f, 0.00336f, 1.5f, 1.35f},
                         MGEMM_SK_I8_ALL(128, 128, 128, 2, 4, true, 2)),
        // rows 4-byte aligned (and K a multiple of 4), every tile: 16-byte
        // copies on all but a tile's last slab (4-byte copies).  Estimates from
        // a same-box fit against the two-stage siblings, scaled by their
        // table/fit ratios: 1.4 to 1.5 times their time per K
        MGEMM_VARIANT_I8_ALL(128, 128, 128, 2, 2, false, 4, "mgemm_i8_128x128x128_w2x2_d4_u",
                             {4.2f, 0.0046f, 1.0f, 1.35f},
                         MGEMM_SK_I8_ALL(128, 128, 128, 2, 2, false, 4)),
        MGEMM_VARIANT_I8_ALL(128, 128, 128, 2, 2, false, 1, "mgemm_i8_128x128x128_w2x2_u", {},
                         MGEMM_SK_I8_ALL(128, 128, 128, 2, 2, false, 1)),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, true, 1, "mgemm_i8_64x64x128_w2x2", {0.64f, 0.00195f, 1.5f, 2.6f},
                         MGEMM_SK_I8(64, 64, 128, 2, 2, true, 1)),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, true, 2, "mgemm_i8_64x64x128_w2x2_d2", {0.82f, 0.00139f, 1.5f, 3.16f},
                         MGEMM_SK_I8(64, 64, 128, 2, 2, true, 2)),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 4, "mgemm_i8_64x64x128_w2x2_d4_u",
                         {0.84f, 0.00206f, 1.0f, 2.8f},
                         MGEMM_SK_I8(64, 64, 128, 2, 2, false, 4)),
        MGEMM_VARIANT_I8(64, 64, 128, 2, 2, false, 1, "mgemm_i8_64x64x128_w2x2_u", {},
                         MGEMM_SK_I8(64, 64, 128, 2, 2, false, 1)),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
