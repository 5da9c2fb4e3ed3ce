// fp64 kernel variants: v_mfma_f64_16x16x4_f64, double accumulate and double C,
// 16- or 32-element K-slabs, every transpose combination.
#include "variants.hpp"

namespace mgemm {

const Variant *f64_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp): 128x128
    // 0.129 us per K per round (0.83 of the matrix peak per CU), 128x64 0.072
    // (0.74), 64x64 0.0368 (0.72).  The 64x64 tile wins where 128x128 leaves
    // a last round mostly empty (3072^3: 1043 us against 1207).  Builds
    // without an estimate run when forced, or by preference order when no
    // estimated build fits (unaligned rows).  Measured on DGEMM 4096^3 NN:
    // 128x128 with eight waves 63.8 TFLOP/s, with four waves (64x64 per
    // wave: 280 registers, one wave per SIMD) 46.5, 128x64 54.8, 64x64 54.5,
    // 32-deep slabs 43-54.  Every build but the 2x4-wave one also has a
    // stream-K launch (gemm_f64_sk_kernel).
    static const Variant table[] = {
        MGEMM_VARIANT_F64(128, 128, 16, 4, 2, true, "mgemm_f64_128x128x16_w4x2", {0.44f, 0.1291f, 1.0f, 1.12f},
                          MGEMM_SK_F64(128, 128, 16, 4, 2, true)),
        MGEMM_VARIANT_F64(128, 128, 16, 2, 4, true, "mgemm_f64_128x128x16_w2x4", {}),
        MGEMM_VARIANT_F64(128, 64, 16, 2, 2, true, "mgemm_f64_128x64x16_w2x2", {1.78f, 0.0720f, 1.0f, 1.1f},
                          MGEMM_SK_F64(128, 64, 16, 2, 2, true)),
        MGEMM_VARIANT_F64(128, 128, 16, 4, 2, false, "mgemm_f64_128x128x16_w4x2_u", {},
                          MGEMM_SK_F64(128, 128, 16, 4, 2, false)),
        MGEMM_VARIANT_F64(64, 64, 16, 2, 2, true, "mgemm_f64_64x64x16_w2x2", {1.64f, 0.0368f, 1.0f, 1.6f},
                          MGEMM_SK_F64(64, 64, 16, 2, 2, true)),
        MGEMM_VARIANT_F64(64, 64, 16, 2, 2, false, "mgemm_f64_64x64x16_w2x2_u", {},
                          MGEMM_SK_F64(64, 64, 16, 2, 2, false)),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
