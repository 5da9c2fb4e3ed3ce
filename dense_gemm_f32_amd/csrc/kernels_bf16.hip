// bf16-input kernel variants: v_mfma_f32_32x32x16_bf16, fp32 accumulate, 64-element K-slabs.
#include "variants.hpp"

namespace mgemm {

const Variant *bf16_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp: t0 us, tk us
    // per unit of K, register-path factor, one-round factor), fitted on bf16
    // (the two 16-bit types run the same kernels at the same rates): the
    // 256x256 two-stage tile 0.0219 us per K per round (0.61 of the matrix
    // peak per CU; its fit scaled by the 4% that spreading its copies among
    // the MFMAs gained), 128x128 0.0083 to 0.0096 (0.35 to 0.40), 64x64 0.0034 to
    // 0.0039 (0.21 to 0.25).  The 128x128 slopes are set 10% above their fit:
    // their rounds slow down on large problems (twice the operand traffic of
    // the 256x256 tile), and without it the choice took them at 3000^3 and
    // 7000^3 where the large tile is faster.  K <= 128 (store-bound) takes the
    // 256x256 4x2-wave tile first.  Builds without an estimate run when
    // forced, or by preference order when no estimated build fits (rows not
    // 4-byte aligned, or offsets past 32 bits: the register-path builds).
    static const Variant table[] = {
        MGEMM_VARIANT_D(__bf16, 2, 256, 256, 64, 2, 4, true, 2, "mgemm_bf16_256x256x64_w2x4_d2", {10.7f, 0.0219f, 1.6f, 1.0f}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 2, 4, true, "mgemm_bf16_256x256x64_w2x4", {}),
        // one LDS stage for K <= 64 (attention scores): two workgroups per CU
        MGEMM_VARIANT_D(__bf16, 2, 256, 256, 64, 4, 2, true, 3, "mgemm_bf16_256x256x64_w4x2_s1", {}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 4, 2, true, "mgemm_bf16_256x256x64_w4x2", {}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 2, 2, true, "mgemm_bf16_256x256x64_w2x2", {}),
        MGEMM_VARIANT_D(__bf16, 2, 256, 256, 64, 2, 2, true, 2, "mgemm_bf16_256x256x64_w2x2_d2", {}),
        // 128x128 with eight waves: four stages of 32 for one-round grids (the
        // deeper ring hides the loads of a lone workgroup), two of 64 when a CU
        // holds several workgroups
        MGEMM_VARIANT(__bf16, 2, 128, 128, 64, 2, 4, true, "mgemm_bf16_128x128x64_w2x4", {2.35f, 0.00964f, 1.65f, 1.07f},
                      MGEMM_SK16(__bf16, 128, 128, 64, 2, 4, true, 1)),
        MGEMM_VARIANT_D(__bf16, 2, 128, 128, 64, 2, 4, true, 2, "mgemm_bf16_128x128x64_w2x4_d2", {2.46f, 0.00829f, 1.65f, 1.39f},
                        MGEMM_SK16(__bf16, 128, 128, 64, 2, 4, true, 2)),
        // rows 4-byte aligned (and K even), every tile: 16-byte copies on all
        // but a tile's last slab, which takes 4-byte copies.  Estimates: a fit
        // on rows only 4-byte aligned (1.3 to 1.5 times the two-stage
        // siblings' time per K on the same box, bf16 and f16 alike).  On
        // 16-byte aligned rows with a K tail they beat the siblings' register
        // path by 1.3 to 1.65x (bf16 2048^2 x 2046: 28.3 against 44.1 us;
        // 3000^2 x 2998: 94.7 against 119.7; 4096^2 x 4094: 122.8 against
        // 163.3), which is what the siblings' register factors (1.6, 1.65;
        // 1.1 and 1.5 before) now say
        MGEMM_VARIANT_D(__bf16, 2, 128, 128, 64, 2, 2, false, 4, "mgemm_bf16_128x128x64_w2x2_d4_u",
                        {3.06f, 0.00845f, 1.0f, 1.55f},
                        MGEMM_SK16(__bf16, 128, 128, 64, 2, 2, false, 4)),
        MGEMM_VARIANT(__bf16, 2, 128, 128, 64, 2, 2, false, "mgemm_bf16_128x128x64_w2x2_u", {},
                      MGEMM_SK16(__bf16, 128, 128, 64, 2, 2, false, 1)),
        MGEMM_VARIANT(__bf16, 2, 64, 64, 64, 2, 2, true, "mgemm_bf16_64x64x64_w2x2", {0.44f, 0.00391f, 1.6f, 1.73f},
                      MGEMM_SK16(__bf16, 64, 64, 64, 2, 2, true, 1)),
        MGEMM_VARIANT_D(__bf16, 2, 64, 64, 64, 2, 2, true, 2, "mgemm_bf16_64x64x64_w2x2_d2", {0.45f, 0.00335f, 1.6f, 2.32f},
                        MGEMM_SK16(__bf16, 64, 64, 64, 2, 2, true, 2)),
        MGEMM_VARIANT_D(__bf16, 2, 64, 64, 64, 2, 2, false, 4, "mgemm_bf16_64x64x64_w2x2_d4_u",
                        {0.90f, 0.00427f, 1.0f, 2.2f},
                        MGEMM_SK16(__bf16, 64, 64, 64, 2, 2, false, 4)),
        MGEMM_VARIANT(__bf16, 2, 64, 64, 64, 2, 2, false, "mgemm_bf16_64x64x64_w2x2_u", {},
                      MGEMM_SK16(__bf16, 64, 64, 64, 2, 2, false, 1)),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
