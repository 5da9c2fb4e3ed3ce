// bf16-input kernel variants: v_mfma_f32_32x32x16_bf16, fp32 accumulate, 64-element K-slabs.
#include "variants.hpp"

namespace mgemm {

const Variant *bf16_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp: t0 us, tk us
    // per unit of K, register-path factor, one-round factor), fitted on bf16
    // (the two 16-bit types run the same kernels at the same rates): the
    // 256x256 two-stage tile 0.0236 us per K per round (0.57 of the matrix
    // peak per CU), 128x128 0.0085 (0.39), 64x64 0.0040 (0.21).  K <= 128
    // (store-bound) takes the 256x256 4x2-wave tile first.  Builds without
    // an estimate run when forced, or by preference order when no estimated
    // build fits (unaligned rows: 4-byte copies first).
    static const Variant table[] = {
        MGEMM_VARIANT_D(__bf16, 2, 256, 256, 64, 2, 4, true, 2, "mgemm_bf16_256x256x64_w2x4_d2", {11.1f, 0.02356f, 1.6f, 1.0f}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 2, 4, true, "mgemm_bf16_256x256x64_w2x4", {}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 4, 2, true, "mgemm_bf16_256x256x64_w4x2", {}),
        MGEMM_VARIANT(__bf16, 2, 256, 256, 64, 2, 2, true, "mgemm_bf16_256x256x64_w2x2", {}),
        MGEMM_VARIANT_D(__bf16, 2, 256, 256, 64, 2, 2, true, 2, "mgemm_bf16_256x256x64_w2x2_d2", {}),
        MGEMM_VARIANT(__bf16, 2, 128, 128, 64, 2, 2, true, "mgemm_bf16_128x128x64_w2x2", {2.34f, 0.00852f, 1.5f, 1.27f}),
        // rows 4-byte aligned (and K even): 4-byte copies into LDS, every tile
        MGEMM_VARIANT_D(__bf16, 2, 128, 128, 64, 2, 2, false, 4, "mgemm_bf16_128x128x64_w2x2_d4_u", {}),
        MGEMM_VARIANT(__bf16, 2, 128, 128, 64, 2, 2, false, "mgemm_bf16_128x128x64_w2x2_u", {}),
        MGEMM_VARIANT(__bf16, 2, 64, 64, 64, 2, 2, true, "mgemm_bf16_64x64x64_w2x2", {0.41f, 0.00402f, 1.1f, 2.28f}),
        MGEMM_VARIANT_D(__bf16, 2, 64, 64, 64, 2, 2, false, 4, "mgemm_bf16_64x64x64_w2x2_d4_u", {}),
        MGEMM_VARIANT(__bf16, 2, 64, 64, 64, 2, 2, false, "mgemm_bf16_64x64x64_w2x2_u", {}),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
