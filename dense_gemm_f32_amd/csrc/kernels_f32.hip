// fp32 (SGEMM) kernel variants: v_mfma_f32_32x32x2_f32, 32-float K-slabs.
#include "variants.hpp"

namespace mgemm {

const Variant *f32_variants(int *count)
{
    // Chosen by the lowest estimated time (Cost in variants.hpp: t0 us, tk us
    // per unit of K, register-path factor, one-round factor); a build without
    // an estimate runs only when forced or when no estimated build fits.
    // Rounds: 256x256 0.234 us per K (0.91 of the matrix peak per CU),
    // 128x128 0.0605 (0.88), 64x64 two-stage 0.0166 (0.80).  The 4-byte-copy
    // builds copy all but a tile's last slab 16 bytes at a time: on the same
    // box their rate per K matched their aligned siblings' within 2% (odd
    // leading dimensions, 1024^2 to 6144^2, K 256 to 4096), with 0.7 (64x64)
    // and 1.4 us (128x128) more per round; their estimates are the
    // siblings' with that added (with 4-byte copies throughout they were
    // 0.0658 and 0.0185).  The 64x64 tiles lose per flop but win where the
    // larger tiles leave a last round mostly empty (4608^3: 324 tiles of
    // 256x256 are two rounds, 5184 of 64x64 twenty-one).  The 64x64 two-stage
    // build's register factor is its one-round figure (1000^3: 39 us against
    // 26 us for 1024^3 on the DMA path); over several rounds it measured 1.2
    // to 1.3, where the 4-byte-copy build is faster still.
    static const Variant table[] = {
        MGEMM_VARIANT_F32(256, 256, 32, 4, 2, true, "mgemm_f32_256x256x32_w4x2", {13.9f, 0.2344f, 1.10f, 1.0f}),
        MGEMM_VARIANT_F32(256, 256, 32, 2, 2, true, "mgemm_f32_256x256x32_w2x2", {}),
        MGEMM_VARIANT_F32(128, 128, 32, 2, 2, true, "mgemm_f32_128x128x32_w2x2", {6.6f, 0.0605f, 1.15f, 1.25f},
                          MGEMM_SK(float, 128, 128, 32, 2, 2, true, 1)),
        MGEMM_VARIANT_F32_D(128, 128, 32, 2, 2, false, 4, "mgemm_f32_128x128x32_w2x2_d4_u",
                            {8.0f, 0.0606f, 1.0f, 1.2f}, MGEMM_SK(float, 128, 128, 32, 2, 2, false, 4)),
        MGEMM_VARIANT_F32(128, 128, 32, 2, 2, false, "mgemm_f32_128x128x32_w2x2_u", {},
                          MGEMM_SK(float, 128, 128, 32, 2, 2, false, 1)),
        // 64x64: two stages of 32 (one barrier per 16 MFMAs) measured 9-14%
        // faster than four of 16 at 512^3 to 2048^3 (deeper rings of 8 or 16
        // stages gained nothing)
        MGEMM_VARIANT_F32_D(64, 64, 32, 2, 2, true, 2, "mgemm_f32_64x64x32_w2x2_d2", {2.1f, 0.0166f, 1.5f, 1.4f},
                            MGEMM_SK(float, 64, 64, 32, 2, 2, true, 2)),
        // (four stages of 32 with 4-byte copies, ragged 1000x1027x999: one pass
        // 49.0 against 50.6 us, stream-K 36.4 against 37.8, split-K 44.2
        // against 39.9; not kept)
        MGEMM_VARIANT_F32_D(64, 64, 32, 2, 2, false, 4, "mgemm_f32_64x64x32_w2x2_d4_u",
                            {2.8f, 0.0168f, 1.0f, 1.6f}, MGEMM_SK(float, 64, 64, 32, 2, 2, false, 4)),
        MGEMM_VARIANT_F32(64, 64, 32, 2, 2, false, "mgemm_f32_64x64x32_w2x2_u", {},
                          MGEMM_SK(float, 64, 64, 32, 2, 2, false, 1)),
        // small problems: 16x16 tiles, the waves of a workgroup sharing K
        // (t0 + max(tk*K, tw*W*K) us).  Measured per call from HIP-graph
        // replays, against the 64x64 build the model picked before: 256^3 4.2
        // against 7.5 us, 128^3 3.2 against 5.1, 256x256x1024 10.0 against
        // 21.8; the 64x64 build stays ahead at 512^3 (12.3 against 17.3) and
        // 512x512x256 (7.6 against 9.7), where the 16x16 grid is four times
        // larger than one CU-filling round
        MGEMM_VARIANT_F32_SMALL(4, 2, "mgemm_f32_16x16_k4w_256", {2.2f, 0.0076f, 1.0f, 1.0f, 3.05e-5f}),
        MGEMM_VARIANT_F32_SMALL(8, 4, "mgemm_f32_16x16_k8w_1024", {2.2f, 0.0076f, 1.0f, 1.0f, 3.05e-5f}),
    };
    *count = sizeof(table) / sizeof(table[0]);
    return table;
}

}  // namespace mgemm
