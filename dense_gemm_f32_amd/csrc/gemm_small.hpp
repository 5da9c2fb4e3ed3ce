// Small fp32 problems (a few hundred in M, N and K): one workgroup per 16x16
// output tile, its W wavefronts sharing K.
//
// A 256^3 product has 16 tiles of 64x64; on 16 of 256 CUs its matrix-core
// time alone is some 3.4 us, and each slab waits on the previous one's loads.
// Here every CU takes one 16x16 tile (256 workgroups), and each of its four
// wavefronts (one per SIMD) a quarter of K: it loads its whole K range
// straight into registers at once (one latency), runs 16x16x4 fp32 MFMAs,
// and the four partial tiles are added through LDS in wave order, so the
// result does not depend on timing.  Blocking the product, loading operand
// tiles into fast memory and adding per-block partial sums is the block
// tiling of "cuda11/matmul" (section "V1 Tile版本") and of the CSDN
// tile-algorithm page; the K split across the waves of a block is this
// kernel's own.
//
// v_mfma_f32_16x16x4_f32, lane l (i = l % 16, g = l / 16):
//   A operand  A[i][slot g],  B operand  B[slot g][i],
//   result     register r of lane l is row 4g + r, column i.
// Slot g of MFMA s in chunk c of a wave carries k = kb + 32c + 8g + s, so
// each lane reads 8 consecutive k of its row (or column) per chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.hpp"

namespace mgemm {

namespace small {
constexpr int kTile = 16;
constexpr int kSlot = 8;              // consecutive k per lane group and chunk
constexpr int kChunk = 4 * kSlot;     // k per chunk (four lane groups)
}  // namespace small

// W wavefronts per workgroup; each takes at most NCH chunks of 32 k (the
// host keeps K <= W * NCH * 32).  Out-of-range rows, columns and k read as
// zero; C is read only when beta != 0.
template <int W, int NCH, bool TA, bool TB>
__global__ void __launch_bounds__(W * 64) gemm_small_kernel(KernelArgs p)
{
    using namespace small;
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    // one partial tile per wave; a row pitch of 20 floats puts the four lane
    // groups (rows 4 apart, 80 floats) 16 banks apart, so neither the writes
    // below nor the reads of the sum conflict
    __shared__ float red[W][kTile][kTile + 4];
    int bidx, tm, tn;
    map_tile(p, bidx, tm, tn);
    const int m0 = tm * kTile, n0 = tn * kTile;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, g = lane >> 4;
    const float *A = static_cast<const float *>(p.A) + (int64_t)bidx * p.strideA;
    const float *B = static_cast<const float *>(p.B) + (int64_t)bidx * p.strideB;
    // this wave's k range [kb, ke), a whole number of chunks deep
    const int kw = ((p.K + W - 1) / W + kChunk - 1) / kChunk * kChunk;
    const int kb = w * kw, ke = min(p.K, kb + kw);
    const int nch = ke > kb ? (ke - kb + kChunk - 1) / kChunk : 0;
    const int row = m0 + i, col = n0 + i;  // this lane's row of A and column of B
    const bool row_ok = row < p.M, col_ok = col < p.N;

    float a[NCH][kSlot], b[NCH][kSlot];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c < nch) {
#pragma unroll
            for (int s = 0; s < kSlot; ++s) {
                const int k = kb + c * kChunk + g * kSlot + s;
                const bool k_ok = k < ke;
                a[c][s] = (row_ok && k_ok) ? A[TA ? (int64_t)k * p.lda + row : (int64_t)row * p.lda + k] : 0.0f;
                b[c][s] = (col_ok && k_ok) ? B[TB ? (int64_t)col * p.ldb + k : (int64_t)k * p.ldb + col] : 0.0f;
            }
        }
    }
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c < nch) {
#pragma unroll
            for (int s = 0; s < kSlot; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c][s], b[c][s], acc, 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][4 * g + r][i] = acc[r];
    __syncthreads();
    // the tile's elements over the workgroup's threads; waves added in order
    for (int e = tid; e < kTile * kTile; e += W * 64) {
        const int er = e / kTile, ec = e % kTile;
        const int gr = m0 + er, gc = n0 + ec;
        if (gr >= p.M || gc >= p.N) continue;
        float sum = red[0][er][ec];
#pragma unroll
        for (int v = 1; v < W; ++v) sum += red[v][er][ec];
        float *cp = static_cast<float *>(p.C) + (int64_t)bidx * p.strideC + (int64_t)gr * p.ldc + gc;
        const float o = p.beta != 0.0f ? p.alpha * sum + p.beta * *cp : p.alpha * sum;
        __builtin_nontemporal_store(o, cp);
    }
}

}  // namespace mgemm
