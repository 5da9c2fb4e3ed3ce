// Measurement aid for bench.py (not a GEMM entry point): the throughput of the
// 16-bit and int8 matrix cores with no memory traffic, on operand values the
// caller supplies.  Under sustained load the part runs at a power-limited clock that
// depends on what the multipliers see, so this gives, on the same board and
// for the same data distribution as a GEMM workload, the rate that no GEMM
// moving data between HBM, L2 and LDS can exceed.
//
// 256 workgroups of four wavefronts (one per SIMD of every CU).  Each wave
// loads 32 operand fragments once (4 k-groups x (4 A + 4 B)), then issues
// `iters` x 64 v_mfma_f32_32x32x16_{bf16,f16} (or v_mfma_i32_32x32x32_i8,
// int32 accumulate) into 16 independent accumulators (the MFMA order of a
// 128x128 wave tile), and finally writes one sum per lane so that nothing is
// optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/mgemm_diag.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWorkgroups = 256, kWaves = 4, kFrags = 32;

// KIND: 0 binary16, 1 bfloat16, 2 int8
template <int KIND>
__global__ void __launch_bounds__(256) mfma_ceiling(const u32x4 *src, float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
    u32x4 a[4][4], b[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a[g][t] = src[((size_t)wave * kFrags + g * 8 + t) * 64 + lane];
            b[g][t] = src[((size_t)wave * kFrags + g * 8 + 4 + t) * 64 + lane];
        }
    using Acc = typename std::conditional<KIND == 2, i32x16, f32x16>::type;
    Acc acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][u] = Acc{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (KIND == 2)
                        acc[t][u] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            __builtin_bit_cast(i32x4, a[g][t]), __builtin_bit_cast(i32x4, b[g][u]), acc[t][u], 0, 0, 0);
                    else if constexpr (KIND == 1)
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a[g][t]), __builtin_bit_cast(bf16x8, b[g][u]), acc[t][u], 0, 0, 0);
                    else
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, a[g][t]), __builtin_bit_cast(f16x8, b[g][u]), acc[t][u], 0, 0, 0);
                }
    }
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += (float)acc[t][u][r];
    out[(size_t)wave * 64 + lane] = s;
}

}  // namespace

extern "C" {

int64_t mgemm_diag_ceiling_operand_bytes(void) { return (int64_t)kWorkgroups * kWaves * kFrags * 64 * 16; }

int64_t mgemm_diag_ceiling_out_floats(void) { return (int64_t)kWorkgroups * kWaves * 64; }

double mgemm_diag_ceiling_flop(int iters) { return (double)kWorkgroups * kWaves * iters * 64 * 32768.0; }

double mgemm_diag_ceiling_ops(int kind, int iters)
{
    return (kind == MGEMM_DIAG_I8 ? 2.0 : 1.0) * mgemm_diag_ceiling_flop(iters);
}

int mgemm_diag_mfma_ceiling(int kind, const void *operands, float *out, int iters, hipStream_t stream)
{
    if (operands == nullptr || out == nullptr || iters <= 0) return 1;
    if (kind != MGEMM_DIAG_F16 && kind != MGEMM_DIAG_BF16 && kind != MGEMM_DIAG_I8) return 1;
    const u32x4 *src = static_cast<const u32x4 *>(operands);
    if (kind == MGEMM_DIAG_I8)
        hipLaunchKernelGGL(mfma_ceiling<2>, dim3(kWorkgroups), dim3(64 * kWaves), 0, stream, src, out, iters);
    else if (kind == MGEMM_DIAG_BF16)
        hipLaunchKernelGGL(mfma_ceiling<1>, dim3(kWorkgroups), dim3(64 * kWaves), 0, stream, src, out, iters);
    else
        hipLaunchKernelGGL(mfma_ceiling<0>, dim3(kWorkgroups), dim3(64 * kWaves), 0, stream, src, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
