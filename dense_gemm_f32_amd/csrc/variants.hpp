// Registry of compiled GEMM kernel variants (one per tile shape and
// alignment class; each holds the four transpose combinations).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_f64.hpp"
#include "gemm_kernel.hpp"
#include "gemm_small.hpp"

namespace mgemm {

using LaunchFn = hipError_t (*)(const KernelArgs &, unsigned grid, hipStream_t);

// Time model of one build, for the automatic choice: a CU runs its share of the
// workgroups one after another, so a launch of W workgroups takes ceil(W/256)
// "rounds" of t0 + tk*K microseconds on 256 CUs.  reg multiplies the round when
// the tiles take the range-checked register path (a K that is no multiple of
// 16 bytes, or offsets past 32 bits).  solo multiplies a
// launch of one round: a CU holding a single workgroup cannot hide one
// workgroup's load latency behind another's MFMAs.  Measured on MI355X by
// forcing each build over square and oblong shapes from 512 to 8192 (t0, tk:
// least squares over the launches of at least two rounds; solo: launches of
// 256 workgroups).  tk == 0: no estimate; such a build runs only when asked
// for by name or when no estimated build fits.
// Small-problem builds (pipe 6) have workgroups of a few dozen registers that
// share CUs, so rounds do not apply: their launch takes t0 + max(tk*K, tw*W*K)
// us for W workgroups, the longer of one workgroup's load-then-multiply chain
// and the whole launch's rate (measured from HIP-graph replays over shapes
// from 64^3 to 1024x1024x256).
struct Cost {
    float t0, tk, reg, solo;
    float tw = 0.0f;  // us per workgroup per unit of K (pipe 6 only)
};

struct Variant {
    int dtype;            // mgemm_dtype of A and B
    int bm, bn, bk;       // workgroup tile and K-slab
    int wm, wn;           // wavefront grid
    bool vec;             // needs 16-byte aligned A/B rows (dwordx4 loads)
    int pipe;             // DMA-path schedule (1: 4 stages of bk/2, 2: 2 stages of bk,
                          // 3: 1 stage of bk, K <= bk only, 4: rows 4-byte aligned, 2
                          // stages of bk, 16-byte copies but 4-byte ones on a tile's last
                          // slab, every tile); 6: small-problem kernel (gemm_small.hpp,
                          // registers only, K <= bk, wn waves sharing K)
    const char *name;
    LaunchFn fn[2][2];    // [transA][transB], fp32 C (int32 C for int8, double C for fp64 inputs)
    LaunchFn fn16[2][2];  // [transA][transB], C in the inputs' 16-bit type (16-bit tables only)
    Cost cost;            // zero: no estimate
    LaunchFn sk[2][2];    // stream-K launch of the same tile, fp32 C (int32 for int8); null: none
    LaunchFn sk16[2][2];  // stream-K launch with C in the inputs' 16-bit type (16-bit tables only)
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V, int D, typename CT>
hipError_t launch_gemm(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    KernelArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<T, BM, BN, BK, WM, WN, TA, TB, V, D, CT>),
                           dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V, int D, typename CT>
hipError_t launch_gemm_sk(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    KernelArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_sk_kernel<T, BM, BN, BK, WM, WN, TA, TB, V, D, CT>),
                           dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

template <int W, int NCH, bool TA, bool TB>
hipError_t launch_gemm_small(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    KernelArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_small_kernel<W, NCH, TA, TB>), dim3(grid),
                           dim3(W * 64), args, 0, s);
}

template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V>
hipError_t launch_gemm_f64(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    KernelArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f64_kernel<BM, BN, BK, WM, WN, TA, TB, V>),
                           dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V>
hipError_t launch_gemm_f64_sk(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    KernelArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f64_sk_kernel<BM, BN, BK, WM, WN, TA, TB, V>),
                           dim3(grid), dim3(WM * WN * 64), args, 0, s);
}

// stream-K launchers of an fp64 build (the trailing argument after its Cost)
#define MGEMM_SK_F64(BM, BN, BK, WM, WN, V)                                                  \
    {{launch_gemm_f64_sk<BM, BN, BK, WM, WN, false, false, V>,                               \
      launch_gemm_f64_sk<BM, BN, BK, WM, WN, false, true, V>},                               \
     {launch_gemm_f64_sk<BM, BN, BK, WM, WN, true, false, V>,                                \
      launch_gemm_f64_sk<BM, BN, BK, WM, WN, true, true, V>}}

// fp64 inputs: double C
#define MGEMM_VARIANT_F64(BM, BN, BK, WM, WN, V, NAME, ...)                                  \
    {5, BM, BN, BK, WM, WN, V, 1, NAME,                                                      \
     {{launch_gemm_f64<BM, BN, BK, WM, WN, false, false, V>,                                \
       launch_gemm_f64<BM, BN, BK, WM, WN, false, true, V>},                                \
      {launch_gemm_f64<BM, BN, BK, WM, WN, true, false, V>,                                 \
       launch_gemm_f64<BM, BN, BK, WM, WN, true, true, V>}},                                \
     {{nullptr, nullptr}, {nullptr, nullptr}}, __VA_ARGS__}

#define MGEMM_LAUNCHERS(T, BM, BN, BK, WM, WN, V, D, CT)                                     \
    {{launch_gemm<T, BM, BN, BK, WM, WN, false, false, V, D, CT>,                            \
      launch_gemm<T, BM, BN, BK, WM, WN, false, true, V, D, CT>},                            \
     {launch_gemm<T, BM, BN, BK, WM, WN, true, false, V, D, CT>,                             \
      launch_gemm<T, BM, BN, BK, WM, WN, true, true, V, D, CT>}}

// The trailing argument of each macro is the build's Cost, {t0, tk, reg, solo}
// ({}: no estimate), optionally followed by its stream-K launchers
// (MGEMM_SK, MGEMM_SK16 for both C types of 16-bit inputs, MGEMM_SK_I8 /
// MGEMM_SK_I8_ALL, MGEMM_SK_F64; omitted: none).
#define MGEMM_SK_C(T, BM, BN, BK, WM, WN, V, D, CT)                                          \
    {{launch_gemm_sk<T, BM, BN, BK, WM, WN, false, false, V, D, CT>,                         \
      launch_gemm_sk<T, BM, BN, BK, WM, WN, false, true, V, D, CT>},                         \
     {launch_gemm_sk<T, BM, BN, BK, WM, WN, true, false, V, D, CT>,                          \
      launch_gemm_sk<T, BM, BN, BK, WM, WN, true, true, V, D, CT>}}
#define MGEMM_SK(T, BM, BN, BK, WM, WN, V, D) MGEMM_SK_C(T, BM, BN, BK, WM, WN, V, D, float)
// 16-bit inputs: stream-K with fp32 C, then with C in the inputs' own type
#define MGEMM_SK16(T, BM, BN, BK, WM, WN, V, D)                                              \
    MGEMM_SK_C(T, BM, BN, BK, WM, WN, V, D, float), MGEMM_SK_C(T, BM, BN, BK, WM, WN, V, D, T)
#define MGEMM_SK_I8(BM, BN, BK, WM, WN, V, D)                                                 \
    {{nullptr, launch_gemm_sk<int8_t, BM, BN, BK, WM, WN, false, true, V, D, int32_t>},       \
     {nullptr, nullptr}}
#define MGEMM_SK_I8_ALL(BM, BN, BK, WM, WN, V, D)                                             \
    {{launch_gemm_sk<int8_t, BM, BN, BK, WM, WN, false, false, V, D, int32_t>,                \
      launch_gemm_sk<int8_t, BM, BN, BK, WM, WN, false, true, V, D, int32_t>},                \
     {launch_gemm_sk<int8_t, BM, BN, BK, WM, WN, true, false, V, D, int32_t>,                 \
      launch_gemm_sk<int8_t, BM, BN, BK, WM, WN, true, true, V, D, int32_t>}}
// small fp32 problems: 16x16 tiles, W waves sharing K <= W * NCH * 32 (pipe 6)
#define MGEMM_VARIANT_F32_SMALL(W, NCH, NAME, ...)                                          \
    {0, 16, 16, (W) * (NCH) * 32, 1, W, false, 6, NAME,                                      \
     {{launch_gemm_small<W, NCH, false, false>, launch_gemm_small<W, NCH, false, true>},     \
      {launch_gemm_small<W, NCH, true, false>, launch_gemm_small<W, NCH, true, true>}},      \
     {{nullptr, nullptr}, {nullptr, nullptr}}, __VA_ARGS__}

// fp32 inputs: fp32 C only
#define MGEMM_VARIANT_F32_D(BM, BN, BK, WM, WN, V, D, NAME, ...)                              \
    {0, BM, BN, BK, WM, WN, V, D, NAME, MGEMM_LAUNCHERS(float, BM, BN, BK, WM, WN, V, D, float), \
     {{nullptr, nullptr}, {nullptr, nullptr}}, __VA_ARGS__}
#define MGEMM_VARIANT_F32(BM, BN, BK, WM, WN, V, NAME, ...) \
    MGEMM_VARIANT_F32_D(BM, BN, BK, WM, WN, V, 1, NAME, __VA_ARGS__)

// int8 inputs: int32 C; every transpose (_ALL), or A K-contiguous (op N) and
// B K-contiguous (op T) only (tiles whose MN-contiguous LDS rows, 64 bytes,
// are too short for the transposing layout)
#define MGEMM_VARIANT_I8_ALL(BM, BN, BK, WM, WN, V, D, NAME, ...)                            \
    {3, BM, BN, BK, WM, WN, V, D, NAME, MGEMM_LAUNCHERS(int8_t, BM, BN, BK, WM, WN, V, D, int32_t), \
     {{nullptr, nullptr}, {nullptr, nullptr}}, __VA_ARGS__}
#define MGEMM_VARIANT_I8(BM, BN, BK, WM, WN, V, D, NAME, ...)                                \
    {3, BM, BN, BK, WM, WN, V, D, NAME,                                                      \
     {{nullptr, launch_gemm<int8_t, BM, BN, BK, WM, WN, false, true, V, D, int32_t>},         \
      {nullptr, nullptr}},                                                                   \
     {{nullptr, nullptr}, {nullptr, nullptr}}, __VA_ARGS__}

// 16-bit inputs: fp32 C or C of the input type
#define MGEMM_VARIANT_D(T, DT, BM, BN, BK, WM, WN, V, D, NAME, ...)                          \
    {DT, BM, BN, BK, WM, WN, V, D, NAME, MGEMM_LAUNCHERS(T, BM, BN, BK, WM, WN, V, D, float), \
     MGEMM_LAUNCHERS(T, BM, BN, BK, WM, WN, V, D, T), __VA_ARGS__}

#define MGEMM_VARIANT(T, DT, BM, BN, BK, WM, WN, V, NAME, ...) \
    MGEMM_VARIANT_D(T, DT, BM, BN, BK, WM, WN, V, 1, NAME, __VA_ARGS__)

// Host-side variant tables, one per input type (function-local statics, so
// that the device compilation never sees the host launch pointers).
const Variant *f32_variants(int *count);
const Variant *f16_variants(int *count);
const Variant *bf16_variants(int *count);
const Variant *i8_variants(int *count);
const Variant *f64_variants(int *count);

hipError_t launch_scale_c(int c_dtype, void *C, int M, int N, int64_t ldc, int64_t strideC, int batch,
                          double beta, int beta_i, hipStream_t s);

hipError_t launch_splitk_reduce(int c_dtype, const void *W, int splits, int M, int N, void *C,
                                int64_t ldc, double alpha, double beta, int alpha_i, int beta_i,
                                hipStream_t s);

}  // namespace mgemm
