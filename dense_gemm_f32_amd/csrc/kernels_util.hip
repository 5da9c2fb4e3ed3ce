// C = beta * C for the alpha == 0 and K == 0 cases (fp32, 16-bit, int32 or
// double C).  beta arrives as a double; for fp32 and 16-bit C it is a float
// widened on the host, and the product is formed in fp32 as before.
#include "variants.hpp"

namespace mgemm {

template <typename CT>
__global__ void __launch_bounds__(256) scale_c_kernel(CT *C, int M, int N, int64_t ldc,
                                                      int64_t strideC, int batch, double beta,
                                                      int beta_i)
{
    const int64_t total = (int64_t)batch * M * N;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        const int64_t b = e / ((int64_t)M * N);
        const int64_t rem = e - b * M * N;
        const int64_t i = rem / N, j = rem - i * N;
        CT *c = C + b * strideC + i * ldc + j;
        if constexpr (__is_same(CT, int32_t))  // int32 C: wrapping integer product
            __builtin_nontemporal_store(beta_i == 0 ? 0 : (int32_t)((uint32_t)beta_i * (uint32_t)*c), c);
        else if constexpr (__is_same(CT, double))
            __builtin_nontemporal_store(beta == 0.0 ? 0.0 : beta * *c, c);
        else
            __builtin_nontemporal_store((CT)(beta == 0.0 ? 0.0f : (float)beta * (float)*c), c);
    }
}

// Split-K reduction: C = alpha * sum_z W[z] + beta * C over the M x N output,
// with W = [splits][M][N] partial products (fp32 for fp32/16-bit inputs,
// int32 for int8, double for fp64).  The chunks are summed in ascending z,
// so the result does not depend on the launch.  C is read only when
// beta != 0; 16-bit C is rounded to nearest even, int32 wraps.
template <typename WT, typename CT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const WT *W, int splits, int M, int N,
                                                            CT *C, int64_t ldc, double alpha,
                                                            double beta, int alpha_i, int beta_i)
{
    const int64_t total = (int64_t)M * N;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        const int64_t i = e / N, j = e - i * N;
        CT *c = C + i * ldc + j;
        if constexpr (__is_same(WT, int32_t)) {
            uint32_t acc = 0;
            for (int z = 0; z < splits; ++z) acc += (uint32_t)__builtin_nontemporal_load(W + z * total + e);
            uint32_t o = (uint32_t)alpha_i * acc;
            if (beta_i != 0) o += (uint32_t)beta_i * (uint32_t)*c;
            __builtin_nontemporal_store((int32_t)o, c);
        } else if constexpr (__is_same(WT, double)) {
            double acc = 0.0;
            for (int z = 0; z < splits; ++z) acc += __builtin_nontemporal_load(W + z * total + e);
            double o = alpha * acc;
            if (beta != 0.0) o += beta * *c;
            __builtin_nontemporal_store(o, c);
        } else {
            float acc = 0.0f;
            for (int z = 0; z < splits; ++z) acc += __builtin_nontemporal_load(W + z * total + e);
            float o = (float)alpha * acc;
            if (beta != 0.0) o += (float)beta * (float)*c;
            __builtin_nontemporal_store((CT)o, c);
        }
    }
}

// Stream-K fix-up.  Workgroup (t, y) takes elements 1024y .. 1024y+1023 of
// tile t (row-major in the tile), four adjacent ones per thread, so that
// the partial tiles stream in with many loads in flight.  Tile t holds
// iterations a = t*iters .. z = a + iters - 1; the workgroups whose shares
// hold them are g0 = owner(a) .. g1 = owner(z), where owner(x), the largest
// g with T*g/G <= x, is ((x+1)*G - 1) / T.  With g0 == g1 the tile was whole
// and is in C already.  Otherwise its partials are g0's slot 0 if g0's share
// starts at a, else its slot 1, then slot 0 of g0+1 .. g1, summed in that
// order (ascending K); then alpha and beta (C read only when beta != 0) as
// in the one-pass epilogue.  int32 wraps.
template <typename PT, typename CT>
__global__ void __launch_bounds__(256) sk_fixup_kernel(KernelArgs p, int bm, int bn)
{
    using AT = typename std::conditional<__is_same(PT, int32_t), uint32_t, float>::type;
    using V4 = typename std::conditional<__is_same(PT, int32_t), i32x4, f32x4>::type;
    const int tile = blockIdx.x;
    const int64_t T = p.sk_total, G = p.sk_grid;
    const int64_t a = (int64_t)tile * p.sk_iters, z = a + p.sk_iters - 1;
    const int64_t g0 = ((a + 1) * G - 1) / T, g1 = ((z + 1) * G - 1) / T;
    const int e = (blockIdx.y * blockDim.x + threadIdx.x) * 4;  // bn is a multiple of 4
    if (g0 == g1 || e >= bm * bn) return;
    int b, tm, tn;
    tile_coords(p, tile, b, tm, tn);
    const int i = e / bn, j = e - i * bn;
    const int row = tm * bm + i, col = tn * bn + j;
    if (row >= p.M || col >= p.N) return;
    const int64_t tsz = (int64_t)bm * bn;
    const PT *part = static_cast<const PT *>(p.sk_part);
    const int first_slot = T * g0 / G == a ? 0 : 1;
    const V4 v0 = *reinterpret_cast<const V4 *>(part + (g0 * 2 + first_slot) * tsz + e);
    AT s[4] = {(AT)v0[0], (AT)v0[1], (AT)v0[2], (AT)v0[3]};
    for (int64_t g = g0 + 1; g <= g1; ++g) {
        const V4 v = *reinterpret_cast<const V4 *>(part + g * 2 * tsz + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] += (AT)v[u];
    }
    CT *cp = static_cast<CT *>(p.C) + (int64_t)b * p.strideC + (int64_t)row * p.ldc + col;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (col + u >= p.N) break;
        if constexpr (__is_same(CT, int32_t)) {
            uint32_t v = (uint32_t)p.alpha_i * s[u];
            if (p.beta_i != 0) v += (uint32_t)p.beta_i * (uint32_t)cp[u];
            cp[u] = (int32_t)v;
        } else {
            float v = p.alpha * s[u];
            if (p.beta != 0.0f) v = v + p.beta * (float)cp[u];
            cp[u] = (CT)v;
        }
    }
}

hipError_t launch_sk_fixup(int c_dtype, const KernelArgs &a, int bm, int bn, unsigned tiles, hipStream_t s)
{
    if (tiles == 0) return hipSuccess;
    KernelArgs copy = a;
    int bm_ = bm, bn_ = bn;
    void *args[] = {&copy, &bm_, &bn_};
    const void *fn = c_dtype == 4 ? reinterpret_cast<const void *>(&sk_fixup_kernel<int32_t, int32_t>)
                                  : reinterpret_cast<const void *>(&sk_fixup_kernel<float, float>);
    return hipLaunchKernel(fn, dim3(tiles, (unsigned)((bm * bn + 1023) / 1024)), dim3(256), args, 0, s);
}

hipError_t launch_splitk_reduce(int c_dtype, const void *W, int splits, int M, int N, void *C,
                                int64_t ldc, double alpha, double beta, int alpha_i, int beta_i,
                                hipStream_t s)
{
    const int64_t total = (int64_t)M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    void *args[] = {&W, &splits, &M, &N, &C, &ldc, &alpha, &beta, &alpha_i, &beta_i};
    const void *fn = c_dtype == 1   ? reinterpret_cast<const void *>(&splitk_reduce_kernel<float, _Float16>)
                     : c_dtype == 2 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<float, __bf16>)
                     : c_dtype == 4 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<int32_t, int32_t>)
                     : c_dtype == 5 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<double, double>)
                                    : reinterpret_cast<const void *>(&splitk_reduce_kernel<float, float>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

hipError_t launch_scale_c(int c_dtype, void *C, int M, int N, int64_t ldc, int64_t strideC, int batch,
                          double beta, int beta_i, hipStream_t s)
{
    const int64_t total = (int64_t)batch * M * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    void *args[] = {&C, &M, &N, &ldc, &strideC, &batch, &beta, &beta_i};
    const void *fn = c_dtype == 1   ? reinterpret_cast<const void *>(&scale_c_kernel<_Float16>)
                     : c_dtype == 2 ? reinterpret_cast<const void *>(&scale_c_kernel<__bf16>)
                     : c_dtype == 4 ? reinterpret_cast<const void *>(&scale_c_kernel<int32_t>)
                     : c_dtype == 5 ? reinterpret_cast<const void *>(&scale_c_kernel<double>)
                                    : reinterpret_cast<const void *>(&scale_c_kernel<float>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

}  // namespace mgemm
