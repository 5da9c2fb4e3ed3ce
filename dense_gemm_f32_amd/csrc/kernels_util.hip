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
