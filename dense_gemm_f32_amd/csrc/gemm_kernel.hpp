// Templated MFMA GEMM kernel family for gfx950 (CDNA4, wave64).
//
//     C = alpha * op(A) * op(B) + beta * C        (row-major, fp32 C)
//
// The GEMM form and the row-major convention are those of "Sgemm [128,128,8]"
// (jianshu, the kernel's design comment).  Design ideas kept from the pages,
// re-done for CDNA4:
//   * block tiling with a K-slab staged in on-chip memory ("cuda11/matmul",
//     section "V1 Tile版本") -> LDS tiles;
//   * 16-byte vector global accesses ("V2 Tile"; the float4 loads of the
//     jianshu kernel) -> dwordx4 loads and 16-byte LDS writes/reads;
//   * a transposed on-chip tile so that a thread reads several rows with one
//     vector access ("V3 双缓冲", the transposed SA; jianshu's transposed A)
//     -> the fp32 "MN-contiguous" LDS layout read with ds_read_b128;
//   * double buffering with the next slab fetched to registers while the
//     current one is consumed, one barrier per slab ("V3 双缓冲"; the
//     jianshu kernel's two shared stages and peeled tail);
//   * zero-filled residual tiles and guarded stores (the CSDN tile-algorithm
//     page, "使用CUDA和瓦片算法计算矩阵乘法", MatrixMulCUDA);
//   * grouped tile ordering for cache reuse ("cuda11/matmul", Triton
//     section) -> XCD-aware workgroup rasterisation.
// What replaces the NVIDIA-era pieces: the per-thread 8x8 FMA micro-tile and
// the WMMA fragments become 32x32 MFMA blocks per wavefront
// (v_mfma_f32_32x32x2_f32 for fp32, v_mfma_f32_32x32x16_{f16,bf16} for
// 16-bit inputs), with fp32 accumulators held in registers.
//
// MFMA operand/result placement used below (wave64, lane l, i' = l % 32,
// h = l / 32):
//   32x32x2 f32 : lane supplies A[i'][k_h] and B[k_h][i'] (one value each);
//   32x32x16    : lane supplies 8 values A[i'][k in group h] and B[k][i'];
//   result      : accumulator element r (0..15) of lane l is row
//                 8*(r/4) + 4*h + r%4, column i'.
// Only the result placement and "lanes index rows of A / columns of B" matter:
// a sum over k does not depend on which k each (h, element) slot carries, as
// long as A and B agree, so the kernel assigns k to slots to suit its LDS
// layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Everything a GEMM launch needs; built on the host after validation.
struct KernelArgs {
    const void *A;
    const void *B;
    float *C;
    int64_t lda, ldb, ldc;
    int64_t strideA, strideB, strideC;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;      // tile rows per raster group
    float alpha, beta;
    int c_vec;        // C pointer/ldc/strideC allow 16-byte accesses
};

// ---------------------------------------------------------------------------
// Workgroup -> (batch, tile row, tile column).
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  The id is first remapped so that every XCD receives one
// contiguous range of logical ids, and that range is walked in groups of
// `group_m` tile rows, so the tiles resident on one XCD share A rows and B
// columns in its L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void map_tile(const KernelArgs &p, int &b, int &tm, int &tn)
{
    const int nwg = gridDim.x;
    const int w = blockIdx.x;
    const int q = nwg >> 3, rem = nwg & 7;
    const int x = w & 7, i = w >> 3;
    const int L = x * q + min(x, rem) + i;
    const int per_b = p.tiles_m * p.tiles_n;
    b = L / per_b;
    const int t = L - b * per_b;
    const int width = p.group_m * p.tiles_n;
    const int g = t / width;
    const int first = g * p.group_m;
    const int gsz = min(p.tiles_m - first, p.group_m);
    const int w2 = t - g * width;
    tm = first + w2 % gsz;
    tn = w2 / gsz;
}

template <int BYTES> struct RawOf;
template <> struct RawOf<16> { using type = u32x4; };
template <> struct RawOf<4> { using type = uint32_t; };
template <> struct RawOf<2> { using type = uint16_t; };

// K-contiguous LDS tile: ROWS rows of BK elements (one row = ROWB bytes =
// NCH 16-byte chunks).  Chunk c of row r is stored at chunk c ^ ((r/IL) % NCH),
// where IL is the operand's sub-tile interleave: lanes i' = 0..7 of a fragment
// read rows IL*i' + t, which land in 8 distinct chunk columns.
template <int ROWB, int IL>
__device__ __forceinline__ int kc_off(int row, int kbyte)
{
    constexpr int NCH = ROWB / 16;
    const int chunk = (kbyte >> 4) ^ ((row / IL) & (NCH - 1));
    return row * ROWB + (chunk << 4) + (kbyte & 15);
}

// ---------------------------------------------------------------------------
// Global -> register loader for one operand tile of one K-slab.
// The tile is R memory rows by CC contiguous elements; each of the NT threads
// owns NPT vectors of VEC elements, consecutive threads owning consecutive
// vectors of a row (coalesced).  Out-of-range elements are loaded as 0.
// ---------------------------------------------------------------------------
template <int ES, int R, int CC, int VEC, int NT>
struct TileLoader {
    static constexpr int VPR = CC / VEC;
    static constexpr int NV = R * VPR;
    static constexpr int NPT = NV / NT;
    static_assert(NV % NT == 0, "tile not divisible among threads");
    using Raw = typename RawOf<VEC * ES>::type;
    Raw regs[NPT];

    __device__ __forceinline__ static int row_of(int tid, int q) { return (tid + q * NT) / VPR; }
    __device__ __forceinline__ static int col_of(int tid, int q) { return ((tid + q * NT) % VPR) * VEC; }

    // base points at memory element (r0, c0); rows < rlim and cols < clim are in range
    // (limits already relative to r0/c0).  `full` = the whole tile is in range.
    __device__ __forceinline__ void load(const char *base, int64_t ld, int rlim, int clim,
                                         bool full, int tid)
    {
        if (full) {
#pragma unroll
            for (int q = 0; q < NPT; ++q) {
                const int r = row_of(tid, q), c = col_of(tid, q);
                regs[q] = *reinterpret_cast<const Raw *>(base + ((int64_t)r * ld + c) * ES);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NPT; ++q) {
                const int r = row_of(tid, q), c = col_of(tid, q);
                const char *ptr = base + ((int64_t)r * ld + c) * ES;
                if (r < rlim && c + VEC <= clim) {
                    regs[q] = *reinterpret_cast<const Raw *>(ptr);
                } else if constexpr (VEC == 1) {
                    regs[q] = 0;
                } else {
                    regs[q] = masked_vec(ptr, r < rlim ? clim - c : 0);
                }
            }
        }
    }

    // A vector of which only the first `n` elements are in range.
    __device__ __forceinline__ static Raw masked_vec(const char *ptr, int n)
    {
        Raw v = {};
        if constexpr (ES == 4) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e < n) v[e] = reinterpret_cast<const uint32_t *>(ptr)[e];
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (e < n) {
                    const uint32_t h = reinterpret_cast<const uint16_t *>(ptr)[e];
                    v[e >> 1] |= h << (16 * (e & 1));
                }
        }
        return v;
    }

    // 16-bit element e of register vector q.
    __device__ __forceinline__ uint16_t half_of(int q, int e) const
    {
        if constexpr (VEC == 1) {
            return (uint16_t)regs[q];
        } else {
            return (uint16_t)(regs[q][e >> 1] >> (16 * (e & 1)));
        }
    }
};

// N adjacent floats from LDS with one access (N = 1, 2 or 4; ptr aligned to 4*N bytes).
template <int N>
__device__ __forceinline__ void lds_floats(const float *ptr, float (&out)[N])
{
    if constexpr (N == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(ptr);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (N == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(ptr);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = ptr[0];
    }
}

// ---------------------------------------------------------------------------
// The kernel.
//   T          float, _Float16 or __bf16 (A and B element type)
//   BM, BN, BK workgroup tile and K-slab
//   WM, WN     wavefront grid; each wave owns a (BM/WM) x (BN/WN) sub-tile
//              made of TM x TN MFMA blocks of 32x32, interleaved: block (t,u)
//              covers wave rows TM*i'+t and wave columns TN*j'+u, so each lane
//              ends with TN adjacent columns (one vector store).
//   TA, TB     op(A) = A^T, op(B) = B^T
//   VECOK      A and B allow 16-byte global accesses
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VECOK>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(KernelArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int ES = sizeof(T);
    constexpr bool F32 = (ES == 4);
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1 && TM * 32 * WM == BM && TN * 32 * WN == BN, "tile");
    static_assert(TN == 1 || TN == 2 || TN == 4, "TN");
    constexpr int VEC = VECOK ? 16 / ES : 1;
    constexpr int ROWB = BK * ES;  // bytes per K-contiguous LDS row
    static_assert(ROWB == 128, "LDS rows are 128 bytes (8 chunks)");
    // LDS layouts: fp32 keeps the operand's global orientation; 16-bit
    // operands are always stored K-contiguous (the MFMA reads 8 k per lane).
    constexpr bool A_KC = !TA || !F32;
    constexpr bool B_KC = TB || !F32;
    constexpr int A_BYTES = BM * BK * ES, B_BYTES = BN * BK * ES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    // memory-order tile shapes: rows x contiguous elements
    constexpr int A_R = TA ? BK : BM, A_C = TA ? BM : BK;
    constexpr int B_R = TB ? BN : BK, B_C = TB ? BK : BN;
    TileLoader<ES, A_R, A_C, VEC, NT> la;
    TileLoader<ES, B_R, B_C, VEC, NT> lb;

    int bidx, tm, tn;
    map_tile(p, bidx, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 31, lh = lane >> 5;

    const char *Ab = static_cast<const char *>(p.A) + (int64_t)bidx * p.strideA * ES;
    const char *Bb = static_cast<const char *>(p.B) + (int64_t)bidx * p.strideB * ES;
    // tile origin in memory coordinates
    const char *Ap = Ab + (TA ? (int64_t)m0 : (int64_t)m0 * p.lda) * ES;
    const char *Bp = Bb + (TB ? (int64_t)n0 * p.ldb : (int64_t)n0) * ES;
    const int64_t a_kstep = (TA ? (int64_t)BK * p.lda : (int64_t)BK) * ES;
    const int64_t b_kstep = (TB ? (int64_t)BK : (int64_t)BK * p.ldb) * ES;
    const bool a_in = m0 + BM <= p.M, b_in = n0 + BN <= p.N;
    const int mrem = p.M - m0, nrem = p.N - n0;

    auto load_slab = [&](int k0) {
        const int krem = p.K - k0;
        const bool kfull = krem >= BK;
        if constexpr (TA) la.load(Ap, p.lda, krem, mrem, a_in && kfull, tid);
        else              la.load(Ap, p.lda, mrem, krem, a_in && kfull, tid);
        if constexpr (TB) lb.load(Bp, p.ldb, nrem, krem, b_in && kfull, tid);
        else              lb.load(Bp, p.ldb, krem, nrem, b_in && kfull, tid);
    };

    // registers -> LDS stage
    auto store_slab = [&](int stage) {
        char *sa = smem + stage * STAGE;
        char *sb = sa + A_BYTES;
#pragma unroll
        for (int q = 0; q < decltype(la)::NPT; ++q) {
            const int r = decltype(la)::row_of(tid, q), c = decltype(la)::col_of(tid, q);
            if constexpr (!TA) {  // memory row = m, contiguous = k -> K-contiguous rows
                if constexpr (VEC > 1)
                    *reinterpret_cast<u32x4 *>(sa + kc_off<ROWB, TM>(r, c * ES)) = la.regs[q];
                else
                    *reinterpret_cast<typename decltype(la)::Raw *>(sa + kc_off<ROWB, TM>(r, c * ES)) = la.regs[q];
            } else if constexpr (F32) {  // memory row = k, contiguous = m -> [BK][BM]
                *reinterpret_cast<typename decltype(la)::Raw *>(sa + (r * BM + c) * 4) = la.regs[q];
            } else {  // 16-bit, memory row = k: transpose into K-contiguous rows
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    *reinterpret_cast<uint16_t *>(sa + kc_off<ROWB, TM>(c + e, r * 2)) = la.half_of(q, e);
            }
        }
#pragma unroll
        for (int q = 0; q < decltype(lb)::NPT; ++q) {
            const int r = decltype(lb)::row_of(tid, q), c = decltype(lb)::col_of(tid, q);
            if constexpr (TB) {  // memory row = n, contiguous = k
                if constexpr (VEC > 1)
                    *reinterpret_cast<u32x4 *>(sb + kc_off<ROWB, TN>(r, c * ES)) = lb.regs[q];
                else
                    *reinterpret_cast<typename decltype(lb)::Raw *>(sb + kc_off<ROWB, TN>(r, c * ES)) = lb.regs[q];
            } else if constexpr (F32) {  // memory row = k, contiguous = n -> [BK][BN]
                *reinterpret_cast<typename decltype(lb)::Raw *>(sb + (r * BN + c) * 4) = lb.regs[q];
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    *reinterpret_cast<uint16_t *>(sb + kc_off<ROWB, TN>(c + e, r * 2)) = lb.half_of(q, e);
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = f32x16{};

    const int a_row0 = wm * WTM + TM * li;  // LDS row of sub-tile t is a_row0 + t
    const int b_row0 = wn * WTN + TN * li;

    auto compute_slab = [&](int stage) {
        const char *sa = smem + stage * STAGE;
        const char *sb = sa + A_BYTES;
        if constexpr (F32) {
            // 8 k per group: slot (h, s) carries k = 8*g + 4*h + s, s = 0..3
#pragma unroll
            for (int g = 0; g < BK / 8; ++g) {
                float av[TM][4], bv[TN][4];
                if constexpr (A_KC) {
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(
                            sa + kc_off<ROWB, TM>(a_row0 + t, (8 * g + 4 * lh) * 4));
#pragma unroll
                        for (int s = 0; s < 4; ++s) av[t][s] = v[s];
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        float v[TM];
                        lds_floats<TM>(reinterpret_cast<const float *>(sa) + (8 * g + 4 * lh + s) * BM + a_row0, v);
#pragma unroll
                        for (int t = 0; t < TM; ++t) av[t][s] = v[t];
                    }
                }
                if constexpr (B_KC) {
#pragma unroll
                    for (int u = 0; u < TN; ++u) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(
                            sb + kc_off<ROWB, TN>(b_row0 + u, (8 * g + 4 * lh) * 4));
#pragma unroll
                        for (int s = 0; s < 4; ++s) bv[u][s] = v[s];
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        float v[TN];
                        lds_floats<TN>(reinterpret_cast<const float *>(sb) + (8 * g + 4 * lh + s) * BN + b_row0, v);
#pragma unroll
                        for (int u = 0; u < TN; ++u) bv[u][s] = v[u];
                    }
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
#pragma unroll
                        for (int u = 0; u < TN; ++u)
                            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[t][s], bv[u][s], acc[t][u], 0, 0, 0);
            }
        } else {
            // 16 k per group: lane half h carries k = 16*g + 8*h + (0..7)
#pragma unroll
            for (int g = 0; g < BK / 16; ++g) {
                u32x4 av[TM], bv[TN];
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    av[t] = *reinterpret_cast<const u32x4 *>(sa + kc_off<ROWB, TM>(a_row0 + t, (16 * g + 8 * lh) * 2));
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    bv[u] = *reinterpret_cast<const u32x4 *>(sb + kc_off<ROWB, TN>(b_row0 + u, (16 * g + 8 * lh) * 2));
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int u = 0; u < TN; ++u) {
                        if constexpr (sizeof(T) == 2 && __is_same(T, _Float16))
                            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                __builtin_bit_cast(f16x8, av[t]), __builtin_bit_cast(f16x8, bv[u]), acc[t][u], 0, 0, 0);
                        else
                            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, av[t]), __builtin_bit_cast(bf16x8, bv[u]), acc[t][u], 0, 0, 0);
                    }
            }
        }
    };

    // ---- software pipeline: one LDS stage being consumed, the next slab in flight
    const int nk = (p.K + BK - 1) / BK;
    load_slab(0);
    store_slab(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {
            Ap += a_kstep;
            Bp += b_kstep;
            load_slab((kt + 1) * BK);
        }
        compute_slab(kt & 1);
        if (more) store_slab((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: C = alpha*acc + beta*C, C read only when beta != 0
    float *Cb = p.C + (int64_t)bidx * p.strideC;
    const int col = n0 + wn * WTN + TN * li;
    const bool col_full = col + TN <= p.N;
    const bool use_beta = p.beta != 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ip = 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int row = m0 + wm * WTM + TM * ip + t;
            if (row >= p.M) continue;
            float *cp = Cb + (int64_t)row * p.ldc + col;
            float v[TN];
#pragma unroll
            for (int u = 0; u < TN; ++u) v[u] = p.alpha * acc[t][u][r];
            if (TN > 1 && col_full && p.c_vec) {
                if constexpr (TN == 4) {
                    f32x4 o = {v[0], v[1], v[2], v[3]};
                    if (use_beta) o += p.beta * *reinterpret_cast<const f32x4 *>(cp);
                    *reinterpret_cast<f32x4 *>(cp) = o;
                } else if constexpr (TN == 2) {
                    f32x2 o = {v[0], v[1]};
                    if (use_beta) o += p.beta * *reinterpret_cast<const f32x2 *>(cp);
                    *reinterpret_cast<f32x2 *>(cp) = o;
                }
            } else {
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    if (col + u < p.N) cp[u] = use_beta ? v[u] + p.beta * cp[u] : v[u];
            }
        }
    }
}

// C = beta * C over a strided batch (alpha == 0 or K == 0).  beta == 0 writes
// zeros without reading C.
__global__ void __launch_bounds__(256) scale_c_kernel(float *C, int M, int N, int64_t ldc,
                                                      int64_t strideC, int batch, float beta);

}  // namespace mgemm
