// fp64 GEMM on the CDNA4 matrix cores: C = alpha * op(A) * op(B) + beta * C
// with double A, B, C, alpha and beta (the double x double -> double row of
// the WMMA API page's type table, section "1. 概述").
//
// The instruction is v_mfma_f64_16x16x4_f64: a 16x16 block of D from 16x4 of
// A and 4x16 of B.  Lane layout (pinned by an in-bounds one-wave probe):
//   A[i][k] comes from lane 16k + i, B[k][j] from lane 16k + j, and register
//   r of lane L holds D[4r + L/16][L%16].
// The matrix cores run fp64 at the vector rate (78.6 TFLOP/s on MI355X,
// 32 flop per clock per SIMD): one 16x16x4 block takes about 64 clocks, so
// operand traffic per flop is small and a register-staged, double-buffered
// tile keeps the matrix cores fed.  Every tile uses range-checked loads
// (out-of-range elements read as zero), so edges and unaligned leading
// dimensions need no second path.  The tile (F64Tile) serves the one-pass
// kernel and the stream-K kernel, whose segments run it over a K range.
//
// LDS holds both operands k-major, [BK][P] doubles.  At MFMA step s of a
// 16-deep group, lane (g = lane/16, i = lane%16) reads row
// 8(g&1) + 4(g>>1) + s, column i of its 16-wide block: the four steps cover
// the 16 rows once, and A and B use the same k-slot, which is all the dot
// product needs.  Bank arithmetic, as the counters show it for 64-bit
// accesses: 32 banks of 4 bytes, 16 lanes served together.
//   - fragment reads: 16 lanes read 16 consecutive doubles of one row, 32
//     distinct banks whatever the row pitch P;
//   - transposing stores (memory rows along m/n): with P = MN + 2, LDS rows
//     c and c' of one column are 2(c - c')P = 4(c - c') mod 32 dwords apart.
//     A 16-lane group that covered 8 k-pairs of 2 memory rows (16-byte loads)
//     put k-pairs j and j + 4 on the same banks: 2-way conflicts, 1/9 of the
//     LDS cycles of 4096^3 NN.  Each 16-lane group now covers 4 k-pairs of 4
//     memory rows (8 k of 2 rows for 8-byte loads): 8j + 2r' (+1), all 32
//     banks; the two k-halves of a 32-lane half-wave land 32 dwords apart;
//   - k-row operands are stored 16 bytes per lane, 16 consecutive doubles of
//     one row per 8 lanes.
#pragma once

#include "gemm_kernel.hpp"

namespace mgemm {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// One operand's tile for one K-slab: memory tile [R][CC] (CC contiguous);
// KROW: memory rows are k (R = BK, CC = MN), else memory rows are m or n
// (R = MN, CC = BK).  VEC doubles per global load (2 when 16-byte aligned).
template <int MN, int BK, int NT, bool KROW, int VEC>
struct F64Operand {
    static constexpr int R = KROW ? BK : MN;
    static constexpr int CC = KROW ? MN : BK;
    static constexpr int VPR = CC / VEC;        // vectors per memory row
    static constexpr int NPT = R * VPR / NT;    // vectors per thread
    static_assert(NPT * NT == R * VPR, "tile not divisible among threads");
    static constexpr int P = MN + 2;            // padded LDS row (doubles)
    f64x2 regs[NPT];

    // Element (row, column) of vector q of thread tid.  A k-row operand walks
    // the tile row by row.  A transposing one (memory rows m/n) gives each
    // wave RW = 64/VPR whole memory rows (the same bytes either way) and its
    // 16-lane groups a block of H = VPR/2 vectors by 16/H rows: group (h, g)
    // takes vector columns h*H .. h*H+H-1 of rows g*16/H ...  See above for
    // the banks.
    static constexpr int RW = 64 / VPR, H = VPR / 2;
    static_assert(KROW || (VPR == 8 || VPR == 16), "transposing tile: 8 or 16 vectors per row");
    __device__ __forceinline__ static int row_of(int tid, int q)
    {
        const int idx = tid + q * NT;
        if constexpr (KROW) return idx / VPR;
        const int l = idx & 63, m = l & 15, qw = l >> 4;
        return (idx >> 6) * RW + (qw >> 1) * (16 / H) + m / H;
    }
    __device__ __forceinline__ static int col_of(int tid, int q)
    {
        const int idx = tid + q * NT;
        if constexpr (KROW) return (idx % VPR) * VEC;
        const int l = idx & 63, m = l & 15, qw = l >> 4;
        return ((qw & 1) * H + m % H) * VEC;
    }

    // rows < rlim and columns < clim of the memory tile at `base` are in range.
    __device__ __forceinline__ void load(const double *base, int64_t ld, int rlim, int clim, int tid)
    {
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
            const int r = row_of(tid, q), c = col_of(tid, q);
            const double *ptr = base + (int64_t)r * ld + c;
            f64x2 v = {0.0, 0.0};
            if (r < rlim) {
                if constexpr (VEC == 2) {
                    if (c + 1 < clim)
                        v = *reinterpret_cast<const f64x2 *>(ptr);
                    else if (c < clim)
                        v[0] = ptr[0];
                } else {
                    if (c < clim) v[0] = ptr[0];
                }
            }
            regs[q] = v;
        }
    }

    // registers -> k-major LDS tile s[BK][P]
    __device__ __forceinline__ void store(double *s, int tid) const
    {
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
            const int r = row_of(tid, q), c = col_of(tid, q);
            if constexpr (KROW) {          // memory row = k: already k-major
                if constexpr (VEC == 2)
                    *reinterpret_cast<f64x2 *>(s + r * P + c) = regs[q];
                else
                    s[r * P + c] = regs[q][0];
            } else {                       // memory row = m/n: transpose into k rows
                s[c * P + r] = regs[q][0];
                if constexpr (VEC == 2) s[(c + 1) * P + r] = regs[q][1];
            }
        }
    }
};

// BM x BN workgroup tile, WM x WN waves, each owning a (BM/WM) x (BN/WN)
// sub-tile of TM x TN blocks of 16x16; BK-deep K-slabs (a multiple of 16).
// V2: A and B allow 16-byte loads.
template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V2>
struct F64Tile {
    static_assert(BK % 16 == 0, "K-slab");
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 16, TN = WTN / 16;
    static_assert(TM * 16 * WM == BM && TN * 16 * WN == BN, "tile");
    static constexpr int VEC = V2 ? 2 : 1;
    using OpA = F64Operand<BM, BK, NT, TA, VEC>;    // A^T in memory: rows are k
    using OpB = F64Operand<BN, BK, NT, !TB, VEC>;   // B in memory: rows are k
    static constexpr int A_ELEMS = BK * OpA::P, B_ELEMS = BK * OpB::P, STAGE = A_ELEMS + B_ELEMS;
    static constexpr int SMEM = 2 * STAGE;          // doubles of LDS

    // acc += op(A) x op(B) over K columns of A (rows of B) for the tile at
    // (m0, n0) of batch entry bidx, starting `k_off` columns in (a stream-K
    // segment); rows past M, columns past N and k past K read as zero.
    __device__ __forceinline__ static void run(const KernelArgs &p, double *smem, int bidx, int m0, int n0,
                                               int64_t k_off, int K, f64x4 (&acc)[TM][TN])
    {
        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = wave / WN, wn = wave % WN;
        const int g = lane >> 4, li = lane & 15;
        const double *Ap = static_cast<const double *>(p.A) + (int64_t)bidx * p.strideA +
                           (TA ? (int64_t)m0 + k_off * p.lda : (int64_t)m0 * p.lda + k_off);
        const double *Bp = static_cast<const double *>(p.B) + (int64_t)bidx * p.strideB +
                           (TB ? (int64_t)n0 * p.ldb + k_off : (int64_t)n0 + k_off * p.ldb);
        const int64_t a_kstep = TA ? (int64_t)BK * p.lda : (int64_t)BK;
        const int64_t b_kstep = TB ? (int64_t)BK : (int64_t)BK * p.ldb;
        const int mrem = p.M - m0, nrem = p.N - n0;

        OpA la;
        OpB lb;
        auto load_slab = [&](int kt) {
            const int krem = K - kt * BK;
            const double *a = Ap + (int64_t)kt * a_kstep;
            const double *b = Bp + (int64_t)kt * b_kstep;
            if constexpr (TA) la.load(a, p.lda, krem, mrem, tid);
            else              la.load(a, p.lda, mrem, krem, tid);
            if constexpr (TB) lb.load(b, p.ldb, nrem, krem, tid);
            else              lb.load(b, p.ldb, krem, nrem, tid);
        };
        // MFMA steps of k = 4; in each 16-deep group h of the slab, lane group g
        // takes k = 16h + 8(g&1) + 4(g>>1) + s at step s
        const int g_row = 8 * (g & 1) + 4 * (g >> 1);
        auto compute = [&](int stage) {
            const double *sa = smem + stage * STAGE + wm * WTM + li;
            const double *sb = smem + stage * STAGE + A_ELEMS + wn * WTN + li;
#pragma unroll
            for (int hs = 0; hs < BK / 4; ++hs) {
                const int kr = 16 * (hs >> 2) + g_row + (hs & 3);
                double a[TM], b[TN];
#pragma unroll
                for (int t = 0; t < TM; ++t) a[t] = sa[kr * OpA::P + 16 * t];
#pragma unroll
                for (int u = 0; u < TN; ++u) b[u] = sb[kr * OpB::P + 16 * u];
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int u = 0; u < TN; ++u)
                        acc[t][u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[t], b[u], acc[t][u], 0, 0, 0);
            }
        };

        // two LDS stages; the next slab is fetched to registers during the current one
        const int nk = (K + BK - 1) / BK;
        lds_poison<2 * STAGE * 8>(smem);
        load_slab(0);
        la.store(smem, tid);
        lb.store(smem + A_ELEMS, tid);
        __syncthreads();
        for (int kt = 0; kt + 1 < nk; ++kt) {
            load_slab(kt + 1);
            // a wave multiplying outranks one at its stores and barrier (four
            // waves share each SIMD): about 1% in a same-box A/B
            __builtin_amdgcn_s_setprio(1);
            compute(kt & 1);
            __builtin_amdgcn_s_setprio(0);
            double *st = smem + ((kt + 1) & 1) * STAGE;
            la.store(st, tid);
            lb.store(st + A_ELEMS, tid);
            __syncthreads();
            lds_poison<STAGE * 8>(smem + (kt & 1) * STAGE);  // read by every wave
        }
        compute((nk - 1) & 1);
    }

    // Element (row, column) of the tile that register r of block (t, u) of
    // this lane holds: register r of lane L is D[4r + L/16][L%16].
    __device__ __forceinline__ static int row_of(int t, int r)
    {
        return (threadIdx.x >> 6) / WN * WTM + 16 * t + 4 * r + ((threadIdx.x & 63) >> 4);
    }
    __device__ __forceinline__ static int col_of(int u)
    {
        return (threadIdx.x >> 6) % WN * WTN + 16 * u + (threadIdx.x & 15);
    }

    // Block (t, u) of C: C = alpha*v + beta*C (C read only when beta != 0)
    __device__ __forceinline__ static void store_block(const KernelArgs &p, int bidx, int m0, int n0, int t,
                                                       int u, const f64x4 &v)
    {
        const int col = n0 + col_of(u);
        if (col >= p.N) return;
        double *Cb = static_cast<double *>(p.C) + (int64_t)bidx * p.strideC + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + row_of(t, r);
            if (row >= p.M) continue;
            double *c = Cb + (int64_t)row * p.ldc;
            double x = p.alpha_d * v[r];
            if (p.beta_d != 0.0) x += p.beta_d * *c;
            __builtin_nontemporal_store(x, c);
        }
    }

    __device__ __forceinline__ static void epilogue(const KernelArgs &p, int bidx, int m0, int n0,
                                                    const f64x4 (&acc)[TM][TN])
    {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                store_block(p, bidx, m0, n0, t, u, acc[t][u]);
    }

    // stream-K: this workgroup's partial tile, BM x BN doubles row-major, with
    // agent-scope stores (visible to every XCD once acknowledged)
    __device__ __forceinline__ static void store_partial(void *part, const f64x4 (&acc)[TM][TN])
    {
        uint64_t *P = static_cast<uint64_t *>(part);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    // the element as a scalar first: a bit cast applied to a vector
                    // element read element 0 whatever the index
                    const double d = acc[t][u][r];
                    __hip_atomic_store(P + row_of(t, r) * BN + col_of(u), __builtin_bit_cast(uint64_t, d),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
    }

    // stream-K: the last contributor me of split tile (bidx, m0, n0), whose
    // iterations start at a0 and belong to workgroups g0..g1, adds the terms
    // in ascending K (g0 first, its own sums from registers in their place;
    // the others' partial tiles with agent-scope loads) and writes C.  One
    // 16x16 block at a time, so that only its four sums are live beside the
    // accumulators.
    __device__ __forceinline__ static void finish(const KernelArgs &p, int bidx, int m0, int n0, int64_t a0,
                                                  int64_t g0, int64_t g1, int64_t me,
                                                  const f64x4 (&acc)[TM][TN])
    {
        constexpr int TSZ = BM * BN;
        const uint64_t *part = static_cast<const uint64_t *>(p.sk_part);
        const int first_slot = p.sk_total * g0 / p.sk_grid == a0 ? 0 : 1;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                f64x4 sum;
                for (int64_t g = g0; g <= g1; ++g) {
                    f64x4 v = acc[t][u];
                    if (g != me) {
                        const uint64_t *pg = part + (g * 2 + (g == g0 ? first_slot : 0)) * TSZ + col_of(u);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = __builtin_bit_cast(double, __hip_atomic_load(pg + row_of(t, r) * BN,
                                                                                __ATOMIC_RELAXED,
                                                                                __HIP_MEMORY_SCOPE_AGENT));
                    }
                    sum = g == g0 ? v : sum + v;
                }
                store_block(p, bidx, m0, n0, t, u, sum);
            }
    }
};

template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V2>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_f64_kernel(KernelArgs p)
{
    using F = F64Tile<BM, BN, BK, WM, WN, TA, TB, V2>;
    __shared__ __attribute__((aligned(16))) double smem[F::SMEM];
    int bidx, tm, tn;
    map_tile(p, bidx, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = bidx == p.tail_batch ? p.k_tail : p.K;  // split-K's last chunk may be shorter
    f64x4 acc[F::TM][F::TN];
#pragma unroll
    for (int t = 0; t < F::TM; ++t)
#pragma unroll
        for (int u = 0; u < F::TN; ++u)
            acc[t][u] = f64x4{0.0, 0.0, 0.0, 0.0};
    F::run(p, smem, bidx, m0, n0, 0, K, acc);
    F::epilogue(p, bidx, m0, n0, acc);
}

// Stream-K for fp64: the partition, segments and completion of gemm_sk_kernel
// (gemm_kernel.hpp), with double partial tiles.
template <int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool V2>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_f64_sk_kernel(KernelArgs p)
{
    using F = F64Tile<BM, BN, BK, WM, WN, TA, TB, V2>;
    __shared__ __attribute__((aligned(16))) double smem[F::SMEM];
    __shared__ int last_arrival;
    const int L = logical_wg();
    const int iters = p.sk_iters;
    const int64_t beg = p.sk_total * L / p.sk_grid, end = p.sk_total * (L + 1) / p.sk_grid;
    for (int64_t it = beg; it < end;) {
        const int tile = (int)(it / iters);
        const int k0 = (int)(it - (int64_t)tile * iters);
        const int k1 = end - it < iters - k0 ? k0 + (int)(end - it) : iters;
        int bidx, tm, tn;
        tile_coords(p, tile, bidx, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int64_t ko = (int64_t)k0 * p.sk_unit;  // first k of the segment
        const int K = k1 == iters ? p.K - (int)ko : (k1 - k0) * p.sk_unit;
        f64x4 acc[F::TM][F::TN];
#pragma unroll
        for (int t = 0; t < F::TM; ++t)
#pragma unroll
            for (int u = 0; u < F::TN; ++u)
                acc[t][u] = f64x4{0.0, 0.0, 0.0, 0.0};
        F::run(p, smem, bidx, m0, n0, ko, K, acc);
        if (k0 == 0 && k1 == iters) {
            F::epilogue(p, bidx, m0, n0, acc);
        } else {
            const int64_t a0 = (int64_t)tile * iters;
            int64_t g0, g1;
            sk_owners(p, a0, g0, g1);
            const bool last = sk_arrive(p, g0, g1, last_arrival, [&] {
                F::store_partial(static_cast<double *>(p.sk_part) +
                                     ((int64_t)L * 2 + (it == beg ? 0 : 1)) * (BM * BN), acc);
            });
            if (last) F::finish(p, bidx, m0, n0, a0, g0, g1, L, acc);
        }
        it += k1 - k0;
        __syncthreads();  // the next segment refills the LDS stages
    }
}

}  // namespace mgemm
