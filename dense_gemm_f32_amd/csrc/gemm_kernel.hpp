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
//     jianshu kernel) -> dwordx4 loads, here issued straight into LDS;
//   * a transposed on-chip tile so that one access serves several rows
//     ("V3 双缓冲", the transposed SA; jianshu's transposed A tile) -> on
//     CDNA4 the transpose happens in the LDS read (ds_read_b64_tr_b16) or,
//     for fp32, in the choice of which index a lane's vector read runs along;
//   * overlapping the fetch of later slabs with the math on the current one
//     ("V3 双缓冲"; the jianshu kernel's double buffer and prefetch) ->
//     a 4-stage LDS ring filled three slabs ahead;
//   * zero-filled residual tiles and guarded stores (the CSDN tile-algorithm
//     page, "使用CUDA和瓦片算法计算矩阵乘法", MatrixMulCUDA);
//   * grouped tile ordering for cache reuse ("cuda11/matmul", Triton
//     section) -> XCD-aware workgroup rasterisation.
// What replaces the NVIDIA-era pieces: the per-thread 8x8 FMA micro-tile and
// the WMMA fragments become 32x32 MFMA blocks per wavefront
// (v_mfma_f32_32x32x2_f32 for fp32, v_mfma_f32_32x32x16_{f16,bf16} for
// 16-bit inputs) with fp32 accumulators.
//
// MFMA operand/result placement (wave64, lane l, i' = l % 32, h = l / 32):
//   32x32x2 f32 : lane supplies A[i'][k_h] and B[k_h][i'] (one value each);
//   32x32x16    : lane supplies 8 values A[i'][k in group h] and B[k][i'];
//   result      : accumulator element r (0..15) of lane l is row
//                 8*(r/4) + 4*h + r%4, column i'.
// A sum over k does not depend on which k each (h, element) slot carries as
// long as A and B agree, so each path assigns k to slots to suit its LDS
// layout.
//
// Each workgroup takes one of two paths (uniform branch):
//   DmaPath  every tile of 16-byte aligned problems with K a multiple of 16
//            bytes: global -> LDS by buffer_load ... lds, a ring of stages;
//   RegPath  everything else: range-checked loads through registers,
//            out-of-range elements read as zero, 2 LDS stages.
// gemm_kernel gives each workgroup one tile; gemm_sk_kernel (stream-K)
// gives each an equal share of the (tile, K-iteration) pairs and runs the
// same paths over K ranges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));  // 16 bytes at a 4-byte aligned address
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Everything a GEMM launch needs; built on the host after validation.
struct KernelArgs {
    const void *A;
    const void *B;
    void *C;          // fp32, the inputs' 16-bit type, int32 (int8 inputs) or double
    int64_t lda, ldb, ldc;
    int64_t strideA, strideB, strideC;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;      // tile rows per raster group
    float alpha, beta;
    int alpha_i, beta_i;  // integral alpha and beta for int8 inputs (int32 C)
    int c_vec;        // C pointer/ldc/strideC allow one vector access per 4 elements
    int fast_ok;      // operand tiles addressable with 32-bit byte offsets
    double alpha_d, beta_d;  // alpha and beta of fp64 GEMM
    int k_tail, tail_batch;  // batch entry tail_batch runs K = k_tail (split-K's last chunk); -1: none
    // stream-K launches (gemm_sk_kernel): every tile is sk_iters
    // K-iterations of sk_unit elements (the last one may be shorter); the
    // sk_total = tiles * sk_iters iterations, tile-major, are shared out
    // evenly over sk_grid workgroups; sk_part holds two partial tiles per
    // workgroup, sk_count one arrival counter per workgroup (zero between
    // launches)
    int sk_iters, sk_unit, sk_grid;
    int64_t sk_total;
    void *sk_part;
    unsigned *sk_count;
};

// ---------------------------------------------------------------------------
// Workgroup -> (batch, tile row, tile column).
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  The id is first remapped so that every XCD receives one
// contiguous range of logical ids, and that range is walked in groups of
// `group_m` tile rows, so the tiles resident on one XCD share A rows and B
// columns in its L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int logical_wg()
{
    const int nwg = gridDim.x;
    const int w = blockIdx.x;
    const int q = nwg >> 3, rem = nwg & 7;
    const int x = w & 7, i = w >> 3;
    return x * q + min(x, rem) + i;
}

// logical tile L -> (batch, tile row, tile column), grouped order
__device__ __forceinline__ void tile_coords(const KernelArgs &p, int L, int &b, int &tm, int &tn)
{
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

__device__ __forceinline__ void map_tile(const KernelArgs &p, int &b, int &tm, int &tn)
{
    tile_coords(p, logical_wg(), b, tm, tn);
}

template <int BYTES> struct RawOf;
template <> struct RawOf<16> { using type = u32x4; };
template <> struct RawOf<8> { using type = u32x2; };
template <> struct RawOf<4> { using type = uint32_t; };
template <> struct RawOf<2> { using type = uint16_t; };
template <> struct RawOf<1> { using type = uint8_t; };

// Buffer resource over [base, base + 2 GiB): raw addressing, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             0x00020000);
}

// 16-byte global -> LDS copy: lane l's 16 bytes from rsrc[voff + soff] land at
// LDS byte lds_addr + 16*l.  Issued through inline asm so that the compiler's
// memory-counter tracking does not see it: it would otherwise wait for every
// outstanding copy before any LDS read it cannot prove disjoint (the
// transposing reads among them), serialising the ring.  Callers order these
// copies with explicit vmcnt waits.  The LDS destination goes in M0 through
// an "{m0}" operand: the compiler writes M0 itself before the copy, and so
// knows that M0 changes there (M0 is a reserved register, which a clobber
// list cannot name).
// The compiler inserts the wait states a memory instruction needs after the
// writes of its scalar operands only for instructions it can see, not for
// inline asm, so the copy opens with s_nop 4 (five wait states): a vector
// instruction that writes an SGPR (v_readfirstlane, which forms soff and may
// form M0 or the resource) must be five wait states ahead of a vector-memory
// instruction that reads it, and a scalar write of M0 one ahead of an LDS-DMA
// read of M0.  Without them a copy can take the SGPR's previous value: an
// interior-tile prologue whose soff came from v_readfirstlane one wait state
// earlier loaded 1 KB of B from a wrong address.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr, int voff, int soff)
{
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr) : "memory");
}

// 4-byte global -> LDS copy: lane l's 4 bytes from rsrc[voff] land at LDS byte
// lds_addr + 4*l.  A lane whose voff is past the buffer's range (kOutOfRange)
// is masked by the hardware's range check: no memory is read and a zero is
// written to its LDS word (checked with a one-wave probe).
constexpr int kOutOfRange = 0x7fffffff;

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr, int voff)
{
    // s_nop 4: the wait states of dma16
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rs), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const char *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// s_waitcnt with vmcnt = VM (<= 63), lgkmcnt = LGKM (<= 15), expcnt unrestricted.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts()
{
    static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "waitcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier that orders LDS accesses in the compiler but leaves the
// hardware counters to explicit waits (so loads further ahead stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Race check of the LDS rings (debug builds, -DMGEMM_DEBUG_POISON; a no-op
// otherwise): every thread of the workgroup fills its share of LDS bytes
// [p, p + BYTES) with 0xFF (NaN in every floating type, -1 in int8), waits
// for its LDS writes and meets the others at a barrier.  Vector-memory
// counters are not waited on, so copies in flight stay in flight.  Each ring
// poisons all of its stages before its first copy and each stage again once
// every wave has read it, before its refill is issued: a fragment read that
// runs ahead of its slab's copies, or a stage refilled while a wave still
// reads it, then takes poison instead of a plausible value.
template <int BYTES>
__device__ __forceinline__ void lds_poison(void *p)
{
#ifdef MGEMM_DEBUG_POISON
    static_assert(BYTES % 4 == 0, "whole words");
    uint32_t *w = static_cast<uint32_t *>(p);
    for (int i = threadIdx.x; i < BYTES / 4; i += blockDim.x) w[i] = 0xffffffffu;
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#else
    (void)p;
#endif
}

// Physical order of the rows of a K-contiguous LDS tile.  A wavefront's
// 32*IL rows hold its IL interleaved MFMA sub-tiles (logical row IL*i' + t);
// physical row 32*t + i' holds logical row IL*i' + t, so the lanes of one
// fragment read touch consecutive physical rows.
template <int IL>
__device__ __forceinline__ int phys_row(int r)
{
    constexpr int WT = 32 * IL;
    const int w = r / WT, rr = r % WT;
    return w * WT + (rr % IL) * 32 + rr / IL;
}

template <int IL>
__device__ __forceinline__ int logical_row(int p)
{
    constexpr int WT = 32 * IL;
    const int w = p / WT, pp = p % WT;
    return w * WT + (pp % 32) * IL + pp / 32;
}

// Two 16-bit halves -> one dword: lo16(a) | lo16(b) << 16 (hi = 0) or
// hi16(a) | hi16(b) << 16 (hi = 1).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, int hi)
{
    return hi ? __builtin_amdgcn_perm(b, a, 0x07060302u) : __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// ---------------------------------------------------------------------------
// Instruction-group ordering hints for the scheduler (sched_group_barrier):
// mask 0x008 = MFMA, 0x020 = VMEM read, 0x100 = DS read, 0x200 = DS write.
// sched_interleave<X, NX, Y, NY>() asks for X, Y, X, Y, ... then the rest of
// the longer group.
// ---------------------------------------------------------------------------
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;

template <int MX, int NX, int MY, int NY>
__device__ __forceinline__ void sched_interleave()
{
    constexpr int P = NX < NY ? NX : NY;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        __builtin_amdgcn_sched_group_barrier(MX, 1, 0);
        __builtin_amdgcn_sched_group_barrier(MY, 1, 0);
    }
    if constexpr (NX > P) __builtin_amdgcn_sched_group_barrier(MX, NX - P, 0);
    if constexpr (NY > P) __builtin_amdgcn_sched_group_barrier(MY, NY - P, 0);
}

// sched_front<X, NX, Y, NY, R>() asks for X followed by R of Y, until Y runs
// out, then the rest of X: the Y (fragment reads) are issued early in the
// group, so they have completed well before its last X (MFMA).
template <int MX, int NX, int MY, int NY, int R, int I = 0>
__device__ __forceinline__ void sched_front()
{
    constexpr int left = NY - I * R;
    if constexpr (I < NX && left > 0) {
        __builtin_amdgcn_sched_group_barrier(MX, 1, 0);
        __builtin_amdgcn_sched_group_barrier(MY, left < R ? left : R, 0);
        sched_front<MX, NX, MY, NY, R, I + 1>();
    } else {
        if constexpr (NX > I) __builtin_amdgcn_sched_group_barrier(MX, NX - I, 0);
        if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(MY, left, 0);
    }
}

// N adjacent floats from LDS with one access (N = 1, 2 or 4; ptr aligned to 4*N bytes).
template <int N>
__device__ __forceinline__ void lds_floats(const char *ptr, float (&out)[N])
{
    if constexpr (N == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(ptr);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (N == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2 *>(ptr);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = *reinterpret_cast<const float *>(ptr);
    }
}

// ---------------------------------------------------------------------------
// Operand fragments of one k-group and the MFMAs that consume them.
// fp32: 4 k-slots per operand row (k = 8g + 4h + s); 16-bit: one 8-element
// vector per row (k = 16g + 8h + 0..7); int8: one 16-element vector per row
// (k = 32g + 16h + 0..15), v_mfma_i32_32x32x32_i8 with int32 accumulators
// kept in the same registers (the f32x16 type only names 16 dwords).
// ---------------------------------------------------------------------------
template <typename T, int TM, int TN>
struct Frags {
    static constexpr bool F32 = sizeof(T) == 4;
    float a32[F32 ? TM : 1][4], b32[F32 ? TN : 1][4];
    u32x4 a16[F32 ? 1 : TM], b16[F32 ? 1 : TN];

    // the 16-bit / int8 MFMA of sub-tile (I / TN, I % TN)
    template <int I>
    __device__ __forceinline__ void mfma_at(f32x16 (&acc)[TM][TN]) const
    {
        static_assert(!F32 && I < TM * TN, "one 16-bit or int8 MFMA");
        constexpr int t = I / TN, u = I % TN;
        if constexpr (__is_same(T, int8_t))
            acc[t][u] = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, a16[t]), __builtin_bit_cast(i32x4, b16[u]),
                __builtin_bit_cast(i32x16, acc[t][u]), 0, 0, 0));
        else if constexpr (__is_same(T, _Float16))
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, a16[t]), __builtin_bit_cast(f16x8, b16[u]), acc[t][u], 0, 0, 0);
        else
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a16[t]), __builtin_bit_cast(bf16x8, b16[u]), acc[t][u], 0, 0, 0);
    }

    __device__ __forceinline__ void mfmas(f32x16 (&acc)[TM][TN]) const
    {
        if constexpr (F32) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int u = 0; u < TN; ++u)
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x2f32(a32[t][s], b32[u][s], acc[t][u], 0, 0, 0);
        } else {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    if constexpr (__is_same(T, int8_t))
                        acc[t][u] = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            __builtin_bit_cast(i32x4, a16[t]), __builtin_bit_cast(i32x4, b16[u]),
                            __builtin_bit_cast(i32x16, acc[t][u]), 0, 0, 0));
                    else if constexpr (__is_same(T, _Float16))
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, a16[t]), __builtin_bit_cast(f16x8, b16[u]), acc[t][u], 0, 0, 0);
                    else
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a16[t]), __builtin_bit_cast(bf16x8, b16[u]), acc[t][u], 0, 0, 0);
                }
        }
    }
};

// ===========================================================================
// RegPath: range-checked global loads through registers, 2 LDS stages.
// K-contiguous LDS rows hold BK elements = 128 bytes, half of the 64-bank x
// 4-byte LDS line; a 16-byte access is served 16 lanes at a time, so the 16
// lanes of a fragment read, which touch 16 consecutive physical rows,
// alternate between the two halves of a line, and chunk c of physical row p
// sits at chunk c ^ ((p >> 1) & 7), spreading each half over 8 chunks.
// ===========================================================================
__device__ __forceinline__ int kc128_off(int p, int kbyte)
{
    const int chunk = (kbyte >> 4) ^ ((p >> 1) & 7);
    return p * 128 + (chunk << 4) + (kbyte & 15);
}

// int8 operands whose memory rows are k (MN-contiguous, "MC"): LDS rows of
// ROWB bytes (the tile's MN), 16-byte chunks permuted per row, chunk c of row
// k at c ^ (k % 8) (k % 4 for 64-byte rows).  A transposing fragment read
// (tr8_frag) takes one 16-byte chunk from each of 8 consecutive rows per 16
// lanes; the permutation puts those in 8 distinct chunks, i.e. all 32 banks
// of a 128-byte access.  The permutation is its own inverse: physical chunk
// c of row k holds logical chunk c ^ (k % 8).
template <int ROWB>
__device__ __forceinline__ int mc8_chunk(int k, int c)
{
    static_assert(ROWB % 64 == 0, "whole 64-byte pieces");
    return c ^ (k & (ROWB >= 128 ? 7 : 3));
}
template <int ROWB>
__device__ __forceinline__ int mc8_off(int k, int byte)
{
    return k * ROWB + (mc8_chunk<ROWB>(k, byte >> 4) << 4) + (byte & 15);
}

// Fragment of one MC int8 operand: the 16 k-values 32g + 16h + 0..15 of column
// (wave-local) col_base + lane % 32, for v_mfma_i32_32x32x32_i8, via two
// ds_read_b64_tr_b8.  Within a 16-lane group, source lane j supplies 8 bytes
// of row k0 + j/2, columns 8*(j%2) .. +7 of the group's 16, and lane i
// receives column i of rows k0 .. k0+7 in its bytes 0..7 (pinned by an
// in-bounds one-wave probe); the second read covers rows k0+8 .. k0+15.
template <int ROWB>
__device__ __forceinline__ u32x4 tr8_frag(const char *s, int g, int lh, int col_base, int lane)
{
    const int gi = lane & 15;
    const int col = col_base + 16 * ((lane >> 4) & 1) + 8 * (gi & 1);
    const int k0 = 32 * g + 16 * lh + (gi >> 1);
    const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(s + mc8_off<ROWB>(k0, col)));
    const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(s + mc8_off<ROWB>(k0 + 8, col)));
    return u32x4{(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
}

// One operand (A or B) of one K-slab: global -> registers -> LDS.
//   ES    element size (4: fp32, 2: f16/bf16, 1: int8)
//   MN    tile extent along M (for A) or N (for B)
//   KROW  memory rows run along k (A^T or B), i.e. MN is the contiguous dim
//   IL    the operand's sub-tile interleave
//   VECOK 16-byte aligned rows; otherwise every 16-byte vector is assembled
//         from the aligned dwords around it (realigned_vec)
// Modes:
//   vector   (!KROW, fp32 or int8): memory vectors copied as is; LDS rows
//            are K-contiguous (!KROW), the fp32 [BK][MN] layout (fp32 KROW)
//            or the int8 MC layout of mc8_off (int8 KROW, read back with
//            transposing reads).
//   block    (16-bit KROW): KB x 8 blocks transposed in registers so LDS
//            rows stay K-contiguous (the MFMA wants 8 k per lane).
template <int ES, int NT, int MN, int BK, int IL, bool KROW, bool VECOK>
struct RegOperand {
    static constexpr bool F32 = ES == 4;
    static constexpr int ROWB = BK * ES;
    static_assert(ROWB == 128, "K-contiguous rows are 128 bytes");
    static constexpr bool BLOCK = KROW && ES == 2;
    static constexpr bool MC8 = KROW && ES == 1;  // int8 rows of k: MC layout
    static constexpr int VEC = 16 / ES;
    static constexpr int R = KROW ? BK : MN;   // memory rows of the tile
    static constexpr int CC = KROW ? MN : BK;  // contiguous elements per memory row
    static constexpr int VPR = CC / VEC;
    static constexpr int NPT = (R * CC / VEC) / NT;
    static_assert(BLOCK || (R * CC / VEC) % NT == 0, "tile not divisible among threads");
    static constexpr int KB = ((BK / 8) * (MN / 8) >= NT) ? 8 : ((BK / 4) * (MN / 8) >= NT) ? 4 : 2;
    static constexpr int KGS = BK / KB;
    static constexpr int NPB = BLOCK ? (KGS * (MN / 8)) / NT : 1;
    static_assert(!BLOCK || (KGS * (MN / 8)) % NT == 0, "blocks not divisible among threads");
    static constexpr int NREG = BLOCK ? NPB * KB : NPT;
    using Raw = typename RawOf<VEC * ES>::type;
    Raw regs[NREG];

    // vector mode: slot (tid, q) fills tile row vrow (the physical LDS row for
    // K-contiguous layouts) at column vcol, from memory row mem_row(vrow).
    __device__ __forceinline__ static int vrow(int tid, int q) { return (tid + q * NT) / VPR; }
    __device__ __forceinline__ static int vcol(int tid, int q) { return ((tid + q * NT) % VPR) * VEC; }
    __device__ __forceinline__ static int mem_row(int v) { return KROW ? v : logical_row<IL>(v); }
    __device__ __forceinline__ static int bkg(int tid) { return tid % KGS; }
    __device__ __forceinline__ static int bng(int tid, int q) { return tid / KGS + q * (NT / KGS); }

    // rows < rlim and columns < clim (memory order, relative to the tile
    // origin `base`) are in range; everything else reads as zero.
    __device__ __forceinline__ void load(const char *base, int64_t ld, int rlim, int clim, int tid)
    {
        if constexpr (BLOCK) {
#pragma unroll
            for (int q = 0; q < NPB; ++q)
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    const int row = bkg(tid) * KB + r, col = bng(tid, q) * 8;
                    regs[q * KB + r] = load_vec(base + ((int64_t)row * ld + col) * ES,
                                                row < rlim ? clim - col : 0);
                }
        } else {
#pragma unroll
            for (int q = 0; q < NPT; ++q) {
                const int r = mem_row(vrow(tid, q)), c = vcol(tid, q);
                regs[q] = load_vec(base + ((int64_t)r * ld + c) * ES, r < rlim ? clim - c : 0);
            }
        }
    }

    __device__ __forceinline__ static u32x4 load_vec(const char *ptr, int n)
    {
        if constexpr (VECOK) return masked_vec(ptr, n);
        else                 return realigned_vec(ptr, n);
    }

    // masked_vec for an address aligned only to the element size (rows of
    // any length).  The 4-byte aligned dwords that hold in-range bytes are
    // loaded -- four from the aligned-down address (the compiler issues a
    // 4-byte aligned 16-byte access as dword loads), a fifth when the
    // address is not 4-byte aligned -- and shifted into place with
    // v_alignbyte.  A dword holding an in-range byte lies in that byte's
    // page, so no load can fault; bytes past the n elements are cleared.
    __device__ __forceinline__ static u32x4 realigned_vec(const char *ptr, int n)
    {
        constexpr int V = 16 / ES;
        if (n <= 0) return u32x4{0, 0, 0, 0};
        const uintptr_t addr = reinterpret_cast<uintptr_t>(ptr);
        const int o = ES == 4 ? 0 : (int)(addr & 3);
        const uint32_t *p0 = reinterpret_cast<const uint32_t *>(addr - (uintptr_t)o);
        const int nb = (n < V ? n : V) * ES;  // in-range bytes from ptr
        const int end = o + nb;               // in-range bytes end here, from p0
        u32x4 lo = {0, 0, 0, 0};
        uint32_t hi = 0;
        if (end > 12) {
            lo = *reinterpret_cast<const u32x4_a4 *>(p0);
        } else {
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (4 * j < end) lo[j] = p0[j];
        }
        if (end > 16) hi = p0[4];
        u32x4 v;
        v[0] = __builtin_amdgcn_alignbyte(lo[1], lo[0], o);
        v[1] = __builtin_amdgcn_alignbyte(lo[2], lo[1], o);
        v[2] = __builtin_amdgcn_alignbyte(lo[3], lo[2], o);
        v[3] = __builtin_amdgcn_alignbyte(hi, lo[3], o);
        if (nb < 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int keep = nb - 4 * i;  // in-range bytes of dword i
                if (keep <= 0) v[i] = 0;
                else if (keep < 4) v[i] &= (1u << (8 * keep)) - 1u;
            }
        }
        return v;
    }

    // A 16-byte vector of which only the first `n` elements are in range.
    __device__ __forceinline__ static u32x4 masked_vec(const char *ptr, int n)
    {
        constexpr int V = 16 / ES;
        if (n >= V) return *reinterpret_cast<const u32x4 *>(ptr);
        u32x4 v = {0, 0, 0, 0};
        if constexpr (ES == 4) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (e < n) v[e] = reinterpret_cast<const uint32_t *>(ptr)[e];
        } else if constexpr (ES == 1) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (e < n) v[e >> 2] |= (uint32_t)reinterpret_cast<const uint8_t *>(ptr)[e] << (8 * (e & 3));
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (e < n) v[e >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(ptr)[e] << (16 * (e & 1));
        }
        return v;
    }

    // registers -> LDS tile at `s`
    __device__ __forceinline__ void store(char *s, int tid) const
    {
        if constexpr (BLOCK) {
#pragma unroll
            for (int q = 0; q < NPB; ++q) {
                const int kbyte = bkg(tid) * KB * 2, row0 = bng(tid, q) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // column e of the block: KB k-values, two per dword
                    const int d = e >> 1, hi = e & 1;
                    char *dst = s + kc128_off(phys_row<IL>(row0 + e), kbyte);
                    if constexpr (KB == 8) {
                        u32x4 o;
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            o[p] = pack_halves(regs[q * 8 + 2 * p][d], regs[q * 8 + 2 * p + 1][d], hi);
                        *reinterpret_cast<u32x4 *>(dst) = o;
                    } else if constexpr (KB == 4) {
                        u32x2 o;
#pragma unroll
                        for (int p = 0; p < 2; ++p)
                            o[p] = pack_halves(regs[q * 4 + 2 * p][d], regs[q * 4 + 2 * p + 1][d], hi);
                        *reinterpret_cast<u32x2 *>(dst) = o;
                    } else {
                        *reinterpret_cast<uint32_t *>(dst) = pack_halves(regs[q * 2][d], regs[q * 2 + 1][d], hi);
                    }
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < NPT; ++q) {
                const int r = vrow(tid, q), c = vcol(tid, q);
                if constexpr (!KROW) {          // memory row = mn, contiguous = k; r is physical
                    *reinterpret_cast<Raw *>(s + kc128_off(r, c * ES)) = regs[q];
                } else if constexpr (MC8) {     // int8, memory row = k: one 16-byte chunk
                    *reinterpret_cast<Raw *>(s + mc8_off<MN>(r, c)) = regs[q];
                } else {                        // fp32, memory row = k, contiguous = mn -> [BK][MN]
                    *reinterpret_cast<Raw *>(s + (r * MN + c) * 4) = regs[q];
                }
            }
        }
    }
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VECOK>
struct RegPath {
    static constexpr int NT = WM * WN * 64;
    static constexpr int ES = sizeof(T);
    static constexpr bool F32 = (ES == 4);
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1 && TM * 32 * WM == BM && TN * 32 * WN == BN, "tile");
    static_assert(TN == 1 || TN == 2 || TN == 4, "TN");
    // LDS layout of A (B) is K-contiguous; otherwise fp32 [BK][MN] or the int8
    // MC layout (16-bit operands are always stored K-contiguous)
    static constexpr bool A_KC = !TA || ES == 2;
    static constexpr bool B_KC = TB || ES == 2;
    static constexpr bool A_MC8 = !A_KC && ES == 1, B_MC8 = !B_KC && ES == 1;
    static constexpr int A_BYTES = BM * BK * ES, B_BYTES = BN * BK * ES;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static constexpr int G = F32 ? BK / 8 : BK * ES / 32;  // k-groups of 32 bytes per slab
    // C mapping: interleaved rows and columns, except that a transposing read
    // (int8 MC) gives each lane consecutive ones
    static constexpr int IL_A = A_MC8 ? 1 : TM, IL_B = B_MC8 ? 1 : TN;
    // 64x64 tiles keep two register sets in flight: a grid of them is often
    // about one workgroup per CU, with little else to hide the load latency
    // behind.  Larger tiles keep one: a second set would cost them occupancy
    // (128x128 unaligned fp32 would go from 244 to 308 registers).
    static constexpr bool REG2 = BM * BN <= 64 * 64;

    using OpA = RegOperand<ES, NT, BM, BK, TM, TA, VECOK>;
    using OpB = RegOperand<ES, NT, BN, BK, TN, !TB, VECOK>;
    using Fr = Frags<T, TM, TN>;

    // a_row0/b_row0: first interleaved row of this lane in the fp32 [BK][MN]
    // layout; a_prow0/b_prow0: its physical row in the K-contiguous layout.
    __device__ __forceinline__ static void load_frags(const char *sa, const char *sb, int g, int a_row0,
                                                      int b_row0, int a_prow0, int b_prow0, int lh, Fr &f)
    {
        if constexpr (F32) {
            if constexpr (A_KC) {
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(sa + kc128_off(a_prow0 + 32 * t, (8 * g + 4 * lh) * 4));
#pragma unroll
                    for (int s = 0; s < 4; ++s) f.a32[t][s] = v[s];
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float v[TM];
                    lds_floats<TM>(sa + ((8 * g + 4 * lh + s) * BM + a_row0) * 4, v);
#pragma unroll
                    for (int t = 0; t < TM; ++t) f.a32[t][s] = v[t];
                }
            }
            if constexpr (B_KC) {
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(sb + kc128_off(b_prow0 + 32 * u, (8 * g + 4 * lh) * 4));
#pragma unroll
                    for (int s = 0; s < 4; ++s) f.b32[u][s] = v[s];
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float v[TN];
                    lds_floats<TN>(sb + ((8 * g + 4 * lh + s) * BN + b_row0) * 4, v);
#pragma unroll
                    for (int u = 0; u < TN; ++u) f.b32[u][s] = v[u];
                }
            }
        } else {
            // int8 MC operands: transposing reads of the wave's consecutive columns
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if constexpr (A_MC8)
                    f.a16[t] = tr8_frag<BM>(sa, g, lh, (wave / WN) * WTM + 32 * t, lane);
                else
                    f.a16[t] = *reinterpret_cast<const u32x4 *>(sa + kc128_off(a_prow0 + 32 * t, (16 * g + 8 * lh) * 2));
            }
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                if constexpr (B_MC8)
                    f.b16[u] = tr8_frag<BN>(sb, g, lh, (wave % WN) * WTN + 32 * u, lane);
                else
                    f.b16[u] = *reinterpret_cast<const u32x4 *>(sb + kc128_off(b_prow0 + 32 * u, (16 * g + 8 * lh) * 2));
            }
        }
    }

    __device__ __forceinline__ static void run(const KernelArgs &p, char *smem, int bidx, int m0, int n0,
                               f32x16 (&acc)[TM][TN])
    {
        const int tid = threadIdx.x;
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = wave / WN, wn = wave % WN;
        const int li = lane & 31, lh = lane >> 5;
        const char *Ap = static_cast<const char *>(p.A) + (int64_t)bidx * p.strideA * ES +
                         (TA ? (int64_t)m0 : (int64_t)m0 * p.lda) * ES;
        const char *Bp = static_cast<const char *>(p.B) + (int64_t)bidx * p.strideB * ES +
                         (TB ? (int64_t)n0 * p.ldb : (int64_t)n0) * ES;
        const int64_t a_kstep = (TA ? (int64_t)BK * p.lda : (int64_t)BK) * ES;
        const int64_t b_kstep = (TB ? (int64_t)BK : (int64_t)BK * p.ldb) * ES;
        const int mrem = p.M - m0, nrem = p.N - n0;
        const int a_row0 = wm * WTM + TM * li, b_row0 = wn * WTN + TN * li;
        const int a_prow0 = wm * WTM + li, b_prow0 = wn * WTN + li;

        auto load_slab = [&](int kt, OpA &la, OpB &lb) {
            const int krem = p.K - kt * BK;
            const char *a = Ap + (int64_t)kt * a_kstep;
            const char *b = Bp + (int64_t)kt * b_kstep;
            if constexpr (TA) la.load(a, p.lda, krem, mrem, tid);
            else              la.load(a, p.lda, mrem, krem, tid);
            if constexpr (TB) lb.load(b, p.ldb, nrem, krem, tid);
            else              lb.load(b, p.ldb, krem, nrem, tid);
        };
        auto compute = [&](int stage) {
            const char *sa = smem + stage * STAGE;
            const char *sb = sa + A_BYTES;
            Fr f[2];
            load_frags(sa, sb, 0, a_row0, b_row0, a_prow0, b_prow0, lh, f[0]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g + 1 < G) load_frags(sa, sb, g + 1, a_row0, b_row0, a_prow0, b_prow0, lh, f[(g + 1) & 1]);
                f[g & 1].mfmas(acc);
            }
        };
        const int nk = (p.K + BK - 1) / BK;
        lds_poison<2 * STAGE>(smem);
        if constexpr (!REG2) {
            // two LDS stages, the next slab fetched to registers during the current one
            OpA la;
            OpB lb;
            load_slab(0, la, lb);
            la.store(smem, tid);
            lb.store(smem + A_BYTES, tid);
            __syncthreads();
            for (int kt = 0; kt + 1 < nk; ++kt) {
                load_slab(kt + 1, la, lb);
                compute(kt & 1);
                char *st = smem + ((kt + 1) & 1) * STAGE;
                la.store(st, tid);
                lb.store(st + A_BYTES, tid);
                __syncthreads();
                lds_poison<STAGE>(smem + (kt & 1) * STAGE);  // read by every wave
            }
            compute((nk - 1) & 1);
        } else {
            // Two LDS stages and two register sets: the loads of slab kt+2 are
            // issued before slab kt is computed and written to LDS only after
            // slab kt+1 has been, so each load has two slabs of compute to
            // arrive.  At step kt, LDS stage kt&1 holds slab kt and register
            // set (kt+1)&1 holds slab kt+1; set kt&1 (stored one step ago) is
            // free.  The loop is unrolled by two so that the register sets are
            // distinct variables.
            OpA la0, la1;
            OpB lb0, lb1;
            load_slab(0, la0, lb0);
            if (nk > 1) load_slab(1, la1, lb1);
            la0.store(smem, tid);
            lb0.store(smem + A_BYTES, tid);
            __syncthreads();
            auto step = [&](int kt, OpA &free_a, OpB &free_b, const OpA &next_a, const OpB &next_b) {
                if (kt + 2 < nk) load_slab(kt + 2, free_a, free_b);
                compute(kt & 1);
                if (kt + 1 < nk) {
                    char *st = smem + ((kt + 1) & 1) * STAGE;
                    next_a.store(st, tid);
                    next_b.store(st + A_BYTES, tid);
                    __syncthreads();
                    lds_poison<STAGE>(smem + (kt & 1) * STAGE);  // read by every wave
                }
            };
            int kt = 0;
            for (; kt + 1 < nk; kt += 2) {
                step(kt, la0, lb0, la1, lb1);
                step(kt + 1, la1, lb1, la0, lb0);
            }
            if (kt < nk) step(kt, la0, lb0, la1, lb1);
        }
    }
};

// ===========================================================================
// DmaPath: every tile of a 16-byte aligned problem whose K is a multiple of
// the 16-byte chunk (CH elements).  Global -> LDS with buffer_load_dwordx4
// ... lds (no registers in between) into a ring of NS LDS stages of BK
// elements.  Chunks past K, and rows past the matrix, are masked to zero by
// the buffer range check, so edge tiles and the slab past the last whole one
// take the same copies.
// Schedules (PIPE):
//   1  BK = BKR/2 (32 for 16-bit, 16 for fp32), NS = 4, loads issued 3 slabs
//      ahead; every wave reads and multiplies each slab, with one barrier per
//      slab placed before the MFMAs of its last k-group so that the next
//      slab's first fragment reads overlap them.
//   2  the same with BK = BKR, NS = 2 (one slab ahead, half the barriers).
//   3  one stage of BK = BKR, for K <= BKR only (one slab, e.g. attention
//      scores over a 64-wide head): half the LDS, so that two workgroups
//      share a CU and one's C stores overlap the other's loads;
//   4  for every tile of a problem whose rows are 4-byte aligned (and, for
//      8/16-bit elements, whose K is a multiple of the 4-byte piece), BK =
//      BKR, NS = 2.  Whole slabs with operand rows after them are copied 16
//      bytes per lane at 4-byte aligned addresses (a multi-dword access
//      needs only dword alignment; fp32 measured as fast as on 16-byte
//      aligned rows, 16-bit and int8 1.3 to 1.5 times slower per K, still
//      well ahead of the register path).  The last slab of a tile takes
//      4-byte copies: each lane copies one piece, and lanes whose piece lies
//      past the matrix (row, column or k) are masked to zero by the buffer
//      range check, so edges, K tails and leading dimensions that are no
//      multiple of 16 bytes need no register path.
//
// LDS layouts (bank-conflict free for every access of this path):
//   KC  operand K-contiguous in memory: rows of BK elements (RB = 64 or 128
//       bytes, a quarter or half of a 256-byte bank line); physical row order
//       as phys_row; chunk c of physical row p at c ^ swz(p), with
//       swz(p) = (p >> 2) & 3 for 64-byte rows and (p >> 1) & 7 for 128-byte
//       rows.  A fragment read touches 16 consecutive physical rows per 16
//       lanes, which then cover the 16 distinct 16-byte slots of a line.
//   MC  operand MN-contiguous in memory: BK rows of MN elements, stored as
//       in memory but with its 64-byte pieces permuted per row
//       (piece ^ key(k)), so the 4 rows read together land in 4 distinct
//       64-byte groups of banks.  16-bit MC operands are read with
//       ds_read_b64_tr_b16: within a 16-lane group, source lane j supplies
//       4 values at row k0 + j/4, columns n0 + 4*(j%4) .. +3, and lane i
//       receives column n0 + i of rows k0 .. k0+3.  The MFMA lanes of a
//       16-bit MC operand therefore index consecutive (not interleaved)
//       rows/columns (interleave 1).
// ===========================================================================
template <typename T, int BM, int BN, int BKR, int WM, int WN, bool TA, bool TB, int PIPE>
struct DmaPath {
    static constexpr int NT = WM * WN * 64;
    static constexpr int NW = WM * WN;
    static constexpr int ES = sizeof(T);
    static constexpr bool F32 = (ES == 4);
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr bool DW = PIPE == 4;  // every tile; 4-byte copies on the last slab
    static constexpr bool ONE = PIPE == 3;  // one stage, one slab (K <= BKR)
    static constexpr int BK = PIPE == 2 || DW || ONE ? BKR : BKR / 2;
    static constexpr int NS = PIPE == 1 ? 4 : ONE ? 1 : 2;
    static constexpr int RB = BK * ES;          // K-contiguous row bytes
    static_assert(RB == 64 || RB == 128, "64- or 128-byte K-contiguous rows");
    static constexpr int CPR = RB / 16;         // 16-byte chunks per row
    static constexpr int CH = 16 / ES;          // elements per 16-byte chunk: K % CH == 0 on this path
    static constexpr int G = F32 ? BK / 8 : BK * ES / 32;  // k-groups (32 bytes of k) per slab
    static constexpr bool A_KC = !TA, B_KC = TB;
    static constexpr bool A_TR = TA && !F32, B_TR = !TB && !F32;
    // raised priority while multiplying (with 4-byte copies on every slab
    // the 4-byte-copy builds lost 4% to it on the ragged fp32 shape; with
    // 16-byte copies on all but the last slab they gain 0-2%, same-box A/B
    // over odd leading dimensions from 1000x1024x999 to 3000x3001x2999)
    static constexpr bool PRIO = F32 || B_KC;
    // 256x256 16-bit tiles whose B is MN-contiguous (transposing fragment
    // reads): each group's fragment reads are issued at two per MFMA from
    // its start, and after the slab barrier the copies of the next slab
    // alternate one by one with the last group's MFMAs instead of issuing as
    // one block.  Same-box A/Bs, bf16 NN and TN: 4 to 5% faster at 4096^3
    // and 8192^3, 7 to 11% at 2048^3.  With a K-contiguous B the order
    // measured level, and on 128x128 and 64x64 tiles between 7% faster and
    // 6% slower by shape, so those keep the compiler's order.
    static constexpr bool SPREAD = !F32 && !DW && B_TR && BM == 256 && BN == 256;
    static constexpr int IL_A = A_TR ? 1 : TM, IL_B = B_TR ? 1 : TN;
    static constexpr int A_BYTES = BM * BK * ES, B_BYTES = BN * BK * ES;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = NS * STAGE;
    static constexpr int A_ROWB = BM * ES, B_ROWB = BN * ES;  // MC row bytes
    static constexpr int CPY = DW ? 256 : 1024;  // LDS bytes one copy instruction fills
    static_assert(A_BYTES % (CPY * NW) == 0 && B_BYTES % (CPY * NW) == 0, "DMA split");
    static constexpr int A_IPW = A_BYTES / CPY / NW, B_IPW = B_BYTES / CPY / NW;
    // 4-byte-copy builds copy every slab but a tile's last with 16-byte
    // copies (issue()); those counts per wave
    static constexpr int A_IPW16 = A_BYTES / 1024 / NW, B_IPW16 = B_BYTES / 1024 / NW;
    static_assert(!DW || (A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0), "16-byte DMA split");
    // DMA loads per slab per thread, as the waits count them: the 16-byte
    // count in the 4-byte-copy builds, whose only slab of 4-byte copies is
    // the last (a wait that allows fewer loads in flight than there are
    // waits longer, never too short)
    static constexpr int LPS = DW ? A_IPW16 + B_IPW16 : A_IPW + B_IPW;
    static_assert((NS - 1) * LPS <= 63, "vmcnt range");
    static_assert(A_KC || A_ROWB >= 128, "MC rows of at least 128 bytes");
    static_assert(B_KC || B_ROWB >= 128, "MC rows of at least 128 bytes");

    using Fr = Frags<T, TM, TN>;

    __device__ __forceinline__ static int swz(int p) { return RB == 64 ? ((p >> 2) & 3) : ((p >> 1) & 7); }

    __device__ __forceinline__ static int kc_off(int p, int kbyte)
    {
        const int chunk = (kbyte >> 4) ^ swz(p);
        return p * RB + (chunk << 4) + (kbyte & 15);
    }

    template <int ROWB>
    __device__ __forceinline__ static int mc_key(int k)
    {
        return ROWB >= 256 ? (k & 3) : ((k >> 1) & 1);
    }

    template <int ROWB>
    __device__ __forceinline__ static int mc_off(int k, int byte)
    {
        if constexpr (ES == 1) return mc8_off<ROWB>(k, byte);
        return k * ROWB + (((byte >> 6) ^ mc_key<ROWB>(k)) << 6) + (byte & 63);
    }

    // byte column of the memory tile that physical byte bb of MC row k holds
    // (both permutations are their own inverses)
    template <int ROWB>
    __device__ __forceinline__ static int mc_logical(int k, int bb)
    {
        if constexpr (ES == 1) return (mc8_chunk<ROWB>(k, bb >> 4) << 4) | (bb & 15);
        return (((bb >> 6) ^ mc_key<ROWB>(k)) << 6) | (bb & 63);
    }

    // DMA instruction q (of IPW) of wave `w` for one operand's slab: 1 KB into
    // the operand's region `dst` of a stage, from tile origin `src`.  Memory
    // tile rows < rows_ok and columns < cols_ok exist (rows k and columns m/n
    // for an MC operand, rows m/n and columns k for a KC one).  A chunk of a
    // row past rows_ok, or starting at or past cols_ok, gets an out-of-range
    // offset: the copy writes zeros to its 16 LDS bytes and reads no memory.
    // K is a multiple of CH, so no KC chunk straddles the end of K.  An MC
    // chunk that straddles the m/n edge is read whole: it is 16-byte aligned
    // and holds a valid element, so it lies inside a mapped page, and its
    // values past the edge feed only rows or columns of C that are not stored.
    // (The 4-byte-copy builds also use these copies on rows that are only
    // 4-byte aligned, on whole slabs that end before row K-1; see issue().)
    // CHECK false (interior tiles with whole slabs): no masking, and the
    // offsets do not depend on the slab.
    template <bool KC, int IL, int ROWB, int IPW, bool CHECK>
    __device__ __forceinline__ static void dma_one(__amdgpu_buffer_rsrc_t rs, char *dst, int ld_bytes, int w,
                                                   int lane, int q, int rows_ok, int cols_ok)
    {
        const int ins = w * IPW + q;
        if constexpr (KC) {
            // 1024/RB physical rows pb.. of RB bytes; lane -> row pb + lane/CPR, physical
            // chunk lane%CPR holding logical chunk (lane%CPR) ^ swz(row); the logical
            // rows are logical_row(pb) + (lane/CPR)*IL.
            constexpr int RPI = 1024 / RB;
            const int pb = ins * RPI;
            const int j = lane / CPR;
            const int c = (lane % CPR) ^ swz(pb + j);
            const int row0 = logical_row<IL>(pb);
            int voff = j * IL * ld_bytes + (c << 4);
            if (CHECK && (row0 + j * IL >= rows_ok || c * CH >= cols_ok)) voff = kOutOfRange;
            const int soff = __builtin_amdgcn_readfirstlane(row0 * ld_bytes);
            dma16(rs, lds_addr_of(dst + pb * RB), voff, soff);
        } else {
            // bytes b = ins*1024 + 16*lane of the [BK][MN] region: row k = b / ROWB,
            // physical byte b % ROWB holds logical byte mc_logical(k, b % ROWB)
            const int b = ins * 1024 + 16 * lane;
            const int k = b / ROWB, bb = b % ROWB;
            const int lb = mc_logical<ROWB>(k, bb);
            const int voff = (CHECK && (k >= rows_ok || lb >= cols_ok * ES)) ? kOutOfRange : k * ld_bytes + lb;
            dma16(rs, lds_addr_of(dst + ins * 1024), voff, 0);
        }
    }

    // 4-byte copy instruction q (of IPW) of wave `w`: 256 bytes of the
    // operand's region `dst`, laid out exactly as dma_one lays them (KC rows
    // with swizzled chunks, or MC rows with permuted pieces).  Each lane
    // copies one 4-byte piece (1, 2 or 4 elements) of 4-byte aligned rows.
    // Memory tile rows < rows_ok and columns < cols_ok exist; a piece in a
    // row past rows_ok, or starting at or past cols_ok, reads as zero through
    // an out-of-range offset.  For KC operands K is a multiple of the piece;
    // an MC piece that straddles the m/n edge is read whole (it lies in the
    // page of its first element and feeds only C elements that are not stored).
    template <bool KC, int IL, int ROWB, int IPW>
    __device__ __forceinline__ static void dma_dw(__amdgpu_buffer_rsrc_t rs, char *dst, int ld_bytes, int w,
                                                  int lane, int q, int rows_ok, int cols_ok)
    {
        const int ins = w * IPW + q;
        const int b = ins * 256 + 4 * lane;  // byte of the operand's LDS region
        int r, cb;                           // memory row and byte column of the tile
        if constexpr (KC) {
            const int pr = b / RB, within = b % RB;   // physical row, byte within it
            r = logical_row<IL>(pr);
            cb = (((within >> 4) ^ swz(pr)) << 4) | (within & 15);
        } else {
            const int k = b / ROWB, bb = b % ROWB;
            r = k;
            cb = mc_logical<ROWB>(k, bb);
        }
        const int voff = (r < rows_ok && cb < cols_ok * ES) ? r * ld_bytes + cb : kOutOfRange;
        dma4(rs, lds_addr_of(dst + ins * 256), voff);
    }

    // Fragment of one MC 16-bit operand (rows k, columns mn): the 8 k-values
    // 16g + 8h + 0..7 of column (wave-local) base + 16*((lane/16)&1) + lane%16,
    // via two transposing reads.
    template <int ROWB>
    __device__ __forceinline__ static u32x4 tr_frag(const char *s, int g, int lh, int col_base, int lane)
    {
        const int gi = lane & 15;
        const int col = col_base + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
        const int k0 = 16 * g + 8 * lh + (gi >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(s + mc_off<ROWB>(k0, col * 2)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(s + mc_off<ROWB>(k0 + 4, col * 2)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }

    struct Lane {
        int lane, li, lh;
        int a_row0, b_row0;    // fp32 MC: first interleaved row/column of this lane
        int a_prow0, b_prow0;  // KC: physical row of sub-tile 0
        int a_blk, b_blk;      // 16-bit MC: wave-local base of sub-tile 0
    };

    __device__ __forceinline__ static void load_frags(const char *sa, const char *sb, int g, const Lane &L, Fr &f)
    {
        if constexpr (F32) {
            if constexpr (A_KC) {
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(sa + kc_off(L.a_prow0 + 32 * t, (8 * g + 4 * L.lh) * 4));
#pragma unroll
                    for (int s = 0; s < 4; ++s) f.a32[t][s] = v[s];
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float v[TM];
                    lds_floats<TM>(sa + mc_off<A_ROWB>(8 * g + 4 * L.lh + s, L.a_row0 * 4), v);
#pragma unroll
                    for (int t = 0; t < TM; ++t) f.a32[t][s] = v[t];
                }
            }
            if constexpr (B_KC) {
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(sb + kc_off(L.b_prow0 + 32 * u, (8 * g + 4 * L.lh) * 4));
#pragma unroll
                    for (int s = 0; s < 4; ++s) f.b32[u][s] = v[s];
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float v[TN];
                    lds_floats<TN>(sb + mc_off<B_ROWB>(8 * g + 4 * L.lh + s, L.b_row0 * 4), v);
#pragma unroll
                    for (int u = 0; u < TN; ++u) f.b32[u][s] = v[u];
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if constexpr (A_KC)
                    f.a16[t] = *reinterpret_cast<const u32x4 *>(sa + kc_off(L.a_prow0 + 32 * t, (16 * g + 8 * L.lh) * 2));
                else if constexpr (ES == 1)
                    f.a16[t] = tr8_frag<A_ROWB>(sa, g, L.lh, L.a_blk + 32 * t, L.lane);
                else
                    f.a16[t] = tr_frag<A_ROWB>(sa, g, L.lh, L.a_blk + 32 * t, L.lane);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                if constexpr (B_KC)
                    f.b16[u] = *reinterpret_cast<const u32x4 *>(sb + kc_off(L.b_prow0 + 32 * u, (16 * g + 8 * L.lh) * 2));
                else if constexpr (ES == 1)
                    f.b16[u] = tr8_frag<B_ROWB>(sb, g, L.lh, L.b_blk + 32 * u, L.lane);
                else
                    f.b16[u] = tr_frag<B_ROWB>(sb, g, L.lh, L.b_blk + 32 * u, L.lane);
            }
        }
    }

    // per-group instruction counts (for the schedule hints)
    static constexpr int DSR_A = F32 ? (A_KC ? TM : 4) : (A_KC ? TM : 2 * TM);
    static constexpr int DSR_B = F32 ? (B_KC ? TN : 4) : (B_KC ? TN : 2 * TN);
    static constexpr int DSR = DSR_A + DSR_B;
    static constexpr int MF = F32 ? 4 * TM * TN : TM * TN;

    template <int N>
    __device__ __forceinline__ static void wait_ahead()
    {
        wait_counts<N * LPS, 0>();
    }

    // wait_ahead<n> for a run-time n in [0, N] (n above N waits as N)
    template <int N>
    __device__ __forceinline__ static void wait_ahead_upto(int n)
    {
        if constexpr (N == 0) {
            wait_ahead<0>();
        } else {
            if (n >= N) wait_ahead<N>();
            else        wait_ahead_upto<N - 1>(n);
        }
    }

    // MFMA I, then copy I, for I = 0 .. max(NM, NC) - 1, in that order
    // (sched_barrier keeps the scheduler from regrouping them)
    template <int I, int NM, int NC, typename FM, typename FC>
    __device__ __forceinline__ static void alternate(FM &mfma, FC &copy)
    {
        if constexpr (I < NM || I < NC) {
            if constexpr (I < NM) mfma(std::integral_constant<int, I>{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (I < NC) copy(I);
            __builtin_amdgcn_sched_barrier(0);
            alternate<I + 1, NM, NC>(mfma, copy);
        }
    }

    // CHECK: mask copies against the matrix edges and K (edge tiles, a K
    // tail); without it the tile must be interior with whole slabs.
    // k_more: the operands have rows past this K (a split-K chunk or
    // stream-K segment that ends before the end of K)
    template <bool CHECK>
    __device__ __forceinline__ static void run(const KernelArgs &p, char *smem, int bidx, int m0, int n0,
                                               f32x16 (&acc)[TM][TN], bool k_more = false)
    {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = w / WN, wn = w % WN;
        Lane L;
        L.lane = lane;
        L.li = lane & 31;
        L.lh = lane >> 5;
        L.a_row0 = wm * WTM + TM * L.li;
        L.b_row0 = wn * WTN + TN * L.li;
        L.a_prow0 = wm * WTM + L.li;
        L.b_prow0 = wn * WTN + L.li;
        L.a_blk = wm * WTM;
        L.b_blk = wn * WTN;

        const char *Ap = static_cast<const char *>(p.A) + (int64_t)bidx * p.strideA * ES +
                         (TA ? (int64_t)m0 : (int64_t)m0 * p.lda) * ES;
        const char *Bp = static_cast<const char *>(p.B) + (int64_t)bidx * p.strideB * ES +
                         (TB ? (int64_t)n0 * p.ldb : (int64_t)n0) * ES;
        const int64_t a_kstep = (TA ? (int64_t)BK * p.lda : (int64_t)BK) * ES;
        const int64_t b_kstep = (TB ? (int64_t)BK : (int64_t)BK * p.ldb) * ES;
        const int lda_b = (int)(p.lda * ES), ldb_b = (int)(p.ldb * ES);

        auto stage = [&](int s) { return smem + (s % NS) * STAGE; };
        const int mrem = p.M - m0, nrem = p.N - n0;
        // 4-byte-copy builds: rows of at least 16 bytes take 16-byte copies
        // on every slab but the last
        const bool wide = DW && p.M * ES >= 16 && p.N * ES >= 16;
        // 16-byte copy q (of LPS: A's first, then B's) of slab s into stage
        // st, the same copies as issue(s) makes
        auto copy_of = [&](int s, char *st, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int q) {
            const int krem = p.K - s * BK;
            if (q < A_IPW)
                dma_one<A_KC, IL_A, A_ROWB, A_IPW, CHECK>(ra, st, lda_b, w, lane, q, A_KC ? mrem : krem,
                                                          A_KC ? krem : mrem);
            else
                dma_one<B_KC, IL_B, B_ROWB, B_IPW, CHECK>(rb, st + A_BYTES, ldb_b, w, lane, q - A_IPW,
                                                          B_KC ? nrem : krem, B_KC ? krem : nrem);
        };
        auto issue = [&](int s) {
            char *st = stage(s);
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ap + (int64_t)s * a_kstep);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bp + (int64_t)s * b_kstep);
            if constexpr (DW) {
                const int krem = p.K - s * BK;
                if (wide && (krem > BK || (krem == BK && k_more))) {
                    // 16-byte copies of rows that may be only 4-byte aligned
                    // (a multi-dword access needs dword alignment alone): the
                    // slab is whole, so no KC chunk straddles the end of K,
                    // and a row of the operand follows its last row, so an MC
                    // chunk that straddles the m/n edge reads at most 16-ES
                    // bytes past its row's last element, which lie in a later
                    // row (wide: at least 16 bytes per row)
#pragma unroll
                    for (int q = 0; q < A_IPW16; ++q)
                        dma_one<A_KC, IL_A, A_ROWB, A_IPW16, true>(ra, st, lda_b, w, lane, q, A_KC ? mrem : krem,
                                                                   A_KC ? krem : mrem);
#pragma unroll
                    for (int q = 0; q < B_IPW16; ++q)
                        dma_one<B_KC, IL_B, B_ROWB, B_IPW16, true>(rb, st + A_BYTES, ldb_b, w, lane, q,
                                                                   B_KC ? nrem : krem, B_KC ? krem : nrem);
                } else {
                    // the last slab: 4-byte pieces, each checked against K and the edges
#pragma unroll
                    for (int q = 0; q < A_IPW; ++q)
                        dma_dw<A_KC, IL_A, A_ROWB, A_IPW>(ra, st, lda_b, w, lane, q, A_KC ? mrem : krem,
                                                          A_KC ? krem : mrem);
#pragma unroll
                    for (int q = 0; q < B_IPW; ++q)
                        dma_dw<B_KC, IL_B, B_ROWB, B_IPW>(rb, st + A_BYTES, ldb_b, w, lane, q,
                                                          B_KC ? nrem : krem, B_KC ? krem : nrem);
                }
            } else {
                // CHECK is fixed for the whole tile: a branch between checked
                // and unchecked copies inside one loop cost the LDS address
                // its scalar register
                const int krem = p.K - s * BK;
#pragma unroll
                for (int q = 0; q < A_IPW; ++q)
                    dma_one<A_KC, IL_A, A_ROWB, A_IPW, CHECK>(ra, st, lda_b, w, lane, q, A_KC ? mrem : krem,
                                                              A_KC ? krem : mrem);
#pragma unroll
                for (int q = 0; q < B_IPW; ++q)
                    dma_one<B_KC, IL_B, B_ROWB, B_IPW, CHECK>(rb, st + A_BYTES, ldb_b, w, lane, q,
                                                              B_KC ? nrem : krem, B_KC ? krem : nrem);
            }
        };
        auto frags = [&](int s, int g, Fr &f) {
            const char *st = stage(s);
            load_frags(st, st + A_BYTES, g, L, f);
        };

        const int nk = (p.K + BK - 1) / BK;  // a K tail is one more slab, zero-filled past K
        lds_poison<LDS_BYTES>(smem);
        // prologue: slabs 0..NS-1 in flight, wait for slab 0
        issue(0);
#pragma unroll
        for (int s = 1; s < NS; ++s)
            if (s < nk) issue(s);
        {
            const int inflight = nk < NS ? nk : NS;  // slabs issued
            wait_ahead_upto<NS - 1>(inflight - 1);
        }
        lds_barrier();

        Fr f[2];
        frags(0, 0, f[0]);
        // one slab: groups 0..G-2 with the next group's fragments read under
        // the MFMAs; then wait for slab kt+1 (my copies), barrier, refill the
        // freed stage, read slab kt+1's first group under the last group's MFMAs
        auto body_head = [&](int kt) {
#pragma unroll
            for (int g = 0; g + 1 < G; ++g) {
                frags(kt, g + 1, f[(g + 1) & 1]);
                f[g & 1].mfmas(acc);
                if constexpr (SPREAD) sched_front<SG_MFMA, MF, SG_DS_READ, DSR, 2>();
                else                  sched_interleave<SG_MFMA, MF, SG_DS_READ, DSR>();
            }
        };
        int kt = 0;
        // steady state: slab kt+NS exists; at the wait, slabs kt+2 .. kt+NS-1
        // may still be in flight (a one-stage build has a single slab)
        if constexpr (NS >= 2)
        for (; kt + NS < nk; ++kt) {
            // A wave multiplying a slab outranks one at its copies and waits
            // (two waves share each SIMD).  Measured in a same-box A/B: fp32
            // 4096^3 within 0.8%, 16-bit with a K-contiguous B -1.5%, int8
            // -1.5 to -2.5%, while 16-bit with an MN-contiguous B
            // (transposing reads) lost 0.6%: it keeps the default priority.
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
            body_head(kt);
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            wait_ahead<NS - 2>();
            lds_barrier();
            lds_poison<STAGE>(stage(kt));  // read by every wave; refilled below
            if constexpr (SPREAD) {
                frags(kt + 1, 0, f[G & 1]);
                __builtin_amdgcn_sched_barrier(0);
                const int sn = kt + NS;
                char *st = stage(sn);
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ap + (int64_t)sn * a_kstep);
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bp + (int64_t)sn * b_kstep);
                const Fr &fl = f[(G - 1) & 1];
                auto mfma = [&](auto i) { fl.template mfma_at<decltype(i)::value>(acc); };
                auto copy = [&](int q) { copy_of(sn, st, ra, rb, q); };
                alternate<0, MF, LPS>(mfma, copy);
            } else {
                issue(kt + NS);
                frags(kt + 1, 0, f[G & 1]);
                f[(G - 1) & 1].mfmas(acc);
                sched_interleave<SG_MFMA, MF, SG_DS_READ, DSR>();
            }
        }
        // last slabs: everything already issued
        for (; kt < nk; ++kt) {
            body_head(kt);
            if constexpr (NS >= 2) {
                if (kt + 1 < nk) {
                    const int ahead = nk - kt - 2;  // slabs after kt+1 still possibly in flight
                    wait_ahead_upto<NS - 2>(ahead);
                    lds_barrier();
                    frags(kt + 1, 0, f[G & 1]);
                }
            }
            f[(G - 1) & 1].mfmas(acc);
        }
    }
};

// ---------------------------------------------------------------------------
// Epilogue: C = alpha*acc + beta*C (C read only when beta != 0).  IL_A / IL_B
// give the sub-tile interleave of rows / columns: row of (t, i') is
// IL_A == 1 ? 32t + i' : TM*i' + t, likewise for columns; with interleaved
// columns each lane holds TN adjacent columns and stores them as one vector.
// C is written with non-temporal stores: it is not read again by this kernel,
// and streaming it past the caches raised the store-bound shallow-K batch
// (attention scores, K = 64) from 5.6 to 6.5 TB/s, with no change on the
// compute-bound shapes.
// ---------------------------------------------------------------------------
template <typename CT, int N>
struct CVec {
    typedef CT type __attribute__((ext_vector_type(N)));
};

// N adjacent elements of C at cp (aligned to N elements when N > 1):
// v + beta * C_old, rounded to CT (round to nearest even), stored as one
// non-temporal vector.
// int32 C of int8 inputs: alpha*acc + beta*C in 32-bit two's-complement
// arithmetic (wrapping), stored as N adjacent ints.
template <int N>
__device__ __forceinline__ void store_c_int(int32_t *cp, const uint32_t *v, bool use_beta, uint32_t beta)
{
    if constexpr (N == 1) {
        const uint32_t o = use_beta ? v[0] + beta * (uint32_t)*cp : v[0];
        __builtin_nontemporal_store((int32_t)o, cp);
    } else {
        using V = typename CVec<int32_t, N>::type;
        V o;
        if (use_beta) {
            const V old = *reinterpret_cast<const V *>(cp);
#pragma unroll
            for (int u = 0; u < N; ++u) o[u] = (int32_t)(v[u] + beta * (uint32_t)old[u]);
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u) o[u] = (int32_t)v[u];
        }
        __builtin_nontemporal_store(o, reinterpret_cast<V *>(cp));
    }
}

template <typename CT, int N>
__device__ __forceinline__ void store_c(CT *cp, const float *v, bool use_beta, float beta)
{
    if constexpr (N == 1) {
        const float o = use_beta ? v[0] + beta * (float)*cp : v[0];
        __builtin_nontemporal_store((CT)o, cp);
    } else {
        using V = typename CVec<CT, N>::type;
        V o;
        if (use_beta) {
            const V old = *reinterpret_cast<const V *>(cp);
#pragma unroll
            for (int u = 0; u < N; ++u) o[u] = (CT)(v[u] + beta * (float)old[u]);
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u) o[u] = (CT)v[u];
        }
        __builtin_nontemporal_store(o, reinterpret_cast<V *>(cp));
    }
}

template <bool EDGE, int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN, typename CT>
__device__ __forceinline__ void epilogue_fp(const KernelArgs &p, int bidx, int m0, int n0,
                                            const f32x16 (&acc)[TM][TN]);

// Register r of an int32 accumulator held in an f32x16.  The whole vector is
// reinterpreted before indexing: a bit cast applied to one element of an
// ext_vector lvalue compiled to a read of element 0 whatever the index.
__device__ __forceinline__ uint32_t acc_u32(const f32x16 &v, int r)
{
    return (uint32_t)__builtin_bit_cast(i32x16, v)[r];
}

// The same mapping for int32 accumulators (int8 inputs) and int32 C.
template <bool EDGE, int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN>
__device__ __forceinline__ void epilogue_int(const KernelArgs &p, int bidx, int m0, int n0,
                                             const f32x16 (&acc)[TM][TN])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 31, lh = lane >> 5;
    int32_t *Cb = static_cast<int32_t *>(p.C) + (int64_t)bidx * p.strideC;
    const bool use_beta = p.beta_i != 0;
    const uint32_t alpha = (uint32_t)p.alpha_i, beta = (uint32_t)p.beta_i;
    constexpr bool VCOL = IL_B > 1;
    const int colv = n0 + wn * WTN + TN * li;
    const bool vec_store = VCOL && p.c_vec && (!EDGE || colv + TN <= p.N);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ip = 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int row = m0 + wm * WTM + (IL_A == 1 ? 32 * t + ip : TM * ip + t);
            if (EDGE && row >= p.M) continue;
            int32_t *crow = Cb + (int64_t)row * p.ldc;
            if constexpr (VCOL) {
                uint32_t v[TN];
#pragma unroll
                for (int u = 0; u < TN; ++u) v[u] = alpha * acc_u32(acc[t][u], r);
                int32_t *cp = crow + colv;
                if (vec_store) {
                    store_c_int<TN>(cp, v, use_beta, beta);
                } else {
#pragma unroll
                    for (int u = 0; u < TN; ++u)
                        if (!EDGE || colv + u < p.N) store_c_int<1>(cp + u, v + u, use_beta, beta);
                }
            } else {
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    const int col = n0 + wn * WTN + 32 * u + li;
                    if (EDGE && col >= p.N) continue;
                    const uint32_t v = alpha * acc_u32(acc[t][u], r);
                    store_c_int<1>(crow + col, &v, use_beta, beta);
                }
            }
        }
    }
}

template <bool EDGE, int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN, typename CT>
__device__ __forceinline__ void epilogue(const KernelArgs &p, int bidx, int m0, int n0,
                                         const f32x16 (&acc)[TM][TN])
{
    if constexpr (__is_same(CT, int32_t))
        epilogue_int<EDGE, IL_A, IL_B, TM, TN, WTM, WTN, WN>(p, bidx, m0, n0, acc);
    else
        epilogue_fp<EDGE, IL_A, IL_B, TM, TN, WTM, WTN, WN, CT>(p, bidx, m0, n0, acc);
}

template <bool EDGE, int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN, typename CT>
__device__ __forceinline__ void epilogue_fp(const KernelArgs &p, int bidx, int m0, int n0,
                                            const f32x16 (&acc)[TM][TN])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 31, lh = lane >> 5;
    CT *Cb = static_cast<CT *>(p.C) + (int64_t)bidx * p.strideC;
    const bool use_beta = p.beta != 0.0f;
    constexpr bool VCOL = IL_B > 1;  // TN adjacent columns per lane
    const int colv = n0 + wn * WTN + TN * li;
    const bool vec_store = VCOL && p.c_vec && (!EDGE || colv + TN <= p.N);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ip = 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int row = m0 + wm * WTM + (IL_A == 1 ? 32 * t + ip : TM * ip + t);
            if (EDGE && row >= p.M) continue;
            CT *crow = Cb + (int64_t)row * p.ldc;
            if constexpr (VCOL) {
                float v[TN];
#pragma unroll
                for (int u = 0; u < TN; ++u) v[u] = p.alpha * acc[t][u][r];
                CT *cp = crow + colv;
                if (vec_store) {
                    store_c<CT, TN>(cp, v, use_beta, p.beta);
                } else {
#pragma unroll
                    for (int u = 0; u < TN; ++u)
                        if (!EDGE || colv + u < p.N) store_c<CT, 1>(cp + u, v + u, use_beta, p.beta);
                }
            } else {
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    const int col = n0 + wn * WTN + 32 * u + li;
                    if (EDGE && col >= p.N) continue;
                    const float v = p.alpha * acc[t][u][r];
                    store_c<CT, 1>(crow + col, &v, use_beta, p.beta);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel.
//   T          float, _Float16, __bf16 or int8_t (A and B element type)
//   BM, BN     workgroup tile
//   BK         K-slab of the register path (the DMA path uses BK/2)
//   WM, WN     wavefront grid; each wave owns a (BM/WM) x (BN/WN) sub-tile
//              made of TM x TN MFMA blocks of 32x32
//   TA, TB     op(A) = A^T, op(B) = B^T
//   VECOK      A and B allow 16-byte global accesses (enables DmaPath)
//   PIPE       DmaPath schedule: 1 -> 4 stages of BK/2, 2 -> 2 stages of BK,
//              3 -> 1 stage of BK (K <= BK), 4 -> 4-byte copies, 2 stages of BK
//   CT         C element type: float, T itself (16-bit output), or int32_t
//              (int8 inputs)
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VECOK, int PIPE,
          typename CT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(KernelArgs p)
{
    using R = RegPath<T, BM, BN, BK, WM, WN, TA, TB, VECOK>;
    using D = DmaPath<T, BM, BN, BK, WM, WN, TA, TB, PIPE>;
    constexpr int TM = R::TM, TN = R::TN, WTM = R::WTM, WTN = R::WTN;
    // 4-byte copies serve every tile, and one-stage builds run only where the
    // DMA path serves every tile: no register path
    constexpr bool ALL_DMA = D::DW || D::ONE;
    constexpr int LDS = ALL_DMA ? D::LDS_BYTES
                        : (VECOK && D::LDS_BYTES > R::LDS_BYTES) ? D::LDS_BYTES : R::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[LDS];
    int bidx, tm, tn;
    map_tile(p, bidx, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    KernelArgs pk = p;  // this workgroup's K: split-K's last chunk may be shorter
    if (bidx == p.tail_batch) pk.K = p.k_tail;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = f32x16{};
    if constexpr (ALL_DMA) {
        const bool full = m0 + BM <= pk.M && n0 + BN <= pk.N;
        if constexpr (D::ONE) {
            if (full && pk.K == D::BK) D::template run<false>(pk, smem, bidx, m0, n0, acc);
            else                       D::template run<true>(pk, smem, bidx, m0, n0, acc);
        } else {
            // a split-K chunk before the last has the next chunk's rows after it
            D::template run<true>(pk, smem, bidx, m0, n0, acc, p.tail_batch >= 0 && bidx != p.tail_batch);
        }
        if (full)
            epilogue<false, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
        else
            epilogue<true, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
    } else {
        if constexpr (VECOK) {
            if (pk.fast_ok && pk.K % D::CH == 0) {
                const bool full = m0 + BM <= pk.M && n0 + BN <= pk.N;
                if (full && pk.K % D::BK == 0)
                    D::template run<false>(pk, smem, bidx, m0, n0, acc);
                else
                    D::template run<true>(pk, smem, bidx, m0, n0, acc);
                if (full)
                    epilogue<false, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
                else
                    epilogue<true, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
                return;
            }
        }
        R::run(pk, smem, bidx, m0, n0, acc);
        epilogue<true, R::IL_A, R::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
    }
}

// ---------------------------------------------------------------------------
// Stream-K: a grid of sk_grid workgroups shares one GEMM evenly, whatever
// the tile count.  The work is the list of (tile, K-iteration) pairs in
// tile-major order; logical workgroup L takes pairs [T*L/G, T*(L+1)/G)
// (T = sk_total, G = sk_grid) and walks them as segments, each within one
// tile.  A segment that covers a whole tile writes C as gemm_kernel does;
// any other writes its sums (fp32; int32 for int8 inputs) to one of the
// workgroup's two partial tiles in sk_part, slot 0 for its first segment
// and slot 1 for its last.  Only a workgroup's first and last segments can
// be partial, so a split tile's contributors are the consecutive
// workgroups g0..g1 that own its first and last iterations, and each
// workgroup is g0 of at most one split tile (the one its range ends in).
//
// Completion without a second launch: a contributor writes its partial tile
// with agent-scope stores, waits until they are acknowledged (then visible
// to every XCD), and counts itself in at sk_count[g0] with a wrapping
// increment (limit g1 - g0).  The contributor that reads g1 - g0 is the last
// to arrive; the same increment has put the counter back to zero, ready for
// the next launch.  That workgroup reads the partials with agent-scope loads,
// adds them in ascending K order, g0 first, and writes C.  No workgroup
// waits on another, and the sum order is fixed, whichever arrives last.
// (Agent-scope fences instead cost an L2-wide write-back per contribution
// and an L2 invalidate per tile: 1000x1027x999 fp32 took 108 us instead of
// 33.)  The host keeps G <= T, so every workgroup has at least one pair.
// ---------------------------------------------------------------------------

// Agent-scope accesses (one 32-bit value, or two adjacent as one 64-bit
// store): stores written through to the device-wide point of coherence and
// loads served from it, so partial sums pass between XCDs (each with its own
// L2) without an L2-wide write-back or invalidate.
__device__ __forceinline__ void sk_put2(void *at, uint32_t lo, uint32_t hi)
{
    __hip_atomic_store(static_cast<uint64_t *>(at), (uint64_t)hi << 32 | lo, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sk_put1(void *at, uint32_t v)
{
    __hip_atomic_store(static_cast<uint32_t *>(at), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A split tile's partial sums (fp32 bits, or int32 for int8 inputs) into
// `part`, the whole BM x BN tile row-major, with the C mapping of the
// epilogue below (IL_A / IL_B as there).
template <int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN, int BN>
__device__ __forceinline__ void sk_store_partial(void *part, const f32x16 (&acc)[TM][TN])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 31, lh = lane >> 5;
    uint32_t *P = static_cast<uint32_t *>(part);
    constexpr bool VCOL = IL_B > 1;  // TN adjacent columns per lane
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ip = 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            uint32_t *prow = P + (wm * WTM + (IL_A == 1 ? 32 * t + ip : TM * ip + t)) * BN;
            if constexpr (VCOL && TN % 2 == 0) {
#pragma unroll
                for (int u = 0; u < TN; u += 2)
                    sk_put2(prow + wn * WTN + TN * li + u, acc_u32(acc[t][u], r), acc_u32(acc[t][u + 1], r));
            } else {
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    sk_put1(prow + wn * WTN + (VCOL ? TN * li + u : 32 * u + li), acc_u32(acc[t][u], r));
            }
        }
    }
}

__device__ __forceinline__ uint32_t sk_get1(const uint32_t *at)
{
    return __hip_atomic_load(at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count-in of one contribution to a split tile whose contributors are the
// stream-K workgroups g0..g1; true when this workgroup completes the tile.
// Each contributor counts in once.  If all the others already have (the
// counter reads g1 - g0), this one is the last: it skips its partial tile,
// finishes from its registers and clears the counter for the next launch.
// Otherwise `store` writes its partial tile with agent-scope stores, every
// wave waits until they are acknowledged (then visible to every XCD), and
// the workgroup counts in with a wrapping increment (limit g1 - g0): the one
// that reads g1 - g0 is the last, and the same increment has reset the
// counter.  `flag` is a workgroup-shared int.  Call from uniform control flow.
template <typename Store>
__device__ __forceinline__ bool sk_arrive(const KernelArgs &p, int64_t g0, int64_t g1, int &flag, Store &&store)
{
    unsigned *count = p.sk_count + g0;
    const unsigned others = (unsigned)(g1 - g0);
    if (threadIdx.x == 0)
        flag = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == others;
    __syncthreads();
    // one value for the whole workgroup (read back from LDS): a uniform branch
    bool last = __builtin_amdgcn_readfirstlane(flag);
    if (!last) {
        store();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0)
            flag = __builtin_amdgcn_atomic_inc32(count, others, __ATOMIC_RELAXED, "agent") == others;
        __syncthreads();
        last = __builtin_amdgcn_readfirstlane(flag);
    } else if (threadIdx.x == 0) {
        __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return last;
}

// Stream-K partition: stream-K workgroup L takes (tile, iteration) pairs
// [T*L/G, T*(L+1)/G) (T = sk_total, G = sk_grid); a split tile whose pairs
// start at a0 belongs to workgroups g0 .. g1, the owners of its first and
// last pairs (owner(x) = ((x+1)*G - 1) / T).
__device__ __forceinline__ void sk_owners(const KernelArgs &p, int64_t a0, int64_t &g0, int64_t &g1)
{
    g0 = ((a0 + 1) * p.sk_grid - 1) / p.sk_total;
    g1 = ((a0 + p.sk_iters) * p.sk_grid - 1) / p.sk_total;
}

// The last contributor's share of stream-K: split tile (bidx, m0, n0), whose
// iterations start at a0 and belong to workgroups g0..g1, this one (me)
// among them.  Its own sums are still in `acc`; the others' partial tiles
// are read at the same C positions (the epilogue's mapping), the terms are
// added in ascending K order, g0 first (fp32, or wrapping int32 for int8
// inputs), and the epilogue writes C.
template <bool EDGE, int IL_A, int IL_B, int TM, int TN, int WTM, int WTN, int WN, int BM, int BN, typename PT,
          typename CT>
__device__ __forceinline__ void sk_finish(const KernelArgs &p, int bidx, int m0, int n0, int64_t a0, int64_t g0,
                                          int64_t g1, int64_t me, const f32x16 (&acc)[TM][TN])
{
    constexpr int TSZ = BM * BN;
    constexpr bool INT = __is_same(PT, int32_t);
    constexpr bool VCOL = IL_B > 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int li = lane & 31, lh = lane >> 5;
    const uint32_t *part = static_cast<const uint32_t *>(p.sk_part);
    const int first_slot = p.sk_total * g0 / p.sk_grid == a0 ? 0 : 1;
    f32x16 sum[TM][TN];
    for (int64_t g = g0; g <= g1; ++g) {
        const bool first = g == g0;
        if (g == me) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    if (first) {
                        sum[t][u] = acc[t][u];
                    } else if constexpr (INT) {
                        const u32x16 x = __builtin_bit_cast(u32x16, sum[t][u]) + __builtin_bit_cast(u32x16, acc[t][u]);
                        sum[t][u] = __builtin_bit_cast(f32x16, x);
                    } else {
                        sum[t][u] = sum[t][u] + acc[t][u];
                    }
                }
            continue;
        }
        const uint32_t *pg = part + (g * 2 + (first ? first_slot : 0)) * TSZ;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int col = wn * WTN + (VCOL ? TN * li + u : 32 * u + li);
                u32x16 v;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ip = 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int row = wm * WTM + (IL_A == 1 ? 32 * t + ip : TM * ip + t);
                    v[r] = sk_get1(pg + row * BN + col);
                }
                if (first) {
                    sum[t][u] = __builtin_bit_cast(f32x16, v);
                } else if constexpr (INT) {
                    sum[t][u] = __builtin_bit_cast(f32x16, __builtin_bit_cast(u32x16, sum[t][u]) + v);
                } else {
                    sum[t][u] = sum[t][u] + __builtin_bit_cast(f32x16, v);
                }
            }
    }
    epilogue<EDGE, IL_A, IL_B, TM, TN, WTM, WTN, WN, CT>(p, bidx, m0, n0, sum);
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VECOK, int PIPE,
          typename CT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_sk_kernel(KernelArgs p)
{
    using R = RegPath<T, BM, BN, BK, WM, WN, TA, TB, VECOK>;
    using D = DmaPath<T, BM, BN, BK, WM, WN, TA, TB, PIPE>;
    using PT = typename std::conditional<__is_same(T, int8_t), int32_t, float>::type;
    constexpr int TM = R::TM, TN = R::TN, WTM = R::WTM, WTN = R::WTN;
    constexpr bool ALL_DMA = D::DW;
    constexpr int LDS = ALL_DMA ? D::LDS_BYTES
                        : (VECOK && D::LDS_BYTES > R::LDS_BYTES) ? D::LDS_BYTES : R::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[LDS];
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
        KernelArgs pk = p;
        pk.A = static_cast<const T *>(p.A) + (TA ? ko * p.lda : ko);
        pk.B = static_cast<const T *>(p.B) + (TB ? ko : ko * p.ldb);
        pk.K = k1 == iters ? p.K - (int)ko : (k1 - k0) * p.sk_unit;
        pk.tail_batch = -1;
        f32x16 acc[TM][TN];
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                acc[t][u] = f32x16{};
        const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
        bool dma = ALL_DMA;
        if constexpr (ALL_DMA) {
            D::template run<true>(pk, smem, bidx, m0, n0, acc, k1 < iters);
        } else {
            if constexpr (VECOK) {
                if (pk.fast_ok && pk.K % D::CH == 0) {
                    dma = true;
                    if (full && pk.K % D::BK == 0)
                        D::template run<false>(pk, smem, bidx, m0, n0, acc);
                    else
                        D::template run<true>(pk, smem, bidx, m0, n0, acc);
                }
            }
            if (!dma) R::run(pk, smem, bidx, m0, n0, acc);
        }
        if (k0 == 0 && k1 == iters) {
            if (dma) {
                if (full) epilogue<false, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
                else      epilogue<true, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
            } else {
                epilogue<true, R::IL_A, R::IL_B, TM, TN, WTM, WTN, WN, CT>(pk, bidx, m0, n0, acc);
            }
        } else {
            const int64_t a0 = (int64_t)tile * iters;
            int64_t g0, g1;
            sk_owners(p, a0, g0, g1);
            const bool last = sk_arrive(p, g0, g1, last_arrival, [&] {
                // the whole BM x BN tile, row-major, into partial slot (L, first or last)
                void *slot = static_cast<PT *>(p.sk_part) + ((int64_t)L * 2 + (it == beg ? 0 : 1)) * (BM * BN);
                if (dma) sk_store_partial<D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, BN>(slot, acc);
                else     sk_store_partial<R::IL_A, R::IL_B, TM, TN, WTM, WTN, WN, BN>(slot, acc);
            });
            // (the range-checked epilogue for every finished tile: one more
            // instance of the unchecked one ran the 16-bit 4-byte-copy builds
            // out of scalar registers for their copies' buffer resources)
            if (last) {
                if (dma) sk_finish<true, D::IL_A, D::IL_B, TM, TN, WTM, WTN, WN, BM, BN, PT, CT>(
                             pk, bidx, m0, n0, a0, g0, g1, L, acc);
                else     sk_finish<true, R::IL_A, R::IL_B, TM, TN, WTM, WTN, WN, BM, BN, PT, CT>(
                             pk, bidx, m0, n0, a0, g0, g1, L, acc);
            }
        }
        it += k1 - k0;
        __syncthreads();  // the next segment refills the LDS stages
    }
}

// C = beta * C over a strided batch (alpha == 0 or K == 0), in C's own type.
// beta == 0 writes zeros without reading C.
template <typename CT>
__global__ void __launch_bounds__(256) scale_c_kernel(CT *C, int M, int N, int64_t ldc,
                                                      int64_t strideC, int batch, double beta,
                                                      int beta_i);

}  // namespace mgemm
