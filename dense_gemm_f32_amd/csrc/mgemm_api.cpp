// C-ABI entry points: argument validation, variant selection, launch.
//
// Validation and selection are pure host code (no HIP call), so the
// introspection functions work on machines without a GPU.
#include <atomic>
#include <climits>
#include <mutex>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/mgemm.h"
#include "variants.hpp"

namespace mgemm {
namespace {

struct Table {
    const Variant *v;
    int n;
    int first_id;  // global id of v[0]
};

Table table_for(int dtype)
{
    int n32, n16, nb16, n8, n64;
    const Variant *v32 = f32_variants(&n32);
    const Variant *v16 = f16_variants(&n16);
    const Variant *vb16 = bf16_variants(&nb16);
    const Variant *v8 = i8_variants(&n8);
    const Variant *v64 = f64_variants(&n64);
    switch (dtype) {
    case MGEMM_F32: return {v32, n32, 0};
    case MGEMM_F16: return {v16, n16, n32};
    case MGEMM_BF16: return {vb16, nb16, n32 + n16};
    case MGEMM_I8: return {v8, n8, n32 + n16 + nb16};
    case MGEMM_F64: return {v64, n64, n32 + n16 + nb16 + n8};
    default: return {nullptr, 0, 0};
    }
}

// input types with a variant table: f32, f16, bf16, i8 and f64 (codes 0-3 and 5)
constexpr int N_CODES = MGEMM_F64 + 1;
std::atomic<int> g_forced[N_CODES] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}};

bool is_input_type(int dtype) { return (dtype >= MGEMM_F32 && dtype <= MGEMM_I8) || dtype == MGEMM_F64; }

int total_variants() { return table_for(MGEMM_F64).first_id + table_for(MGEMM_F64).n; }

const Variant *variant_by_id(int id)
{
    for (int d = 0; d < N_CODES; ++d) {
        if (!is_input_type(d)) continue;
        Table t = table_for(d);
        if (id >= t.first_id && id < t.first_id + t.n) return &t.v[id - t.first_id];
    }
    return nullptr;
}

// Builds whose tiles are copied 4 bytes at a time (pipe 4): one path for
// every tile, rows only 4-byte aligned, offsets within 32 bits.
bool dw_copies(const Variant &v) { return v.pipe == 4; }

int elem_size(int dtype)
{
    return dtype == MGEMM_F64 ? 8 : dtype == MGEMM_F32 || dtype == MGEMM_I32 ? 4 : dtype == MGEMM_I8 ? 1 : 2;
}

// alpha or beta usable as an int32 multiplier (int8 inputs): integral and in range
bool int32_scalar(double x) { return x == (double)(int64_t)x && x >= -2147483648.0 && x < 2147483648.0; }

// What a validated call will do.
struct Plan {
    enum Kind { NOTHING, SCALE, GEMM } kind;
    const Variant *var;
    int id;
    KernelArgs args;
    int64_t grid;
};

bool aligned(const void *p, int64_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// Smallest element span one stored matrix occupies: (rows-1)*ld + cols.
int64_t span(int64_t rows, int64_t cols, int64_t ld) { return rows == 0 || cols == 0 ? 0 : (rows - 1) * ld + cols; }

// k_total >= 0: the batch entries are K-chunks of one operand pair of depth
// k_total (split-K's partial products), so strideA/strideB step along K
// inside one matrix and are not required to cover a whole matrix; the last
// chunk is shorter than K.
mgemm_status validate_and_plan(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N,
                               int64_t K, double alpha, const void *A, int64_t lda, int64_t strideA,
                               const void *B, int64_t ldb, int64_t strideB, double beta,
                               const void *C, int64_t ldc, int64_t strideC, int64_t batch,
                               Plan *plan, int64_t k_total = -1, bool need_sk = false)
{
    const bool k_chunks = k_total >= 0;
    if (!is_input_type(dtype)) return MGEMM_INVALID_ARG;
    if (dtype == MGEMM_F64) {
        if (c_dtype != MGEMM_F64) return MGEMM_INVALID_ARG;  // double C only
    } else if (dtype == MGEMM_I8) {
        // int32 C; integral alpha and beta
        if (c_dtype != MGEMM_I32) return MGEMM_INVALID_ARG;
        if (!int32_scalar(alpha) || !int32_scalar(beta)) return MGEMM_INVALID_ARG;
    } else if (c_dtype != MGEMM_F32 && c_dtype != dtype) {
        return MGEMM_INVALID_ARG;  // fp32 C, or the inputs' own 16-bit type
    }
    if ((transA != MGEMM_OP_N && transA != MGEMM_OP_T) || (transB != MGEMM_OP_N && transB != MGEMM_OP_T))
        return MGEMM_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return MGEMM_INVALID_ARG;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX || batch > INT_MAX) return MGEMM_INVALID_ARG;
    const int64_t a_rows = transA ? K : M, a_cols = transA ? M : K;
    const int64_t b_rows = transB ? N : K, b_cols = transB ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return MGEMM_INVALID_ARG;
    if (strideA < 0 || strideB < 0 || strideC < 0) return MGEMM_INVALID_ARG;
    if (batch > 1 && !k_chunks) {
        if (strideA != 0 && strideA < span(a_rows, a_cols, lda)) return MGEMM_INVALID_ARG;
        if (strideB != 0 && strideB < span(b_rows, b_cols, ldb)) return MGEMM_INVALID_ARG;
    }
    if (batch > 1) {
        if (M > 0 && N > 0 && strideC < span(M, N, ldc)) return MGEMM_INVALID_ARG;
    }
    const int es = elem_size(dtype);
    const bool writes_c = M > 0 && N > 0 && batch > 0;
    const bool reads_ab = writes_c && K > 0 && alpha != 0.0;
    const int ces = elem_size(c_dtype);
    if (writes_c && (C == nullptr || !aligned(C, ces))) return MGEMM_INVALID_ARG;
    if (reads_ab && (A == nullptr || B == nullptr || !aligned(A, es) || !aligned(B, es)))
        return MGEMM_INVALID_ARG;

    plan->kind = Plan::NOTHING;
    plan->var = nullptr;
    plan->id = -1;
    plan->grid = 0;
    if (!writes_c) return MGEMM_OK;
    KernelArgs &a = plan->args;
    a.A = A;
    a.B = B;
    a.C = const_cast<void *>(C);
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.strideA = strideA;
    a.strideB = strideB;
    a.strideC = strideC;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.alpha = (float)alpha;  // exact: the fp32/16-bit/int8 entry points take float scalars
    a.beta = (float)beta;
    a.alpha_i = dtype == MGEMM_I8 ? (int)(int64_t)alpha : 0;
    a.beta_i = dtype == MGEMM_I8 ? (int)(int64_t)beta : 0;
    a.alpha_d = alpha;
    a.beta_d = beta;
    a.k_tail = a.K;
    a.tail_batch = -1;
    // a lane stores up to 4 adjacent C elements as one vector
    a.c_vec = aligned(C, 4 * ces) && ldc % 4 == 0 && (batch == 1 || strideC % 4 == 0);
    // Interior tiles address their operands with 32-bit byte offsets from the
    // tile origin: at most 256 rows of the larger leading dimension.
    const int64_t max_ld = lda > ldb ? lda : ldb;
    a.fast_ok = (256 + 1) * max_ld * es < ((int64_t)1 << 31);
    if (!reads_ab) {
        plan->kind = Plan::SCALE;
        return MGEMM_OK;
    }

    // 16-byte global accesses need 16-byte aligned operand rows in every batch entry.
    const int vec = 16 / es;
    const bool vec_ok = aligned(A, 16) && aligned(B, 16) && lda % vec == 0 && ldb % vec == 0 &&
                        strideA % vec == 0 && strideB % vec == 0;

    // Builds with 4-byte copies (pipe 4) address their tiles with 32-bit
    // offsets too, and copy 4-byte pieces: 8/16-bit operands need 4-byte
    // aligned rows and a K (every chunk's, under split-K) that is a multiple
    // of the piece.
    const int64_t piece = es >= 4 ? 1 : 4 / es, k_all = k_chunks ? k_total : K;
    const bool dw_rows = es >= 4 || (aligned(A, 4) && aligned(B, 4) && lda % piece == 0 && ldb % piece == 0 &&
                                     strideA % piece == 0 && strideB % piece == 0 && k_all % piece == 0);
    // One-stage builds (pipe 3) hold a single K-slab and have no register
    // path: K at most their slab, every workgroup's K a multiple of 16 bytes,
    // 32-bit offsets.  Under split-K, K is the chunk length (a multiple of the
    // slab) and the last chunk takes the rest of k_all, so the chunk multiple
    // is checked on k_all: the last chunk's remainder is k_all's.
    // (and a build of this transpose and C type: the 64x64 int8 tiles take
    // A K-contiguous and B K-contiguous only)
    const bool wide_c = c_dtype == MGEMM_F32 || c_dtype == MGEMM_I32 || c_dtype == MGEMM_F64;
    auto sk_launcher = [&](const Variant &v) { return (wide_c ? v.sk : v.sk16)[transA][transB]; };
    auto offsets_ok = [&](const Variant &v) {
        return (wide_c ? v.fn : v.fn16)[transA][transB] != nullptr &&
               (!dw_copies(v) || (a.fast_ok && dw_rows)) &&
               (v.pipe != 3 || (a.fast_ok && K <= v.bk && k_all % (16 / es) == 0)) &&
               // the small-problem kernel: its waves share at most bk of K, and it
               // has no shorter last chunk (split-K) of its own
               (v.pipe != 6 || (K <= v.bk && !k_chunks));
    };
    Table t = table_for(dtype);
    const int forced = g_forced[dtype].load();
    int pick = -1;
    if (forced >= 0) {
        const Variant *v = variant_by_id(forced);
        if (v && (!v->vec || vec_ok) && offsets_ok(*v) && (!need_sk || sk_launcher(*v)))
            pick = forced - t.first_id;
        // a forced variant the operands do not allow falls back to the automatic choice
    }
    auto wgs_of = [&](const Variant &v) {
        return ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn) * batch;
    };
    // need_sk: only builds with a stream-K launch for this transpose
    auto has_sk = [&](const Variant &v) { return !need_sk || sk_launcher(v) != nullptr; };
    auto eligible = [&](const Variant &v) { return v.vec == vec_ok && offsets_ok(v) && has_sk(v); };
    if (pick < 0 && !need_sk && (dtype == MGEMM_F16 || dtype == MGEMM_BF16) && K <= 128) {
        // A shallow K (the whole product is a couple of slabs, e.g. attention
        // scores with a 64-wide head) is bound by the C store rather than the
        // matrix cores: the 256x256 tile with 4x2 wavefronts, whose lanes
        // store four adjacent elements, while it still gives one workgroup
        // per CU.  (Two 128x128 workgroups per CU ran 4% faster on the
        // attention-score batch with an fp32 C from a cool start, but slowed
        // from 82 to 120 us per launch over 50 back-to-back launches, where
        // this tile goes from 86 to 99.)
        for (int i = 0; i < t.n && pick < 0; ++i) {
            const Variant &v = t.v[i];
            if (eligible(v) && v.bm == 256 && v.bn == 256 && v.wm == 4 && wgs_of(v) >= 256) pick = i;
        }
    }
    if (pick < 0) {
        // Builds with a time estimate (Cost in variants.hpp): the lowest one.
        // Builds without 16-byte loads serve aligned operands too.  A build
        // with a DMA path and a register path pays the register factor when
        // its tiles take the latter (K not a multiple of 16 bytes, or offsets
        // past 32 bits; the 4-byte-copy builds have no second path); a grid
        // of one round pays the one-round factor.
        // The small-problem builds (pipe 6) load one element at a time and
        // take any alignment; where no estimated build fits the operands, the
        // unestimated ones below run the register path, and a small build
        // must beat that path's estimate (the 16-byte builds' times with the
        // register factor) rather than nothing.
        double best_us = 0.0, small_us = 0.0, reg_us = -1.0;
        int small = -1;
        for (int i = 0; i < t.n; ++i) {
            const Variant &v = t.v[i];
            if (v.cost.tk <= 0.0f || !has_sk(v)) continue;
            const int64_t rounds = (wgs_of(v) + 255) / 256;
            double us = (double)rounds * (v.cost.t0 + v.cost.tk * (double)K);
            if (rounds == 1) us *= v.cost.solo;
            if (v.pipe == 6) {  // workgroups share CUs: no rounds (Cost in variants.hpp)
                const double chain = v.cost.tk * (double)K;
                const double rate = v.cost.tw * (double)wgs_of(v) * (double)K;
                us = v.cost.t0 + (chain > rate ? chain : rate);
                if (offsets_ok(v) && (small < 0 || us < small_us)) {
                    small = i;
                    small_us = us;
                }
                continue;
            }
            if ((v.vec && !vec_ok) || !offsets_ok(v)) {
                if (!dw_copies(v) && (reg_us < 0.0 || us * v.cost.reg < reg_us)) reg_us = us * v.cost.reg;
                continue;
            }
            // the 16-byte DMA path takes every tile when K is a multiple of 16 bytes
            const bool reg_tiles = !dw_copies(v) && (!a.fast_ok || K % (16 / es) != 0);
            if (reg_tiles) us *= v.cost.reg;
            if (pick < 0 || us < best_us) {
                pick = i;
                best_us = us;
            }
        }
        if (small >= 0 && (pick >= 0 ? small_us < best_us : (reg_us < 0.0 || small_us < reg_us))) pick = small;
    }
    if (pick < 0) {
        // No estimated build fits (unaligned rows, or offsets past 32 bits):
        // the table is in order of preference; take the first variant that
        // still gives at least one workgroup per CU (256 CUs); if none does,
        // the smallest tile, to spread a small problem over more CUs.
        const int64_t min_wgs = 256;
        int best = -1, smallest = -1;
        for (int i = 0; i < t.n; ++i) {
            const Variant &v = t.v[i];
            if (!eligible(v)) continue;
            if (smallest < 0 || v.bm * v.bn < t.v[smallest].bm * t.v[smallest].bn) smallest = i;
            if (best < 0 && wgs_of(v) >= min_wgs) best = i;
        }
        pick = best >= 0 ? best : smallest;
    }
    if (pick < 0) return MGEMM_INVALID_ARG;
    const Variant &v = t.v[pick];
    a.tiles_m = (int)((M + v.bm - 1) / v.bm);
    a.tiles_n = (int)((N + v.bn - 1) / v.bn);
    const int64_t grid = (int64_t)a.tiles_m * a.tiles_n * batch;
    if (grid > INT_MAX) return MGEMM_INVALID_ARG;
    // raster group: tile rows walked together (cache reuse of B columns)
    a.group_m = a.tiles_m < 8 ? a.tiles_m : 8;
    if (a.group_m < 1) a.group_m = 1;
    plan->kind = Plan::GEMM;
    plan->var = &v;
    plan->id = t.first_id + pick;
    plan->grid = grid;
    return MGEMM_OK;
}

// ---------------------------------------------------------------------------
// Split-K.  K is cut into chunks of ks (a multiple of the type's K-slab); the
// partial products of the chunks go to the caller's workspace as a batch
// ([splits][M][N], fp32 / int32 / double), then one reduction kernel forms
// C = alpha * sum of the chunks (ascending) + beta * C.
// ---------------------------------------------------------------------------
int64_t k_granule(int dtype)
{
    return dtype == MGEMM_F32 ? 32 : dtype == MGEMM_I8 ? 128 : dtype == MGEMM_F64 ? 16 : 64;
}

int partial_dtype(int dtype) { return dtype == MGEMM_I8 ? MGEMM_I32 : dtype == MGEMM_F64 ? MGEMM_F64 : MGEMM_F32; }

// chunk length for `splits` requested chunks, and the number of chunks it gives
int64_t k_chunk(int dtype, int64_t K, int64_t splits, int64_t *used)
{
    const int64_t g = k_granule(dtype);
    int64_t ks = (K + splits - 1) / splits;
    ks = (ks + g - 1) / g * g;
    if (ks < g) ks = g;
    *used = (K + ks - 1) / ks;
    return ks;
}

// Automatic split count, for deep-K shapes that leave the device idle: when
// 128x128 tiles give fewer than 256 workgroups and K >= 2 max(M, N), enough
// chunks for one workgroup per CU, each at least 512 deep; otherwise 1.
// (Measured: 512x512x4096 fp32 91 -> 28 us with 8 chunks, 256x256x8192
// 176 -> 24 us with 16; on 1024^3 and 256^3 the extra pass and the
// workspace traffic cost more than the fuller grid gives.)
int64_t auto_splits(int dtype, int64_t M, int64_t N, int64_t K)
{
    (void)dtype;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles >= 256 || tiles == 0 || K < 2 * (M > N ? M : N)) return 1;
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t by_k = K / 512;
    if (s > by_k) s = by_k;
    return s < 1 ? 1 : s;
}

// The partial-product launch: `used` chunks of ks (the last K - (used-1)*ks)
// as a batch over the workspace W = [used][M][N].
mgemm_status plan_chunks(int dtype, int transA, int transB, int64_t M, int64_t N, int64_t K, int64_t ks,
                         int64_t used, const void *A, int64_t lda, const void *B, int64_t ldb,
                         const void *W, Plan *part)
{
    const int64_t sA = transA ? ks * lda : ks;  // chunk z starts at column (or row) z*ks
    const int64_t sB = transB ? ks : ks * ldb;
    mgemm_status st = validate_and_plan(dtype, partial_dtype(dtype), transA, transB, M, N, ks, 1.0, A,
                                        lda, sA, B, ldb, sB, 0.0, W, N, M * N, used, part, K);
    if (st != MGEMM_OK) return st;
    if (part->kind != Plan::GEMM) return MGEMM_INVALID_ARG;
    part->args.k_tail = (int)(K - (used - 1) * ks);
    part->args.tail_batch = (int)(used - 1);
    return MGEMM_OK;
}

// What gemm_splitk does for one call: the plain kernel (chunks == 1), or all
// of C in `chunks` K-chunks of ks (the last chunk takes the rest of K).
struct SplitPlan {
    int64_t chunks, ks;
    int64_t workspace_bytes;
};

// stands in for C or the workspace when only the variant choice is wanted
const void *const kAnyAligned = reinterpret_cast<const void *>((uintptr_t)256);

// Small grids of builds without 16-byte aligned rows: when the plain grid is
// at most one and a half rounds of 256 workgroups (a second round at most
// half full) and its build is one of the 4-byte-copy or range-checked
// register builds, three chunks of all of C spread the last round's tiles
// and put two or three workgroups on every CU to hide each other's loads.
// Applied only where one tile's MFMA work is at least 5 us at the matrix
// peak, so that the two extra launches stay small beside it.  Measured,
// plain -> 3 chunks (fp32 with odd leading dimensions unless noted): 600^2 x
// 999, 100 tiles, 32.0 -> 23.4 us; 1000x1024x999, 256 tiles, 31.3 -> 31.9;
// 1000^2 x 2000, 256 tiles, 54.2 -> 48.1; ragged 1000x1027x999, 272 tiles,
// 44.1 -> 37.4; 1100^3, 324 tiles, 47.4 -> 41.4; the ragged shape in fp64
// 89.7 -> 65.6.  A second round more than half full loses: 1300^2 x 999, 441
// tiles, 43.9 -> 54.3.  The rule leaves alone bf16 ragged (31 -> 34),
// aligned fp32 1024^3 (26 -> 28) and aligned fp64 1024^3 (65 -> 70).
int64_t small_grid_splits(int dtype, int transA, int transB, int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, const void *B, int64_t ldb)
{
    Plan full;
    if (validate_and_plan(dtype, partial_dtype(dtype), transA, transB, M, N, K, 1.0, A, lda, 0, B, ldb,
                          0, 0.0, kAnyAligned, N, 0, 1, &full) != MGEMM_OK ||
        full.kind != Plan::GEMM)
        return 1;
    if (full.grid > 384 || full.var->vec) return 1;
    // matrix peak per CU, flop/s: fp32 157.3 T, fp64 78.6 T, 16-bit 2516.6 T, int8 5000 T over 256 CUs
    const double per_cu = dtype == MGEMM_F32 ? 157.3e12 / 256 : dtype == MGEMM_F64 ? 78.6e12 / 256
                        : dtype == MGEMM_I8 ? 5000e12 / 256 : 2516.6e12 / 256;
    const double tile_s = 2.0 * full.var->bm * full.var->bn * (double)K / per_cu;
    if (tile_s < 5e-6) return 1;
    return K >= 6 * k_granule(dtype) ? 3 : 1;
}

mgemm_status make_split_plan(int dtype, int transA, int transB, int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda, const void *B, int64_t ldb, int64_t splits,
                             SplitPlan *sp)
{
    *sp = SplitPlan{1, K, 0};
    if (splits < 0) return MGEMM_INVALID_ARG;
    if (M == 0 || N == 0 || K == 0) return MGEMM_OK;
    const int64_t wes = elem_size(partial_dtype(dtype));
    if (splits == 0) {
        splits = auto_splits(dtype, M, N, K);
        if (splits <= 1) splits = small_grid_splits(dtype, transA, transB, M, N, K, A, lda, B, ldb);
    }
    if (splits > 1) {
        int64_t used;
        const int64_t ks = k_chunk(dtype, K, splits, &used);
        if (used > 1) *sp = SplitPlan{used, ks, used * M * N * wes};
    }
    return MGEMM_OK;
}

LaunchFn launcher_for(const Plan &p, int c_dtype, int transA, int transB)
{
    const bool wide_c = c_dtype == MGEMM_F32 || c_dtype == MGEMM_I32 || c_dtype == MGEMM_F64;
    return wide_c ? p.var->fn[transA][transB] : p.var->fn16[transA][transB];
}

mgemm_status run_splitk(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N,
                        int64_t K, double alpha, const void *A, int64_t lda, const void *B,
                        int64_t ldb, double beta, void *C, int64_t ldc, int64_t splits,
                        void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    if (splits < 0) return MGEMM_INVALID_ARG;
    Plan full;
    mgemm_status st = validate_and_plan(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, 0, B,
                                        ldb, 0, beta, C, ldc, 0, 1, &full);
    if (st != MGEMM_OK || full.kind == Plan::NOTHING) return st;
    hipError_t err;
    if (full.kind == Plan::SCALE) {
        err = launch_scale_c(c_dtype, C, (int)M, (int)N, ldc, 0, 1, beta, full.args.beta_i, stream);
        return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
    }
    SplitPlan sp;
    st = make_split_plan(dtype, transA, transB, M, N, K, A, lda, B, ldb, splits, &sp);
    if (st != MGEMM_OK) return st;
    if (sp.chunks == 1) {  // one kernel, no workspace
        const LaunchFn fn = launcher_for(full, c_dtype, transA, transB);
        if (fn == nullptr) return MGEMM_INVALID_ARG;
        err = fn(full.args, (unsigned)full.grid, stream);
        return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
    }
    if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < sp.workspace_bytes)
        return MGEMM_INVALID_ARG;
    Plan part;
    st = plan_chunks(dtype, transA, transB, M, N, K, sp.ks, sp.chunks, A, lda, B, ldb, workspace, &part);
    if (st != MGEMM_OK) return st;
    const LaunchFn pfn = part.var->fn[transA][transB];
    if (pfn == nullptr) return MGEMM_INVALID_ARG;
    err = pfn(part.args, (unsigned)part.grid, stream);
    if (err == hipSuccess)
        err = launch_splitk_reduce(c_dtype, workspace, (int)sp.chunks, (int)M, (int)N, C, ldc, alpha, beta,
                                   full.args.alpha_i, full.args.beta_i, stream);
    return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
}

// ---------------------------------------------------------------------------
// Stream-K.  One launch of G workgroups shares the (tile, K-iteration) pairs
// of the whole product evenly (gemm_sk_kernel), so a tile count that leaves
// the last round of CUs part-empty costs no idle round; the last workgroup
// to finish its part of a split tile completes it in the same launch.  The
// caller's workspace holds the arrival counters (MGEMM_STREAMK_COUNTER_BYTES
// at its start, one 32-bit word per workgroup, zero between calls) and then
// the partial tiles ([G][2][bm*bn], fp32; int32 for int8).  The counters
// keep one place in every call, so calls of any size can share a workspace
// without one call's partial tiles landing on another's counters.
// Iterations are the split-K granule of K (whole slabs of every build).
// ---------------------------------------------------------------------------
constexpr int64_t kStreamkWorkgroups = 512;  // default: two per CU
static_assert(MGEMM_STREAMK_MAX_WORKGROUPS * 4 <= MGEMM_STREAMK_COUNTER_BYTES, "one counter per workgroup");

struct StreamPlan {
    Plan plan;  // the stream-K launch (kind GEMM), or SCALE / NOTHING
    int64_t tiles, workspace_bytes;
};

mgemm_status make_streamk_plan(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N,
                               int64_t K, double alpha, const void *A, int64_t lda, const void *B,
                               int64_t ldb, double beta, const void *C, int64_t ldc, int64_t workgroups,
                               void *W, StreamPlan *sp)
{
    sp->tiles = 0;
    sp->workspace_bytes = 0;
    // C of the partial sums' type, or (16-bit inputs) of the inputs' own type
    const bool c16 = (dtype == MGEMM_F16 || dtype == MGEMM_BF16) && c_dtype == dtype;
    if (workgroups < 0 || (c_dtype != partial_dtype(dtype) && !c16)) return MGEMM_INVALID_ARG;
    mgemm_status st = validate_and_plan(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb,
                                        0, beta, C, ldc, 0, 1, &sp->plan, -1, true);
    if (st != MGEMM_OK || sp->plan.kind != Plan::GEMM) return st;
    KernelArgs &a = sp->plan.args;
    const Variant &v = *sp->plan.var;
    const int64_t unit = k_granule(dtype);
    const int64_t iters = (K + unit - 1) / unit;
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    const int64_t total = tiles * iters;
    int64_t g = workgroups > 0 ? workgroups : kStreamkWorkgroups;
    if (g > MGEMM_STREAMK_MAX_WORKGROUPS) g = MGEMM_STREAMK_MAX_WORKGROUPS;
    if (g > total) g = total;  // every workgroup gets at least one iteration
    // the kernels form total * (workgroup + 1) in 64 bits
    if (g > INT_MAX || iters > INT_MAX || total > ((int64_t)1 << 62) / g) return MGEMM_INVALID_ARG;
    a.sk_iters = (int)iters;
    a.sk_unit = (int)unit;
    a.sk_grid = (int)g;
    a.sk_total = total;
    a.sk_count = static_cast<unsigned *>(W);
    a.sk_part = W ? static_cast<char *>(W) + MGEMM_STREAMK_COUNTER_BYTES : nullptr;
    sp->plan.grid = g;
    sp->tiles = tiles;
    sp->workspace_bytes =
        MGEMM_STREAMK_COUNTER_BYTES + g * 2 * (int64_t)v.bm * v.bn * elem_size(partial_dtype(dtype));
    return MGEMM_OK;
}

mgemm_status run_streamk(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N, int64_t K,
                         double alpha, const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                         void *C, int64_t ldc, int64_t workgroups, void *workspace, int64_t workspace_bytes,
                         hipStream_t stream)
{
    StreamPlan sp;
    mgemm_status st = make_streamk_plan(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                                        C, ldc, workgroups, workspace, &sp);
    if (st != MGEMM_OK || sp.plan.kind == Plan::NOTHING) return st;
    hipError_t err;
    if (sp.plan.kind == Plan::SCALE) {
        err = launch_scale_c(c_dtype, C, (int)M, (int)N, ldc, 0, 1, beta, sp.plan.args.beta_i, stream);
        return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
    }
    if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < sp.workspace_bytes)
        return MGEMM_INVALID_ARG;
    const bool wide_c = c_dtype == MGEMM_F32 || c_dtype == MGEMM_I32 || c_dtype == MGEMM_F64;
    const LaunchFn fn = (wide_c ? sp.plan.var->sk : sp.plan.var->sk16)[transA][transB];
    if (fn == nullptr) return MGEMM_INVALID_ARG;
    err = fn(sp.plan.args, (unsigned)sp.plan.grid, stream);
    return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
}

// ---------------------------------------------------------------------------
// Fixed scratch for gemm_splitk_noalloc: split-K's partial products on a GPU
// whose caller cannot allocate.  The array's host-side name is not a device
// address: the device address is looked up once per device, with that device
// current, and only that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this GPU's scratch for work on `stream` (which must
// belong to the current device).
mgemm_status scratch_for(hipStream_t stream, void **out)
{
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
        return MGEMM_HIP_ERROR;
    if (sdev != cur) return MGEMM_INVALID_ARG;
    if (cur < 0 || cur >= kMaxDevices) return MGEMM_HIP_ERROR;
    void *p = g_scratch_ptr[cur].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[cur].load(std::memory_order_acquire);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return MGEMM_HIP_ERROR;
            g_scratch_ptr[cur].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MGEMM_OK;
}

mgemm_status run_splitk_noalloc(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N,
                                int64_t K, double alpha, const void *A, int64_t lda, const void *B,
                                int64_t ldb, double beta, void *C, int64_t ldc, int64_t splits,
                                hipStream_t stream)
{
    // argument errors and the size limit first, before any device call
    Plan full;
    mgemm_status st = validate_and_plan(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, 0, B,
                                        ldb, 0, beta, C, ldc, 0, 1, &full);
    if (st != MGEMM_OK) return st;
    void *ws = nullptr;
    if (full.kind == Plan::GEMM) {
        SplitPlan sp;
        st = make_split_plan(dtype, transA, transB, M, N, K, A, lda, B, ldb, splits, &sp);
        if (st != MGEMM_OK) return st;
        if (sp.workspace_bytes > MGEMM_NOALLOC_SCRATCH_BYTES) return MGEMM_SCRATCH_TOO_SMALL;
        if (sp.chunks > 1) {
            st = scratch_for(stream, &ws);
            if (st != MGEMM_OK) return st;
        }
    }
    return run_splitk(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                      ws, ws ? MGEMM_NOALLOC_SCRATCH_BYTES : 0, stream);
}

void fill_info(const Variant &v, int id, mgemm_variant_info *out)
{
    out->id = id;
    out->dtype = v.dtype;
    out->block_m = v.bm;
    out->block_n = v.bn;
    out->block_k = v.bk;
    out->waves_m = v.wm;
    out->waves_n = v.wn;
    out->threads = v.wm * v.wn * 64;
    // two stages of bk in either path (fp64 rows carry a 2-element pad,
    // gemm_f64.hpp; the DMA path's PIPE 1 has four of bk/2)
    const int pad = v.dtype == MGEMM_F64 ? 2 : 0;
    out->lds_bytes = v.pipe == 6 ? v.wn * 16 * 20 * 4  // small builds: one padded partial tile per wave
                                 : (v.pipe == 3 ? 1 : 2) * (v.bm + v.bn + 2 * pad) * v.bk * elem_size(v.dtype);
    out->pipe = v.pipe;
    std::snprintf(out->name, sizeof(out->name), "%s", v.name);
}

mgemm_status run(int dtype, int c_dtype, int transA, int transB, int64_t M, int64_t N, int64_t K,
                 double alpha, const void *A, int64_t lda, int64_t strideA, const void *B,
                 int64_t ldb, int64_t strideB, double beta, void *C, int64_t ldc, int64_t strideC,
                 int64_t batch, hipStream_t stream)
{
    Plan plan;
    mgemm_status st = validate_and_plan(dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda,
                                        strideA, B, ldb, strideB, beta, C, ldc, strideC, batch, &plan);
    if (st != MGEMM_OK || plan.kind == Plan::NOTHING) return st;
    hipError_t err;
    if (plan.kind == Plan::SCALE) {
        err = launch_scale_c(c_dtype, C, (int)M, (int)N, ldc, strideC, (int)batch, beta,
                             plan.args.beta_i, stream);
    } else {
        const bool wide_c = c_dtype == MGEMM_F32 || c_dtype == MGEMM_I32 || c_dtype == MGEMM_F64;
        const LaunchFn fn = wide_c ? plan.var->fn[transA][transB] : plan.var->fn16[transA][transB];
        if (fn == nullptr) return MGEMM_INVALID_ARG;
        err = fn(plan.args, (unsigned)plan.grid, stream);
    }
    return err == hipSuccess ? MGEMM_OK : MGEMM_HIP_ERROR;
}

}  // namespace
}  // namespace mgemm

using namespace mgemm;

extern "C" {

mgemm_status gemm_f32(mgemm_op transA, mgemm_op transB, int64_t M, int64_t N, int64_t K,
                      float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                      float beta, float *C, int64_t ldc, hipStream_t stream)
{
    return run(MGEMM_F32, MGEMM_F32, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C,
               ldc, 0, 1, stream);
}

mgemm_status gemm_f16(mgemm_op transA, mgemm_op transB, int64_t M, int64_t N, int64_t K,
                      float alpha, const mgemm_f16 *A, int64_t lda, const mgemm_f16 *B,
                      int64_t ldb, float beta, float *C, int64_t ldc, hipStream_t stream)
{
    return run(MGEMM_F16, MGEMM_F32, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C,
               ldc, 0, 1, stream);
}

mgemm_status gemm_bf16(mgemm_op transA, mgemm_op transB, int64_t M, int64_t N, int64_t K,
                       float alpha, const mgemm_bf16 *A, int64_t lda, const mgemm_bf16 *B,
                       int64_t ldb, float beta, float *C, int64_t ldc, hipStream_t stream)
{
    return run(MGEMM_BF16, MGEMM_F32, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C,
               ldc, 0, 1, stream);
}

mgemm_status gemm_strided_batched(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB,
                                  int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                  int64_t lda, int64_t strideA, const void *B, int64_t ldb,
                                  int64_t strideB, float beta, float *C, int64_t ldc,
                                  int64_t strideC, int64_t batch, hipStream_t stream)
{
    if (in_dtype == MGEMM_F64) return MGEMM_INVALID_ARG;  // fp64 has its own entry points
    return run(in_dtype, MGEMM_F32, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
               beta, C, ldc, strideC, batch, stream);
}

mgemm_status gemm_strided_batched_ex(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                                     mgemm_op transB, int64_t M, int64_t N, int64_t K, float alpha,
                                     const void *A, int64_t lda, int64_t strideA, const void *B,
                                     int64_t ldb, int64_t strideB, float beta, void *C, int64_t ldc,
                                     int64_t strideC, int64_t batch, hipStream_t stream)
{
    if (in_dtype == MGEMM_F64) return MGEMM_INVALID_ARG;  // fp64 has its own entry points
    return run(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
               beta, C, ldc, strideC, batch, stream);
}

mgemm_status gemm_f64(mgemm_op transA, mgemm_op transB, int64_t M, int64_t N, int64_t K,
                      double alpha, const double *A, int64_t lda, const double *B, int64_t ldb,
                      double beta, double *C, int64_t ldc, hipStream_t stream)
{
    return run(MGEMM_F64, MGEMM_F64, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C,
               ldc, 0, 1, stream);
}

mgemm_status gemm_f64_strided_batched(mgemm_op transA, mgemm_op transB, int64_t M, int64_t N,
                                      int64_t K, double alpha, const double *A, int64_t lda,
                                      int64_t strideA, const double *B, int64_t ldb,
                                      int64_t strideB, double beta, double *C, int64_t ldc,
                                      int64_t strideC, int64_t batch, hipStream_t stream)
{
    return run(MGEMM_F64, MGEMM_F64, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
               strideB, beta, C, ldc, strideC, batch, stream);
}

mgemm_status gemm_splitk(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                         mgemm_op transB, int64_t M, int64_t N, int64_t K, double alpha,
                         const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                         void *C, int64_t ldc, int64_t splits, void *workspace,
                         int64_t workspace_bytes, hipStream_t stream)
{
    // 32-bit, 16-bit and int8 paths take float scalars: refuse what a float cannot hold
    if (in_dtype != MGEMM_F64 && ((double)(float)alpha != alpha || (double)(float)beta != beta))
        return MGEMM_INVALID_ARG;
    return run_splitk(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                      splits, workspace, workspace_bytes, stream);
}

mgemm_status gemm_splitk_noalloc(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                                 mgemm_op transB, int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                                 void *C, int64_t ldc, int64_t splits, hipStream_t stream)
{
    if (in_dtype != MGEMM_F64 && ((double)(float)alpha != alpha || (double)(float)beta != beta))
        return MGEMM_INVALID_ARG;
    return run_splitk_noalloc(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                              ldc, splits, stream);
}

mgemm_status mgemm_splitk_plan(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB, int64_t M,
                               int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                               int64_t ldb, int64_t splits, mgemm_splitk_plan_info *out)
{
    if (!out) return MGEMM_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    out->variant.id = -1;
    SplitPlan sp;
    mgemm_status st = make_split_plan(in_dtype, transA, transB, M, N, K, A, lda, B, ldb, splits, &sp);
    if (st != MGEMM_OK) return st;
    out->workspace_bytes = sp.workspace_bytes;
    out->chunks = sp.chunks;
    out->chunk_len = sp.ks;
    if (M == 0 || N == 0 || K == 0) return MGEMM_OK;
    Plan p;
    if (sp.chunks > 1)
        st = plan_chunks(in_dtype, transA, transB, M, N, K, sp.ks, sp.chunks, A, lda, B, ldb, kAnyAligned, &p);
    else
        st = validate_and_plan(in_dtype, partial_dtype(in_dtype), transA, transB, M, N, K, 1.0, A, lda, 0, B,
                               ldb, 0, 0.0, kAnyAligned, N, 0, 1, &p);
    if (st != MGEMM_OK) return st;
    if (p.kind == Plan::GEMM) {
        fill_info(*p.var, p.id, &out->variant);
        out->grid = p.grid;
    }
    return MGEMM_OK;
}

mgemm_status gemm_streamk(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                          mgemm_op transB, int64_t M, int64_t N, int64_t K, double alpha,
                          const void *A, int64_t lda, const void *B, int64_t ldb, double beta,
                          void *C, int64_t ldc, int64_t workgroups, void *workspace,
                          int64_t workspace_bytes, hipStream_t stream)
{
    if (in_dtype != MGEMM_F64 && ((double)(float)alpha != alpha || (double)(float)beta != beta))
        return MGEMM_INVALID_ARG;
    return run_streamk(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                       workgroups, workspace, workspace_bytes, stream);
}

mgemm_status mgemm_streamk_plan(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB, int64_t M,
                                int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                                int64_t ldb, int64_t workgroups, mgemm_streamk_plan_info *out)
{
    if (!out) return MGEMM_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    out->variant.id = -1;
    StreamPlan sp;
    const mgemm_status st = make_streamk_plan(in_dtype, partial_dtype(in_dtype), transA, transB, M, N, K, 1.0,
                                              A, lda, B, ldb, 0.0, kAnyAligned, N, workgroups, nullptr, &sp);
    if (st != MGEMM_OK) return st;
    if (sp.plan.kind == Plan::GEMM) {
        fill_info(*sp.plan.var, sp.plan.id, &out->variant);
        out->workspace_bytes = sp.workspace_bytes;
        out->workgroups = sp.plan.grid;
        out->tiles = sp.tiles;
        out->iterations = sp.plan.args.sk_iters;
        out->k_per_iteration = sp.plan.args.sk_unit;
    }
    return MGEMM_OK;
}

const char *mgemm_status_string(mgemm_status s)
{
    switch (s) {
    case MGEMM_OK: return "MGEMM_OK";
    case MGEMM_INVALID_ARG: return "MGEMM_INVALID_ARG: an argument failed validation; nothing was launched";
    case MGEMM_HIP_ERROR: return "MGEMM_HIP_ERROR: the HIP runtime refused the kernel launch";
    case MGEMM_SCRATCH_TOO_SMALL:
        return "MGEMM_SCRATCH_TOO_SMALL: the split-K partial sums need more than the fixed "
               "scratch of gemm_splitk_noalloc (MGEMM_NOALLOC_SCRATCH_BYTES); nothing was launched";
    default: return "unknown mgemm_status";
    }
}

int mgemm_num_variants(void) { return total_variants(); }

int mgemm_build_flags(void)
{
#ifdef MGEMM_DEBUG_POISON
    return MGEMM_BUILD_LDS_POISON;
#else
    return 0;
#endif
}

mgemm_status mgemm_variant(int id, mgemm_variant_info *out)
{
    const Variant *v = variant_by_id(id);
    if (!v || !out) return MGEMM_INVALID_ARG;
    fill_info(*v, id, out);
    return MGEMM_OK;
}

mgemm_status mgemm_select(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB, int64_t M,
                          int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
                          int64_t strideA, const void *B, int64_t ldb, int64_t strideB,
                          float beta, const float *C, int64_t ldc, int64_t strideC,
                          int64_t batch, mgemm_variant_info *out, int64_t *grid)
{
    // C as fp32 (int32 for int8, double for fp64 inputs)
    const mgemm_dtype c_dtype = in_dtype == MGEMM_I8    ? MGEMM_I32
                                : in_dtype == MGEMM_F64 ? MGEMM_F64
                                                        : MGEMM_F32;
    return mgemm_select_ex(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                           strideB, beta, C, ldc, strideC, batch, out, grid);
}

mgemm_status mgemm_select_ex(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                             mgemm_op transB, int64_t M, int64_t N, int64_t K, double alpha,
                             const void *A, int64_t lda, int64_t strideA, const void *B,
                             int64_t ldb, int64_t strideB, double beta, const void *C,
                             int64_t ldc, int64_t strideC, int64_t batch, mgemm_variant_info *out,
                             int64_t *grid)
{
    Plan plan;
    mgemm_status st = validate_and_plan(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda,
                                        strideA, B, ldb, strideB, beta, C, ldc, strideC, batch, &plan);
    if (st != MGEMM_OK) return st;
    if (out) {
        if (plan.kind == Plan::GEMM) {
            fill_info(*plan.var, plan.id, out);
        } else {
            std::memset(out, 0, sizeof(*out));
            out->id = -1;
            std::snprintf(out->name, sizeof(out->name), "%s",
                          plan.kind == Plan::SCALE ? "mgemm_scale_c" : "none");
        }
    }
    if (grid) *grid = plan.kind == Plan::GEMM ? plan.grid : 0;
    return MGEMM_OK;
}

mgemm_status mgemm_force_variant(mgemm_dtype dtype, int id)
{
    if (!is_input_type(dtype)) return MGEMM_INVALID_ARG;
    if (id >= 0) {
        const Variant *v = variant_by_id(id);
        if (!v || v->dtype != dtype) return MGEMM_INVALID_ARG;
    } else {
        id = -1;
    }
    g_forced[dtype].store(id);
    return MGEMM_OK;
}

}  // extern "C"
