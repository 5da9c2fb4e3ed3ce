"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact on integer-valued inputs whose partial sums stay below 2^24
(2^53 for fp64 inputs; the result is then unique) and for int8; otherwise
max|err| <= c*sqrt(K)*max|ref|, with c = 1e-5 for fp32 inputs, 2e-3 for
f16/bf16 inputs and 1e-5 * 2^-29 for fp64 inputs.
Small problems are compared element by element over the whole output; the
full-size workloads, in the launch configuration the benchmark times, on
sampled elements (whole boundary rows/columns plus random positions).
"""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

from dense_gemm_f32_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dense_gemm_f32_amd as mg
    import oracle
    from parity import Run, check_exact, check_tolerance, expected_exact, log, sample_positions


@pytest.fixture(autouse=True)
def _auto_variant():
    yield
    for dt in ("f32", "f16", "bf16", "i8", "f64"):
        mg.force_variant(dt, None)


def full_check(p, exact=False, c_fill=None, what=""):
    log(f"[{what}] {p.dtype}->{p.c_dtype} tA={int(p.transA)} tB={int(p.transB)} M={p.M} N={p.N} "
        f"K={p.K} batch={p.batch} lda={p.lda} ldb={p.ldb} ldc={p.ldc} alpha={p.alpha} "
        f"beta={p.beta} dist={p.dist} seed={p.seed}")
    r = Run(p, c_fill=c_fill)
    r.launch()
    got = r.result()
    ref = r.oracle_full()
    if exact:
        check_exact(got, expected_exact(p, ref), what)
    else:
        check_tolerance(got, ref, p, what)
    return got


def sampled_check(p, exact=False, what="", n_random=20000):
    log(f"[{what}] {p.dtype}->{p.c_dtype} tA={int(p.transA)} tB={int(p.transB)} M={p.M} N={p.N} "
        f"K={p.K} batch={p.batch} alpha={p.alpha} beta={p.beta} dist={p.dist} seed={p.seed} "
        f"(sampled)")
    info, grid = mg.select(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                           16, p.lda, p.strideA, 16, p.ldb, p.strideB, p.beta, 16, p.ldc,
                           p.strideC, p.batch)
    log(f"  variant {info['name']} grid {grid}")
    r = Run(p)
    r.launch()
    got = r.result()
    b, i, j = sample_positions(p, n_random=n_random)
    ref = r.oracle_elems(b, i, j)
    vals = got[b, i, j]
    if exact:
        check_exact(vals, expected_exact(p, ref), what)
    else:
        check_tolerance(vals, ref, p, what)
    assert not np.isnan(got).any()


def _round8(x):
    return (x + 7) // 8 * 8


ES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "f64": 8}


def _narrow_dw(v, dtype):
    """An 8/16-bit build with 4-byte copies: rows 4-byte aligned, K a multiple of the piece."""
    return v["pipe"] == 4 and ES[dtype] < 4


def _ld_unaligned(v, dtype, cols):
    """A leading dimension with no 16-byte rows that the unaligned build v accepts: odd,
    or (8/16-bit 4-byte-copy builds) a multiple of the 4-byte piece."""
    if _narrow_dw(v, dtype):
        piece = 4 // ES[dtype]
        ld = -(-cols // piece) * piece
        return ld + piece if (ld * ES[dtype]) % 16 == 0 else ld
    return cols + 1


def transposes_of(v, dtype):
    """(transA, transB) pairs build v has launchers for: all four, except the 64x64 int8
    tiles (A and B K-contiguous only)."""
    if dtype == "i8" and v["block_m"] < 128:
        return [(False, True)]
    return list(itertools.product((False, True), repeat=2))


def _assert_selected(p, v):
    # a forced aligned-only variant falls back to the automatic choice on unaligned
    # operands: make sure the case really runs the variant it is meant to cover
    info, _ = mg.select(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                        16, p.lda, p.strideA, 16, p.ldb, p.strideB, p.beta, 16, p.ldc,
                        p.strideC, p.batch)
    assert info["name"] == v["name"], (info["name"], v["name"])


def variants_of(dtype, one_stage=False, small=False):
    """The dtype's tile builds; the one-stage ones (pipe 3, K of one slab only) or the
    small-problem ones (pipe 6, K at most their block_k) when asked."""
    code = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "f64": 5}[dtype]
    if not torch.cuda.is_available():
        return []
    return [v for v in mg.variants() if v["dtype"] == code and (v["pipe"] == 3) == one_stage
            and (v["pipe"] == 6) == small]


# ------------------------------------------------------------------ every variant, every op

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_variant_every_transpose_ragged(dtype):
    for v in variants_of(dtype):
        if _narrow_dw(v, dtype):
            continue    # needs an even K: test_four_byte_copy_variants covers it
        mg.force_variant(dtype, v["id"])
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        M, N, K = 2 * bm + 17, 2 * bn + 9, 3 * bk + 5
        aligned = not v["name"].endswith("_u")
        for tA, tB in itertools.product((False, True), repeat=2):
            a_cols = M if tA else K
            b_cols = K if tB else N
            # the aligned builds need 16-byte rows; the others get the tight, odd ones
            base = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, alpha=1.5, beta=0.5,
                              lda=_round8(a_cols) if aligned else a_cols,
                              ldb=_round8(b_cols) if aligned else b_cols,
                              dist="uniform" if dtype == "f32" else "normal",
                              c_dist="uniform", pad_value=float("nan"), seed=11)
            _assert_selected(base, v)
            full_check(base, what=f"{v['name']} float")
            full_check(wl.int_shadow(base, -8, 8), exact=True, what=f"{v['name']} int")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dma_path_every_variant_every_transpose(dtype):
    # K a multiple of every slab depth: interior tiles take the unchecked LDS-DMA
    # copies, the ragged last tile row/column the range-checked ones; leading
    # dimensions padded by 8 elements (16-byte rows stay aligned) with NaN in the
    # padding.
    for v in variants_of(dtype):
        if v["name"].endswith("_u"):
            continue
        mg.force_variant(dtype, v["id"])
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        M, N, K = 2 * bm + 17, 2 * bn + 9, 4 * bk
        for tA, tB in itertools.product((False, True), repeat=2):
            a_cols = M if tA else K
            b_cols = K if tB else N
            base = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=_round8(a_cols) + 8,
                              ldb=_round8(b_cols) + 8, ldc=N + 4, alpha=1.5, beta=0.5,
                              dist="uniform" if dtype == "f32" else "normal", c_dist="uniform",
                              pad_value=float("nan"), seed=31)
            _assert_selected(base, v)
            full_check(base, what=f"{v['name']} DMA float")
            full_check(wl.int_shadow(base, -8, 8), exact=True, what=f"{v['name']} DMA int")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dma_path_short_k(dtype):
    # one to four LDS slabs: the prologue and the drain of every schedule,
    # with interior tiles (M, N multiples of the tile) and a ragged edge
    for v in variants_of(dtype):
        if v["name"].endswith("_u"):
            continue
        mg.force_variant(dtype, v["id"])
        half = v["block_k"] // 2
        for nslab in (1, 2, 3, 4, 5):
            K = nslab * half
            base = wl.Problem(dtype, v["block_m"] + 40, 2 * v["block_n"], K, transB=nslab % 2 == 1,
                              dist="int", int_lo=-8, int_hi=8, alpha=1.0, beta=-1.0,
                              c_dist="int", seed=40 + nslab)
            _assert_selected(base, v)
            full_check(base, exact=True, what=f"{v['name']} K={K}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_dma_path_k_tails(dtype):
    # K a multiple of the 16-byte chunk but not of the slab: interior tiles
    # stay on the LDS-DMA path and copy one more slab whose chunks past K are
    # masked to zero.  NaN fills the row padding past K, so a chunk read
    # past K would show; a K shorter than one slab, and a tail after several.
    es = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}[dtype]
    ch = 16 // es
    for v in variants_of(dtype):
        if v["name"].endswith("_u"):
            continue
        mg.force_variant(dtype, v["id"])
        bm, bn = v["block_m"], v["block_n"]
        slab = v["block_k"] // 2 if v["pipe"] == 1 else v["block_k"]
        combos = transposes_of(v, dtype)
        M, N = 2 * bm + 17, 2 * bn + 9
        pad = 16 if dtype == "i8" else 8
        padded = lambda cols: -(-cols // pad) * pad + pad   # 16-byte rows, padding after
        for K in (ch, 3 * slab + slab - ch, slab + slab // 2 + ch):
            for tA, tB in combos:
                kw = dict(c_dtype="i32", int_lo=-100, int_hi=100, pad_value=77) if dtype == "i8" else \
                    dict(int_lo=-8, int_hi=8, pad_value=float("nan"))
                p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=padded(M if tA else K),
                               ldb=padded(K if tB else N), alpha=1.0, beta=-1.0, dist="int",
                               c_dist="int", seed=90 + K % 7, **kw)
                _assert_selected(p, v)
                full_check(p, exact=True, what=f"{v['name']} K={K} tA={tA} tB={tB}")
        if dtype in ("f32", "bf16"):
            K = 2 * slab + ch
            p = wl.Problem(dtype, M, N, K, alpha=1.5, beta=0.5, lda=padded(K), ldb=padded(N),
                           dist="uniform" if dtype == "f32" else "normal", c_dist="uniform",
                           pad_value=float("nan"), seed=97)
            _assert_selected(p, v)
            full_check(p, what=f"{v['name']} float K tail")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_four_byte_copy_variants(dtype):
    # builds whose every tile copies 4-byte pieces into LDS (1 fp32, 2 16-bit
    # or 4 int8 elements), with out-of-matrix lanes masked to zero: leading
    # dimensions with no 16-byte rows and filler in the padding, K tails of
    # every length mod the slab (whole pieces), slab counts through the steady
    # state, every transpose, a batch with a shared operand
    es = ES[dtype]
    piece = 4 // es
    up = lambda x: -(-x // piece) * piece
    i8 = dtype == "i8"
    for v in variants_of(dtype):
        if v["pipe"] != 4:
            continue
        mg.force_variant(dtype, v["id"])
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        for i, K in enumerate((1, bk - 1, bk, bk + 1, 3 * bk + 17, 9 * bk + 5)):
            K = up(K)
            tA, tB = (False, True) if i8 else (bool(i & 1), bool(i & 2))
            M, N = bm + 3 + i, 2 * bn - 7
            kw = dict(c_dtype="i32", alpha=2.0, beta=-1.0, int_lo=-100, int_hi=100, pad_value=77) if i8 \
                else dict(alpha=1.5, beta=0.5, int_lo=-20, int_hi=20, pad_value=float("nan"))
            p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB,
                           lda=_ld_unaligned(v, dtype, M if tA else K),
                           ldb=_ld_unaligned(v, dtype, K if tB else N), ldc=N + 1,
                           dist="int", c_dist="int", seed=70 + i, **kw)
            _assert_selected(p, v)
            full_check(p, exact=True, what=f"{v['name']} K={K} tA={int(tA)} tB={int(tB)}")
        K = up(2 * bk + 3)
        q = wl.Problem(dtype, bm + 5, bn + 9, K, transB=True, batch=3, strideB=0,
                       lda=_ld_unaligned(v, dtype, K), ldb=_ld_unaligned(v, dtype, K + 1),
                       dist="int" if i8 else "uniform", int_lo=-100, int_hi=100,
                       c_dtype="i32" if i8 else "f32", seed=77)
        q.force_batched = True
        _assert_selected(q, v)
        full_check(q, exact=i8, what=f"{v['name']} batched, B shared")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dma_path_batched_and_broadcast(dtype):
    # interior tiles in several batch entries, B shared by all entries (stride 0)
    v = variants_of(dtype)[0]
    mg.force_variant(dtype, v["id"])
    K = 2 * v["block_k"]
    p = wl.Problem(dtype, v["block_m"], v["block_n"], K, batch=3, strideB=0, transB=True,
                   dist="int", int_lo=-8, int_hi=8, seed=32)
    _assert_selected(p, v)
    full_check(p, exact=True, what=f"{v['name']} DMA batched, strideB=0")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_unaligned_leading_dims_and_nan_padding(dtype):
    # odd leading dimensions (no 16-byte rows) and NaN in every padding element
    for tA, tB in itertools.product((False, True), repeat=2):
        M, N, K = 77, 91, 83
        a_cols = M if tA else K
        b_cols = K if tB else N
        p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=a_cols + 3, ldb=b_cols + 5,
                       ldc=N + 7, dist="int", int_lo=-9, int_hi=9, pad_value=float("nan"),
                       seed=12)
        full_check(p, exact=True, c_fill=float("nan"), what="odd ld, NaN padding")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_aligned_padded_leading_dims(dtype):
    vec = 4 if dtype == "f32" else 8
    for tA, tB in itertools.product((False, True), repeat=2):
        M, N, K = 300, 260, 140
        a_cols = M if tA else K
        b_cols = K if tB else N
        p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=a_cols + vec, ldb=b_cols + 2 * vec,
                       ldc=N + 4, alpha=-1.0, beta=2.0, dist="int", int_lo=-9, int_hi=9,
                       pad_value=float("nan"), seed=13)
        full_check(p, exact=True, what="aligned padded ld")


# ------------------------------------------------------------------ the named workloads

def test_sgemm_256():
    p = wl.sgemm_256()
    full_check(p, c_fill=float("nan"), what="sgemm 256^3, beta=0 with NaN C")
    full_check(wl.int_shadow(p, -50, 50), exact=True, what="sgemm 256^3 int shadow")


def test_sgemm_ragged_bit_exact():
    full_check(wl.sgemm_ragged(), exact=True, c_fill=float("nan"), what="sgemm 1000x1027x999 ints")


def test_sgemm_4096():
    p = wl.sgemm_4096()
    sampled_check(p, what="sgemm 4096^3 alpha=1.5 beta=0.5")
    sampled_check(wl.int_shadow(p, -7, 7), exact=True, what="sgemm 4096^3 int shadow")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gemm16_8192(dtype):
    p = wl.gemm16_8192(dtype)
    sampled_check(p, what=f"{dtype} 8192^3")
    sampled_check(wl.int_shadow(p, -8, 8), exact=True, what=f"{dtype} 8192^3 int shadow")


def test_qkt_batched():
    p = wl.qkt_batched()
    sampled_check(p, what="QK^T 128 x 1024x1024x64 fp16")
    sampled_check(wl.int_shadow(p, -8, 8), exact=True, what="QK^T int shadow")


def test_qkt_batched_f16_out():
    p = wl.qkt_batched_f16_out()
    sampled_check(p, what="QK^T 128 x 1024x1024x64 fp16 -> fp16 C")
    sampled_check(wl.int_shadow(p, -8, 8), exact=True, what="QK^T -> fp16 C, int shadow")


# ------------------------------------------------------------------ 16-bit C output

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_c16_every_variant_every_transpose(dtype):
    # C in the inputs' 16-bit type: interior (LDS-DMA) and edge tiles; integer
    # inputs accumulate exactly in fp32, so the stored value is that exact sum
    # rounded to nearest-even, bit for bit (most sums are not representable)
    for v in variants_of(dtype):
        mg.force_variant(dtype, v["id"])
        aligned = not v["name"].endswith("_u")
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        M, N, K = 2 * bm + 17, 2 * bn + 9, 4 * bk
        for tA, tB in itertools.product((False, True), repeat=2):
            a_cols = M if tA else K
            b_cols = K if tB else N
            base = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, c_dtype=dtype,
                              lda=_round8(a_cols) if aligned else _ld_unaligned(v, dtype, a_cols),
                              ldb=_round8(b_cols) if aligned else _ld_unaligned(v, dtype, b_cols),
                              alpha=1.5, beta=0.5, dist="normal", c_dist="uniform", seed=51)
            _assert_selected(base, v)
            full_check(base, what=f"{v['name']} -> {dtype} C, float")
            full_check(wl.int_shadow(base, -20, 20), exact=True, what=f"{v['name']} -> {dtype} C, int")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_c16_odd_ldc_padding_untouched(dtype):
    # ldc not a multiple of 4: element stores; the padding keeps its NaNs
    for tA, tB in itertools.product((False, True), repeat=2):
        p = wl.Problem(dtype, 300, 277, 192, transA=tA, transB=tB, c_dtype=dtype, ldc=277 + 3,
                       dist="int", int_lo=-20, int_hi=20, pad_value=float("nan"), seed=52)
        full_check(p, exact=True, c_fill=float("nan"), what=f"-> {dtype} C, ldc odd")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_c16_quick_returns_scale_c(dtype):
    for alpha, K in ((0.0, 64), (1.0, 0)):
        p = wl.Problem(dtype, 70, 90, K, alpha=alpha, beta=-1.25, c_dtype=dtype, dist="int",
                       int_lo=-30, int_hi=30, c_dist="uniform", seed=53)
        full_check(p, exact=True, what=f"-> {dtype} C, alpha={alpha} K={K}")
    p = wl.Problem(dtype, 70, 90, 0, beta=0.0, c_dtype=dtype, seed=54)
    got = full_check(p, exact=True, c_fill=float("nan"), what=f"-> {dtype} C, beta=0 K=0")
    assert not np.isnan(got).any()


# ------------------------------------------------------------------ int8 inputs, int32 C

def test_i8_every_variant():
    # every transpose each build has (an MN-contiguous operand through transposing LDS
    # reads); interior (LDS-DMA) and edge tiles, aligned and odd leading dimensions,
    # integral alpha and beta, exact
    for v in variants_of("i8"):
        mg.force_variant("i8", v["id"])
        aligned = not v["name"].endswith("_u")
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        ld = lambda cols: -(-cols // 16) * 16 + 16 if aligned else _ld_unaligned(v, "i8", cols)
        for n, (tA, tB) in enumerate(transposes_of(v, "i8")):
            for (M, N, K) in ((2 * bm + 17, 2 * bn + 9, 4 * bk), (bm + 3, bn + 40, 3 * bk + 29)):
                if _narrow_dw(v, "i8"):
                    K -= K % 4      # 4-byte pieces of k
                for alpha, beta in ((1.0, 0.0), (-3.0, 2.0)):
                    p = wl.Problem("i8", M, N, K, transA=tA, transB=tB, c_dtype="i32", alpha=alpha,
                                   beta=beta, lda=ld(M if tA else K), ldb=ld(K if tB else N),
                                   dist="int", int_lo=-128, int_hi=127, c_dist="int", seed=71 + n,
                                   pad_value=77)
                    _assert_selected(p, v)
                    full_check(p, exact=True, what=f"{v['name']} i8 tA={int(tA)} tB={int(tB)} "
                                                   f"alpha={alpha} beta={beta}")


def test_i8_wraps_like_int32():
    # alpha * acc overflows int32: the stored value is the exact one modulo 2^32
    p = wl.Problem("i8", 300, 260, 256, transB=True, c_dtype="i32", alpha=float(1 << 20),
                   beta=-(1 << 30), dist="int", int_lo=-128, int_hi=127, c_dist="int", seed=72)
    full_check(p, exact=True, what="i8 int32 wrap-around")
    ref = Run(p).oracle_full()
    assert np.abs(ref).max() > 2 ** 31          # the case really overflows


def test_i8_quick_returns_and_empty():
    for alpha, K in ((0.0, 128), (1.0, 0)):
        p = wl.Problem("i8", 70, 90, K, transB=True, c_dtype="i32", alpha=alpha, beta=-5.0,
                       dist="int", int_lo=-100, int_hi=100, c_dist="int", seed=73)
        full_check(p, exact=True, what=f"i8 alpha={alpha} K={K}")


def test_gemm_i8_8192():
    sampled_check(wl.gemm_i8_8192(), exact=True, what="int8 8192^3 -> int32")


# ------------------------------------------------------------------ fp64 inputs

def test_f64_every_variant_every_transpose():
    # integer-valued doubles (every partial sum exact): bit-exact, with several
    # tiles plus a ragged tail, padded (NaN) or odd leading dimensions
    for v in variants_of("f64"):
        mg.force_variant("f64", v["id"])
        aligned = not v["name"].endswith("_u")
        bm, bn = v["block_m"], v["block_n"]
        for tA, tB in itertools.product((False, True), repeat=2):
            M, N, K = 2 * bm + 19, bn + 37, 3 * 16 + 7
            a_cols = M if tA else K
            b_cols = K if tB else N
            p = wl.Problem("f64", M, N, K, transA=tA, transB=tB, alpha=-1.5, beta=0.25,
                           lda=_round8(a_cols) if aligned else a_cols + 1,
                           ldb=_round8(b_cols) if aligned else b_cols + 3,
                           ldc=N + 5, dist="int", int_lo=-1000, int_hi=1000, c_dist="int",
                           seed=81, pad_value=float("nan"))
            _assert_selected(p, v)
            full_check(p, exact=True, what=f"{v['name']} f64 tA={int(tA)} tB={int(tB)}")


def test_f64_float_inputs_within_tolerance():
    for v in variants_of("f64"):
        mg.force_variant("f64", v["id"])
        aligned = not v["name"].endswith("_u")
        for tA, tB in ((False, False), (True, True)):
            M, N, K = 300, 221, 515
            a_cols, b_cols = (M if tA else K), (K if tB else N)
            p = wl.Problem("f64", M, N, K, transA=tA, transB=tB, alpha=1.5, beta=0.5,
                           lda=_round8(a_cols) if aligned else a_cols + 1,
                           ldb=_round8(b_cols) if aligned else b_cols + 1,
                           dist="uniform", seed=82)
            _assert_selected(p, v)
            full_check(p, what=f"{v['name']} f64 uniform tA={int(tA)} tB={int(tB)}")


def test_f64_batched_and_broadcast():
    p = wl.Problem("f64", 130, 70, 90, transB=True, batch=5, alpha=2.0, beta=-1.0,
                   dist="int", int_lo=-500, int_hi=500, c_dist="int", seed=83)
    full_check(p, exact=True, what="f64 batched")
    q = dataclasses.replace(p, strideA=0, seed=84)
    q.force_batched = True
    full_check(q, exact=True, what="f64 batched, A shared (stride 0)")


def test_f64_quick_returns_and_nan_c():
    for alpha, K in ((0.0, 64), (1.0, 0)):
        p = wl.Problem("f64", 70, 90, K, alpha=alpha, beta=-0.75, dist="uniform", seed=85)
        full_check(p, exact=True, what=f"f64 alpha={alpha} K={K}")
    # beta == 0: C is never read, so NaN in C does not leak
    p = wl.Problem("f64", 100, 80, 40, dist="int", int_lo=-9, int_hi=9, seed=86)
    full_check(p, exact=True, c_fill=float("nan"), what="f64 beta=0 over NaN C")


def test_dgemm_4096():
    sampled_check(wl.dgemm_4096(), what="DGEMM 4096^3 alpha=1.5 beta=0.5")


def test_dgemm_4096_integer_shadow():
    sampled_check(wl.int_shadow(wl.dgemm_4096(), -1000, 1000), exact=True,
                  what="DGEMM 4096^3 integer shadow")


# ------------------------------------------------------------------ split-K

SPLITK_TYPES = [("f32", "f32", 1000), ("f16", "f32", 8), ("bf16", "bf16", 8), ("i8", "i32", 127),
                ("f64", "f64", 1000)]


@pytest.mark.parametrize("dtype,c_dtype,hi", SPLITK_TYPES)
def test_splitk_every_type_and_transpose_exact(dtype, c_dtype, hi):
    # integer-valued inputs: the chunked sum is exact, so bit-exact; K is no
    # multiple of the chunk, so the last chunk is short (and takes the edge path)
    lo = -128 if dtype == "i8" else -hi
    trans = list(itertools.product((False, True), repeat=2))
    for tA, tB in trans:
        for splits, (M, N, K) in ((2, (150, 133, 700)), (5, (70, 300, 1111)), (0, (200, 190, 2050))):
            ab = (3.0, -2.0) if dtype == "i8" else (1.5, 0.5)
            p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, alpha=ab[0], beta=ab[1],
                           dist="int", int_lo=lo, int_hi=hi, c_dist="int", c_dtype=c_dtype,
                           seed=91, splitk=splits)
            if dtype == "f32":   # keep every partial sum below 2^24
                p = dataclasses.replace(p, int_lo=-20, int_hi=20)
            if dtype in ("f16", "bf16") and c_dtype != "f32":
                p = dataclasses.replace(p, int_lo=-4, int_hi=4)
            n = mg.splitk_chunks(dtype, M, N, K, splits, transA=int(tA), transB=int(tB),
                                 lda=p.lda, ldb=p.ldb)
            assert n > 1
            full_check(p, exact=True, what=f"split-K {dtype}->{c_dtype} x{n} tA={int(tA)} tB={int(tB)}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_splitk_float_inputs_within_tolerance(dtype):
    p = wl.Problem(dtype, 257, 190, 3000, transA=True, alpha=0.75, beta=-1.25,
                   dist="normal" if dtype == "bf16" else "uniform", c_dist="uniform", seed=92,
                   splitk=6)
    full_check(p, what=f"split-K {dtype} x{mg.splitk_chunks(dtype, 257, 190, 3000, 6, transA=1)}")


def test_splitk_workspace_reused_by_a_smaller_call():
    p = wl.Problem("f32", 300, 260, 1500, dist="int", int_lo=-9, int_hi=9, seed=93, splitk=4)
    ws = torch.empty(mg.splitk_workspace_bytes("f32", 300, 260, 1500, 4), dtype=torch.uint8,
                     device="cuda")
    for q in (p, dataclasses.replace(p, M=120, N=77, K=900, seed=94)):
        r = Run(q)
        r.launch(workspace=ws)
        check_exact(r.result(), r.oracle_full(), f"split-K {q.M}x{q.N}x{q.K} in a shared workspace")


def test_splitk_quick_returns_and_one_chunk():
    for alpha, K in ((0.0, 512), (1.0, 0)):
        p = wl.Problem("f32", 90, 70, K, alpha=alpha, beta=-0.5, dist="uniform", seed=95, splitk=4)
        full_check(p, exact=True, what=f"split-K alpha={alpha} K={K} (no chunks)")
    # a request that gives one chunk runs the plain kernel, with no workspace
    p = wl.Problem("f32", 64, 64, 32, dist="int", int_lo=-9, int_hi=9, seed=96, splitk=8)
    assert mg.splitk_chunks("f32", 64, 64, 32, 8) == 1
    full_check(p, exact=True, what="split-K with one chunk")


def test_sgemm_ragged_splitk_bit_exact():
    p = wl.sgemm_ragged_splitk()
    assert mg.splitk_chunks("f32", p.M, p.N, p.K, p.splitk, lda=p.lda, ldb=p.ldb) == 3
    full_check(p, exact=True, what="ragged 1000x1027x999 through split-K")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_splitk_auto_small_unaligned_grid(dtype):
    # odd leading dimensions, a grid of 16 x 17 tiles: the automatic plan
    # chunks all of C in three; integer data bit-exact, float data in tolerance
    for tA, tB in itertools.product((False, True), repeat=2):
        p = wl.Problem(dtype, 1000, 1027, 999, transA=tA, transB=tB, alpha=2.0, beta=-1.0,
                       dist="int", int_lo=-20, int_hi=20, c_dist="int", seed=98, splitk=0)
        plan = mg.splitk_plan(dtype, 1000, 1027, 999, 0, transA=int(tA), transB=int(tB),
                              lda=p.lda, ldb=p.ldb)
        assert plan["chunks"] == 3, plan
        full_check(p, exact=True, what=f"automatic split-K {dtype} tA={int(tA)} tB={int(tB)}")
    q = wl.Problem(dtype, 1000, 1027, 999, alpha=0.5, beta=0.25, dist="uniform", c_dist="uniform",
                   seed=99, splitk=0)
    full_check(q, what=f"automatic split-K {dtype} uniform")


@pytest.mark.parametrize("K", [196, 200])
def test_splitk_attention_layout_with_padded_rows(K):
    # QK^T layout (16-bit, B stored [n][k]) with rows padded to 200 elements of NaN-free
    # data and NaN in the padding, four 64-deep chunks, 256 workgroups.  With K = 196 the
    # last chunk is 4 deep: the one-stage builds (no register path) must not take it,
    # else the row padding past K would be multiplied in.  K = 200 keeps them.
    p = wl.Problem("f16", 2048, 2048, K, transB=True, lda=200, ldb=200, dist="int", int_lo=-8,
                   int_hi=8, seed=120 + K, splitk=4, pad_value=float("nan"))
    plan = mg.splitk_plan("f16", 2048, 2048, K, 4, transB=1, lda=200, ldb=200)
    assert plan["chunks"] == 4 and plan["grid"] >= 256, plan
    assert plan["variant"]["name"].endswith("_s1") == (K % 8 == 0), plan
    full_check(p, exact=True, what=f"split-K QK^T layout K={K} ({plan['variant']['name']})")


def test_splitk_own_workspace_on_an_explicit_stream():
    # no workspace given: the binding allocates it on the launch stream, here a side stream
    # passed by handle while torch's current stream is another one
    p = wl.Problem("f32", 300, 260, 1500, dist="int", int_lo=-9, int_hi=9, seed=125, splitk=4)
    r = Run(p)
    s = torch.cuda.Stream()
    r.launch(stream=s.cuda_stream)
    s.synchronize()
    check_exact(r.result(), r.oracle_full(), "split-K, binding-allocated workspace, side stream")


def test_splitk_auto_on_a_deep_k_shape():
    p = wl.Problem("f32", 256, 256, 8192, alpha=2.0, dist="int", int_lo=-9, int_hi=9, seed=97,
                   splitk=0)
    assert mg.splitk_chunks("f32", 256, 256, 8192, 0) == 16
    full_check(p, exact=True, what="256x256x8192 automatic split-K")


@pytest.mark.parametrize("dtype,c_dtype", [("f32", "f32"), ("f16", "f32"), ("bf16", "f32"), ("i8", "i32"),
                                           ("f64", "f64"), ("f16", "f16"), ("bf16", "bf16")])
def test_streamk_exact(dtype, c_dtype):
    # integer-valued inputs: bit-exact however the tiles are split between
    # workgroups; shapes with edge tiles and K tails, the 4-byte-copy builds
    # (odd leading dimensions), one workgroup, and one workgroup per
    # (tile, iteration) pair.  A 16-bit C holds the exact sum rounded once
    # (the data stay small enough for binary16's range).
    i8 = dtype == "i8"
    lo, hi = (-128, 127) if i8 else (-4, 4) if c_dtype in ("f16", "bf16") else (-20, 20)
    trans = [(False, False), (False, True), (True, False), (True, True)]
    cases = [((1000, 1027, 999), 0), ((1000, 1027, 999), 37), ((150, 133, 700), 0),
             ((70, 300, 1111), 5), ((200, 190, 2050), 1), ((64, 64, 300), None)]
    for n, (tA, tB) in enumerate(trans):
        for (M, N, K), wgs in cases[n % 2::2]:
            plan = mg.streamk_plan(dtype, M, N, K, 0, transA=int(tA), transB=int(tB))
            if wgs is None:   # one workgroup per (tile, iteration) pair
                wgs = plan["tiles"] * plan["iterations"]
            ab = (3.0, -2.0) if i8 else (1.5, 0.5)
            p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, alpha=ab[0], beta=ab[1], dist="int",
                           int_lo=lo, int_hi=hi, c_dist="int", c_dtype=c_dtype, seed=131 + n,
                           streamk=wgs)
            plan = mg.streamk_plan(dtype, M, N, K, wgs, transA=int(tA), transB=int(tB), lda=p.lda,
                                   ldb=p.ldb)
            full_check(p, exact=True, what=f"stream-K {dtype}->{c_dtype} tA={int(tA)} tB={int(tB)} "
                       f"{plan['variant']['name']} x{plan['workgroups']} over {plan['tiles']} tiles "
                       f"of {plan['iterations']} iterations")


SK_ES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "f64": 8}
SK_GRANULE = {"f32": 32, "f16": 64, "bf16": 64, "i8": 128, "f64": 16}


@pytest.mark.parametrize("dtype,c_dtype", [("f32", "f32"), ("f16", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                           ("bf16", "bf16"), ("i8", "i32"), ("f64", "f64")])
def test_streamk_every_build_exact(dtype, c_dtype):
    # each build's stream-K launch, forced, on every transpose it has: edge tiles, a last
    # iteration shorter than the granule (a whole number of 16-byte chunks on the
    # aligned builds, so that the DMA ring takes it), 37 workgroups over a few
    # dozen (tile, iteration) pairs, so that most tiles are split
    es, unit = SK_ES[dtype], SK_GRANULE[dtype]
    code = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "f64": 5}[dtype]
    i8 = dtype == "i8"
    seen = set()
    try:
        for v in mg.variants():
            if v["dtype"] != code or v["pipe"] == 6:
                continue
            mg.force_variant(dtype, v["id"])
            aligned = not v["name"].endswith("_u")
            narrow_dw = v["pipe"] == 4 and es < 4
            M, N = 2 * v["block_m"] + 17, 2 * v["block_n"] + 9
            K = 4 * unit + (3 * 16 // es if aligned else 5 if not narrow_dw else 4 // es * 3)

            def ld(cols):
                if aligned:
                    return -(-cols // (16 // es)) * (16 // es)
                if narrow_dw:   # whole 4-byte pieces, not whole 16-byte chunks
                    piece = 4 // es
                    x = -(-cols // piece) * piece
                    return x + piece if (x * es) % 16 == 0 else x
                return cols + 1 if cols % 2 == 0 else cols

            hits = 0
            for n, (tA, tB) in enumerate(itertools.product((False, True), repeat=2)):
                lda, ldb = ld(M if tA else K), ld(K if tB else N)
                plan = mg.streamk_plan(dtype, M, N, K, 37, transA=int(tA), transB=int(tB), lda=lda, ldb=ldb)
                if plan["variant"]["name"] != v["name"]:
                    continue   # no stream-K launch of this build for this transpose
                ab = (3.0, -2.0) if i8 else (1.5, 0.5)
                lo, hi = (-128, 127) if i8 else (-4, 4)
                p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=lda, ldb=ldb, alpha=ab[0],
                               beta=ab[1], dist="int", int_lo=lo, int_hi=hi, c_dist="int", c_dtype=c_dtype,
                               seed=150 + n, streamk=37)
                full_check(p, exact=True, what=f"stream-K forced {v['name']} ({c_dtype} C) tA={int(tA)} "
                           f"tB={int(tB)} over {plan['tiles']} tiles of {plan['iterations']} iterations")
                hits += 1
            if hits:
                seen.add(v["name"])
    finally:
        mg.force_variant(dtype, None)
    log(f"  stream-K builds run: {sorted(seen)}")
    # every 128x128 and 64x64 build of the 32-bit-accumulating types has a launch; fp64 all but 2x4 waves
    want = {"f32": 6, "f16": 8, "bf16": 8, "i8": 8, "f64": 5}[dtype]
    assert len(seen) == want, sorted(seen)


@pytest.mark.parametrize("dtype,c_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16"),
                                           ("f64", "f64")])
def test_streamk_float_inputs_within_tolerance(dtype, c_dtype):
    p = wl.Problem(dtype, 1000, 1027, 999, alpha=0.75, beta=-1.25,
                   dist="normal" if dtype in ("bf16", "f16") else "uniform", c_dist="uniform",
                   c_dtype=c_dtype, seed=141, streamk=0)
    full_check(p, what=f"stream-K {dtype}->{c_dtype} 1000x1027x999")


def test_streamk_quick_returns_and_shared_workspace():
    for alpha, K in ((0.0, 512), (1.0, 0)):
        p = wl.Problem("f32", 90, 70, K, alpha=alpha, beta=-0.5, dist="uniform", seed=142, streamk=0)
        full_check(p, exact=True, what=f"stream-K alpha={alpha} K={K} (nothing but beta*C)")
    # one zero-filled workspace for calls of different sizes, workgroup counts and tile
    # counts, smaller after larger and larger after smaller: each call's last contributors
    # put the arrival counters back to zero, and the partial tiles never reach them
    shapes = ((300, 260, 1500, 100, 143), (120, 77, 900, 60, 144), (1000, 1027, 999, 0, 145),
              (64, 64, 300, None, 146), (300, 260, 1500, 100, 147))
    probs = []
    for M, N, K, wgs, seed in shapes:
        if wgs is None:   # one workgroup per (tile, iteration) pair
            plan = mg.streamk_plan("f32", M, N, K, 0)
            wgs = plan["tiles"] * plan["iterations"]
        probs.append(wl.Problem("f32", M, N, K, dist="int", int_lo=-9, int_hi=9, seed=seed,
                                streamk=wgs))
    need = max(mg.streamk_plan("f32", q.M, q.N, q.K, q.streamk, lda=q.lda, ldb=q.ldb)["workspace_bytes"]
               for q in probs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for q in probs:
        r = Run(q)
        ws[mg.STREAMK_COUNTER_BYTES:].fill_(0xA5)   # stale partial sums from anything before
        r.launch(workspace=ws)
        check_exact(r.result(), r.oracle_full(),
                    f"stream-K {q.M}x{q.N}x{q.K} x{q.streamk} in a shared workspace")
        left = int(torch.count_nonzero(ws[:mg.STREAMK_COUNTER_BYTES]))
        assert left == 0, f"{left} counter bytes non-zero after stream-K {q.M}x{q.N}x{q.K}"


ODD_ROW_BUILDS = {"f32": "mgemm_f32_%dx%dx32_w2x2_d4_u", "bf16": "mgemm_bf16_%dx%dx64_w2x2_d4_u",
                  "f16": "mgemm_f16_%dx%dx64_w2x2_d4_u", "i8": "mgemm_i8_%dx%dx128_w2x2_d4_u"}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "i8"])
def test_odd_row_builds_copy_rules_exact(dtype):
    # The builds for rows that are only 4-byte aligned copy 16 bytes per lane on
    # every whole slab with operand rows after it and 4 bytes on a tile's last
    # slab.  Cases: MN-contiguous operands whose edge chunks straddle the m/n
    # edge; M or N too small for 16-byte rows (4-byte copies throughout); K a
    # whole number of slabs (the last one whole but at the end of K); one slab
    # plus one piece; strided batches with rows packed tight.  Integer data,
    # compared exactly.
    es = {"f32": 4, "bf16": 2, "f16": 2, "i8": 1}[dtype]
    piece = 4 // es
    i8 = dtype == "i8"
    ids = {v["name"]: v["id"] for v in mg.variants()}
    bk = {"f32": 32, "bf16": 64, "f16": 64, "i8": 128}[dtype]

    def odd(cols):   # a whole number of 4-byte pieces, not of 16 bytes
        x = -(-cols // piece) * piece
        return x + piece if (x * es) % 16 == 0 else x

    cases = [(133, 129, 3 * bk + piece, 1), (130, 70, 2 * bk, 1), (97, 3 if es == 4 else 6, 3 * bk, 1),
             (3 if es == 4 else 6, 90, 2 * bk + piece, 1), (70, 75, bk + piece, 3), (200, 203, 5 * bk, 2)]
    try:
        for tile in (64, 128):
            name = ODD_ROW_BUILDS[dtype] % (tile, tile)
            mg.force_variant(dtype, ids[name])
            for n, (M, N, K, batch) in enumerate(cases):
                for tA, tB in itertools.product((False, True), repeat=2):
                    if i8 and tile == 64 and (tA or not tB):
                        continue   # the 64x64 int8 tiles take A and B K-contiguous only
                    lda, ldb = odd(M if tA else K), odd(K if tB else N)
                    a_rows, b_rows = (K if tA else M), (N if tB else K)
                    p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=lda, ldb=ldb, batch=batch,
                                   strideA=a_rows * lda, strideB=b_rows * ldb,
                                   alpha=3.0 if i8 else 1.5, beta=-2.0 if i8 else 0.5, dist="int",
                                   int_lo=-128 if i8 else -8, int_hi=127 if i8 else 8, c_dist="int",
                                   c_dtype="i32" if i8 else "f32", seed=170 + n)
                    info, _ = mg.select(dtype, int(tA), int(tB), M, N, K, p.alpha, 16, lda, p.strideA, 16, ldb,
                                        p.strideB, p.beta, 16, p.ldc, p.strideC, batch)
                    assert info["name"] == name, (info["name"], name)
                    full_check(p, exact=True, what=f"{name} tA={int(tA)} tB={int(tB)} {M}x{N}x{K} batch {batch}")
    finally:
        mg.force_variant(dtype, None)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_one_stage_builds_shallow_k_exact(dtype):
    # the one-stage 256x256 builds (K of one slab at most): full and edge tiles, a K tail
    # inside the slab, every transpose, fp32 and 16-bit C, batches; integer data, so each
    # result is the exact sum rounded once to C's type
    builds = variants_of(dtype, one_stage=True)
    assert builds
    for v in builds:
        mg.force_variant(dtype, v["id"])
        for n, (M, N, K, batch) in enumerate(((512, 768, 64, 2), (300, 260, 40, 3), (256, 256, 8, 1),
                                              (1000, 520, 56, 1))):
            for tA, tB in itertools.product((False, True), repeat=2):
                for c_dtype in ("f32", dtype):
                    a_cols = M if tA else K
                    b_cols = K if tB else N
                    p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, batch=batch, alpha=0.5,
                                   beta=0.0 if n % 2 else 2.0, lda=_round8(a_cols), ldb=_round8(b_cols),
                                   dist="int", int_lo=-4, int_hi=4, c_dist="int", c_dtype=c_dtype,
                                   pad_value=float("nan"), seed=151 + n)
                    _assert_selected(p, v)
                    full_check(p, exact=True, what=f"{v['name']} -> {c_dtype}")
    # the automatic choice takes it for the attention-score batch, and not past one slab
    info, _ = mg.select(dtype, 0, 1, 1024, 1024, 64, 0.125, 1 << 20, 64, 65536, 1 << 20, 64, 65536,
                        0.0, 1 << 20, 1024, 1 << 20, 128)
    assert info["name"].endswith("_w4x2_s1"), info["name"]
    info, _ = mg.select(dtype, 0, 1, 1024, 1024, 128, 0.125, 1 << 20, 128, 131072, 1 << 20, 128,
                        131072, 0.0, 1 << 20, 1024, 1 << 20, 128)
    assert info["name"].endswith("_w4x2"), info["name"]


# ------------------------------------------------------------------ shapes from the pages

def test_small_problem_builds_exact_and_in_tolerance():
    # 16x16 tiles whose waves share K: every transpose, edge tiles, K tails inside a
    # wave's share and in the last chunk, a K that leaves waves empty, batches, NaN in
    # the padding and in a beta = 0 C; integer data bit-exact, floats in tolerance
    for v in variants_of("f32", small=True):
        mg.force_variant("f32", v["id"])
        kmax = v["block_k"]
        for tA, tB in itertools.product((False, True), repeat=2):
            for (M, N, K, batch) in ((256, 256, min(256, kmax), 1), (37, 45, kmax, 1),
                                     (100, 130, kmax - 29, 2), (16, 16, 1, 1), (1, 1, 5, 3),
                                     (70, 33, 40, 1)):
                for dist, exact in (("int", True), ("uniform", False)):
                    p = wl.Problem("f32", M, N, K, transA=tA, transB=tB, batch=batch,
                                   alpha=1.5, beta=0.5 if dist == "int" else 0.0, dist=dist,
                                   int_lo=-20, int_hi=20, c_dist=dist, seed=150 + K,
                                   lda=(M if tA else K) + 3, ldb=(K if tB else N) + 5, ldc=N + 2,
                                   pad_value=float("nan"))
                    _assert_selected(p, v)
                    full_check(p, exact=exact, c_fill=float("nan"),
                               what=f"{v['name']} {dist} tA={int(tA)} tB={int(tB)}")
    mg.force_variant("f32", None)


def test_csdn_ragged_integer_example():
    # A 47 x 804, B 804 x 53, rand() % 100 values (CSDN tile-algorithm page, main)
    p = wl.Problem("f32", 47, 53, 804, dist="int", int_lo=0, int_hi=99, seed=14)
    full_check(p, exact=True, what="47x804x53 ints")


def test_dlog_shapes():
    full_check(wl.Problem("f32", 100, 300, 200, dist="normal", seed=15), what="mm 100x200x300")
    full_check(wl.Problem("f32", 16, 128, 64, batch=10, dist="normal", seed=16),
               what="bmm (10,16,64)x(10,64,128)")
    full_check(wl.Problem("f16", 10, 10, 64, transB=True, batch=16, alpha=0.125, dist="normal",
                          seed=17), what="einsum QK^T (2,8,10,64)")


def test_wmma_single_tile_f16_col_major_a():
    # 16x16x16 half inputs, A column-major (= op(A) = A^T row-major), float accumulator
    p = wl.Problem("f16", 16, 16, 16, transA=True, dist="normal", seed=18)
    full_check(p, what="16^3 f16 transA")
    full_check(wl.int_shadow(p, -8, 8), exact=True, what="16^3 f16 transA int")


# ------------------------------------------------------------------ degenerate cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_alpha_zero_and_k_zero_give_beta_c(dtype):
    for p in (wl.Problem(dtype, 70, 50, 30, alpha=0.0, beta=0.5, c_dist="uniform", seed=19),
              wl.Problem(dtype, 70, 50, 0, alpha=1.0, beta=-2.0, c_dist="uniform", seed=20),
              wl.Problem(dtype, 70, 50, 0, alpha=1.0, beta=0.0, seed=21)):
        full_check(p, exact=True, c_fill=float("nan"), what=f"alpha={p.alpha} K={p.K}")


def test_empty_problems_touch_nothing():
    for M, N in ((0, 10), (10, 0)):
        p = wl.Problem("f32", M, N, 5, seed=22)
        log(f"[empty] M={M} N={N}")
        mg.gemm_f32(0, 0, M, N, 5, 1.0, torch.zeros(64, device="cuda"), 5,
                    torch.zeros(64, device="cuda"), max(N, 1), 0.0, torch.zeros(64, device="cuda"),
                    max(N, 1))
    c = torch.full((64,), 3.0, device="cuda")
    mg.gemm_strided_batched("f32", 0, 0, 4, 4, 4, 1.0, c, 4, 16, c, 4, 16, 0.0, c, 4, 16, 0)
    torch.cuda.synchronize()
    assert torch.all(c == 3.0)


def test_minimum_sizes():
    for M, N, K in ((1, 1, 1), (1, 7, 3), (5, 1, 9), (3, 3, 1), (33, 65, 2)):
        for dt in ("f32", "f16", "bf16", "f64"):
            full_check(wl.Problem(dt, M, N, K, dist="int", int_lo=-9, int_hi=9, seed=23),
                       exact=True, what=f"tiny {dt}")
        full_check(wl.Problem("i8", M, N, K, transB=True, c_dtype="i32", dist="int", int_lo=-128,
                              int_hi=127, seed=24), exact=True, what="tiny i8")
        # split-K on tiny shapes: one chunk (plain kernel) or a few short ones
        full_check(wl.Problem("f32", M, N, K, dist="int", int_lo=-9, int_hi=9, seed=25, splitk=4),
                   exact=True, what="tiny split-K")


def test_empty_problems_for_every_entry_point():
    # M, N or batch == 0: OK, nothing launched, nothing written
    c = torch.full((64,), 3.0, device="cuda", dtype=torch.float64)
    mg.gemm_f64(0, 0, 0, 4, 4, 1.0, c, 4, c, 4, 0.0, c, 4)
    mg.gemm_f64_strided_batched(0, 0, 4, 4, 4, 1.0, c, 4, 16, c, 4, 16, 0.0, c, 4, 16, 0)
    ci = torch.full((64,), 3, device="cuda", dtype=torch.int32)
    a8 = torch.zeros(64, device="cuda", dtype=torch.int8)
    mg.gemm_strided_batched_ex("i8", "i32", 0, 1, 4, 0, 4, 1.0, a8, 4, 0, a8, 4, 0, 0.0, ci, 1, 0, 1)
    cf = torch.full((64,), 3.0, device="cuda")
    mg.gemm_splitk("f32", "f32", 0, 0, 0, 4, 64, 1.0, cf, 64, cf, 4, 0.0, cf, 4, splits=4)
    torch.cuda.synchronize()
    assert torch.all(c == 3.0) and torch.all(ci == 3) and torch.all(cf == 3.0)


def test_leading_dimensions_beyond_32bit_tile_offsets():
    # with a leading dimension past 2^31 / (257 * element size), 257 rows no longer
    # fit 32-bit byte offsets from a tile origin: every tile must take the
    # 64-bit-addressed register path and still be exact
    p = wl.Problem("f32", 300, 260, 48, ldb=(1 << 21) + 64, dist="int", int_lo=-9, int_hi=9,
                   seed=27)
    full_check(p, exact=True, what="fp32, ldb 2^21+64")
    p = wl.Problem("bf16", 300, 260, 32, transA=True, lda=(1 << 22) + 64, dist="int", int_lo=-9,
                   int_hi=9, seed=28)
    full_check(p, exact=True, what="bf16, A^T, lda 2^22+64")


def test_output_beyond_2_31_elements():
    # C with more than 2^31 elements (8.6 GB): row * ldc and batch * strideC offsets
    # must be 64-bit; checked on every element of the rows past index 2^31 that we
    # sample, against the oracle element by element
    for (M, N, K, batch) in ((65600, 32768, 32, 1), (32768, 32768, 16, 3)):
        p = wl.Problem("bf16", M, N, K, transB=True, batch=batch, dist="int", int_lo=-4, int_hi=4,
                       seed=29)
        log(f"[>2^31 C] bf16 M={M} N={N} K={K} batch={batch} C elements {p.c_elems}")
        A, B, _ = wl.make_inputs(p)
        dA, dB = A.cuda(), B.cuda()
        dC = torch.full((p.c_elems,), float("nan"), device="cuda")
        mg.gemm_strided_batched("bf16", 0, 1, M, N, K, 1.0, dA, p.lda, p.strideA, dB, p.ldb,
                                p.strideB, 0.0, dC, p.ldc, p.strideC, batch)
        torch.cuda.synchronize()
        rng = np.random.default_rng(5)
        last = batch - 1
        rows = np.array([M - 1, M - 2, (1 << 31) // N if batch == 1 else M // 2])
        bs = np.concatenate([np.full(N, last)] * 3 + [rng.integers(0, batch, 4000)])
        is_ = np.concatenate([np.full(N, r) for r in rows] + [rng.integers(0, M, 4000)])
        js = np.concatenate([np.arange(N)] * 3 + [rng.integers(0, N, 4000)])
        flat = torch.from_numpy(bs * p.strideC + is_ * p.ldc + js).cuda()
        got = dC[flat].cpu().numpy().astype(np.float64)
        assert (bs * p.strideC + is_ * p.ldc + js).max() >= (1 << 31)
        ref = oracle.gemm_elems("bf16", False, True, M, N, K, 1.0, wl.to_numpy_operand(A), p.lda,
                                wl.to_numpy_operand(B), p.ldb, 0.0, None, p.ldc, bs, is_, js,
                                batch=batch, strideA=p.strideA, strideB=p.strideB,
                                strideC=p.strideC)
        check_exact(got, ref, f"C past 2^31 elements, batch={batch}")
        del dA, dB, dC
        torch.cuda.empty_cache()


def test_broadcast_operands_in_batches():
    p = wl.Problem("f32", 40, 36, 44, batch=5, strideA=0, dist="int", int_lo=-9, int_hi=9,
                   seed=24)
    full_check(p, exact=True, what="strideA=0")
    p = wl.Problem("bf16", 40, 36, 44, batch=5, strideB=0, transB=True, dist="int", int_lo=-9,
                   int_hi=9, seed=25)
    full_check(p, exact=True, what="strideB=0")


def test_repeated_runs_are_bitwise_identical():
    p = wl.Problem("f32", 1024, 1024, 1024, alpha=1.0, beta=0.0, dist="uniform", seed=26)
    log("[determinism] f32 1024^3 x3")
    r = Run(p)
    outs = []
    for _ in range(3):
        r.launch()
        outs.append(r.result().copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    q = wl.Problem("bf16", 1024, 1024, 1024, dist="normal", seed=27)
    log("[determinism] bf16 1024^3 x3")
    r = Run(q)
    outs = []
    for _ in range(3):
        r.launch()
        outs.append(r.result().copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_runs_on_a_side_stream():
    p = wl.Problem("bf16", 512, 384, 256, transA=True, dist="normal", seed=28)
    log("[side stream] bf16 512x384x256")
    r = Run(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r.launch()          # binding picks the current (side) stream
    s.synchronize()
    got = r.result()
    check_tolerance(got, r.oracle_full(), p, "side stream")


# ------------------------------------------------------------------ HIP graph capture

def test_launches_replay_in_a_hip_graph():
    # The library only enqueues kernels on the caller's stream, so a capture
    # records them (split-K's and stream-K's two kernels included).  Each replay is checked against the eager result, with
    # eager work and synchronisation between replays.
    p = wl.Problem("f32", 256, 256, 256, alpha=1.5, beta=0.5, dist="int", int_lo=-8, int_hi=8,
                   c_dist="int", seed=120)
    r = Run(p)
    c0 = r.dCbuf.clone()
    r.launch()
    eager = r.result()
    check_exact(eager, r.oracle_full(), "eager 256^3")
    q = wl.Problem("f32", 256, 256, 8192, dist="int", int_lo=-8, int_hi=8, seed=121, splitk=0)
    rq = Run(q)
    ws = torch.empty(mg.splitk_workspace_bytes("f32", 256, 256, 8192, 0), dtype=torch.uint8,
                     device="cuda")
    rq.launch(workspace=ws)
    eager_q = rq.result()
    z = wl.Problem("f32", 1000, 1027, 999, dist="int", int_lo=-8, int_hi=8, seed=122, streamk=0)
    rz = Run(z)
    wz = torch.zeros(mg.streamk_plan("f32", 1000, 1027, 999, 0, lda=z.lda, ldb=z.ldb)["workspace_bytes"],
                     dtype=torch.uint8, device="cuda")
    rz.launch(workspace=wz)
    eager_z = rz.result()
    check_exact(eager_z, rz.oracle_full(), "eager stream-K 1000x1027x999")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # capture on a side stream, as torch requires
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            r.launch()
            rq.launch(workspace=ws)
            rz.launch(workspace=wz)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        r.dCbuf.copy_(c0)                  # beta = 0.5 reads C: restore it eagerly
        rq.dC.fill_(float("nan"))          # beta = 0: C is overwritten (guard bands kept)
        rz.dC.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()      # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        check_exact(r.result(), eager, f"graph replay {rep} (256^3)")
        check_exact(rq.result(), eager_q, f"graph replay {rep} (split-K 256x256x8192)")
        check_exact(rz.result(), eager_z, f"graph replay {rep} (stream-K 1000x1027x999)")
        assert int(torch.count_nonzero(wz[:mg.STREAMK_COUNTER_BYTES])) == 0, "stream-K counters left set"


# ------------------------------------------------------------------ seeded random problems

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8", "f64"])
def test_random_problems_exact(dtype):
    # Seeded random shapes, transposes, leading-dimension padding (aligned and
    # not), C types, batches and split-K plans through the automatic choice:
    # whatever build and path (unchecked or checked DMA copies, 4-byte copies,
    # the realigning register path) the choice lands on must be exact on
    # integer-valued inputs, with NaN (or a filler) in every padding element.
    rng = np.random.default_rng({"f32": 11, "f16": 12, "bf16": 13, "i8": 14, "f64": 15}[dtype])
    i8 = dtype == "i8"
    for case in range(16):
        small = rng.random() < 0.4
        M = int(rng.integers(1, 70 if small else 400))
        N = int(rng.integers(1, 70 if small else 400))
        K = int(rng.integers(1, 64)) if rng.random() < 0.3 else int(rng.integers(64, 500))
        if rng.random() < 0.3:
            K = -(-K // 32) * 32          # whole slabs now and then
        tA, tB = (False, True) if i8 else (bool(rng.integers(2)), bool(rng.integers(2)))
        batch = int(rng.integers(1, 4)) if rng.random() < 0.3 else 1
        splitk = None
        if batch == 1 and rng.random() < 0.25:
            splitk = int(rng.choice([0, 2, 3, 5]))
        pads = [0, 1, 2, 3, 4, 8, 16, 64]
        a_cols, b_cols = (M if tA else K), (K if tB else N)
        lda = max(a_cols, 1) + int(rng.choice(pads))
        ldb = max(b_cols, 1) + int(rng.choice(pads))
        ldc = max(N, 1) + int(rng.choice(pads))
        if i8:
            kw = dict(c_dtype="i32", int_lo=-128, int_hi=127, pad_value=77,
                      alpha=float(rng.choice([1, -3, 2])), beta=float(rng.choice([0, 1, -2])))
        else:
            c16 = dtype in ("f16", "bf16") and rng.random() < 0.4
            kw = dict(c_dtype=dtype if c16 else "f32", int_lo=-8, int_hi=8, pad_value=float("nan"),
                      alpha=float(rng.choice([1.0, -1.0, 2.0, 0.5])),
                      beta=float(rng.choice([0.0, 1.0, -1.0, 0.5])))
        p = wl.Problem(dtype, M, N, K, transA=tA, transB=tB, batch=batch, lda=lda, ldb=ldb, ldc=ldc,
                       dist="int", c_dist="int", seed=1000 * case + 7, splitk=splitk, **kw)
        info, _ = mg.select(p.dtype, int(tA), int(tB), M, N, K, A=16, lda=lda,
                            strideA=p.strideA, B=16, ldb=ldb, strideB=p.strideB, C=16, ldc=ldc,
                            strideC=p.strideC, batch=batch, alpha=p.alpha, beta=p.beta)
        full_check(p, exact=True, what=f"random {dtype} #{case} ({info['name']}, splitk={splitk})")
