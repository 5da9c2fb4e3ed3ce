"""Every LDS schedule under the race-check build of the library.

libmgemm_poison.so is built from the same sources with -DMGEMM_DEBUG_POISON.
Each LDS ring fills all of its stages with 0xFF bytes before its first copy,
and refills each stage the same way once every wave has read it, before the
stage's refill is issued. 0xFF bytes are NaN in every floating type and -1
in int8. A fragment read that overtakes its slab's copies (a wait too
short), or a refill that overtakes a read (a missing barrier), then reads
poison instead of a plausible stale value.

The data are integer-valued and compared exactly with the oracle. The test
covers every build of every type:
- the 4-stage and 2-stage DMA rings (PIPE 1 and 2) and their register path
  (K not a whole number of 16-byte chunks);
- the one-stage builds (PIPE 3) and the 4-byte-copy builds (PIPE 4);
- the SPREAD order of the 256x256 16-bit builds (MN-contiguous B, that is
  transB = N);
- int8 (transposing 8-bit reads for MN-contiguous operands) and fp64;
- split-K chunks and stream-K segments, whose rings restart per segment
  (fp32, bf16 with fp32 and bf16 C, int8 and fp64).
"""
import itertools

import pytest
import torch

from dense_gemm_f32_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import _lib
    from parity import Run, check_exact, expected_exact, log

ES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "f64": 8}
CODE = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "f64": 5}


@pytest.fixture(scope="module", autouse=True)
def poison_library():
    with _lib.using_library(_lib.POISON_LIB_PATH) as lib:
        assert mg.load() is lib
        assert _lib.build_flags() == _lib.BUILD_LDS_POISON, "not the race-check build"
        try:
            yield lib
        finally:
            for dt in CODE:
                mg.force_variant(dt, None)
    assert _lib.build_flags() == 0


def exact(p, what):
    log(f"[poison: {what}] {p.dtype} tA={int(p.transA)} tB={int(p.transB)} M={p.M} N={p.N} K={p.K} "
        f"lda={p.lda} ldb={p.ldb} splitk={p.splitk} streamk={p.streamk} seed={p.seed}")
    r = Run(p)
    r.launch()
    check_exact(r.result(), expected_exact(p, r.oracle_full()), f"poison build: {what}")


def selected(p):
    info, _ = mg.select(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, 16, p.lda,
                        p.strideA, 16, p.ldb, p.strideB, p.beta, 16, p.ldc, p.strideC, p.batch)
    return info["name"]


def builds(dtype):
    return [v for v in mg.variants() if v["dtype"] == CODE[dtype] and v["pipe"] != 6]


def int_problem(dtype, M, N, K, tA, tB, lda, ldb, seed, c_dtype="f32"):
    if dtype == "i8":
        return wl.Problem("i8", M, N, K, transA=tA, transB=tB, lda=lda, ldb=ldb, alpha=3.0, beta=-2.0,
                          dist="int", int_lo=-128, int_hi=127, c_dist="int", c_dtype="i32", seed=seed)
    return wl.Problem(dtype, M, N, K, transA=tA, transB=tB, lda=lda, ldb=ldb, alpha=1.0, beta=-1.0,
                      dist="int", int_lo=-8, int_hi=8, c_dist="int", c_dtype=c_dtype, seed=seed)


def lds(dtype, cols, aligned, narrow_dw):
    """A leading dimension for `cols` columns: 16-byte rows for the aligned builds, else
    odd (or, for the 8/16-bit 4-byte-copy builds, a whole number of 4-byte pieces that is
    not one of 16 bytes)."""
    es = ES[dtype]
    if aligned:
        step = 16 // es
        return -(-cols // step) * step
    if narrow_dw:
        piece = 4 // es
        ld = -(-cols // piece) * piece
        return ld + piece if (ld * es) % 16 == 0 else ld
    return cols + 1 if cols % 2 == 0 else cols


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8", "f64"])
def test_every_build_under_lds_poison(dtype):
    combos = list(itertools.product((False, True), repeat=2))
    seen = 0
    for v in builds(dtype):
        mg.force_variant(dtype, v["id"])
        bm, bn, bk = v["block_m"], v["block_n"], v["block_k"]
        aligned = not v["name"].endswith("_u")
        narrow_dw = v["pipe"] == 4 and ES[dtype] < 4
        M, N = 2 * bm + 17, 2 * bn + 9
        if v["pipe"] == 3:            # one stage: K of one slab at most
            ks = [bk, bk - 16 // ES[dtype]]
        elif dtype == "f64":
            ks = [6 * bk + 3]
        else:
            # whole slabs through the ring's steady state; then a K that is no whole
            # number of 16-byte chunks (the register path of the 16-byte builds; a K
            # tail for the others)
            chunk = 16 // ES[dtype]
            tail = 4 // ES[dtype] if narrow_dw else (chunk if dtype == "i8" else 1)
            ks = [6 * bk, 3 * bk + tail]
        for (tA, tB), K in itertools.product(combos, ks):
            lda = lds(dtype, M if tA else K, aligned, narrow_dw)
            ldb = lds(dtype, K if tB else N, aligned, narrow_dw)
            p = int_problem(dtype, M, N, K, tA, tB, lda, ldb, seed=200 + seen % 50)
            if selected(p) != v["name"]:
                continue   # this K or layout is outside the build (e.g. the one-stage K rule)
            exact(p, f"{v['name']} pipe {v['pipe']} K={K}")
            seen += 1
        mg.force_variant(dtype, None)
    assert seen >= len(builds(dtype)), (seen, len(builds(dtype)))


# (K, lda, ldb) per type: fp32 with odd rows (the 4-byte-copy build), bf16 with
# 16-byte rows (the DMA ring), int8 N x N with 16-byte rows, fp64 with 16-byte
# rows and a K tail
STREAM_SHAPES = {"f32": (999, 999, 1027), "bf16": (1000, 1000, 1032), "i8": (1024, 1024, 1040),
                 "f64": (999, 1000, 1028)}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8", "f64"])
def test_streamk_and_splitk_under_lds_poison(dtype):
    tB = False   # B MN-contiguous: int8 through its transposing reads
    K, lda, ldb = STREAM_SHAPES[dtype]
    for wgs in (0, 37):
        p = int_problem(dtype, 1000, 1027, K, False, tB, lda, ldb, seed=260 + wgs)
        p.streamk = wgs
        exact(p, f"stream-K x{wgs or 512}")
    if dtype == "bf16":   # C in the inputs' own type
        p = int_problem(dtype, 1000, 1027, K, False, tB, lda, ldb, seed=265, c_dtype="bf16")
        p.streamk = 0
        exact(p, "stream-K, bf16 C")
    K3 = 3 * K
    p = int_problem(dtype, 300, 260, K3, False, tB, K3, K3 if tB else (260 if dtype != "bf16" else 264),
                    seed=270)
    p.splitk = 3
    exact(p, "split-K, 3 chunks")


def test_poison_build_is_only_used_inside_the_fixture(poison_library):
    assert mg.load() is poison_library
