"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol its header declares, validates arguments on the host and selects
variants.  No kernel is launched here: every call either fails validation
(which happens before any HIP call) or is a pure-host introspection call."""
import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_f32_amd as mg
from dense_gemm_f32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgemm.h")


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB_PATH):
        from dense_gemm_f32_amd import build
        build.build()
    return mg.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("gemm_f32", "gemm_f16", "gemm_bf16", "gemm_f64", "gemm_strided_batched",
                 "gemm_strided_batched_ex", "gemm_f64_strided_batched", "mgemm_status_string",
                 "mgemm_select", "mgemm_force_variant"):
        assert want in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = mg.load()
    for n in declared_functions():
        assert getattr(lib, n) is not None


def test_race_check_build_exports_the_header_and_says_what_it_is():
    # libmgemm_poison.so: the same sources with -DMGEMM_DEBUG_POISON (a GPU test runs it)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.POISON_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert not [n for n in declared_functions() if n not in exported]
    assert "mgemm_build_flags" in declared_functions()
    assert _lib.build_flags() == 0
    with _lib.using_library(_lib.POISON_LIB_PATH) as lib:
        assert mg.load() is lib and _lib.build_flags() == _lib.BUILD_LDS_POISON
        assert lib.mgemm_num_variants() == mg.load().mgemm_num_variants()
    assert _lib.build_flags() == 0 and mg.load() is not lib


def test_diag_library_exports_its_header():
    # the benchmark's measurement aid: built beside libmgemm.so, loaded by bench.py only
    diag_header = os.path.join(ROOT, "include", "mgemm_diag.h")
    diag_lib = os.path.join(os.path.dirname(_lib.LIB_PATH), "libmgemm_diag.so")
    if not os.path.exists(diag_lib):
        from dense_gemm_f32_amd import build
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(diag_header).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))
    assert "mgemm_diag_mfma_ceiling" in names
    out = subprocess.run(["nm", "-D", "--defined-only", diag_lib], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert not [n for n in names if n not in exported]
    lib = ctypes.CDLL(diag_lib)
    lib.mgemm_diag_ceiling_flop.restype = ctypes.c_double
    lib.mgemm_diag_ceiling_flop.argtypes = [ctypes.c_int]
    assert lib.mgemm_diag_ceiling_flop(1) == 256 * 4 * 64 * 32768.0
    lib.mgemm_diag_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]
    assert lib.mgemm_diag_mfma_ceiling(1, None, None, 10, None) == 1   # refused, no launch
    assert lib.mgemm_diag_mfma_ceiling(7, 16, 16, 10, None) == 1        # unknown kind, no launch
    lib.mgemm_diag_ceiling_ops.restype = ctypes.c_double
    lib.mgemm_diag_ceiling_ops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.mgemm_diag_ceiling_ops(2, 1) == 2 * lib.mgemm_diag_ceiling_flop(1)   # int8: 32x32x32
    assert lib.mgemm_diag_ceiling_ops(1, 3) == lib.mgemm_diag_ceiling_flop(3)


def test_status_strings():
    assert mg.status_string(0) == "MGEMM_OK"
    assert "INVALID_ARG" in mg.status_string(1)
    assert "HIP" in mg.status_string(2)
    assert "unknown" in mg.status_string(99)


def test_variant_table():
    vs = mg.variants()
    assert len(vs) == mg.load().mgemm_num_variants() >= 3
    for i, v in enumerate(vs):
        assert v["id"] == i
        assert v["threads"] == v["waves_m"] * v["waves_n"] * 64
        assert v["lds_bytes"] <= 160 * 1024
        assert v["pipe"] in (1, 2, 3, 4, 6)
        assert v["name"].startswith("mgemm_")
    assert {v["dtype"] for v in vs} == {0, 1, 2, 3, 5}
    info = _lib.VariantInfo()
    assert mg.load().mgemm_variant(len(vs), ctypes.byref(info)) == 1


ALIGNED = 1 << 20  # a 16-byte aligned fake address; select() never dereferences it


def sel(dtype="f32", tA=0, tB=0, M=64, N=64, K=64, **kw):
    kw.setdefault("A", ALIGNED)
    kw.setdefault("B", ALIGNED)
    kw.setdefault("C", ALIGNED)
    return mg.select(dtype, tA, tB, M, N, K, **kw)


@pytest.mark.parametrize("bad", [
    dict(M=-1), dict(N=-1), dict(K=-1), dict(batch=-1),
    dict(lda=63), dict(ldb=63), dict(ldc=63),
    dict(A=0), dict(B=0), dict(C=0),
    dict(A=ALIGNED + 2), dict(C=ALIGNED + 2),
    dict(M=2 ** 31), dict(strideA=-1),
    dict(batch=2, strideC=64 * 64 - 1), dict(batch=2, strideA=100, strideC=4096),
])
def test_validation_rejects(bad):
    with pytest.raises(mg.MgemmError) as e:
        sel(**bad)
    assert e.value.status == 1


def test_validation_bad_op_and_dtype():
    with pytest.raises(mg.MgemmError):
        sel(tA=2)
    with pytest.raises(mg.MgemmError):
        sel(dtype=7)


def test_transposed_leading_dimension_rules():
    # op(A)=A^T: A stored K x M -> lda >= M ; op(B)=B^T: B stored N x K -> ldb >= K
    sel(tA=1, tB=1, M=100, N=30, K=20, lda=100, ldb=20, ldc=30)
    with pytest.raises(mg.MgemmError):
        sel(tA=1, M=100, N=30, K=20, lda=99, ldb=30, ldc=30)
    with pytest.raises(mg.MgemmError):
        sel(tB=1, M=100, N=30, K=20, lda=20, ldb=19, ldc=30)


def test_quick_returns_launch_no_gemm():
    info, grid = sel(M=0)
    assert info["id"] == -1 and grid == 0 and info["name"] == "none"
    info, grid = sel(batch=0)
    assert info["name"] == "none"
    # alpha == 0 or K == 0: C = beta*C, A/B not read (NULL allowed)
    info, grid = sel(alpha=0.0, A=0, B=0, beta=2.0)
    assert info["name"] == "mgemm_scale_c" and grid == 0
    info, grid = sel(K=0, A=0, B=0, lda=1, ldb=64)
    assert info["name"] == "mgemm_scale_c"


def test_broadcast_strides_allowed():
    sel(batch=4, strideA=0, strideB=64 * 64, strideC=64 * 64)
    sel(batch=4, strideA=64 * 64, strideB=0, strideC=64 * 64)


def test_unaligned_operands_get_unaligned_variant():
    info, _ = sel(M=1000, N=1027, K=999, lda=999, ldb=1027, ldc=1027)
    assert info["name"].endswith("_u")
    big = dict(M=1024, N=1024, K=1024, lda=1024, ldb=1024, ldc=1024)
    info, _ = sel(A=ALIGNED + 4, **big)
    assert info["name"].endswith("_u")
    info, _ = sel(**big)
    assert not info["name"].endswith("_u")
    # the small-problem build loads one element at a time: any 4-byte alignment
    info, _ = sel(A=ALIGNED + 4)
    assert info["name"].startswith("mgemm_f32_16x16")


def test_selection_for_the_named_workloads():
    big, g = sel(M=4096, N=4096, K=4096, alpha=1.5, beta=0.5)
    assert g == (4096 // big["block_m"]) * (4096 // big["block_n"]) and g >= 256
    info, g = sel("bf16", M=8192, N=8192, K=8192)
    assert info["dtype"] == 2 and g >= 256
    info, g = sel("f16", 0, 1, M=1024, N=1024, K=64, lda=64, ldb=64, ldc=1024, batch=128,
                  strideA=65536, strideB=65536, strideC=1048576, alpha=0.125)
    assert info["dtype"] == 1 and g == 128 * (1024 // info["block_m"]) * (1024 // info["block_n"])


def test_fp32_choice_by_estimated_time():
    """fp32 builds carry a measured time model (rounds of 256 workgroups, a
    register-path factor, a one-round factor); the lowest estimate wins."""
    def name(M, N, K, **kw):
        return sel(M=M, N=N, K=K, **kw)[0]["name"]
    # whole rounds of the large tile stay there
    assert name(4096, 4096, 4096) == "mgemm_f32_256x256x32_w4x2"
    assert name(8192, 8192, 8192) == "mgemm_f32_256x256x32_w4x2"
    # 324 tiles of 256x256 are two rounds, the second a quarter full (measured
    # 2172 us against 1568 for 64x64); 576 of them are three (4392 against 3383)
    assert name(4608, 4608, 4608) == "mgemm_f32_64x64x32_w2x2_d2"
    assert name(6144, 6144, 6144) == "mgemm_f32_128x128x32_w2x2"
    assert name(3072, 3072, 3072) == "mgemm_f32_64x64x32_w2x2_d2"
    # aligned rows, K a multiple of 16 bytes: the 16-byte builds copy every
    # tile by DMA, edges and K tails included
    assert name(3000, 3000, 3000) == "mgemm_f32_64x64x32_w2x2_d2"
    assert name(1000, 1000, 1000) == "mgemm_f32_64x64x32_w2x2_d2"
    assert name(1024, 1024, 1024) == "mgemm_f32_64x64x32_w2x2_d2"
    # aligned rows but K no multiple of 4: the 16-byte builds would take the
    # register path for every tile; the 4-byte-copy builds keep the DMA
    assert name(1000, 1000, 1001, lda=1004) == "mgemm_f32_64x64x32_w2x2_d4_u"
    assert name(3000, 3000, 3001, lda=3004).endswith("_d4_u")
    # offsets past 32 bits: no 4-byte-copy build; aligned rows keep the
    # 16-byte builds (their register path), unaligned ones the plain builds
    big = 2_100_000
    n = name(1024, 1024, 1000, lda=big, ldb=big)
    assert n == "mgemm_f32_64x64x32_w2x2_d2"
    n = name(1024, 1024, 1000, lda=big + 1, ldb=big + 1)
    assert n.endswith("_u") and "_d4" not in n
    # the 16-bit, int8 and fp64 tables carry estimates too (below)
    assert sel("bf16", M=8192, N=8192, K=8192)[0]["block_m"] == 256


def test_other_types_choice_by_estimated_time():
    def name(dtype, M, N, K, tB=0, **kw):
        return sel(dtype, 0, tB, M=M, N=N, K=K, **kw)[0]["name"]
    # the headline shapes keep their builds
    assert name("bf16", 8192, 8192, 8192) == "mgemm_bf16_256x256x64_w2x4_d2"
    assert name("i8", 8192, 8192, 8192, tB=1) == "mgemm_i8_256x256x128_w2x4_d2"
    assert name("f64", 4096, 4096, 4096) == "mgemm_f64_128x128x16_w4x2"
    # 144 tiles of 256x256 beat 576 of 128x128 (three rounds; measured bf16
    # 3072^3 66 us against 78)
    assert name("bf16", 3072, 3072, 3072) == "mgemm_bf16_256x256x64_w2x4_d2"
    # 128x128 with eight waves: one round of 256 tiles takes the four-stage
    # build, several rounds the two-stage one (bf16 2048^3 22 us, 2560^3 38;
    # int8 4608^3 104 us against 116 for 256x256)
    assert name("bf16", 2048, 2048, 2048) == "mgemm_bf16_128x128x64_w2x4"
    assert name("bf16", 2560, 2560, 2560) == "mgemm_bf16_128x128x64_w2x4_d2"
    assert name("i8", 4608, 4608, 4608, tB=1) == "mgemm_i8_128x128x128_w2x4_d2"
    # fp64: 2304 tiles of 64x64 beat 576 of 128x128 (1043 us against 1207)
    assert name("f64", 3072, 3072, 3072) == "mgemm_f64_64x64x16_w2x2"
    # a shallow K is store-bound: the attention-score batch takes the 256x256
    # tile whose lanes store four adjacent elements, with either C type
    qkt = dict(tB=1, lda=64, ldb=64, batch=128, strideA=65536, strideB=65536, strideC=1048576)
    # the attention-score batch (K = 64, one slab): the one-stage build; K = 128: two stages
    assert name("f16", 1024, 1024, 64, **qkt) == "mgemm_f16_256x256x64_w4x2_s1"
    assert name("f16", 1024, 1024, 64, c_dtype="f16", **qkt) == "mgemm_f16_256x256x64_w4x2_s1"
    qkt128 = dict(qkt, lda=128, ldb=128, strideA=131072, strideB=131072)
    assert name("f16", 1024, 1024, 128, **qkt128) == "mgemm_f16_256x256x64_w4x2"
    # mgemm_select_ex checks C's type like the entry points do
    with pytest.raises(mg.MgemmError):
        sel("f16", M=64, N=64, K=64, c_dtype="bf16")
    with pytest.raises(mg.MgemmError):
        sel("f32", M=64, N=64, K=64, c_dtype="f16")
    # rows with no 16-byte alignment: the preference order, 4-byte copies first
    assert name("i8", 3000, 3000, 3000, tB=1) == "mgemm_i8_128x128x128_w2x2_d4_u"
    assert name("bf16", 1000, 1030, 1000, lda=1002, ldb=1030) == "mgemm_bf16_64x64x64_w2x2_d4_u"
    assert name("bf16", 1000, 1027, 999, lda=999, ldb=1027) == "mgemm_bf16_64x64x64_w2x2_u"
    # 4-byte copies of 16-bit elements need an even K
    assert name("bf16", 1000, 1030, 999, lda=1002, ldb=1030) == "mgemm_bf16_64x64x64_w2x2_u"


def test_int8_rules_without_a_gpu():
    lib = mg.load()
    ex = lib.gemm_strided_batched_ex

    def call(tA=0, tB=1, c_dt=4, alpha=1.0, beta=0.0, M=4, A=ALIGNED):
        return ex(3, c_dt, tA, tB, M, 4, 16, alpha, A, 16, 0, ALIGNED, 16, 0, beta, ALIGNED, 4, 0,
                  1, None)
    # int32 C only; integral alpha and beta only
    assert call(c_dt=0) == 1 and call(c_dt=3) == 1
    assert call(alpha=0.5) == 1 and call(beta=1.5) == 1 and call(alpha=3e9) == 1
    for tA, tB in ((0, 0), (1, 0), (1, 1)):
        assert call(tA=tA, tB=tB, alpha=0.5) == 1
        assert call(tA=tA, tB=tB, M=0) == 0          # every transpose is legal (nothing to do)
        info, _ = sel("i8", tA, tB, M=4, N=4, K=16, lda=4 if tA else 16, ldb=16 if tB else 4)
        assert info["dtype"] == 3
    # int32 C is for int8 inputs only
    assert ex(0, 4, 0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 0, ALIGNED, 4, 0, 0.0, ALIGNED, 4, 0, 1,
              None) == 1
    # legal calls with nothing to do return OK without touching the GPU
    assert call(M=0) == 0 and call(M=0, alpha=-7.0, beta=2.0) == 0
    info, grid = sel("i8", 0, 1, M=8192, N=8192, K=8192)
    assert info["dtype"] == 3 and grid == 1024 and info["block_k"] == 128


def test_fp64_rules_without_a_gpu():
    lib = mg.load()
    # fp64 has its own entry points (double scalars): the float-scalar ones refuse it
    assert lib.gemm_strided_batched(5, 0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 0, ALIGNED, 4, 0, 0.0,
                                    ALIGNED, 4, 0, 1, None) == 1
    assert lib.gemm_strided_batched_ex(5, 5, 0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 0, ALIGNED, 4, 0,
                                       0.0, ALIGNED, 4, 0, 1, None) == 1
    f64 = lib.gemm_f64
    # C aligned to 8 bytes; A and B to 8 bytes; the usual shape checks
    assert f64(0, 0, 4, 4, 4, 1.0, ALIGNED, 4, ALIGNED, 4, 0.0, ALIGNED + 4, 4, None) == 1
    assert f64(0, 0, 4, 4, 4, 1.0, ALIGNED + 4, 4, ALIGNED, 4, 0.0, ALIGNED, 4, None) == 1
    assert f64(0, 0, 4, 4, 4, 1.0, ALIGNED, 3, ALIGNED, 4, 0.0, ALIGNED, 4, None) == 1
    assert f64(0, 2, 4, 4, 4, 1.0, ALIGNED, 4, ALIGNED, 4, 0.0, ALIGNED, 4, None) == 1
    # a non-float alpha (not representable in fp32) is fine: nothing to do returns OK
    assert f64(0, 0, 0, 4, 4, 1.0 + 2 ** -40, None, 4, None, 4, 0.0, None, 4, None) == 0
    bat = lib.gemm_f64_strided_batched
    assert bat(0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 16, ALIGNED, 4, 16, 0.0, ALIGNED, 4, 15, 2,
               None) == 1                                      # C entries would overlap
    assert bat(0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 0, ALIGNED, 4, 0, 0.0, ALIGNED, 4, 16, 0,
               None) == 0                                      # batch 0: nothing to do
    info, grid = sel("f64", M=4096, N=4096, K=4096)
    assert info["dtype"] == 5 and grid >= 256 and info["block_k"] == 16
    # odd leading dimensions take the 8-byte-load build
    info, _ = sel("f64", M=1000, N=1027, K=999, lda=999, ldb=1027, ldc=1027)
    assert info["name"].endswith("_u")
    info, _ = sel("f64", 1, 1, M=512, N=512, K=512)
    assert not info["name"].endswith("_u")


def test_i8_every_transpose_has_builds():
    # every transpose is accepted; an MN-contiguous operand rules out the 64x64 tiles
    for tA, tB in ((0, 0), (0, 1), (1, 0), (1, 1)):
        for M, N, K in ((64, 64, 256), (1000, 1027, 1024), (8192, 8192, 8192)):
            lda = M if tA else K
            ldb = K if tB else N
            info, _ = sel("i8", tA, tB, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=N)
            assert info["dtype"] == 3
            if (tA, tB) != (0, 1):
                assert info["block_m"] >= 128, (tA, tB, M, N, K, info["name"])
    assert sel("i8", 0, 1, M=64, N=64, K=256, lda=256, ldb=256)[0]["block_m"] == 64


def test_small_problem_choice():
    # the 16x16 small-problem builds take small grids, and only those
    name = lambda M, N, K, **kw: sel(M=M, N=N, K=K, **kw)[0]["name"]
    assert name(256, 256, 256) == "mgemm_f32_16x16_k4w_256"
    assert name(128, 128, 128) == "mgemm_f32_16x16_k4w_256"
    assert name(256, 256, 1024) == "mgemm_f32_16x16_k8w_1024"
    assert name(128, 128, 1024) == "mgemm_f32_16x16_k8w_1024"
    for M, N, K in ((512, 512, 512), (512, 512, 256), (1024, 1024, 256), (256, 256, 2048),
                    (4096, 4096, 4096)):
        assert "16x16" not in name(M, N, K), (M, N, K)
    # unaligned rows: the small build must beat the register path's estimate
    assert "16x16" not in name(4096, 4096, 4096, lda=4097, ldb=4097)
    assert "16x16" not in name(1024, 1024, 1000, lda=2_100_001, ldb=2_100_001)
    assert name(256, 256, 256, lda=257, ldb=257) == "mgemm_f32_16x16_k4w_256"
    # a batch multiplies the workgroups: 64 entries of 256^3 are a large launch
    assert "16x16" not in name(256, 256, 256, batch=64, strideA=256 * 256, strideB=256 * 256,
                               strideC=256 * 256)


def test_force_variant_roundtrip():
    vs = mg.variants()
    f32_ids = [v["id"] for v in vs if v["dtype"] == 0 and v["pipe"] != 6]
    small = [v for v in vs if v["dtype"] == 0 and v["pipe"] == 6]
    bf16_ids = [v["id"] for v in vs if v["dtype"] == 2]
    try:
        mg.force_variant("f32", f32_ids[-1])
        info, _ = sel(M=4096, N=4096, K=4096)
        assert info["id"] == f32_ids[-1]
        # a small-problem build runs forced while K fits its waves' share, not beyond
        for v in small:
            mg.force_variant("f32", v["id"])
            assert sel(M=300, N=200, K=v["block_k"])[0]["id"] == v["id"]
            assert sel(M=300, N=200, K=v["block_k"] + 1)[0]["id"] != v["id"]
            # nor for split-K's chunks (no shorter last chunk of its own)
            assert mg.splitk_plan("f32", 300, 200, 2 * v["block_k"], 4)["variant"]["id"] != v["id"]
        with pytest.raises(mg.MgemmError):
            mg.force_variant("f32", bf16_ids[0])
    finally:
        mg.force_variant("f32", None)
    info, _ = sel(M=4096, N=4096, K=4096)
    assert info["id"] != f32_ids[-1] or len(f32_ids) == 1


def test_entry_points_reject_bad_arguments_without_a_gpu():
    lib = mg.load()
    # negative M: rejected during host validation, before any HIP call
    assert lib.gemm_f32(0, 0, -1, 4, 4, 1.0, ALIGNED, 4, ALIGNED, 4, 0.0, ALIGNED, 4, None) == 1
    assert lib.gemm_bf16(0, 0, 4, 4, 4, 1.0, None, 4, ALIGNED, 4, 0.0, ALIGNED, 4, None) == 1
    assert lib.gemm_f16(0, 1, 4, 4, 4, 1.0, ALIGNED, 4, ALIGNED, 3, 0.0, ALIGNED, 4, None) == 1
    assert lib.gemm_strided_batched(0, 0, 0, 4, 4, 4, 1.0, ALIGNED, 4, 16, ALIGNED, 4, 16, 0.0,
                                    ALIGNED, 4, 15, 2, None) == 1
    # nothing to do: OK with no launch
    assert lib.gemm_f32(0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None) == 0


def test_c_type_rules_without_a_gpu():
    lib = mg.load()
    ex = lib.gemm_strided_batched_ex

    def call(in_dt, c_dt, C=ALIGNED, ldc=4, M=4):
        return ex(in_dt, c_dt, 0, 0, M, 4, 4, 1.0, ALIGNED, 8, 0, ALIGNED, 8, 0, 0.0, C, ldc, 0, 1,
                  None)
    # C is fp32 or the inputs' own 16-bit type; nothing else
    assert call(0, 1) == 1 and call(0, 2) == 1          # fp32 inputs -> 16-bit C
    assert call(1, 2) == 1 and call(2, 1) == 1          # f16 <-> bf16 mix
    assert call(1, 7) == 1
    # a 16-bit C needs 2-byte alignment only; an odd address is rejected
    assert call(1, 1, C=ALIGNED + 1) == 1
    # empty problems return OK without touching the GPU, for every legal pairing
    for in_dt, c_dt in ((0, 0), (1, 0), (1, 1), (2, 0), (2, 2)):
        assert call(in_dt, c_dt, M=0) == 0


def test_binding_refuses_host_tensors_and_short_buffers():
    import torch
    a = torch.zeros(16)
    with pytest.raises(ValueError):
        mg.gemm_f32(0, 0, 4, 4, 4, 1.0, a, 4, a, 4, 0.0, a, 4)


def test_streamk_rules_without_a_gpu():
    lib = mg.load()
    sk = lib.gemm_streamk

    def call(in_dt=0, c_dt=0, M=64, N=64, K=1024, alpha=1.0, beta=0.0, wgs=0, ws=ALIGNED,
             wbytes=1 << 30, tB=0):
        return sk(in_dt, c_dt, 0, tB, M, N, K, alpha, ALIGNED, K, ALIGNED, K if tB else N, beta,
                  ALIGNED, N, wgs, ws, wbytes, None)
    assert call(wgs=-1) == 1
    assert call(ws=None) == 1                                  # a launch needs the workspace
    assert call(ws=ALIGNED + 8) == 1                           # 16-byte alignment
    need = mg.streamk_plan("f32", 64, 64, 1024)["workspace_bytes"]
    assert need == mg.STREAMK_COUNTER_BYTES + 32 * 2 * 64 * 64 * 4   # 1 tile x 32 iterations: 32 workgroups
    assert call(wbytes=need - 1) == 1
    assert call(alpha=1.0 + 2 ** -40) == 1                     # not a float
    assert call(in_dt=1, c_dt=2) == 1                          # fp32 C or the inputs' own type
    assert call(in_dt=0, c_dt=1) == 1                          # fp32 inputs: fp32 C only
    assert call(in_dt=3, c_dt=4, tB=1, alpha=1.5) == 1         # int8: integral alpha
    assert call(in_dt=5, c_dt=0) == 1                          # fp64 inputs: double C only
    assert call(in_dt=5, c_dt=5, ws=ALIGNED + 8) == 1          # fp64: the same workspace rules
    # nothing to do: OK without a workspace
    for in_dt, c_dt, tB in ((0, 0, 0), (2, 0, 0), (2, 2, 0), (1, 1, 0), (3, 4, 1), (5, 5, 0)):
        assert call(in_dt, c_dt, M=0, ws=None, wbytes=0, tB=tB) == 0
    assert call(5, 5, M=0, alpha=1.0 + 2 ** -40, ws=None, wbytes=0) == 0   # fp64 takes doubles


def test_splitk_rules_without_a_gpu():
    lib = mg.load()
    sk = lib.gemm_splitk

    def call(in_dt=0, c_dt=0, M=64, N=64, K=1024, alpha=1.0, beta=0.0, splits=4, ws=ALIGNED,
             wbytes=1 << 30):
        return sk(in_dt, c_dt, 0, 0, M, N, K, alpha, ALIGNED, K, ALIGNED, N, beta, ALIGNED, N,
                  splits, ws, wbytes, None)
    assert call(splits=-1) == 1
    assert call(ws=None) == 1                                  # chunks > 1 need a workspace
    assert call(ws=ALIGNED + 8) == 1                           # 16-byte alignment
    need = mg.splitk_workspace_bytes("f32", 64, 64, 1024, 4)
    assert need == 4 * 64 * 64 * 4
    assert call(wbytes=need - 1) == 1
    assert call(alpha=1.0 + 2 ** -40) == 1                     # not a float: refused for fp32
    assert call(in_dt=1, c_dt=2) == 1                          # C type rules as the _ex entry point
    assert call(in_dt=3, c_dt=0) == 1                          # int8 needs int32 C
    # nothing to do: OK without a workspace, for every input type
    for in_dt, c_dt in ((0, 0), (1, 1), (2, 0), (5, 5)):
        assert call(in_dt, c_dt, M=0, ws=None, wbytes=0) == 0
    assert call(5, 5, M=0, alpha=1.0 + 2 ** -40, ws=None, wbytes=0) == 0   # fp64 takes doubles
    # chunk planning: whole K-slabs, the automatic count fills the device
    assert mg.splitk_chunks("f32", 512, 512, 4096, 0) == 8     # 16 tiles, chunks >= 512 deep
    assert mg.splitk_chunks("f32", 256, 256, 8192, 0) == 16
    assert mg.splitk_chunks("f32", 4096, 4096, 4096, 0) == 1   # already fills 256 CUs
    assert mg.splitk_chunks("f32", 64, 64, 100, 8) == 4        # 32-deep slabs: 100 -> 4 chunks
    assert mg.splitk_chunks("bf16", 64, 64, 1000, 3) == 3
    assert mg.splitk_chunks("i8", 64, 64, 1000, 16, transB=1) == 8   # 128-byte slabs
    assert mg.splitk_workspace_bytes("f64", 100, 50, 1000, 4) == 4 * 100 * 50 * 8
    assert mg.splitk_workspace_bytes("i8", 100, 50, 1024, 2, transB=1) == 2 * 100 * 50 * 4
    assert mg.splitk_workspace_bytes("f32", 100, 50, 1000, 1) == 0
    info = _lib.SplitkPlanInfo()
    assert lib.mgemm_splitk_plan(0, 0, 0, 4, 4, 4, ALIGNED, 4, ALIGNED, 4, -1, ctypes.byref(info)) == 1
    assert lib.mgemm_splitk_plan(0, 0, 0, 4, 4, 4, ALIGNED, 4, ALIGNED, 4, 0, None) == 1


def test_streamk_plans():
    # the ragged shape: 16 x 17 tiles of the 4-byte-copy 64x64 build, 32 iterations of 32,
    # shared by 512 workgroups (two per CU), two fp32 partial tiles each
    p = mg.streamk_plan("f32", 1000, 1027, 999, lda=999, ldb=1027)
    assert p["variant"]["name"] == "mgemm_f32_64x64x32_w2x2_d4_u"
    assert (p["tiles"], p["iterations"], p["k_per_iteration"], p["workgroups"]) == (272, 32, 32, 512)
    # the arrival counters first (a fixed prefix), then the partial tiles
    assert mg.STREAMK_COUNTER_BYTES == 64 << 10 and mg.STREAMK_MAX_WORKGROUPS * 4 <= mg.STREAMK_COUNTER_BYTES
    assert p["workspace_bytes"] == mg.STREAMK_COUNTER_BYTES + 512 * 2 * 64 * 64 * 4
    # an explicit count, the cap of one workgroup per (tile, iteration) pair, and the cap
    # of one arrival counter per workgroup
    assert mg.streamk_plan("f32", 1000, 1027, 999, 37, lda=999, ldb=1027)["workgroups"] == 37
    assert mg.streamk_plan("f32", 4096, 4096, 4096, 10 ** 6)["workgroups"] == mg.STREAMK_MAX_WORKGROUPS
    one = mg.streamk_plan("f32", 64, 64, 300, 1000)
    assert (one["tiles"], one["iterations"], one["workgroups"]) == (1, 10, 10)
    # the K-iteration is the type's K granule
    assert mg.streamk_plan("bf16", 500, 500, 500)["k_per_iteration"] == 64
    i8 = mg.streamk_plan("i8", 1000, 1027, 999, transB=1)
    assert i8["k_per_iteration"] == 128
    assert i8["workspace_bytes"] == (mg.STREAMK_COUNTER_BYTES +
                                     512 * 2 * i8["variant"]["block_m"] * i8["variant"]["block_n"] * 4)
    # rows of any alignment have a stream-K build (the register path)
    assert mg.streamk_plan("bf16", 1000, 1027, 999, lda=999, ldb=1027)["variant"]["name"].endswith("_u")
    # no tile of 256x256 takes stream-K: a large aligned problem gets a smaller build
    assert mg.streamk_plan("f32", 4096, 4096, 4096)["variant"]["block_m"] <= 128
    # nothing launched: no workspace
    for M, K in ((0, 64), (64, 0)):
        z = mg.streamk_plan("f32", M, 64, K, lda=max(K, 1))
        assert z["workspace_bytes"] == 0 and z["variant"]["id"] == -1
    # fp64: 16-deep iterations and double partial tiles; 16-byte rows take the vector builds
    f64 = mg.streamk_plan("f64", 1000, 1027, 999, lda=1000, ldb=1028)
    assert f64["k_per_iteration"] == 16 and f64["iterations"] == 63
    assert not f64["variant"]["name"].endswith("_u")
    assert f64["workspace_bytes"] == (mg.STREAMK_COUNTER_BYTES +
                                      512 * 2 * f64["variant"]["block_m"] * f64["variant"]["block_n"] * 8)
    assert mg.streamk_plan("f64", 1000, 1027, 999, lda=999, ldb=1027)["variant"]["name"].endswith("_u")
    with pytest.raises(mg.MgemmError):
        mg.streamk_plan("f32", 100, 100, 100, -1)
    # int8 with an MN-contiguous operand: the 128x128 tiles (transposing LDS reads)
    for tA, tB in ((0, 0), (1, 0), (1, 1)):
        assert mg.streamk_plan("i8", 100, 100, 128, transA=tA, transB=tB)["variant"]["block_m"] == 128


def test_splitk_automatic_plans():
    # a small grid of unaligned tiles: three chunks of all of C
    p = mg.splitk_plan("f32", 1000, 1027, 999, 0, lda=999, ldb=1027)
    assert p["chunks"] == 3 and p["chunk_len"] == 352
    assert p["variant"]["name"].endswith("_u") and p["grid"] == 3 * 16 * 17
    assert p["workspace_bytes"] == 3 * 1000 * 1027 * 4
    # the same shape with aligned rows stays one pass (the DMA path hides its loads)
    assert mg.splitk_plan("f32", 1024, 1024, 1024, 0)["chunks"] == 1
    assert mg.splitk_plan("f64", 1024, 1024, 1024, 0)["chunks"] == 1
    # short tiles (16-bit) are not worth two extra launches
    assert mg.splitk_plan("bf16", 1000, 1027, 999, 0, lda=999, ldb=1027)["chunks"] == 1
    # deep K: enough chunks for 256 workgroups
    d = mg.splitk_plan("f32", 256, 256, 8192, 0)
    assert d["chunks"] == 16 and d["grid"] == 256
    # big grids stay one pass; the plan then names the plain kernel
    b = mg.splitk_plan("f32", 4096, 4096, 4096, 0)
    assert b["chunks"] == 1 and b["workspace_bytes"] == 0
    assert b["variant"]["name"] == "mgemm_f32_256x256x32_w4x2" and b["grid"] == 256
    # explicit counts; 1 is the plain kernel
    assert mg.splitk_plan("f32", 1000, 1027, 999, 4)["chunks"] == 4
    assert mg.splitk_plan("f32", 1000, 1027, 999, 1)["chunks"] == 1


def test_splitk_one_stage_needs_whole_chunks_of_k():
    # The one-stage (pipe 3) builds have no register path, so every chunk's K must be a
    # multiple of the 16-byte piece.  Chunks are whole 64-deep slabs and the last takes the
    # rest: with K = 196 the last chunk is 4 deep, and the plan must not pick them.
    p = mg.splitk_plan("f16", 2048, 2048, 196, 4, transB=1, lda=200, ldb=200)
    assert p["chunks"] == 4 and p["chunk_len"] == 64
    assert not p["variant"]["name"].endswith("_s1")
    # with K a multiple of 8 every chunk, the last one included, is whole pieces
    q = mg.splitk_plan("f16", 2048, 2048, 200, 4, transB=1, lda=200, ldb=200)
    assert q["chunks"] == 4 and q["chunk_len"] == 64
    assert q["variant"]["name"].endswith("_s1")


def test_noalloc_refuses_sizes_beyond_its_scratch_without_a_gpu():
    # the plan is checked before any device call: 4 chunks of 4096 x 4096 fp32 partial sums
    # (256 MiB) exceed the fixed scratch, bad arguments are refused as in gemm_splitk
    lib = mg.load()
    na = lib.gemm_splitk_noalloc
    M = N = K = 4096
    assert 4 * M * N * 4 > mg.NOALLOC_SCRATCH_BYTES
    assert na(0, 0, 0, 0, M, N, K, 1.0, ALIGNED, K, ALIGNED, N, 0.0, ALIGNED, N, 4, None) == 3
    assert na(0, 0, 0, 0, M, N, K, 1.0, ALIGNED, K - 1, ALIGNED, N, 0.0, ALIGNED, N, 4, None) == 1
    assert na(0, 0, 0, 0, 64, 64, 1024, 1.0 + 2 ** -40, ALIGNED, 1024, ALIGNED, 64, 0.0, ALIGNED,
              64, 4, None) == 1
    assert na(0, 0, 0, 0, 0, 64, 1024, 1.0, ALIGNED, 1024, ALIGNED, 64, 0.0, ALIGNED, 64, 4,
              None) == 0                                       # nothing to do
    assert "SCRATCH" in mg.status_string(3)
    with open(HEADER) as f:
        assert "#define MGEMM_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)" in f.read()
    assert mg.NOALLOC_SCRATCH_BYTES == 64 << 20


_DISASM = {}


def device_instructions():
    """{code object: [instruction, ...]} of the built library's gfx950 code (our own
    build), disassembled once."""
    if not _DISASM:
        import shutil
        import tempfile
        objdump = "/opt/rocm/llvm/bin/llvm-objdump"
        if not os.path.exists(objdump):
            pytest.skip("llvm-objdump not installed")
        with tempfile.TemporaryDirectory() as d:
            lib = os.path.join(d, "libmgemm.so")
            shutil.copy(_lib.LIB_PATH, lib)
            subprocess.run([objdump, "--offloading", lib], capture_output=True, check=True, cwd=d)
            objs = sorted(f for f in os.listdir(d) if "amdgcn" in f)
            assert objs, "no device code objects in the library"
            for o in objs:
                text = subprocess.run([objdump, "-d", "--no-show-raw-insn", os.path.join(d, o)],
                                      capture_output=True, text=True, check=True).stdout
                ins = []
                for line in text.splitlines():
                    t = line.strip()
                    if not t or t.endswith(":") or t.startswith(("/", ";", "Disassembly")):
                        continue
                    ins.append(t.split("//")[0].strip())
                _DISASM[o] = ins
    return _DISASM


def test_every_lds_copy_in_the_library_opens_with_its_wait_states(built_library):
    # The copies global -> LDS are inline asm, where the compiler inserts no wait states:
    # each must open with s_nop 4, so that a v_readfirstlane that formed one of its scalar
    # operands (the row offset, M0, the buffer resource) is five wait states behind it.
    # Without them an interior-tile prologue loaded 1 KB of B from a stale offset.
    copies = 0
    for o, ins in device_instructions().items():
        prev = ""
        for i in ins:
            if i.startswith("buffer_load") and i.endswith(" lds"):
                copies += 1
                assert prev == "s_nop 4", f"{o}: '{i}' follows '{prev}'"
            prev = i
    assert copies > 1000


def test_atomics_in_the_library_are_vector_memory_ones(built_library):
    # stream-K's arrival counters are the library's only atomics: one wrapping increment
    # per split-tile contribution, through the vector memory path
    found = set()
    for o, ins in device_instructions().items():
        for i in ins:
            op = i.split()[0]
            if "atomic" in op:
                found.add(op)
    assert found == {"global_atomic_inc"}, found
