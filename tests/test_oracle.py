"""Pins for the CPU oracle, each tied to something other than the oracle itself.

Every test here runs on the CPU.  Which mistake each pin would catch:
- golden worked examples from the pages        -> a wrong sum, a wrong element
- exact integer products against numpy int64   -> dropped / extra terms, wrong index,
                                                  transposed operand, wrong ld or stride
- 16-bit decoders against numpy / torch        -> a wrong exponent bias or subnormal rule
- identity / permutation / zero / all-ones     -> sign, alpha/beta and index slips
- beta == 0 with NaN C, NaN padding            -> reading C or padding that must stay unread
- float products against numpy float64 and the exact rational value -> rounding far
                                                  beyond one fp64 summation
- planted mistakes                             -> the pins above really fail on a broken oracle
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_f32_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = [float(t) for t in v.split()]
    return vals


def f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def run(A, B, M, N, K, transA=False, transB=False, alpha=1.0, beta=0.0, C=None,
        lda=None, ldb=None, ldc=None, dtype="f32", gemm=None):
    gemm = gemm or oracle.gemm
    lda = lda or (M if transA else K)
    ldb = ldb or (K if transB else N)
    ldc = ldc or N
    out = gemm(dtype, transA, transB, M, N, K, alpha, A.ravel(), lda, B.ravel(), ldb,
               beta, None if C is None else C.ravel(), ldc)
    return out[0]


# ---------------------------------------------------------------- golden examples

def test_golden_dot_example():
    g = read_golden("dlog_matmul_dot_example.txt")
    out = run(f32(g["a"]), f32(g["b"]), 1, 1, 2)
    assert out[0, 0] == g["product"][0]


def test_golden_inner_and_outer_product_example():
    g = read_golden("dlog_matmul_outer_product_example.txt")
    A = f32(g["A"]).reshape(2, 2)
    B = f32(g["B"]).reshape(2, 2)
    full = run(A, B, 2, 2, 2)
    assert full[0, 0] == g["inner_product_C00"][0]
    # k = 0 rank-1 term: column 0 of A times row 0 of B (K = 1 GEMM)
    r0 = run(f32(A[:, :1]), f32(B[:1, :]), 2, 2, 1)
    assert r0.ravel().tolist() == g["outer_product_k0"]
    # sum of the rank-1 terms over k equals the product
    r1 = run(f32(A[:, 1:]), f32(B[1:, :]), 2, 2, 1)
    assert np.array_equal(r0 + r1, full)


# ---------------------------------------------------------------- exact integer products

def _int_case(rng, M, N, K, transA, transB, lo=-50, hi=50):
    Al = rng.integers(lo, hi + 1, size=(M, K))
    Bl = rng.integers(lo, hi + 1, size=(K, N))
    A = Al.T if transA else Al
    B = Bl.T if transB else Bl
    return Al, Bl, f32(A), f32(B)


def test_tiny_all_shapes_all_trans_exact():
    rng = np.random.default_rng(7)
    for M, N, K in itertools.product(range(1, 6), repeat=3):
        for tA, tB in itertools.product((False, True), repeat=2):
            Al, Bl, A, B = _int_case(rng, M, N, K, tA, tB)
            out = run(A, B, M, N, K, tA, tB)
            assert np.array_equal(out, (Al @ Bl).astype(np.float64)), (M, N, K, tA, tB)


@pytest.mark.parametrize("M,N,K", [(47, 53, 804),    # CSDN tile page: A 47x804, B 804x53
                                   (100, 300, 200),  # dlog mm example (100,200)x(200,300)
                                   (97, 131, 257)])
@pytest.mark.parametrize("tA,tB", list(itertools.product((False, True), repeat=2)))
def test_integer_products_match_numpy_int64(M, N, K, tA, tB):
    rng = np.random.default_rng(M * 7 + N)
    Al, Bl, A, B = _int_case(rng, M, N, K, tA, tB, 0, 99)
    out = run(A, B, M, N, K, tA, tB)
    assert np.array_equal(out, (Al @ Bl).astype(np.float64))


def test_alpha_beta_integer_closed_form():
    rng = np.random.default_rng(3)
    M, N, K = 33, 29, 41
    Al, Bl, A, B = _int_case(rng, M, N, K, False, False, -7, 7)
    C0 = rng.integers(-9, 10, size=(M, N))
    out = run(A, B, M, N, K, alpha=1.5, beta=0.5, C=f32(C0))
    # half-integers well inside 2^52: exact in fp64
    assert np.array_equal(out, 1.5 * (Al @ Bl) + 0.5 * C0)


def test_leading_dims_and_nan_padding_never_read():
    rng = np.random.default_rng(11)
    M, N, K = 13, 17, 19
    Al, Bl, _, _ = _int_case(rng, M, N, K, False, False)
    lda, ldb, ldc = K + 5, N + 3, N + 7
    A = np.full((M, lda), np.nan, np.float32); A[:, :K] = Al
    B = np.full((K, ldb), np.nan, np.float32); B[:, :N] = Bl
    C = np.full((M, ldc), np.nan, np.float32)
    out = run(A, B, M, N, K, lda=lda, ldb=ldb, ldc=ldc, C=C, beta=0.0)
    assert np.array_equal(out, (Al @ Bl).astype(np.float64))


def test_batched_strides_match_per_slice():
    rng = np.random.default_rng(5)
    M, N, K, batch = 9, 11, 7, 4
    sA, sB, sC = M * K + 3, N * K + 5, M * N + 2
    A = f32(rng.integers(-9, 10, size=(batch - 1) * sA + M * K))
    B = f32(rng.integers(-9, 10, size=(batch - 1) * sB + N * K))
    C = f32(rng.integers(-9, 10, size=(batch - 1) * sC + M * N))
    out = oracle.gemm("f32", False, True, M, N, K, 2.0, A, K, B, K, -1.0, C, N,
                      batch=batch, strideA=sA, strideB=sB, strideC=sC)
    for b in range(batch):
        Ab = A[b * sA:b * sA + M * K].reshape(M, K).astype(np.int64)
        Bb = B[b * sB:b * sB + N * K].reshape(N, K).astype(np.int64)
        Cb = C[b * sC:b * sC + M * N].reshape(M, N).astype(np.int64)
        assert np.array_equal(out[b], (2 * (Ab @ Bb.T) - Cb).astype(np.float64))


# ---------------------------------------------------------------- special matrices

def test_identity_permutation_zero_ones():
    rng = np.random.default_rng(9)
    n = 24
    X = f32(rng.uniform(-1, 1, size=(n, n)))
    C0 = f32(rng.uniform(-1, 1, size=(n, n)))
    I = f32(np.eye(n))
    # I*X and X*I return X exactly (one nonzero product per element)
    assert np.array_equal(run(I, X, n, n, n), X.astype(np.float64))
    assert np.array_equal(run(X, I, n, n, n), X.astype(np.float64))
    # permutations move rows / columns bit for bit
    perm = rng.permutation(n)
    P = f32(np.eye(n)[perm])
    assert np.array_equal(run(P, X, n, n, n), X[perm].astype(np.float64))
    assert np.array_equal(run(X, P, n, n, n), (X @ P.astype(np.float64)))
    # A = 0 -> beta*C0 ; alpha = 0 -> beta*C0 (fp64 product of two fp32 is exact)
    Z = f32(np.zeros((n, n)))
    want = 0.25 * C0.astype(np.float64)
    assert np.array_equal(run(Z, X, n, n, n, alpha=3.0, beta=0.25, C=C0), want)
    assert np.array_equal(run(X, X, n, n, n, alpha=0.0, beta=0.25, C=C0), want)
    # all ones -> alpha*K + beta*C0
    K = 37
    ones_a, ones_b = f32(np.ones((n, K))), f32(np.ones((K, n)))
    assert np.array_equal(run(ones_a, ones_b, n, n, K, alpha=-2.0, beta=1.0, C=C0),
                          -2.0 * K + C0.astype(np.float64))


def test_beta_zero_ignores_nan_c_and_empty_k():
    rng = np.random.default_rng(1)
    M, N, K = 6, 5, 4
    A, B = f32(rng.uniform(-1, 1, (M, K))), f32(rng.uniform(-1, 1, (K, N)))
    Cnan = f32(np.full((M, N), np.nan))
    out = run(A, B, M, N, K, C=Cnan, beta=0.0)
    assert not np.isnan(out).any()
    C0 = f32(rng.uniform(-1, 1, (M, N)))
    e = np.zeros(0, np.float32)
    out0 = oracle.gemm("f32", False, False, M, N, 0, 1.0, e, 1, e, N, 0.5, C0.ravel(), N)[0]
    assert np.array_equal(out0, 0.5 * C0.astype(np.float64))


# ---------------------------------------------------------------- 16-bit decoding

def test_f16_decoder_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_bf16_decoder_matches_torch_for_every_pattern():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    want = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.tolist()])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16bit_gemm_matches_float64_of_stored_values(dtype):
    p = wl.Problem(dtype, 21, 19, 37, transA=True, transB=False, dist="normal", seed=4)
    A, B, _ = wl.make_inputs(p)
    An, Bn = wl.to_numpy_operand(A), wl.to_numpy_operand(B)
    out = oracle.gemm(dtype, True, False, p.M, p.N, p.K, 1.0, An, p.lda, Bn, p.ldb, 0.0,
                      None, p.ldc)[0]
    Ad = A.to(torch.float64).numpy().reshape(p.K, p.M).T
    Bd = B.to(torch.float64).numpy().reshape(p.K, p.N)
    np.testing.assert_allclose(out, Ad @ Bd, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- float products

def test_float_products_against_numpy_float64():
    rng = np.random.default_rng(21)
    M, N, K = 64, 48, 300
    A, B = f32(rng.uniform(-1, 1, (M, K))), f32(rng.uniform(-1, 1, (K, N)))
    out = run(A, B, M, N, K)
    want = A.astype(np.float64) @ B.astype(np.float64)
    bound = K * np.finfo(np.float64).eps * (np.abs(A).astype(np.float64) @ np.abs(B))
    assert np.all(np.abs(out - want) <= 2 * bound)


def test_float_products_against_exact_rationals():
    rng = np.random.default_rng(22)
    for M, N, K in [(1, 1, 1), (2, 3, 4), (3, 2, 7), (4, 4, 4)]:
        A, B = f32(rng.uniform(-1, 1, (M, K))), f32(rng.uniform(-1, 1, (K, N)))
        C0 = f32(rng.uniform(-1, 1, (M, N)))
        out = run(A, B, M, N, K, alpha=1.5, beta=-0.75, C=C0)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
                exact = Fraction(1.5) * sum(terms) + Fraction(-0.75) * Fraction(float(C0[i, j]))
                mag = 1.5 * sum(abs(float(t)) for t in terms) + 0.75 * abs(float(C0[i, j]))
                assert abs(float(Fraction(out[i, j]) - exact)) <= (K + 2) * 2.0 ** -52 * mag


def test_elems_matches_full_output_bitwise():
    p = wl.Problem("f32", 37, 41, 53, transB=True, batch=3, alpha=1.5, beta=0.5,
                   dist="uniform", seed=8)
    A, B, C = wl.make_inputs(p)
    An, Bn, Cn = A.numpy(), B.numpy(), C.numpy()
    kw = dict(batch=p.batch, strideA=p.strideA, strideB=p.strideB, strideC=p.strideC)
    full = oracle.gemm("f32", False, True, p.M, p.N, p.K, p.alpha, An, p.lda, Bn, p.ldb,
                       p.beta, Cn, p.ldc, **kw)
    rng = np.random.default_rng(0)
    b, i, j = (rng.integers(0, p.batch, 200), rng.integers(0, p.M, 200), rng.integers(0, p.N, 200))
    el = oracle.gemm_elems("f32", False, True, p.M, p.N, p.K, p.alpha, An, p.lda, Bn, p.ldb,
                           p.beta, Cn, p.ldc, b, i, j, **kw)
    assert np.array_equal(el, full[b, i, j])


def _finite_positive(decoded):
    """Sorted positive finite values of a 16-bit format and their bit patterns."""
    bits = np.arange(1, 0x8000, dtype=np.uint16)
    vals = decoded(bits)
    keep = np.isfinite(vals)
    return vals[keep], bits[keep]


def _round_cases(vals, rng):
    mids = (vals[:-1] + vals[1:]) / 2          # exact ties
    return np.concatenate([
        vals, -vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        rng.standard_normal(20000) * 10.0 ** rng.integers(-45, 40, 20000),
        [0.0, -0.0, vals[-1] * 1.001, vals[-1] * 2, vals[0] / 2, vals[0] / 2 * 1.0001, vals[0] / 3]])


def test_round_to_f16_matches_numpy_conversion():
    # binary16 output rounding: numpy's float64 -> float16 conversion rounds to nearest even
    rng = np.random.default_rng(21)
    vals, _ = _finite_positive(lambda b: b.view(np.float16).astype(np.float64))
    x = _round_cases(vals, rng)
    x = x[np.abs(x) < 1e6]
    got = oracle.round16("f16", x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    # the ties include both directions, so truncation would fail this pin
    mids = (vals[:-1] + vals[1:]) / 2
    assert np.any(oracle.round16("f16", mids) == np.arange(2, 0x7c00, dtype=np.uint16)[:mids.size])


def test_round_to_bf16_matches_brute_force_nearest():
    # bfloat16 output rounding against the nearest representable value found by
    # search over every finite pattern (decoded by torch), ties to the even pattern
    rng = np.random.default_rng(22)
    dec = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    vals, bits = _finite_positive(dec)
    order = np.argsort(vals)
    vals, bits = vals[order], bits[order]
    x = _round_cases(vals, rng)
    a = np.abs(x)
    ulp_top = vals[-1] - vals[-2]
    hi = np.searchsorted(vals, a)               # first value >= a
    want = np.empty(x.size, np.uint16)
    for e, (ae, h) in enumerate(zip(a, hi)):
        if ae == 0:
            w = 0
        elif ae >= vals[-1] + ulp_top / 2:
            w = 0x7f80                           # past the top by half an ulp: infinity
        elif h == 0:                             # below the smallest subnormal
            w = bits[0] if ae > vals[0] / 2 else (bits[0] if (ae == vals[0] / 2 and bits[0] % 2 == 0) else 0)
        elif h == vals.size:
            w = bits[-1]
        else:
            lo_v, hi_v = vals[h - 1], vals[h]
            d_lo, d_hi = ae - lo_v, hi_v - ae
            if d_lo < d_hi:
                w = bits[h - 1]
            elif d_hi < d_lo:
                w = bits[h]
            else:
                w = bits[h - 1] if bits[h - 1] % 2 == 0 else bits[h]
        want[e] = w | (0x8000 if np.signbit(x[e]) else 0)
    got = oracle.round16("bf16", x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("tA,tB", [(False, False), (False, True), (True, False), (True, True)])
def test_int8_products_match_numpy_int64(tA, tB):
    # int8 inputs over their whole range, int32 C with integral alpha and beta
    rng = np.random.default_rng(31)
    M, N, K = 37, 29, 301
    A = rng.integers(-128, 128, (K, M) if tA else (M, K)).astype(np.int8)
    B = rng.integers(-128, 128, (N, K) if tB else (K, N)).astype(np.int8)
    C = rng.integers(-2 ** 31, 2 ** 31, (M, N)).astype(np.int32)
    out = oracle.gemm("i8", tA, tB, M, N, K, -3.0, A.ravel(), A.shape[1], B.ravel(), B.shape[1],
                      5.0, C.ravel(), N)[0]
    opA = (A.T if tA else A).astype(np.int64)
    opB = (B.T if tB else B).astype(np.int64)
    want = -3 * (opA @ opB) + 5 * C.astype(np.int64)
    assert np.array_equal(out, want.astype(np.float64))
    wrapped = oracle.wrap_i32(out)
    assert np.array_equal(wrapped.astype(np.int64), ((want + 2 ** 31) % 2 ** 32) - 2 ** 31)


def test_wrap_to_int32_closed_form():
    x = np.array([0, 1, -1, 2 ** 31 - 1, 2 ** 31, -2 ** 31, -2 ** 31 - 1, 2 ** 32, 2 ** 32 + 7,
                  -2 ** 40 - 3, 2 ** 52 + 1], dtype=np.float64)
    want = np.array([0, 1, -1, 2 ** 31 - 1, -2 ** 31, -2 ** 31, 2 ** 31 - 1, 0, 7, -3, 1],
                    dtype=np.int32)
    assert np.array_equal(oracle.wrap_i32(x), want)
    with pytest.raises(ValueError):
        oracle.wrap_i32(np.array([0.5]))
    with pytest.raises(ValueError):
        oracle.wrap_i32(np.array([2.0 ** 60]))


def test_thread_count_changes_no_bit():
    p = wl.Problem("bf16", 67, 45, 129, transA=True, alpha=0.75, beta=-2.0, dist="normal",
                   c_dist="uniform", seed=9)
    A, B, C = wl.make_inputs(p)
    An, Bn = wl.to_numpy_operand(A), wl.to_numpy_operand(B)
    args = ("bf16", True, False, p.M, p.N, p.K, p.alpha, An, p.lda, Bn, p.ldb, p.beta,
            C.numpy(), p.ldc)
    before = oracle.max_threads()
    try:
        oracle.set_threads(1)
        one = oracle.gemm(*args)
        oracle.set_threads(max(4, before))
        many = oracle.gemm(*args)
    finally:
        oracle.set_threads(before)
    assert np.array_equal(one, many)


def test_bad_arguments_rejected():
    a = f32(np.ones(4))
    with pytest.raises(ValueError):
        oracle.gemm("f32", False, False, 2, 2, 2, 1.0, a, 1, a, 2, 0.0, None, 2)  # lda < K
    with pytest.raises(ValueError):
        oracle.gemm("f32", False, False, 2, 2, 2, 1.0, a, 2, a, 2, 1.0, None, 2)  # C missing


# ---------------------------------------------------------------- planted mistakes

def _pins_hold(gemm):
    """A compact subset of the pins above, run against a given oracle callable."""
    rng = np.random.default_rng(99)
    try:
        for tA, tB in itertools.product((False, True), repeat=2):
            Al, Bl, A, B = _int_case(rng, 7, 5, 9, tA, tB)
            if not np.array_equal(run(A, B, 7, 5, 9, tA, tB, gemm=gemm),
                                  (Al @ Bl).astype(np.float64)):
                return False
        C0 = f32(rng.integers(-5, 5, (4, 4)))
        Z = f32(np.zeros((4, 4)))
        if not np.array_equal(run(Z, Z, 4, 4, 4, beta=0.5, C=C0, gemm=gemm), 0.5 * C0):
            return False
    except Exception:
        return False
    return True


def test_pins_catch_planted_mistakes():
    assert _pins_hold(oracle.gemm)

    def drop_last_k(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, **kw):
        return oracle.gemm(dtype, tA, tB, M, N, max(K - 1, 0), alpha, A, lda, B, ldb,
                           beta, C, ldc, **kw)

    def ignore_trans_b(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, **kw):
        return oracle.gemm(dtype, tA, False, M, N, K, alpha, A, lda, B, N,
                           beta, C, ldc, **kw)

    def negated_beta(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, **kw):
        return oracle.gemm(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, -beta, C, ldc, **kw)

    for broken in (drop_last_k, ignore_trans_b, negated_beta):
        assert not _pins_hold(broken), broken.__name__


def test_workload_generators_are_seeded_and_shaped():
    p = wl.sgemm_ragged()
    A1, B1, C1 = wl.make_inputs(p)
    A2, B2, _ = wl.make_inputs(p)
    assert torch.equal(A1, A2) and torch.equal(B1, B2) and C1 is None
    assert A1.numel() == 1000 * 999 and B1.numel() == 999 * 1027
    assert float(A1.min()) >= 0 and float(A1.max()) <= 99 and torch.all(A1 == A1.round())
    q = wl.qkt_batched()
    assert (q.strideA, q.strideB, q.strideC, q.lda, q.ldb, q.ldc) == (
        65536, 65536, 1048576, 64, 64, 1024)
    assert q.alpha == 0.125


# ---------------------------------------------------------------- double operands

def _exact_f64(A, B, C, alpha, beta, tA, tB):
    """alpha * op(A) op(B) + beta * C in exact rational arithmetic, rounded once to double."""
    opA = A.T if tA else A
    opB = B.T if tB else B
    M, K = opA.shape
    N = opB.shape[1]
    out = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            acc = sum(Fraction(float(opA[i, k])) * Fraction(float(opB[k, j])) for k in range(K))
            v = Fraction(alpha) * acc
            if beta != 0.0:
                v += Fraction(beta) * Fraction(float(C[i, j]))
            out[i, j] = float(v)        # Fraction -> float rounds to nearest
    return out


@pytest.mark.parametrize("tA,tB", list(itertools.product((False, True), repeat=2)))
def test_f64_equals_exact_rational_rounded_once(tA, tB):
    # full 53-bit significands of mixed magnitude, alpha/beta not representable in fp32
    rng = np.random.default_rng(41)
    M, N, K = 9, 7, 33
    A = rng.standard_normal((K, M) if tA else (M, K)) * np.exp2(rng.integers(-20, 20, (K, M) if tA else (M, K)))
    B = rng.standard_normal((N, K) if tB else (K, N))
    C = rng.standard_normal((M, N))
    alpha, beta = 1.0 + 2.0 ** -40, -0.3
    got = oracle.gemm("f64", tA, tB, M, N, K, alpha, A.ravel(), A.shape[1], B.ravel(), B.shape[1],
                      beta, C.ravel(), N)[0]
    assert np.array_equal(got, _exact_f64(A, B, C, alpha, beta, tA, tB))


def test_f64_accumulates_beyond_double_precision():
    # 2^60 + 1 - 2^60: a double accumulator loses the 1, the definition keeps it
    A = np.array([[2.0 ** 60, 1.0, -(2.0 ** 60)]])
    B = np.ones((3, 1))
    got = oracle.gemm("f64", False, False, 1, 1, 3, 1.0, A.ravel(), 3, B.ravel(), 1, 0.0, None, 1)
    assert got[0, 0, 0] == 1.0
    # a product whose low half lies below a double's ulp: (1 + 2^-30)^2 - 1 - 2^-29 = 2^-60
    x = 1.0 + 2.0 ** -30
    A = np.array([[x, -1.0, -(2.0 ** -29)]])
    B = np.array([[x], [1.0], [1.0]])
    got = oracle.gemm("f64", False, False, 1, 1, 3, 1.0, A.ravel(), 3, B.ravel(), 1, 0.0, None, 1)
    assert got[0, 0, 0] == 2.0 ** -60


@pytest.mark.parametrize("tA,tB", list(itertools.product((False, True), repeat=2)))
def test_f64_integer_products_match_numpy_int64(tA, tB):
    rng = np.random.default_rng(43)
    M, N, K = 23, 31, 77
    Ai = rng.integers(-2 ** 20, 2 ** 20, (K, M) if tA else (M, K))
    Bi = rng.integers(-2 ** 20, 2 ** 20, (N, K) if tB else (K, N))
    Ci = rng.integers(-2 ** 40, 2 ** 40, (M, N))
    got = oracle.gemm("f64", tA, tB, M, N, K, 3.0, Ai.astype(np.float64).ravel(), Ai.shape[1],
                      Bi.astype(np.float64).ravel(), Bi.shape[1], -2.0,
                      Ci.astype(np.float64).ravel(), N)[0]
    want = 3 * ((Ai.T if tA else Ai) @ (Bi.T if tB else Bi)) - 2 * Ci   # |want| < 2^53
    assert np.abs(want).max() < 2 ** 53
    assert np.array_equal(got, want.astype(np.float64))


def test_f64_batched_strides_padding_and_elems():
    rng = np.random.default_rng(45)
    M, N, K, batch, lda, ldb, ldc = 6, 5, 11, 3, 13, 7, 9
    sA, sB, sC = M * lda + 4, K * ldb + 2, M * ldc + 1
    A = np.full(batch * sA, np.nan)
    B = np.full(batch * sB, np.nan)
    C = np.full(batch * sC, np.nan)
    Al = rng.integers(-9, 9, (batch, M, K)).astype(np.float64)
    Bl = rng.integers(-9, 9, (batch, K, N)).astype(np.float64)
    Cl = rng.integers(-9, 9, (batch, M, N)).astype(np.float64)
    for b in range(batch):
        for i in range(M):
            A[b * sA + i * lda:b * sA + i * lda + K] = Al[b, i]
            C[b * sC + i * ldc:b * sC + i * ldc + N] = Cl[b, i]
        for k in range(K):
            B[b * sB + k * ldb:b * sB + k * ldb + N] = Bl[b, k]
    out = oracle.gemm("f64", False, False, M, N, K, 0.5, A, lda, B, ldb, 2.0, C, ldc,
                      batch=batch, strideA=sA, strideB=sB, strideC=sC)
    want = 0.5 * np.einsum("bik,bkj->bij", Al, Bl) + 2.0 * Cl     # small integers: exact
    assert np.array_equal(out, want)
    bi = rng.integers(0, batch, 40)
    ii = rng.integers(0, M, 40)
    jj = rng.integers(0, N, 40)
    el = oracle.gemm_elems("f64", False, False, M, N, K, 0.5, A, lda, B, ldb, 2.0, C, ldc,
                           bi, ii, jj, batch=batch, strideA=sA, strideB=sB, strideC=sC)
    assert np.array_equal(el, out[bi, ii, jj])


def test_f64_operands_must_be_float64():
    a = np.zeros(4, np.float32)
    with pytest.raises(TypeError):
        oracle.gemm("f64", False, False, 2, 2, 2, 1.0, a, 2, a, 2, 0.0, None, 2)
    d = np.zeros(4)
    with pytest.raises(TypeError):
        oracle.gemm("f64", False, False, 2, 2, 2, 1.0, d, 2, d, 2, 1.0, np.zeros(4, np.float32), 2)


def _f64_pins_hold(gemm):
    """The fp64 pins above against a given oracle callable."""
    try:
        rng = np.random.default_rng(47)
        for tA, tB in itertools.product((False, True), repeat=2):
            A = rng.standard_normal((6, 5) if tA else (5, 6))
            B = rng.standard_normal((4, 6) if tB else (6, 4))
            C = rng.standard_normal((5, 4))
            got = gemm("f64", tA, tB, 5, 4, 6, 0.7, A.ravel(), A.shape[1], B.ravel(), B.shape[1],
                       1.5, C.ravel(), 4)[0]
            if not np.array_equal(got, _exact_f64(A, B, C, 0.7, 1.5, tA, tB)):
                return False
        A = np.array([2.0 ** 60, 1.0, -(2.0 ** 60)])
        if gemm("f64", False, False, 1, 1, 3, 1.0, A, 3, np.ones(3), 1, 0.0, None, 1)[0, 0, 0] != 1.0:
            return False
    except Exception:
        return False
    return True


def test_f64_pins_catch_planted_mistakes():
    assert _f64_pins_hold(oracle.gemm)

    def double_accumulator(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, **kw):
        opA = A.reshape(-1, lda)[:, :(M if tA else K)]
        opA = opA.T if tA else opA
        opB = B.reshape(-1, ldb)[:, :(K if tB else N)]
        opB = opB.T if tB else opB
        out = alpha * (opA @ opB)
        if beta != 0.0:
            out = out + beta * C.reshape(-1, ldc)[:, :N]
        return out[None]

    def ignore_trans_b(dtype, tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, **kw):
        return oracle.gemm(dtype, tA, False, M, N, K, alpha, A, lda, B, N, beta, C, ldc, **kw)

    for broken in (double_accumulator, ignore_trans_b):
        assert not _f64_pins_hold(broken), broken.__name__
