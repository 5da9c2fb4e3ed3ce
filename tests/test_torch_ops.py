"""The torch front end (mm, bmm, matmul, attention_scores) against the oracle.

Layout mapping is host logic and is checked on the CPU; the products run on
the GPU and are compared with the oracle on the operands' contiguous copies,
bit-exactly (integer-valued inputs) or within the fp32/16-bit tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_f32_amd import torch_ops
from dense_gemm_f32_amd import workloads as wl

GPU = torch.cuda.is_available()


def ints(shape, dtype, gen, lo=-8, hi=8):
    return torch.randint(lo, hi + 1, shape, generator=gen).to(dtype)


def ref_mm(a, b, alpha=1.0, c0=None, beta=0.0):
    """Oracle product of the CPU contiguous copies, (M, N) float64."""
    name = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[a.dtype]
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    M, K = a.shape
    N = b.shape[1]
    cn = None if c0 is None else c0.detach().cpu().float().contiguous().numpy().ravel()
    return oracle.gemm(name, False, False, M, N, K, alpha, wl.to_numpy_operand(a.ravel()), K,
                       wl.to_numpy_operand(b.ravel()), N, beta, cn, N)[0]


# ------------------------------------------------------------------ host logic (no GPU)

def test_layout_of_views():
    x = torch.zeros(6, 10)
    assert torch_ops._matrix_layout(x) == (0, 10)
    assert torch_ops._matrix_layout(x.t()) == (1, 10)          # transposed view: op = T
    assert torch_ops._matrix_layout(x[:, :7]) == (0, 10)       # column slice keeps ld
    assert torch_ops._matrix_layout(x[1:5].t()) == (1, 10)
    assert torch_ops._matrix_layout(x[:, ::2]) is None         # strided columns: copy
    assert torch_ops._matrix_layout(torch.zeros(1, 5)) == (0, 5)
    assert torch_ops._matrix_layout(torch.zeros(5, 1)) in ((0, 1), (1, 5))


def test_batched_layouts():
    x = torch.zeros(4, 6, 10)
    assert torch_ops._batched_operand(x)[1:] == (0, 10, 60)
    t = x.transpose(1, 2)                                      # (4, 10, 6), column-major inner
    assert torch_ops._batched_operand(t)[1:] == (1, 10, 60)
    e = torch.zeros(1, 6, 10).expand(4, 6, 10)                 # broadcast batch: stride 0
    assert torch_ops._batched_operand(e)[1:] == (0, 10, 0)


def test_shape_errors_before_any_gpu_work():
    a, b = torch.zeros(3, 4), torch.zeros(5, 6)
    with pytest.raises(ValueError):
        torch_ops.mm(a, b)
    with pytest.raises(ValueError):
        torch_ops.bmm(torch.zeros(2, 3, 4), torch.zeros(3, 4, 5))
    with pytest.raises(ValueError):
        torch_ops.attention_scores(torch.zeros(1, 2, 3, 4), torch.zeros(1, 2, 3, 5))
    with pytest.raises(TypeError):
        torch_ops.mm(torch.zeros(3, 4, dtype=torch.int32), torch.zeros(4, 5, dtype=torch.int32))
    with pytest.raises(ValueError):                            # CPU tensors are refused
        torch_ops.mm(torch.zeros(3, 4), torch.zeros(4, 5))


# ------------------------------------------------------------------ on the GPU

@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_mm_views_exact(dtype):
    gen = torch.Generator().manual_seed(61)
    for (M, K, N) in ((70, 45, 33), (256, 128, 192)):
        a = ints((M, K), dtype, gen).cuda()
        b = ints((K, N), dtype, gen).cuda()
        at = ints((K, M), dtype, gen).cuda().t()               # transposed views
        bt = ints((N, K), dtype, gen).cuda().t()
        wide = ints((M, K + 9), dtype, gen).cuda()[:, 3:3 + K]  # slice with ld > K
        for x, y in ((a, b), (at, b), (a, bt), (at, bt), (wide, b), (a[:, ::1], b[:, ::1])):
            got = torch_ops.mm(x, y).double().cpu().numpy()
            assert np.array_equal(got, ref_mm(x, y))
        strided = ints((M, 2 * K), dtype, gen).cuda()[:, ::2]    # needs a copy
        assert np.array_equal(torch_ops.mm(strided, b).double().cpu().numpy(), ref_mm(strided, b))


@pytest.mark.gpu
def test_mm_alpha_beta_and_16bit_out():
    gen = torch.Generator().manual_seed(62)
    a = ints((96, 80), torch.bfloat16, gen).cuda()
    b = ints((80, 72), torch.bfloat16, gen).cuda()
    c0 = ints((96, 72), torch.float32, gen).cuda()
    out = c0.clone()
    torch_ops.mm(a, b, alpha=1.5, beta=-0.5, out=out)
    assert np.array_equal(out.double().cpu().numpy(), ref_mm(a, b, 1.5, c0, -0.5))
    h = torch_ops.mm(a, b, out_dtype=torch.bfloat16)
    assert h.dtype == torch.bfloat16
    want = oracle.decode16("bf16", oracle.round16("bf16", ref_mm(a, b)))
    assert np.array_equal(h.double().cpu().numpy(), want)
    with pytest.raises(TypeError):
        torch_ops.mm(a, b, out_dtype=torch.float16)            # C type: fp32 or the inputs' own


@pytest.mark.gpu
def test_matmul_broadcasts_like_the_tutorial_example():
    # a (10, 3, 4) batch against one (4, 5) matrix, and the mirror case
    gen = torch.Generator().manual_seed(63)
    a = ints((10, 3, 4), torch.float32, gen).cuda()
    b = ints((4, 5), torch.float32, gen).cuda()
    got = torch_ops.matmul(a, b).double().cpu().numpy()
    assert got.shape == (10, 3, 5)
    for i in range(10):
        assert np.array_equal(got[i], ref_mm(a[i], b))
    m = ints((3, 4), torch.float32, gen).cuda()
    bb = ints((6, 4, 5), torch.float32, gen).cuda()
    got = torch_ops.matmul(m, bb).double().cpu().numpy()
    for i in range(6):
        assert np.array_equal(got[i], ref_mm(m, bb[i]))
    # two leading batch dimensions
    x = ints((2, 3, 7, 9), torch.bfloat16, gen).cuda()
    y = ints((2, 3, 9, 4), torch.bfloat16, gen).cuda()
    got = torch_ops.matmul(x, y).double().cpu().numpy()
    for i in range(2):
        for j in range(3):
            assert np.array_equal(got[i, j], ref_mm(x[i, j], y[i, j]))


@pytest.mark.gpu
def test_bmm_transposed_and_expanded_batches():
    gen = torch.Generator().manual_seed(64)
    a = ints((5, 40, 36), torch.float16, gen).cuda()
    b = ints((5, 28, 36), torch.float16, gen).cuda().transpose(1, 2)   # (5, 36, 28) views
    got = torch_ops.bmm(a, b).double().cpu().numpy()
    for i in range(5):
        assert np.array_equal(got[i], ref_mm(a[i], b[i]))
    shared = ints((1, 36, 28), torch.float16, gen).cuda().expand(5, 36, 28)
    got = torch_ops.bmm(a, shared).double().cpu().numpy()
    for i in range(5):
        assert np.array_equal(got[i], ref_mm(a[i], shared[0]))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_attention_scores_match_einsum_definition(dtype):
    # scores[b,h,s,t] = scale * sum_d q[b,h,s,d] k[b,h,t,d]
    gen = torch.Generator().manual_seed(65)
    B, H, S, T, D = 2, 3, 70, 90, 64
    q = ints((B, H, S, D), dtype, gen).cuda()
    k = ints((B, H, T, D), dtype, gen).cuda()
    got = torch_ops.attention_scores(q, k).double().cpu().numpy()   # scale 1/8: exact
    for b in range(B):
        for h in range(H):
            assert np.array_equal(got[b, h], ref_mm(q[b, h], k[b, h].t(), 1.0 / math.sqrt(D)))
    # float inputs, 16-bit scores, a non-default scale, k given as a transposed view
    qf = torch.randn(B, H, S, D, generator=gen).to(dtype).cuda()
    kf = torch.randn(B, H, D, T, generator=gen).to(dtype).cuda().transpose(2, 3)
    got = torch_ops.attention_scores(qf, kf, 0.3, out_dtype=dtype).double().cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = ref_mm(qf[b, h], kf[b, h].t(), 0.3)
            tol = (2e-3 * math.sqrt(D) + (2.0 ** -11 if dtype == torch.float16 else 2.0 ** -8))
            assert np.max(np.abs(got[b, h] - ref)) <= tol * np.max(np.abs(ref))


def test_dtype_names_and_default_outputs():
    assert torch_ops._dtype_name(torch.float64) == "f64"
    assert torch_ops._dtype_name(torch.int8) == "i8"
    assert torch_ops._default_out("f64") == torch.float64
    assert torch_ops._default_out("i8") == torch.int32
    assert torch_ops._default_out("bf16") == torch.float32
    with pytest.raises(TypeError):
        torch_ops._dtype_name(torch.int32)


@pytest.mark.gpu
def test_mm_f64_views_and_alpha_beta():
    gen = torch.Generator().manual_seed(66)
    for (M, K, N) in ((70, 45, 33), (200, 130, 150)):
        a = torch.randn(M, K, generator=gen, dtype=torch.float64).cuda()
        b = torch.randn(N, K, generator=gen, dtype=torch.float64).cuda().t()   # transposed view
        c0 = torch.randn(M, N, generator=gen, dtype=torch.float64).cuda()
        out = c0.clone()
        torch_ops.mm(a, b, alpha=0.3, beta=1.7, out=out)
        ref = oracle.gemm("f64", False, False, M, N, K, 0.3, a.cpu().numpy().ravel(), K,
                          b.cpu().contiguous().numpy().ravel(), N, 1.7, c0.cpu().numpy().ravel(), N)[0]
        tol = 1e-5 * 2.0 ** -29 * math.sqrt(K) * np.max(np.abs(ref))
        assert out.dtype == torch.float64
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= tol


@pytest.mark.gpu
def test_mm_and_bmm_int8_any_view():
    gen = torch.Generator().manual_seed(67)
    M, K, N = 70, 160, 50
    a = torch.randint(-128, 128, (M, K), generator=gen).to(torch.int8)
    b = torch.randint(-128, 128, (K, N), generator=gen).to(torch.int8)
    want = (a.long() @ b.long()).numpy()
    # row-major or transposed storage of each operand, read in place (all four transposes)
    at = a.t().contiguous().cuda().t()
    bt = b.t().contiguous().cuda().t()
    for x, y in ((a.cuda(), b.cuda()), (at, b.cuda()), (a.cuda(), bt), (at, bt)):
        got = torch_ops.mm(x, y)
        assert got.dtype == torch.int32
        assert np.array_equal(got.cpu().numpy(), want)
    a3 = torch.randint(-128, 128, (3, M, K), generator=gen).to(torch.int8)
    b3 = torch.randint(-128, 128, (3, K, N), generator=gen).to(torch.int8)
    got = torch_ops.bmm(a3.cuda(), b3.cuda(), alpha=2.0)
    assert np.array_equal(got.cpu().numpy(), 2 * (a3.long() @ b3.long()).numpy())
    with pytest.raises(Exception):
        torch_ops.mm(a.cuda(), b.cuda(), alpha=0.5)                    # int8: integral alpha only


@pytest.mark.gpu
def test_mm_takes_split_k_on_deep_k_and_matches():
    gen = torch.Generator().manual_seed(68)
    M, K, N = 256, 8192, 256
    assert torch_ops._lib.splitk_chunks("f32", M, N, K, 0) > 1          # auto split applies
    a = ints((M, K), torch.float32, gen).cuda()
    b = ints((K, N), torch.float32, gen).cuda()
    got = torch_ops.mm(a, b).double().cpu().numpy()
    assert np.array_equal(got, ref_mm(a, b))
    off = torch_ops.mm(a, b, splitk=1).double().cpu().numpy()           # one pass, same result
    assert np.array_equal(off, got)
    h = torch_ops.mm(a.to(torch.bfloat16), b.to(torch.bfloat16), out_dtype=torch.bfloat16)
    want = oracle.decode16("bf16", oracle.round16("bf16", ref_mm(a.to(torch.bfloat16),
                                                                 b.to(torch.bfloat16))))
    assert np.array_equal(h.double().cpu().numpy(), want)
