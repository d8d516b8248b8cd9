"""Per-kernel parity: each HIP kernel (through include/gpt2_ops.h) against the CPU oracle's function
for the same step, on the same seeded inputs, element by element.

Tolerances (max-norm relative to the reference unless stated):
  fp32 kernels: 2e-5 (accumulation order only);
  bf16 outputs: 8e-3 (one bf16 rounding of the result is 2^-9 relative, plus bf16 inputs);
  bf16 attention gradients: 2e-2 (probabilities are rounded to bf16 before the second MFMA).
"""
import numpy as np
import pytest

import oracle as O
from gpt_transformer_step_train_amd import binding as bd

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def lib(gpu_lib):
    return gpu_lib


def stream():
    return torch.cuda.current_stream().cuda_stream


TD = {bd.GPT2_FP32: torch.float32, bd.GPT2_BF16: torch.bfloat16}


def dev(x, dt):
    return torch.tensor(np.asarray(x, np.float32)).to("cuda").to(TD[dt]).contiguous()


def h64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel(a, ref):
    return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30))


def tol(dt, f32=2e-5, b16=8e-3):
    return f32 if dt == bd.GPT2_FP32 else b16


DTS = [bd.GPT2_FP32, bd.GPT2_BF16]


# ---------------------------------------------------------------------------- GEMM

GEMM_SHAPES = [(200, 136, 72), (256, 384, 256), (36, 16, 2), (130, 264, 520), (260, 392, 512)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("akc,bkc", [(1, 1), (1, 0), (0, 0), (0, 1)])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_layouts_bias(dt, akc, bkc, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N + K)
    vec = 8
    A = rng.normal(0, 1, (M, K))
    Bm = rng.normal(0, 1, (N, K))
    bias = rng.normal(0, 1, N)
    lda = -(-K // vec) * vec if akc else -(-M // vec) * vec
    ldb = -(-K // vec) * vec if bkc else -(-N // vec) * vec
    As = np.zeros((M, lda)) if akc else np.zeros((K, lda))
    if akc:
        As[:, :K] = A
    else:
        As[:, :M] = A.T
    Bs = np.zeros((N, ldb)) if bkc else np.zeros((K, ldb))
    if bkc:
        Bs[:, :K] = Bm
    else:
        Bs[:, :N] = Bm.T
    Ad, Bd, bd_ = dev(As, dt), dev(Bs, dt), dev(bias, dt)
    ldc = -(-N // vec) * vec
    Cd = torch.zeros((M, ldc), dtype=TD[dt], device="cuda")
    rc = bd.load().gpt2op_gemm(dt, akc, bkc, bd.EPI_BIAS, M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb,
                               Cd.data_ptr(), ldc, bd_.data_ptr(), None, 0, None, 0, None, 0, stream())
    assert rc == 0, bd.last_error()
    torch.cuda.synchronize()
    a64 = h64(Ad)[:, :K] if akc else h64(Ad)[:, :M].T
    b64 = h64(Bd)[:, :K] if bkc else h64(Bd)[:, :N].T
    ref = O.matmul_nt(a64, b64) + h64(bd_)
    assert rel(h64(Cd)[:, :N], ref) <= tol(dt)


def test_gemm_rejects_bad_operands():
    """Leading dimensions that are not whole 16-byte vectors or do not cover a row, unaligned
    pointers, and epilogues missing their second input are refused before any launch."""
    lib = bd.load()
    M, N, K = 64, 64, 64
    buf = [torch.zeros(M * 80 + 64, dtype=torch.bfloat16, device="cuda") for _ in range(5)]
    A, Bm, C, aux, C2 = (t.data_ptr() for t in buf)

    def call(dt=bd.GPT2_BF16, epi=bd.EPI_BIAS, lda=K, ldb=K, ldc=N, a=A, b=Bm, c=C, bias=None, x=None, ldx=0,
             c2=None, akc=1, bkc=1):
        return lib.gpt2op_gemm(dt, akc, bkc, epi, M, N, K, a, lda, b, ldb, c, ldc, bias, x, ldx, c2, 0, None, 0,
                               stream())
    assert call() == bd.GPT2_OK
    assert call(lda=K + 1) == bd.GPT2_EINVAL            # not a whole number of 16-byte vectors
    assert call(ldb=K + 4) == bd.GPT2_EINVAL
    assert call(dt=bd.GPT2_FP32, ldc=N + 2) == bd.GPT2_EINVAL
    assert call(lda=K - 8) == bd.GPT2_EINVAL            # shorter than the row it strides over
    assert call(akc=0, lda=M - 8) == bd.GPT2_EINVAL
    assert call(ldc=N - 8) == bd.GPT2_EINVAL
    assert call(a=A + 2) == bd.GPT2_EINVAL              # unaligned pointers
    assert call(c=C + 8) == bd.GPT2_EINVAL
    assert call(bias=aux + 4) == bd.GPT2_EINVAL
    assert call(epi=bd.EPI_RESID) == bd.GPT2_EINVAL     # residual epilogue without its input
    assert call(epi=bd.EPI_RESID, x=aux, ldx=N - 8) == bd.GPT2_EINVAL
    assert call(epi=bd.EPI_GELU) == bd.GPT2_EINVAL      # GELU epilogue without its second output
    assert call(epi=bd.EPI_RESID, x=aux, ldx=N) == bd.GPT2_OK
    assert call(epi=bd.EPI_GELU, c2=C2) == bd.GPT2_OK
    assert lib.gpt2op_gemm(bd.GPT2_BF16, 1, 1, bd.EPI_BIAS, -1, N, K, A, K, Bm, K, C, N, None, None, 0, None, 0,
                           None, 0, stream()) == bd.GPT2_EINVAL
    torch.cuda.synchronize()


BIG_CASES = [((1, 1), bd.EPI_BIAS), ((1, 0), bd.EPI_BIAS), ((0, 0), bd.EPI_BIAS), ((0, 1), bd.EPI_BIAS),
             ((1, 1), bd.EPI_GELU), ((1, 1), bd.EPI_RESID), ((1, 0), bd.EPI_GELU_BWD), ((0, 0), bd.EPI_F32),
             ((1, 1), bd.EPI_GELU_GRAD), ((1, 0), bd.EPI_MUL)]


@pytest.mark.parametrize("K", [72, 192])
@pytest.mark.parametrize("layout,epi", BIG_CASES)
def test_gemm_bf16_256_tile_path(layout, epi, K):
    """Shapes with >= 384 tiles of 256 x 256 take the large-tile kernel; ragged M and N. With K a
    multiple of 64 the interior tiles take the direct global -> LDS copies, the edge tiles the
    register path; with K = 72 every tile has a ragged K tail."""
    check_big_gemm(layout, epi, K, 4100, 6392)


@pytest.mark.parametrize("K", [72, 192])
@pytest.mark.parametrize("epi", [bd.EPI_BIAS, bd.EPI_GELU, bd.EPI_RESID, bd.EPI_GELU_GRAD, bd.EPI_MUL])
def test_gemm_bf16_256x192_tile_path(epi, K):
    """K-contiguous products where 192-wide column tiles fill the CU rounds better than 256-wide
    ones (here 17 x 12 = 204 tiles against 17 x 9 = 153) take the 256 x 192 kernel: ragged M and
    N, direct copies and register-path edge tiles, ragged K tail with K = 72."""
    check_big_gemm((1, 1), epi, K, 4100, 2300)


@pytest.mark.parametrize("dt,M,N,K,epi", [
    (bd.GPT2_BF16, 200, 136, 72, bd.EPI_MUL),         # 128 x 128 tiles, ragged M, N and K
    (bd.GPT2_FP32, 200, 136, 72, bd.EPI_BIAS),
    (bd.GPT2_BF16, 4100, 6392, 192, bd.EPI_MUL),      # 256 x 256 tiles (column sums in the epilogue)
    (bd.GPT2_BF16, 4100, 2296, 192, bd.EPI_BIAS),     # 256 x 192 tiles (separate column-sum pass)
])
@pytest.mark.parametrize("accumulate", [0, 1])
def test_gemm_colsum(dt, M, N, K, epi, accumulate):
    """colsum[n] (+)= sum over rows of the stored C, whichever tile the shape takes; the product
    itself matches the plain gpt2op_gemm bit for bit."""
    rng = np.random.default_rng(M + N + K + epi)
    A, W, b, aux = rng.normal(0, 1, (M, K)), rng.normal(0, 0.2, (N, K)), rng.normal(0, 0.5, N), rng.normal(0, 1, (M, N))
    Ad, Wd, bd_, auxd = dev(A, dt), dev(W, dt), dev(b, dt), dev(aux, dt)
    C = torch.zeros((M, N), dtype=TD[dt], device="cuda")
    Cref = torch.zeros((M, N), dtype=TD[dt], device="cuda")
    cs0 = rng.normal(0, 1, N)
    cs = torch.tensor(cs0, dtype=torch.float32, device="cuda")
    scr = torch.zeros(-(-M // 128) * 2 * N, dtype=torch.float32, device="cuda")
    lib = bd.load()
    rc = lib.gpt2op_gemm_colsum(dt, 1, 1, epi, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, C.data_ptr(), N,
                                bd_.data_ptr(), auxd.data_ptr(), N, None, cs.data_ptr(), accumulate, scr.data_ptr(),
                                scr.numel(), stream())
    assert rc == 0, bd.last_error()
    rc = lib.gpt2op_gemm(dt, 1, 1, epi, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, Cref.data_ptr(), N,
                         bd_.data_ptr(), auxd.data_ptr(), N, None, 0, None, 0, stream())
    assert rc == 0, bd.last_error()
    torch.cuda.synchronize()
    assert torch.equal(C, Cref)
    c64 = h64(C)
    want = c64.sum(0) + (cs0.astype(np.float32) if accumulate else 0.0)
    bound = 2e-5 * (np.abs(c64).sum(0) + (np.abs(cs0) if accumulate else 0.0)) + 1e-30
    assert np.all(np.abs(cs.cpu().numpy().astype(np.float64) - want) <= bound)
    # too small a scratch is refused
    rc = lib.gpt2op_gemm_colsum(dt, 1, 1, epi, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, C.data_ptr(), N,
                                bd_.data_ptr(), auxd.data_ptr(), N, None, cs.data_ptr(), accumulate, scr.data_ptr(),
                                scr.numel() - 1, stream())
    assert rc == bd.GPT2_EINVAL


def check_big_gemm(layout, epi, K, M, N):
    akc, bkc = layout
    rng = np.random.default_rng(epi * 10 + akc * 2 + bkc)
    A, Bm = rng.normal(0, 1, (M, K)), rng.normal(0, 1, (N, K))
    bias = rng.normal(0, 1, N)
    dt = bd.GPT2_BF16
    # ragged N, leading dimensions padded to whole 16-byte vectors (the ops' contract)
    ldn = -(-N // 8) * 8
    aux = np.zeros((M, ldn))
    aux[:, :N] = rng.normal(0, 1, (M, N))
    lda = K if akc else -(-M // 8) * 8
    ldb = K if bkc else ldn
    As = A if akc else np.zeros((K, lda))
    if not akc:
        As[:, :M] = A.T
    if bkc:
        Bs = Bm
    else:
        Bs = np.zeros((K, ldn))
        Bs[:, :N] = Bm.T
    Ad, Bd, bd_, auxd = dev(As, dt), dev(Bs, dt), dev(bias, dt), dev(aux, dt)
    out_dt = torch.float32 if epi == bd.EPI_F32 else torch.bfloat16
    Cd = torch.zeros((M, ldn), dtype=out_dt, device="cuda")
    C2 = torch.zeros((M, ldn), dtype=out_dt, device="cuda")
    rc = bd.load().gpt2op_gemm(dt, akc, bkc, epi, M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, Cd.data_ptr(),
                               ldn, bd_.data_ptr(), auxd.data_ptr(), ldn, C2.data_ptr(), 0, None, 0, stream())
    assert rc == 0, bd.last_error()
    torch.cuda.synchronize()
    a64 = h64(Ad) if akc else h64(Ad)[:, :M].T
    b64 = h64(Bd) if bkc else h64(Bd)[:, :N].T
    acc = O.matmul_nt(a64, b64)
    b = h64(bd_)
    x64 = h64(auxd)[:, :N]
    want = {bd.EPI_BIAS: acc + b, bd.EPI_GELU: acc + b, bd.EPI_RESID: x64 + acc + b,
            bd.EPI_GELU_BWD: acc * O.gelu_grad(x64), bd.EPI_F32: acc,
            bd.EPI_GELU_GRAD: O.gelu_grad(acc + b), bd.EPI_MUL: acc * x64}[epi]
    assert rel(h64(Cd)[:, :N], want) <= (2e-5 if epi == bd.EPI_F32 else 8e-3)
    # the padding columns of the outputs are never written
    assert not h64(Cd)[:, N:].any() and not h64(C2)[:, N:].any()
    if epi in (bd.EPI_GELU, bd.EPI_GELU_GRAD):
        assert rel(h64(C2)[:, :N], O.gelu(acc + b)) <= 8e-3


@pytest.mark.parametrize("dt", DTS)
def test_gemm_gelu_resid_and_gelu_backward_epilogues(dt):
    M, N, K = 160, 200, 96
    rng = np.random.default_rng(3)
    A, W, b = rng.normal(0, 1, (M, K)), rng.normal(0, 0.2, (N, K)), rng.normal(0, 0.5, N)
    aux = rng.normal(0, 1, (M, N))
    Ad, Wd, bd_, auxd = dev(A, dt), dev(W, dt), dev(b, dt), dev(aux, dt)
    lib = bd.load()
    pre = torch.zeros((M, N), dtype=TD[dt], device="cuda")
    g = torch.zeros_like(pre)
    rc = lib.gpt2op_gemm(dt, 1, 1, bd.EPI_GELU, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, pre.data_ptr(), N,
                         bd_.data_ptr(), None, 0, g.data_ptr(), 0, None, 0, stream())
    assert rc == 0
    res = torch.zeros_like(pre)
    rc = lib.gpt2op_gemm(dt, 1, 1, bd.EPI_RESID, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, res.data_ptr(), N,
                         bd_.data_ptr(), auxd.data_ptr(), N, None, 0, None, 0, stream())
    assert rc == 0
    gb = torch.zeros_like(pre)
    rc = lib.gpt2op_gemm(dt, 1, 1, bd.EPI_GELU_BWD, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, gb.data_ptr(), N,
                         None, auxd.data_ptr(), N, None, 0, None, 0, stream())
    assert rc == 0
    torch.cuda.synchronize()
    acc = O.matmul_nt(h64(Ad), h64(Wd))
    pre_ref = acc + h64(bd_)
    assert rel(h64(pre), pre_ref) <= tol(dt)
    assert rel(h64(g), O.gelu(pre_ref)) <= tol(dt, 5e-5)
    assert rel(h64(res), h64(auxd) + pre_ref) <= tol(dt)
    assert rel(h64(gb), acc * O.gelu_grad(h64(auxd))) <= tol(dt, 5e-5)


@pytest.mark.parametrize("dt", DTS)
def test_gemm_gelu_grad_and_mul_epilogues(dt):
    """The MLP forward keeps gelu'(z) next to gelu(z); the backward multiplies by it."""
    M, N, K = 160, 200, 96
    rng = np.random.default_rng(4)
    A, W, b = rng.normal(0, 1, (M, K)), rng.normal(0, 0.2, (N, K)), rng.normal(0, 0.5, N)
    aux = rng.normal(0, 1, (M, N))
    Ad, Wd, bd_, auxd = dev(A, dt), dev(W, dt), dev(b, dt), dev(aux, dt)
    lib = bd.load()
    dg = torch.zeros((M, N), dtype=TD[dt], device="cuda")
    g = torch.zeros_like(dg)
    rc = lib.gpt2op_gemm(dt, 1, 1, bd.EPI_GELU_GRAD, M, N, K, Ad.data_ptr(), K, Wd.data_ptr(), K, dg.data_ptr(), N,
                         bd_.data_ptr(), None, 0, g.data_ptr(), 0, None, 0, stream())
    assert rc == 0
    mu = torch.zeros_like(dg)
    rc = lib.gpt2op_gemm(dt, 1, 0, bd.EPI_MUL, M, N, K, Ad.data_ptr(), K, Wd.t().contiguous().data_ptr(), N,
                         mu.data_ptr(), N, None, auxd.data_ptr(), N, None, 0, None, 0, stream())
    assert rc == 0
    torch.cuda.synchronize()
    acc = O.matmul_nt(h64(Ad), h64(Wd))
    z = acc + h64(bd_)
    assert rel(h64(dg), O.gelu_grad(z)) <= tol(dt, 5e-5)
    assert rel(h64(g), O.gelu(z)) <= tol(dt, 5e-5)
    assert rel(h64(mu), acc * h64(auxd)) <= tol(dt)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("M,N,K", [(128, 136, 4096), (96, 64, 520), (768, 256, 2048)])
def test_gemm_f32_weight_gradient_split_k_accumulate(dt, M, N, K):
    # dW[M,N] (+)= dY^T X with both operands row-contiguous (K = rows of the batch)
    rng = np.random.default_rng(M + N + K)
    dY, X = rng.normal(0, 1, (K, M)), rng.normal(0, 1, (K, N))
    dYd, Xd = dev(dY, dt), dev(X, dt)
    C0 = rng.normal(0, 1, (M, N)).astype(np.float32)
    lib = bd.load()
    scratch = torch.empty(16 * M * N, dtype=torch.float32, device="cuda")
    ref = O.matmul_nt(h64(dYd).T, h64(Xd).T)
    for accumulate in (0, 1):
        Cd = torch.tensor(C0, device="cuda")
        rc = lib.gpt2op_gemm(dt, 0, 0, bd.EPI_F32, M, N, K, dYd.data_ptr(), M, Xd.data_ptr(), N, Cd.data_ptr(), N,
                             None, None, 0, None, accumulate, scratch.data_ptr(), scratch.numel(), stream())
        assert rc == 0
        torch.cuda.synchronize()
        want = ref + (C0 if accumulate else 0)
        assert rel(Cd.cpu().numpy().astype(np.float64), want) <= 2e-5
    # split-K partials are summed in a fixed order: bitwise reproducible
    outs = []
    for _ in range(2):
        Cd = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        lib.gpt2op_gemm(dt, 0, 0, bd.EPI_F32, M, N, K, dYd.data_ptr(), M, Xd.data_ptr(), N, Cd.data_ptr(), N,
                        None, None, 0, None, 0, scratch.data_ptr(), scratch.numel(), stream())
        torch.cuda.synchronize()
        outs.append(Cd.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("dt,C", [(dt, C) for dt in DTS for C in (0, 6, 8192)]
                         + [(bd.GPT2_FP32, 4096), (bd.GPT2_FP32, 2056)])
def test_layernorm_rejects_bad_widths(dt, C):
    rows, cap = 2, 2 * 8192 + 4096
    # every pointer sits 4 KiB into a buffer that would hold rows x 8192 elements
    buf = [torch.zeros(cap, dtype=torch.float32, device="cuda") for _ in range(8)]
    p = [t.data_ptr() + 4096 for t in buf]
    part = torch.zeros(int(bd.load().gpt2op_layernorm_backward_scratch(rows, 8192)) + 1024, dtype=torch.float32,
                       device="cuda")
    lib = bd.load()
    assert lib.gpt2op_layernorm_forward(dt, rows, C, p[0], p[1], p[2], p[3], p[4], p[5], stream()) == bd.GPT2_EINVAL
    assert lib.gpt2op_layernorm_backward(dt, rows, C, p[0], p[3], p[1], p[4], p[5], p[6], p[7], None, None, 0,
                                         part.data_ptr(), stream()) == bd.GPT2_EINVAL
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("rows,C,has_b", [(37, 16, True), (300, 768, True), (65, 200, False), (1030, 1600, True),
                                          (70, 2048, True)])
def test_layernorm_forward_backward(dt, rows, C, has_b):
    if dt == bd.GPT2_BF16 and C % 8:
        pytest.skip("bf16 needs C % 8 == 0")
    rng = np.random.default_rng(rows + C)
    x = rng.normal(0.5, 2.0, (rows, C))
    w = 1.0 + rng.normal(0, 0.2, C)
    b = rng.normal(0, 0.2, C)
    dy = rng.normal(0, 1, (rows, C))
    dres0 = rng.normal(0, 1, (rows, C))
    xd, wd, bdv, dyd, dres = dev(x, dt), dev(w, dt), dev(b, dt), dev(dy, dt), dev(dres0, dt)
    y = torch.empty_like(xd)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    lib = bd.load()
    rc = lib.gpt2op_layernorm_forward(dt, rows, C, xd.data_ptr(), wd.data_ptr(), bdv.data_ptr() if has_b else None,
                                      y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), stream())
    assert rc == 0
    dw = torch.full((C,), 0.25, dtype=torch.float32, device="cuda")
    db = torch.full((C,), -0.5, dtype=torch.float32, device="cuda")
    part = torch.empty(lib.gpt2op_layernorm_backward_scratch(rows, C), dtype=torch.float32, device="cuda")
    dsum = torch.full((C,), 1.5, dtype=torch.float32, device="cuda")
    dres_before = h64(dres)
    rc = lib.gpt2op_layernorm_backward(dt, rows, C, dyd.data_ptr(), xd.data_ptr(), wd.data_ptr(), mean.data_ptr(),
                                       rstd.data_ptr(), dres.data_ptr(), dw.data_ptr(), db.data_ptr(),
                                       dsum.data_ptr(), 1, part.data_ptr(), stream())
    assert rc == 0
    torch.cuda.synchronize()
    x64, w64, b64 = h64(xd), h64(wd), h64(bdv) if has_b else None
    yref, (mu, rs, xhat) = O.layernorm_forward(x64, w64, b64)
    assert rel(h64(y), yref) <= tol(dt)
    np.testing.assert_allclose(mean.cpu().numpy(), mu, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(rstd.cpu().numpy(), rs, rtol=1e-5)
    dx, dwr, dbr = O.layernorm_backward(h64(dyd), xhat, rs, w64)
    got = h64(dres) - dres_before if dt == bd.GPT2_FP32 else h64(dres)
    want = dx if dt == bd.GPT2_FP32 else dres_before + dx
    assert rel(got, want) <= tol(dt, 5e-5)
    assert rel(dw.cpu().numpy(), dwr + 0.25) <= 5e-5
    # column sums of the updated dres rows (taken before their rounding to the storage type)
    assert rel(dsum.cpu().numpy(), (dres_before + dx).sum(0) + 1.5) <= tol(dt, 5e-5)
    assert rel(db.cpu().numpy(), dbr - 0.5) <= 5e-5


# ---------------------------------------------------------------------------- attention

# bf16 shapes: ragged last tiles (T = 33, 200, 777) with several sequences, whose rows past T must
# read as zeros rather than the next sequence's rows; the 350M (16) and 1558M (25) head counts
ATT_CASES = [(bd.GPT2_FP32, 2, 3, 4, 4), (bd.GPT2_FP32, 1, 130, 2, 64), (bd.GPT2_BF16, 2, 256, 2, 64),
             (bd.GPT2_BF16, 1, 200, 3, 64), (bd.GPT2_BF16, 1, 1024, 1, 64), (bd.GPT2_BF16, 1, 33, 1, 64),
             (bd.GPT2_BF16, 1, 1024, 16, 64), (bd.GPT2_BF16, 3, 777, 25, 64)]


@pytest.mark.parametrize("dt,B,T,H,hs", ATT_CASES)
def test_attention_forward_backward(dt, B, T, H, hs):
    C = H * hs
    rng = np.random.default_rng(T + H)
    qkv = rng.normal(0, 1, (B, T, 3 * C))
    dout = rng.normal(0, 1, (B, T, C))
    qd, dod = dev(qkv, dt), dev(dout, dt)
    out = torch.empty((B, T, C), dtype=TD[dt], device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    lib = bd.load()
    assert lib.gpt2op_attention_forward(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), lse.data_ptr(), stream()) == 0
    dq = torch.full((B, T, 3 * C), float("nan"), dtype=TD[dt], device="cuda")
    dvec = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    assert lib.gpt2op_attention_backward(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), dod.data_ptr(),
                                         lse.data_ptr(), dq.data_ptr(), dvec.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    q64, o_gpu, do64 = h64(qd), h64(out), h64(dod)
    for b in range(B):
        o_ref, probs, lse_ref = O.attention_forward(q64[b], H)
        assert rel(o_gpu[b], o_ref) <= tol(dt, 2e-5, 1e-2)
        # bf16: the scores are exact products of the bf16 inputs summed in fp32 (error ~1e-6 of
        # |s|), but the denominators sum the probabilities after their rounding to bf16 (the same
        # values that enter P V): each is within 2^-8 relative, so the sum and exp(LSE) are too,
        # i.e. |LSE - LSE_ref| <= 2^-8 plus the fp32 exponent error; 4.5e-3 in all. A denominator
        # wrong by 1 % (0.01 in LSE) fails it.
        np.testing.assert_allclose(lse.cpu().numpy()[b], lse_ref, atol=1e-4 if dt == bd.GPT2_FP32 else 4.5e-3)
        # gradient with the GPU's own output as O (D = rowsum(dO * O) uses it); reference uses oracle probs
        dq_ref = O.attention_backward(do64[b], q64[b], probs, H)
        assert rel(h64(dq)[b], dq_ref) <= tol(dt, 5e-5, 2e-2)


@pytest.mark.parametrize("dt,B,T,H,hs", [(bd.GPT2_BF16, 2, 200, 3, 64), (bd.GPT2_BF16, 1, 384, 2, 64),
                                         (bd.GPT2_FP32, 2, 70, 2, 16)])
@pytest.mark.parametrize("accumulate", [0, 1])
def test_attention_backward_colsum(dt, B, T, H, hs, accumulate):
    """The qkv bias gradient that comes with the attention backward equals the column sums of the
    dqkv it stores (ragged last tile at T = 200 and 70), and dqkv is the plain backward's."""
    C = H * hs
    rng = np.random.default_rng(T + H + accumulate)
    qd, dod = dev(rng.normal(0, 1, (B, T, 3 * C)), dt), dev(rng.normal(0, 1, (B, T, C)), dt)
    out = torch.empty((B, T, C), dtype=TD[dt], device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    lib = bd.load()
    assert lib.gpt2op_attention_forward(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), lse.data_ptr(), stream()) == 0
    dq = torch.empty((B, T, 3 * C), dtype=TD[dt], device="cuda")
    dq2 = torch.empty((B, T, 3 * C), dtype=TD[dt], device="cuda")
    dvec = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    b0 = rng.normal(0, 1, 3 * C)
    dbias = torch.tensor(b0, dtype=torch.float32, device="cuda")
    nsc = B * -(-T // 128) * 3 * C
    scr = torch.zeros(nsc, dtype=torch.float32, device="cuda")
    rc = lib.gpt2op_attention_backward_colsum(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), dod.data_ptr(),
                                              lse.data_ptr(), dq.data_ptr(), dvec.data_ptr(), dbias.data_ptr(),
                                              accumulate, scr.data_ptr(), nsc, stream())
    assert rc == 0, bd.last_error()
    assert lib.gpt2op_attention_backward(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), dod.data_ptr(),
                                         lse.data_ptr(), dq2.data_ptr(), dvec.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)
    d64 = h64(dq).reshape(B * T, 3 * C)
    want = d64.sum(0) + (b0.astype(np.float32) if accumulate else 0.0)
    bound = 2e-5 * (np.abs(d64).sum(0) + (np.abs(b0) if accumulate else 0.0)) + 1e-30
    assert np.all(np.abs(dbias.cpu().numpy().astype(np.float64) - want) <= bound)
    rc = lib.gpt2op_attention_backward_colsum(dt, B, T, H, hs, qd.data_ptr(), out.data_ptr(), dod.data_ptr(),
                                              lse.data_ptr(), dq.data_ptr(), dvec.data_ptr(), dbias.data_ptr(),
                                              accumulate, scr.data_ptr(), nsc - 1, stream())
    assert rc == bd.GPT2_EINVAL


def test_attention_rejects_unsupported_head_size():
    lib = bd.load()
    x = torch.zeros(8, device="cuda")
    assert lib.gpt2op_attention_forward(bd.GPT2_BF16, 1, 4, 1, 32, x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                        stream()) == bd.GPT2_EINVAL


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("B,T,H,ok", [(-1, -4, 1, False), (2, -1, 1, False), (1, 4, 0, False), (0, 4, 1, True),
                                      (2, 0, 1, True)])
def test_attention_shape_checks(dt, B, T, H, ok):
    """Negative sizes or no head are refused before any launch (B * T alone would let B = T = -1
    through); an empty batch is a no-op."""
    lib = bd.load()
    x = torch.zeros(64, device="cuda")
    p = x.data_ptr()
    want = bd.GPT2_OK if ok else bd.GPT2_EINVAL
    assert lib.gpt2op_attention_forward(dt, B, T, H, 64, p, p, p, stream()) == want
    assert lib.gpt2op_attention_backward(dt, B, T, H, 64, p, p, p, p, p, p, stream()) == want
    torch.cuda.synchronize()
    assert not x.any()


# ---------------------------------------------------------------------------- stochastic rounding

@pytest.mark.parametrize("t,index0", [(1, 0), (7, 123457), (40000, (1 << 31) + 5)])
def test_stochastic_round_matches_oracle_bit_for_bit(t, index0):
    rng = np.random.default_rng(t)
    n = 200_003
    x = (rng.normal(0, 1, n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    x[:6] = [np.inf, -np.inf, 0.0, -0.0, 1.0, 3.0e38]
    xd = torch.tensor(x, device="cuda")
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    seed = 0x1234_5678_9ABC_DEF0
    assert bd.load().gpt2op_stochastic_round(xd.data_ptr(), y.data_ptr(), n, seed, t, index0, stream()) == 0
    torch.cuda.synchronize()
    got = y.cpu().numpy().view(np.uint16)
    want = O.stochastic_round_bf16(x, seed, t, index0)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------- cross-entropy

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("rows,V,ld", [(37, 1000, 1008), (8, 50257, 50304), (36, 2, 8),
                                      # one class: loss 0 and gradient 0; a row with no padded columns
                                      (5, 1, 8), (3, 57344, 57344)])
def test_cross_entropy(dt, rows, V, ld):
    rng = np.random.default_rng(rows + V)
    logits = np.zeros((rows, ld))
    logits[:, :V] = rng.normal(0, 2, (rows, V))
    logits[:, V:] = 77.0  # padded columns must not matter
    tgt = rng.integers(0, V, rows).astype(np.int32)
    tgt[::5] = -1
    n_valid = int((tgt >= 0).sum())
    ld_ = dev(logits, dt)
    x64 = h64(ld_)[:, :V]
    td = torch.tensor(tgt, device="cuda")
    dloss = torch.tensor([1.0 / n_valid], dtype=torch.float32, device="cuda")
    losses = torch.empty(rows, dtype=torch.float32, device="cuda")
    rc = bd.load().gpt2op_cross_entropy(dt, rows, V, ld, ld_.data_ptr(), td.data_ptr(), dloss.data_ptr(),
                                        losses.data_ptr(), stream())
    assert rc == 0
    torch.cuda.synchronize()
    l_ref, d_ref = O.cross_entropy_forward_backward(x64, tgt, 1.0 / n_valid)
    np.testing.assert_allclose(losses.cpu().numpy(), l_ref, rtol=1e-5, atol=1e-5)
    d = h64(ld_)
    assert rel(d[:, :V], d_ref) <= tol(dt, 1e-5, 8e-3)
    assert np.all(d[:, V:] == 0.0)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("V,ld", [(0, 8), (9, 8), (16, 12)])
def test_cross_entropy_rejects_bad_shapes(dt, V, ld):
    x = torch.zeros(2 * 16, dtype=torch.float32, device="cuda")
    losses = torch.empty(2, dtype=torch.float32, device="cuda")
    rc = bd.load().gpt2op_cross_entropy(dt, 2, V, ld, x.data_ptr(), None, None, losses.data_ptr(), stream())
    assert rc == bd.GPT2_EINVAL


# ---------------------------------------------------------------------------- encoder

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,maxT,C", [(8, 4, 16), (4, 4, 0), (4, 4, 6)])
def test_encoder_rejects_bad_shapes(dt, T, maxT, C):
    B, V, lib = 2, 10, bd.load()
    tok = torch.zeros(B * T, dtype=torch.int32, device="cuda")
    # buffers sized for C = 16, so every access of a shape that were accepted stays inside them
    big = [torch.zeros(B * T * 16 + V * 16 + 64, dtype=torch.float32, device="cuda") for _ in range(4)]
    keys = torch.zeros(B * T, dtype=torch.int32, device="cuda")
    part = torch.zeros(int(lib.gpt2op_encoder_backward_scratch(B * T, 16)) + 64, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if C != 16:
        assert lib.gpt2op_encoder_forward(dt, B, T, C, V, tok.data_ptr(), big[0].data_ptr(), big[1].data_ptr(),
                                          big[2].data_ptr(), err.data_ptr(), stream()) == bd.GPT2_EINVAL
    keys.fill_(-7)
    assert lib.gpt2op_encoder_backward(dt, B, T, maxT, C, V, tok.data_ptr(), big[2].data_ptr(), big[0].data_ptr(),
                                       big[1].data_ptr(), 0, keys.data_ptr(), part.data_ptr(),
                                       stream()) == bd.GPT2_EINVAL
    torch.cuda.synchronize()
    assert bool((keys == -7).all())  # refused before the sort wrote its keys


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("B,T,maxT,C,V,p0", [(4, 64, 80, 128, 500, 0.14), (4, 256, 256, 64, 300, 0.5),
                                            (12, 3, 3, 16, 2, 0.5),
                                            # one run over (nearly) every chunk; V = 1: a single token
                                            (2, 1024, 1024, 64, 3, 0.97), (2, 1024, 1024, 64, 1, 0.0)])
def test_encoder_forward_backward_deterministic(dt, B, T, maxT, C, V, p0):
    rng = np.random.default_rng(B * T + V)
    tok = rng.integers(0, V, (B, T)).astype(np.int32)
    tok[rng.random((B, T)) < p0] = 0  # long runs of one id, crossing many 32-entry chunks
    wte, wpe = rng.normal(0, 1, (V, C)), rng.normal(0, 1, (maxT, C))
    dout = rng.normal(0, 1, (B, T, C))
    lib = bd.load()
    wted, wped, dod = dev(wte, dt), dev(wpe, dt), dev(dout, dt)
    tokd = torch.tensor(tok, device="cuda")
    out = torch.empty((B, T, C), dtype=TD[dt], device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert lib.gpt2op_encoder_forward(dt, B, T, C, V, tokd.data_ptr(), wted.data_ptr(), wped.data_ptr(),
                                      out.data_ptr(), err.data_ptr(), stream()) == 0
    keys = torch.empty(B * T, dtype=torch.int32, device="cuda")
    part = torch.empty(lib.gpt2op_encoder_backward_scratch(B * T, C), dtype=torch.float32, device="cuda")
    results = []
    dwte0 = rng.normal(0, 1, (V, C)).astype(np.float32)
    for _ in range(2):
        dwte = torch.tensor(dwte0, device="cuda")
        dwpe = torch.full((maxT, C), 3.0, dtype=torch.float32, device="cuda")
        assert lib.gpt2op_encoder_backward(dt, B, T, maxT, C, V, tokd.data_ptr(), dod.data_ptr(), dwte.data_ptr(),
                                           dwpe.data_ptr(), 0, keys.data_ptr(), part.data_ptr(), stream()) == 0
        torch.cuda.synchronize()
        results.append((dwte.cpu().numpy(), dwpe.cpu().numpy()))
    assert err.item() == 0
    ref_out = np.stack([O.encoder_forward(h64(wted), h64(wped), tok[b]) for b in range(B)])
    assert rel(h64(out), ref_out) <= tol(dt)
    dwte_ref = dwte0.astype(np.float64).copy()
    dwpe_ref = np.zeros((maxT, C))
    for b in range(B):
        O.encoder_backward(dwte_ref, dwpe_ref, h64(dod)[b], tok[b])
    assert rel(results[0][0].astype(np.float64), dwte_ref) <= 2e-5
    assert rel(results[0][1].astype(np.float64), dwpe_ref) <= 2e-5
    assert np.array_equal(results[0][0], results[1][0]) and np.array_equal(results[0][1], results[1][1])


def test_encoder_flags_out_of_range_token():
    lib = bd.load()
    B, T, C, V = 1, 4, 16, 10
    tok = torch.tensor([[1, 2, 10, 3]], dtype=torch.int32, device="cuda")
    w = torch.zeros((V, C), device="cuda")
    p = torch.zeros((T, C), device="cuda")
    out = torch.empty((B, T, C), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert lib.gpt2op_encoder_forward(bd.GPT2_FP32, B, T, C, V, tok.data_ptr(), w.data_ptr(), p.data_ptr(),
                                      out.data_ptr(), err.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert err.item() & 1


# ---------------------------------------------------------------------------- measurement utilities

@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) * 5 + 48, (1 << 22) * 7])
def test_copy_utility_copies_exactly(nbytes):
    """gpt2op_copy (the bandwidth and counter reference) copies exactly `bytes`, including tails
    shorter than a full round of its grid, and nothing past them."""
    lib = bd.load()
    rng = np.random.default_rng(nbytes % 1000)
    src = torch.tensor(rng.integers(0, 256, nbytes + 64, dtype=np.uint8), device="cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    assert lib.gpt2op_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes]) and not dst[nbytes:].any()
    assert lib.gpt2op_copy(dst.data_ptr() + 8, src.data_ptr(), 32, stream()) == bd.GPT2_EINVAL
    assert lib.gpt2op_copy(dst.data_ptr(), src.data_ptr(), 40, stream()) == bd.GPT2_EINVAL


def test_mfma_rate_utility():
    """gpt2op_mfma_rate runs the main loop's MFMAs on the given operand bits: zero operands give zero
    checksums, the same operands the same checksums twice, and bad arguments are refused."""
    lib = bd.load()
    rng = np.random.default_rng(3)
    bits = (rng.integers(0, 1 << 16, 32768, dtype=np.uint32) & 0x807F | 0x3C00).astype(np.uint16)
    ops = torch.tensor(bits.view(np.int16), device="cuda")
    zeros = torch.zeros(32768, dtype=torch.int16, device="cuda")
    out = torch.full((64,), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.gpt2op_mfma_rate(zeros.data_ptr(), out.data_ptr(), 64, 3, stream()) == 0
    torch.cuda.synchronize()
    assert not out.any()
    outs = []
    for _ in range(2):
        assert lib.gpt2op_mfma_rate(ops.data_ptr(), out.data_ptr(), 64, 3, stream()) == 0
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.isfinite(outs[0]).all() and torch.equal(outs[0], outs[1]) and outs[0].abs().sum() > 0
    assert lib.gpt2op_mfma_rate(ops.data_ptr(), out.data_ptr(), 0, 3, stream()) == bd.GPT2_EINVAL
    assert lib.gpt2op_mfma_rate(ops.data_ptr() + 8, out.data_ptr(), 4, 3, stream()) == bd.GPT2_EINVAL
    assert lib.gpt2op_mfma_rate(ops.data_ptr(), out.data_ptr(), 4, -1, stream()) == bd.GPT2_EINVAL
