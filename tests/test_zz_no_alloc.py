"""The attention backward that allocates nothing (gpt2op_attention_backward_noalloc) against the
plain entry point (gpt2op_attention_backward, which takes its scratch from the caller): the same
kernels, so the gradients must agree bit for bit, on two calls in a row, the second with a smaller
input (the library's array keeps the first call's contents in between), and sizes beyond the
array are refused."""
import numpy as np
import pytest

from gpt_transformer_step_train_amd import binding as bd

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TD = {bd.GPT2_FP32: torch.float32, bd.GPT2_BF16: torch.bfloat16}


def run_pair(lib, dt, B, T, H, hs, seed):
    C = H * hs
    rng = np.random.default_rng(seed)
    qkv = torch.tensor(rng.normal(0, 1, (B, T, 3 * C)), dtype=TD[dt], device="cuda")
    dout = torch.tensor(rng.normal(0, 1, (B, T, C)), dtype=TD[dt], device="cuda")
    out = torch.empty((B, T, C), dtype=TD[dt], device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.gpt2op_attention_forward(dt, B, T, H, hs, qkv.data_ptr(), out.data_ptr(), lse.data_ptr(), s) == 0
    ref = torch.full((B, T, 3 * C), float("nan"), dtype=TD[dt], device="cuda")
    dvec = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    assert lib.gpt2op_attention_backward(dt, B, T, H, hs, qkv.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                         lse.data_ptr(), ref.data_ptr(), dvec.data_ptr(), s) == 0
    got = torch.full((B, T, 3 * C), float("nan"), dtype=TD[dt], device="cuda")
    rc = lib.gpt2op_attention_backward_noalloc(dt, B, T, H, hs, qkv.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                               lse.data_ptr(), got.data_ptr(), s)
    assert rc == 0, bd.last_error()
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16 if dt == bd.GPT2_BF16 else torch.int32),
                       ref.view(torch.int16 if dt == bd.GPT2_BF16 else torch.int32))


@pytest.mark.parametrize("dt,big,small", [
    (bd.GPT2_BF16, (4, 1024, 12), (1, 200, 3)),     # GPT-2 124M heads at T = 1024, then a ragged small case
    (bd.GPT2_FP32, (2, 130, 2), (1, 33, 1)),
])
def test_noalloc_attention_backward_matches_the_plain_entry_point(dt, big, small):
    lib = bd.load()
    run_pair(lib, dt, *big[:2], big[2], 64, seed=1)
    run_pair(lib, dt, *small[:2], small[2], 64, seed=2)


def test_noalloc_attention_backward_refuses_more_than_its_scratch():
    lib = bd.load()
    x = torch.zeros(64, device="cuda")
    p = x.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    cap = bd.GPT2_NOALLOC_ATTN_SCRATCH_FLOATS
    assert lib.gpt2op_attention_backward_noalloc(bd.GPT2_BF16, 1, cap // 16 + 1, 16, 64, p, p, p, p, p, s) \
        == bd.GPT2_EINVAL
    assert lib.gpt2op_attention_backward_noalloc(bd.GPT2_BF16, -1, 4, 1, 64, p, p, p, p, p, s) == bd.GPT2_EINVAL
    assert lib.gpt2op_attention_backward_noalloc(bd.GPT2_BF16, 0, 4, 1, 64, p, p, p, p, p, s) == bd.GPT2_OK
    torch.cuda.synchronize()
    assert not x.any()
