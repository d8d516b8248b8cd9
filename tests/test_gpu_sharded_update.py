"""One data-parallel rank's share of a sharded (ZeRO-1) update, on one GPU: gpt2_grad_sumsq_range
and gpt2_adamw_step_range over slices of the flat parameter vector whose ends cut through tensors
(a decayed 2-D weight and an undecayed 1-D vector among them).

Taken together the slices must give, bit for bit, what the full update gives: the squared norm over
[0, N) is the full update's own and the slices' sums add up to it (to double rounding); the
parameters, m and v after the sliced update equal those after gpt2_adamw_step; and so do the next
step's loss and gradients, whose input-gradient products read the transposed bf16 weight copies
(the sliced update leaves them to the next forward to rewrite). Clipping is active (a clip far
below the norm), so the scale formed from the caller's global norm is exercised too."""
import numpy as np
import pytest

import oracle as O
from gpt_transformer_step_train_amd import binding as bd
from gpt_transformer_step_train_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CFG = O.Config(2, 2, 128, 1000, 1024, 128)  # head size 64: the bf16 runs take the MFMA paths
B, T = 2, 128
HP = dict(lr=6e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
CLIP = 1e-2


@pytest.fixture(scope="module", autouse=True)
def lib(gpu_lib):
    yield gpu_lib
    bd.gpt2_free()


def cuda_i32(a):
    return torch.tensor(np.ascontiguousarray(a, np.int32).reshape(-1), device="cuda")


def cuts(cfg, n):
    """Eight equal slices (ends rounded down to multiples of 4) plus cuts in the middle of the token
    embedding, of the first LayerNorm weight and of the second layer's fc weight."""
    offs, o = {}, 0
    for name, shape in O.param_layout(cfg):
        offs[name] = (o, int(np.prod(shape)), len(shape))
        o += offs[name][1]
    assert o == n
    mid = []
    for name in ("wte", "h0.ln1w", "h1.fcw"):
        start, size, dims = offs[name]
        mid.append((start + size // 2) // 4 * 4)
    assert offs["wte"][2] == 2 and offs["h0.ln1w"][2] == 1
    c = sorted(set([0, n] + [(n * k // 8) // 4 * 4 for k in range(1, 8)] + mid))
    return c


def run(precision, no_master, sharded):
    p0 = synth.init_params(CFG.n_layer, CFG.n_embd, CFG.padded_vocab, CFG.max_seq)
    (t0, y0), (t1, y1) = (synth.zipf_batch(CFG.vocab, B, T, s) for s in range(2))
    m = bd.Model(CFG.n_layer, CFG.n_head, CFG.n_embd, CFG.vocab, CFG.padded_vocab, CFG.max_seq, B, T, precision,
                 grad_clip=CLIP, no_master=no_master)
    m.set_params(p0)
    m.forward(cuda_i32(t0), cuda_i32(y0))
    m.backward()
    rc, n2 = bd.gpt2_grad_sumsq_range(0, m.n)
    bd.check(rc, "gpt2_grad_sumsq_range")
    assert np.sqrt(n2) > CLIP  # the clip scale is in play
    parts = None
    if sharded:
        c = cuts(CFG, m.n)
        parts = []
        for a, b in zip(c, c[1:]):
            rc, s = bd.gpt2_grad_sumsq_range(a, b)
            bd.check(rc, "gpt2_grad_sumsq_range")
            parts.append(s)
        for i, (a, b) in enumerate(zip(c, c[1:])):
            bd.check(bd.gpt2_adamw_step_range(HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], 1, a, b, n2,
                                              i == len(c) - 2), "gpt2_adamw_step_range")
    else:
        m.step(HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], 1)
    p = m.params()
    mm, vv = m.adam_state()
    loss1 = m.forward(cuda_i32(t1), cuda_i32(y1))
    m.backward()
    g1 = m.grads()
    del m
    return dict(p=p, m=mm, v=vv, loss1=loss1, g1=g1, n2=n2, parts=parts)


@pytest.mark.parametrize("precision,no_master", [(bd.GPT2_FP32, 0), (bd.GPT2_BF16, 0), (bd.GPT2_BF16, 1)])
def test_sliced_update_equals_the_full_update(precision, no_master):
    full = run(precision, no_master, sharded=False)
    part = run(precision, no_master, sharded=True)
    assert full["n2"] == part["n2"]
    assert abs(sum(part["parts"]) - part["n2"]) <= 1e-12 * part["n2"]
    for k in ("p", "m", "v"):
        assert np.array_equal(full[k], part[k]), k
    assert full["loss1"] == part["loss1"]
    assert np.array_equal(full["g1"], part["g1"])


def test_slice_arguments_are_checked():
    m = bd.Model(CFG.n_layer, CFG.n_head, CFG.n_embd, CFG.vocab, CFG.padded_vocab, CFG.max_seq, B, T,
                 bd.GPT2_BF16, grad_clip=1.0)
    n = m.n
    # no backward yet: the update refuses
    assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 1, 0, n, 1.0, 1) == bd.GPT2_ESTATE
    tok, tgt = synth.zipf_batch(CFG.vocab, B, T, 0)
    m.forward(cuda_i32(tok), cuda_i32(tgt))
    m.backward()
    for a, b in ((2, 8), (0, 6), (8, 4), (0, n + 4)):
        assert bd.gpt2_grad_sumsq_range(a, b)[0] == bd.GPT2_EINVAL, (a, b)
        assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 1, a, b, 1.0, 1) == bd.GPT2_EINVAL, (a, b)
    assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 0, 0, n, 1.0, 1) == bd.GPT2_EINVAL  # t < 1
    # an empty slice is a valid no-op; finish then ends the update
    rc, s = bd.gpt2_grad_sumsq_range(8, 8)
    assert rc == bd.GPT2_OK and s == 0.0
    assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 1, 8, 8, 1.0, 1) == bd.GPT2_OK
    assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 1, 0, n, 1.0, 1) == bd.GPT2_ESTATE
    del m
