"""CPU-side checks of the C-ABI library: it loads, exports every symbol the headers declare,
and its host-only workspace planner agrees with the parameter layout. No GPU calls."""
import ctypes
import os
import re

import pytest

from gpt_transformer_step_train_amd import binding as bd
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("gpt2.h", "gpt2_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(gpt2(?:op)?_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail("libgpt2.so is not built (python -m gpt_transformer_step_train_amd.build)")
    return bd.load()


def test_every_declared_symbol_is_exported(lib):
    declared = declared_functions()
    assert declared == set(bd.EXPORTS), declared ^ set(bd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(os.path.join(ROOT, "include", "gpt2.h")).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (GPT2_[A-Z0-9]+) \(?(-?\d+)\)?", text))
    for k in ("GPT2_OK", "GPT2_EINVAL", "GPT2_ENOMEM", "GPT2_EHIP", "GPT2_ESTATE", "GPT2_ERANGE",
              "GPT2_ENONFINITE", "GPT2_FP32", "GPT2_BF16"):
        assert consts[k] == getattr(bd, k), k
    classes = {k.lower(): int(v) for k, v in re.findall(r"#define GPT2_K_([A-Z0-9_]+) (\d+)", text)}
    assert classes.pop("count") == len(bd.KERNEL_CLASSES)
    for name, i in classes.items():
        assert bd.KERNEL_CLASSES[i] == name
    ops = open(os.path.join(ROOT, "include", "gpt2_ops.h")).read()
    epi = dict((k, int(v)) for k, v in re.findall(r"#define GPT2_(EPI_[A-Z_0-9]+) (\d+)", ops))
    for k, v in epi.items():
        assert getattr(bd, k) == v


def test_config_struct_layout_matches_header():
    # 12 int32 + float + 2 int32 (recompute, no_master) + pad + 3 pointers/uint64 on x86-64
    assert ctypes.sizeof(bd.gpt2_config) == 88
    assert bd.gpt2_config.stream.offset == 64


def _cfg(**kw):
    base = dict(n_layer=12, n_head=12, n_embd=768, vocab=50257, padded_vocab=50304, max_seq=1024, batch=16,
                seq=1024, precision=bd.GPT2_BF16)
    base.update(kw)
    return bd.make_config(**base)


def test_workspace_planner_host_only(lib):
    nb = bd.gpt2_workspace_bytes(_cfg())
    # parameters (fp32 master, grads, m, v + bf16 copy) are all in the arena
    n = O.num_params(O.CFG_124M)
    assert nb > 18 * n
    assert nb % 256 == 0
    # activations scale with the batch
    assert bd.gpt2_workspace_bytes(_cfg(batch=8)) < nb
    # fp32 activations are larger
    assert bd.gpt2_workspace_bytes(_cfg(precision=bd.GPT2_FP32, batch=4)) > bd.gpt2_workspace_bytes(_cfg(batch=4))
    # the 1558M model at B=16 fits one MI355X (288 GB) comfortably
    big = bd.gpt2_workspace_bytes(_cfg(n_layer=48, n_head=25, n_embd=1600))
    assert 30e9 < big < 200e9


@pytest.mark.parametrize("kw,msg", [
    (dict(n_embd=770), "multiple"),
    (dict(n_head=7), "multiple of n_head"),
    (dict(padded_vocab=50000), "vocab"),
    (dict(seq=2048), "seq"),
    (dict(batch=64), "batch"),
    (dict(n_head=24), "head size 64"),
    (dict(precision=7), "precision"),
    (dict(grad_accum=0), "grad_accum"),
    (dict(recompute=3), "recompute"),
    (dict(no_master=2), "no_master"),
    (dict(no_master=1, precision=bd.GPT2_FP32, batch=4), "no_master needs GPT2_BF16"),
])
def test_invalid_configs_rejected_on_host(lib, kw, msg):
    assert bd.gpt2_workspace_bytes(_cfg(**kw)) == 0
    assert bd.gpt2_last_status() == bd.GPT2_EINVAL
    assert msg in bd.last_error()


def test_recompute_saves_workspace(lib):
    # recompute 1 drops one [B*T, 4C] buffer per layer but one (shared); 2 also the two LayerNorm
    # outputs per layer but one
    L, BT, C = 12, 16 * 1024, 768
    w0, w1, w2 = (bd.gpt2_workspace_bytes(_cfg(recompute=r)) for r in range(3))
    assert w0 - w1 >= (L - 1) * BT * 4 * C * 2
    assert w1 - w2 >= (2 * L - 1) * BT * C * 2 - 256 * 2 * L


def test_no_master_saves_the_fp32_parameters(lib):
    n = O.num_params(O.CFG_124M)
    assert bd.gpt2_workspace_bytes(_cfg()) - bd.gpt2_workspace_bytes(_cfg(no_master=1)) >= 4 * n


def test_toy_config_accepted(lib):
    c = bd.make_config(4, 4, 16, 2, 2, 3, 12, 3, precision=bd.GPT2_FP32, linear_bias=0, ln_bias=1)
    assert bd.gpt2_workspace_bytes(c) > 0
