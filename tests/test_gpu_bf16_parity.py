"""Per-tensor gradient parity of the bf16 mixed-precision path, and parity at the GPT-2 1558M widths.

The bf16 path rounds activations, weights and logits to bf16 (8 significant bits: one rounding to
nearest is at most 2^-8 relative, 2^-10 on average) and accumulates in fp32; the oracle is fp64
throughout. A gradient tensor therefore differs from the oracle's by the bf16 roundings along the
backward chain that produced it. The per-tensor bound used here, max |g - g_ref| <= BF16_GRAD_BAND *
max |g_ref|, allows about a dozen such roundings of the largest entry (12 x 2^-8 = 4.7e-2; the
measured worst cases are 1.0e-2 at init and 2.0e-2 after an update, where the two trajectories also
part by the sign of Adam's first step on near-zero gradients); a wrong term, a stale operand or a
transposed index moves a tensor by O(1) of its scale and fails it. Sampled comparisons (the full-size goldens, written by
tests/golden/make_goldens.py from the oracle alone) take max |g_ref| over the whole tensor and
compare 64 seeded entries of it, plus the tensor's own max |g|.

  * a small model (hs 64, ragged tiles), two updates: the first backward reads the transposed
    weight copies made after set_params, the second the copies the AdamW update itself wrote;
    both against the oracle's two-update trajectory; and the second backward bit for bit against
    the same backward after a fresh transpose of the updated weights;
  * the GPT-2 1558M widths (C 1600, 25 heads, 4C 6400, full vocabulary, T = 1024) with two layers:
    fp32 against the oracle at the fp32 bar (loss 1e-5 relative, every tensor 1e-3 of its max),
    bf16 per tensor, and bf16 with two accumulated micro-steps against the oracle's two-sequence
    gradient;
  * GPT-2 124M, B = 16 (the benchmarked workload) and GPT-2 1558M, one sequence, at init:
    loss, norm and sampled gradients against stored oracle values;
  * GPT-2 350M, B = 16: ten updates against the oracle's trajectory; after the loss spike of
    update 3 each update's band widens by twice the oracle's own sensitivity there (its run from
    the bf16-rounded init).
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from gpt_transformer_step_train_amd import binding as bd
from gpt_transformer_step_train_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

BF16_GRAD_BAND = 5e-2       # per tensor, of max |g_ref|
BF16_LOSS_BAND = 2e-2       # absolute: the bar the bf16 path is held to


@pytest.fixture(scope="module", autouse=True)
def lib(gpu_lib):
    yield gpu_lib
    bd.gpt2_free()


def cuda_i32(a):
    return torch.tensor(np.ascontiguousarray(a, np.int32).reshape(-1), device="cuda")


def model(cfg, B, T, precision, grad_accum=1, clip=0.0):
    return bd.Model(cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.vocab, cfg.padded_vocab, cfg.max_seq, B, T, precision,
                    int(cfg.linear_bias), int(cfg.ln_bias), grad_accum, clip)


def init_of(cfg):
    return synth.init_params(cfg.n_layer, cfg.n_embd, cfg.padded_vocab, cfg.max_seq, cfg.linear_bias, cfg.ln_bias)


def per_tensor_rel(cfg, got, ref):
    out = {}
    G, R = O.views(cfg, np.asarray(got, np.float64)), O.views(cfg, np.asarray(ref, np.float64))
    for name, _ in O.param_layout(cfg):
        den = np.abs(R[name]).max()
        out[name] = float(np.abs(G[name] - R[name]).max() / den) if den > 0 else float(np.abs(G[name]).max())
    return out


def report(tag, worst):
    top = sorted(worst.items(), key=lambda kv: -kv[1])[:4]
    print(f"{tag}: worst per-tensor relative errors " + ", ".join(f"{k} {v:.2e}" for k, v in top), flush=True)


def check_sampled(cfg, g, gold, band, tag):
    """Per tensor: |max|g| - gold max| and the 64 sampled entries within band * gold max."""
    offs = np.cumsum([0] + [int(np.prod(s)) for _, s in O.param_layout(cfg)])
    pos, counts, gmax = gold["positions"], gold["counts"], gold["gmax"]
    starts = np.concatenate([[0], np.cumsum(counts)])
    worst = {}
    for t, (name, _) in enumerate(O.param_layout(cfg)):
        sl = slice(starts[t], starts[t + 1])
        gm = np.abs(g[offs[t]:offs[t + 1]]).max()
        e_max = abs(gm - gmax[t]) / gmax[t]
        e_smp = np.abs(g[pos[sl]] - gold["g"][sl]).max() / gmax[t]
        worst[name] = float(max(e_max, e_smp))
    report(tag, worst)
    bad = {k: v for k, v in worst.items() if v > band}
    assert not bad, bad


SMALL = O.Config(2, 2, 128, 1000, 1024, 128)


def test_bf16_small_per_tensor_gradients_over_two_updates():
    cfg, B, T = SMALL, 4, 128
    hp = dict(lr=6e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    p0 = init_of(cfg)
    batches = [synth.zipf_batch(cfg.vocab, B, T, s) for s in range(2)]
    m = model(cfg, B, T, bd.GPT2_BF16, clip=1.0)
    m.set_params(p0)
    grads, losses = [], []
    for s, (tok, tgt) in enumerate(batches):
        losses.append(m.forward(cuda_i32(tok), cuda_i32(tgt)))
        m.backward()
        grads.append(m.grads())
        m.step(hp["lr"], hp["b1"], hp["b2"], hp["eps"], hp["wd"], s + 1)
    p = p0.astype(np.float64)
    mm, vv = np.zeros_like(p), np.zeros_like(p)
    for s, (tok, tgt) in enumerate(batches):
        loss_ref, g_ref = O.forward_backward(cfg, p, tok, tgt)
        assert abs(losses[s] - loss_ref) <= BF16_LOSS_BAND
        worst = per_tensor_rel(cfg, grads[s], g_ref)
        report(f"small bf16 update {s + 1}", worst)
        bad = {k: v for k, v in worst.items() if v > BF16_GRAD_BAND}
        assert not bad, (s, bad)
        p, mm, vv, _ = O.adamw_update(cfg, p, g_ref, mm, vv, t=s + 1, clip=1.0, **hp)


def test_bf16_transposed_copies_written_by_adamw_match_a_fresh_transpose():
    """After an update the input-gradient products read the transposed bf16 weights the AdamW
    kernel wrote; refreshing them from the updated fp32 master (set_params: round to nearest, then
    the transpose kernel) must change nothing: the next backward is the same bit for bit."""
    cfg, B, T = SMALL, 4, 128
    (t0, y0), (t1, y1) = (synth.zipf_batch(cfg.vocab, B, T, s) for s in range(2))
    m = model(cfg, B, T, bd.GPT2_BF16, clip=1.0)
    m.forward(cuda_i32(t0), cuda_i32(y0))
    m.backward()
    m.step(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    l_a = m.forward(cuda_i32(t1), cuda_i32(y1))
    m.backward()
    g_a = m.grads()
    bd.check(bd.gpt2_skip_update(), "gpt2_skip_update")
    m.set_params(m.params())
    l_b = m.forward(cuda_i32(t1), cuda_i32(y1))
    m.backward()
    assert l_a == l_b and np.array_equal(g_a, m.grads())


W1558 = O.Config(2, 25, 1600, 50257, 50304, 1024)   # GPT-2 1558M widths, two layers


@pytest.fixture(scope="module")
def w1558_ref():
    """Oracle loss and gradient of the first sequence at init, and of the first two sequences
    accumulated (mean over both, as two micro-steps of grad_accum = 2 give)."""
    cfg = W1558
    p0 = init_of(cfg)
    tok, tgt = synth.zipf_batch(cfg.vocab, 2, 1024, 0)
    one = O.forward_backward(cfg, p0, tok[:1], tgt[:1])
    two = O.forward_backward(cfg, p0, tok, tgt)
    return p0, tok, tgt, one, two


def test_1558m_widths_fp32_matches_oracle(w1558_ref):
    cfg = W1558
    p0, tok, tgt, (loss_ref, g_ref), _ = w1558_ref
    m = model(cfg, 1, 1024, bd.GPT2_FP32)
    m.set_params(p0)
    loss = m.forward(cuda_i32(tok[:1]), cuda_i32(tgt[:1]))
    m.backward()
    assert abs(loss - loss_ref) <= 1e-5 * abs(loss_ref)
    worst = per_tensor_rel(cfg, m.grads(), g_ref)
    report("1558M widths fp32", worst)
    assert max(worst.values()) <= 1e-3, worst
    del m


def test_1558m_widths_bf16_per_tensor(w1558_ref):
    cfg = W1558
    p0, tok, tgt, (loss_ref, g_ref), _ = w1558_ref
    m = model(cfg, 1, 1024, bd.GPT2_BF16)
    m.set_params(p0)
    loss = m.forward(cuda_i32(tok[:1]), cuda_i32(tgt[:1]))
    m.backward()
    assert abs(loss - loss_ref) <= BF16_LOSS_BAND
    worst = per_tensor_rel(cfg, m.grads(), g_ref)
    report("1558M widths bf16", worst)
    bad = {k: v for k, v in worst.items() if v > BF16_GRAD_BAND}
    assert not bad, bad
    del m


def test_1558m_widths_bf16_two_accumulated_micro_steps(w1558_ref):
    cfg = W1558
    p0, tok, tgt, _, (loss_ref, g_ref) = w1558_ref
    m = model(cfg, 1, 1024, bd.GPT2_BF16, grad_accum=2)
    m.set_params(p0)
    losses = []
    for b in range(2):
        losses.append(m.forward(cuda_i32(tok[b:b + 1]), cuda_i32(tgt[b:b + 1])))
        m.backward()
    assert abs(np.mean(losses) - loss_ref) <= BF16_LOSS_BAND
    worst = per_tensor_rel(cfg, m.grads(), g_ref)
    report("1558M widths bf16, 2 micro-steps", worst)
    bad = {k: v for k, v in worst.items() if v > BF16_GRAD_BAND}
    assert not bad, bad
    del m


def test_124m_bf16_b16_gradients_at_init_vs_oracle():
    gold = np.load(os.path.join(GOLDEN, "gpt2_124m_b16_step1_grads.npz"))
    cfg = O.CFG_124M
    m = model(cfg, 16, 1024, bd.GPT2_BF16, clip=1.0)
    m.set_params(init_of(cfg))
    tok, tgt = synth.zipf_batch(cfg.vocab, 16, 1024, 0)
    loss = m.forward(cuda_i32(tok), cuda_i32(tgt))
    m.backward()
    g = m.grads()
    assert abs(loss - float(gold["loss"])) <= BF16_LOSS_BAND
    nrm = float(np.sqrt(np.dot(g.astype(np.float64), g.astype(np.float64))))
    assert abs(nrm / float(gold["norm"]) - 1) <= BF16_GRAD_BAND
    check_sampled(cfg, g, gold, BF16_GRAD_BAND, "124M bf16 B=16")
    del m


def test_1558m_bf16_one_sequence_gradients_at_init_vs_oracle():
    gold = np.load(os.path.join(GOLDEN, "gpt2_1558m_seq0_grads.npz"))
    cfg = O.CFG_1558M
    m = model(cfg, 1, 1024, bd.GPT2_BF16)
    m.set_params(init_of(cfg))
    tok, tgt = synth.zipf_batch(cfg.vocab, 1, 1024, 0)
    loss = m.forward(cuda_i32(tok), cuda_i32(tgt))
    m.backward()
    g = m.grads()
    assert abs(loss - float(gold["loss"])) <= BF16_LOSS_BAND
    nrm = float(np.sqrt(np.dot(g.astype(np.float64), g.astype(np.float64))))
    assert abs(nrm / float(gold["norm"]) - 1) <= BF16_GRAD_BAND
    check_sampled(cfg, g, gold, BF16_GRAD_BAND, "1558M bf16 one sequence")
    del m


def test_350m_bf16_b16_ten_updates_vs_oracle():
    """GPT-2 350M, B=16, bf16, 10 updates at lr 6e-4 with no warm-up, against the oracle. The loss
    spikes at update 3 and the run is chaotic for a few updates after it: the oracle's own run from
    the same init rounded to bf16 (one perturbation of the size bf16 rounding makes) ends up ~0.4
    away in loss at update 4. Update k is held to 2e-2 plus twice the distance between those two
    oracle runs at update k (0.77 at update 4, 0.03-0.09 at updates 5-10); the first three updates
    come before the spike's effect and take 2e-2 alone. Gradient norms likewise: 5 % plus twice the
    relative distance of the two oracle runs' norms at that update."""
    gold = json.load(open(os.path.join(GOLDEN, "gpt2_350m_b16_10steps.json")))
    pert = json.load(open(os.path.join(GOLDEN, "gpt2_350m_b16_bf16init_10steps.json")))
    assert gold["complete"] and pert["complete"] and pert["hyper"] == gold["hyper"]
    h = gold["hyper"]
    cfg = O.CFG_350M
    m = model(cfg, 16, 1024, bd.GPT2_BF16, clip=h["clip"])
    m.set_params(init_of(cfg))
    losses, norms = [], []
    for s in range(len(gold["losses"])):
        tok, tgt = synth.zipf_batch(cfg.vocab, 16, 1024, s)
        losses.append(m.forward(cuda_i32(tok), cuda_i32(tgt)))
        m.backward()
        m.step(h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], s + 1)
        norms.append(bd.gpt2_grad_norm())
    ref_l, pert_l = np.array(gold["losses"]), np.array(pert["losses"])
    ref_n, pert_n = np.array(gold["norms"]), np.array(pert["norms"])
    band_l = BF16_LOSS_BAND + 2 * np.abs(pert_l - ref_l)
    band_n = 5e-2 + 2 * np.abs(pert_n / ref_n - 1)
    print("350M losses", [round(x, 4) for x in losses], "oracle", [round(x, 4) for x in ref_l],
          "bands", [round(x, 4) for x in band_l], flush=True)
    dl = np.abs(np.array(losses) - ref_l)
    assert np.all(dl[:3] <= BF16_LOSS_BAND), (losses, gold["losses"])
    assert np.all(dl <= band_l), (losses, gold["losses"], band_l)
    assert np.all(np.abs(np.array(norms) / ref_n - 1) <= band_n), (norms, gold["norms"], band_n)
    del m
