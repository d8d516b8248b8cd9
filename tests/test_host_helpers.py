"""Host-side training-loop helpers of the C ABI (learning-rate schedule, spike detector, skipped
update) against the oracle and the values the pages print. No GPU calls."""
import math
import os

import numpy as np
import pytest

from gpt_transformer_step_train_amd import binding as bd
import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail("libgpt2.so is not built (python -m gpt_transformer_step_train_amd.build)")
    return bd.load()


def printed_lr():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "lr_column_1558m.txt")) if l.strip() and l[0] != "#"]
    return [(int(s), float(v)) for s, v in rows]


def test_oracle_schedule_reproduces_the_printed_warmup():
    for step, lr in printed_lr():
        ours = O.lr_schedule(step, 6e-4, 700, 32000, 0.1)
        assert float(f"{ours:.2e}") == lr, (step, ours, lr)


def test_oracle_schedule_closed_forms():
    lr_max, w, n, q = 6e-4, 700, 32000, 0.1
    assert O.lr_schedule(w, lr_max, w, n, q) == pytest.approx(lr_max, rel=1e-15)
    assert O.lr_schedule(n, lr_max, w, n, q) == pytest.approx(q * lr_max, rel=1e-15)
    assert O.lr_schedule(n + 5, lr_max, w, n, q) == pytest.approx(q * lr_max, rel=1e-15)
    mid = (w + n) // 2  # half-way through the decay: cos(pi/2) = 0
    assert O.lr_schedule(mid, lr_max, w, n, q) == pytest.approx((1 + q) / 2 * lr_max, rel=1e-12)
    vals = [O.lr_schedule(s, lr_max, w, n, q) for s in range(1, n + 1, 97)]
    peak = max(range(len(vals)), key=vals.__getitem__)
    assert all(a <= b for a, b in zip(vals[:peak], vals[1:peak + 1]))          # warmup rises
    assert all(a >= b for a, b in zip(vals[peak:], vals[peak + 1:]))            # decay falls


@pytest.mark.parametrize("lr_max,w,n,q", [(6e-4, 700, 32000, 0.1), (1e-3, 0, 50, 0.0), (3e-4, 10, 11, 0.5)])
def test_library_schedule_matches_oracle(lib, lr_max, w, n, q):
    for step in list(range(1, min(n, 800) + 1)) + list(range(n - 3, n + 4)):
        want = O.lr_schedule(step, lr_max, w, n, q)
        got = bd.gpt2_lr_schedule(step, lr_max, w, n, q)
        assert got == pytest.approx(want, rel=2e-7, abs=1e-12), (step, got, want)
    assert math.isnan(bd.gpt2_lr_schedule(0, lr_max, w, n, q))
    assert math.isnan(bd.gpt2_lr_schedule(1, lr_max, 10, 10, q))


def test_library_outlier_detector_matches_oracle(lib):
    rng = np.random.default_rng(7)
    xs = 3.0 + 0.05 * np.cumsum(rng.normal(0, 1, 600)) + rng.normal(0, 0.02, 600)
    xs[[200, 350, 351, 520]] += [2.0, 5.0, -3.0, 8.0]   # spikes
    d = bd.gpt2_outlier()
    bd.gpt2_outlier_reset(d)
    ref = O.OutlierDetector(bd.GPT2_OUTLIER_WINDOW)
    skipped = []
    for i, x in enumerate(xs):
        z = bd.gpt2_outlier_update(d, float(x))
        zr = ref.update(float(x))
        if zr is None:
            assert math.isnan(z), i
        else:
            assert z == pytest.approx(zr, rel=1e-9, abs=1e-12), i
            if zr > 5.0:
                skipped.append(i)
    assert skipped == [200, 350, 520]
    # constant history: no spread, no z-score
    bd.gpt2_outlier_reset(d)
    for _ in range(bd.GPT2_OUTLIER_WINDOW):
        assert math.isnan(bd.gpt2_outlier_update(d, 1.5))
    assert math.isnan(bd.gpt2_outlier_update(d, 100.0))


def test_skip_update_needs_a_model(lib):
    bd.gpt2_free()
    assert bd.gpt2_skip_update() == bd.GPT2_ESTATE


def test_sharded_update_calls_need_a_model(lib):
    """Without a model both calls of the sharded update refuse before any GPU work."""
    bd.gpt2_free()
    assert bd.gpt2_grad_sumsq_range(0, 0)[0] == bd.GPT2_ESTATE
    assert bd.gpt2_adamw_step_range(1e-3, 0.9, 0.95, 1e-8, 0.0, 1, 0, 0, 1.0, 1) == bd.GPT2_ESTATE
