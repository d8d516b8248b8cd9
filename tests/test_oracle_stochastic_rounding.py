"""Pins of the oracle's stochastic rounding (the bf16 update without an fp32 master copy): its
generator against an independent implementation of the same published definition, and the
properties that define stochastic rounding (exact values unchanged, only the two neighbouring
bf16 values produced, rounding up with probability equal to the discarded fraction: unbiased)."""
import numpy as np

import oracle as O
from oracle import gpt2_oracle as OG
from gpt_transformer_step_train_amd import synth


def test_generator_matches_the_other_implementation():
    idx = np.arange(0, 5000, 7, dtype=np.uint64)
    ours = OG._splitmix64_np(12345, idx)
    ref = synth.splitmix64(12345, 0, 5000)[::7]
    assert np.array_equal(ours, ref)
    assert O.splitmix64(12345, 42) == int(ref[6])


def neighbours(x):
    """bf16 bits of the values just below and just above |x| (truncation, truncation + 1 ulp)."""
    u = np.asarray(x, np.float32).view(np.uint32)
    lo = (u >> 16).astype(np.uint16)
    return lo, (lo + 1).astype(np.uint16)


def test_exact_values_and_specials_unchanged():
    x = O.bf16_bits_to_float(np.arange(0, 65536, 97, dtype=np.uint16))
    x = x[np.isfinite(x)]
    assert np.array_equal(O.stochastic_round_bf16(x, 3, 1), x.view(np.uint32) >> 16)
    sp = np.array([np.inf, -np.inf, np.nan], np.float32)
    b = O.stochastic_round_bf16(sp, 3, 1)
    assert b[0] == 0x7F80 and b[1] == 0xFF80
    assert np.isnan(O.bf16_bits_to_float(b[2:3]))[0]


def test_only_the_two_neighbours_and_unbiased():
    rng = np.random.default_rng(0)
    x = (rng.normal(0, 1, 64) * 10.0 ** rng.integers(-6, 6, 64)).astype(np.float32)
    n = 1 << 14
    for j, xv in enumerate(x):
        reps = np.full(n, xv, np.float32)
        b = O.stochastic_round_bf16(reps, 99, 1 + j, 0)  # n different counters
        lo, hi = neighbours(xv)
        assert np.all((b == lo) | (b == hi))
        d = int(np.asarray(xv, np.float32).view(np.uint32)) & 0xFFFF
        p = d / 65536.0
        frac_up = float(np.mean(b == hi))
        assert abs(frac_up - p) <= 5 * np.sqrt(p * (1 - p) / n) + 1e-12, (xv, frac_up, p)
        mean = float(np.mean(O.bf16_bits_to_float(b).astype(np.float64)))
        ulp = float(O.bf16_bits_to_float(np.array([hi]))[0]) - float(O.bf16_bits_to_float(np.array([lo]))[0])
        assert abs(mean - float(xv)) <= 5 * abs(ulp) * np.sqrt(p * (1 - p) / n) + 1e-30


def test_counters_decorrelate_updates_and_elements():
    x = np.full(4096, 1.0 + 2.0 ** -8, np.float32)  # half way between 1 and 1 + 2^-7: p = 1/2
    a = O.stochastic_round_bf16(x, 5, 1)
    b = O.stochastic_round_bf16(x, 5, 2)
    c = O.stochastic_round_bf16(x, 5, 1, index0=4096)
    for u in (a, b, c):
        assert 0.45 < float(np.mean(u == u.max())) < 0.55
    assert np.mean(a == b) < 0.6 and np.mean(a == c) < 0.6
