"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests and the bench.

This module draws random numbers and builds token streams. It holds none of the model's
arithmetic: no layer, loss or update is computed here. Both the HIP library's callers and
the CPU oracle's callers take their inputs from it, so the two implementations see the
same data without sharing any code.

Generators (each written from its published definition):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014): output n of a stream seeded with s is mix(s + (n + 1) * 0x9E3779B97F4A7C15),
    so any element of the stream can be computed independently (counter-based).
  * uniform on (0, 1): u = ((x >> 11) + 0.5) * 2**-53 from a 64-bit output x.
  * Box-Muller (Box & Muller 1958): the pair (u1, u2) taken from outputs 2p and 2p + 1 gives
    r = sqrt(-2 ln u1), z0 = r cos(2 pi u2), z1 = r sin(2 pi u2); normals 2p and 2p + 1.

Workloads:
  * Parameter init, "normal(0, 0.02)" (llm.c reproduction post, training section: a model
    of a given depth is initialised from scratch): every 2-D tensor in layout order draws
    from one normal stream; value = float32(0.02 * z) with z in double. Biases and LN
    biases are 0, LN weights 1.
  * Token streams: the reproduction post trains on tokenized web text in B x T windows; that
    corpus is not available, so ids are drawn i.i.d. from Zipf(s = 1.1) over the 50,257-id
    vocabulary by inverse-CDF sampling (smallest rank k whose CDF >= u), id = k - 1. Each
    micro-step takes a fresh contiguous run of B*T + 1 ids; inputs are ids[0:BT], targets
    ids[1:BT+1].
  * BabyGPT toy data (BabyGPT page: 2 tokens, context 3, the sequence 111101111011110 gives
    12 examples): window i = bits[i:i+3], the next bit is the target of the last position,
    the first two positions carry target -1 (ignored).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

PARAM_SEED = 1337
DATA_SEED = 42
INIT_STD = 0.02
ZIPF_S = 1.1
TOY_BITS = "111101111011110"


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream seeded with `seed` (uint64)."""
    with np.errstate(over="ignore"):
        n = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
        z = np.uint64(seed) + n * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform01(x: np.ndarray) -> np.ndarray:
    """Map 64-bit outputs to doubles strictly inside (0, 1)."""
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normals(seed: int, start: int, count: int) -> np.ndarray:
    """Standard normals start .. start+count-1 of the Box-Muller stream (float64)."""
    if count <= 0:
        return np.zeros(0, np.float64)
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = uniform01(splitmix64(seed, 2 * p0, 2 * (p1 - p0))).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log(u[:, 0]))
    ang = 2.0 * np.pi * u[:, 1]
    z = np.empty(2 * (p1 - p0), np.float64)
    z[0::2] = r * np.cos(ang)
    z[1::2] = r * np.sin(ang)
    off = start - 2 * p0
    return z[off:off + count]


def param_tensor_shapes(n_layer, n_embd, padded_vocab, max_seq, linear_bias=True, ln_bias=True):
    """(name, shape) in the flat layout order both implementations use.

    Order: wte [Vp,C], wpe [max_seq,C]; per layer ln1w, ln1b, qkvw [3C,C], qkvb, attprojw [C,C],
    attprojb, ln2w, ln2b, fcw [4C,C], fcb, fcprojw [C,4C], fcprojb; then lnfw, lnfb. Tensors
    switched off by a bias flag are absent. Weights are [out, in].
    """
    C = n_embd
    out = [("wte", (padded_vocab, C)), ("wpe", (max_seq, C))]
    for l in range(n_layer):
        p = f"h{l}."
        out.append((p + "ln1w", (C,)))
        if ln_bias:
            out.append((p + "ln1b", (C,)))
        out.append((p + "qkvw", (3 * C, C)))
        if linear_bias:
            out.append((p + "qkvb", (3 * C,)))
        out.append((p + "attprojw", (C, C)))
        if linear_bias:
            out.append((p + "attprojb", (C,)))
        out.append((p + "ln2w", (C,)))
        if ln_bias:
            out.append((p + "ln2b", (C,)))
        out.append((p + "fcw", (4 * C, C)))
        if linear_bias:
            out.append((p + "fcb", (4 * C,)))
        out.append((p + "fcprojw", (C, 4 * C)))
        if linear_bias:
            out.append((p + "fcprojb", (C,)))
    out.append(("lnfw", (C,)))
    if ln_bias:
        out.append(("lnfb", (C,)))
    return out


def init_params(n_layer, n_embd, padded_vocab, max_seq, linear_bias=True, ln_bias=True,
                seed=PARAM_SEED, std=INIT_STD) -> np.ndarray:
    """Flat float32 initial parameters (see the module docstring for the recipe)."""
    shapes = param_tensor_shapes(n_layer, n_embd, padded_vocab, max_seq, linear_bias, ln_bias)
    total = sum(int(np.prod(s)) for _, s in shapes)
    out = np.empty(total, np.float32)
    off = 0
    normal_idx = 0
    chunk = 1 << 24
    for name, shape in shapes:
        n = int(np.prod(shape))
        if len(shape) == 2:
            for c0 in range(0, n, chunk):
                c = min(chunk, n - c0)
                out[off + c0:off + c0 + c] = (std * normals(seed, normal_idx + c0, c)).astype(np.float32)
            normal_idx += n
        elif name.endswith("w"):       # LayerNorm weight
            out[off:off + n] = 1.0
        else:                          # biases
            out[off:off + n] = 0.0
        off += n
    return out


_ZIPF_CDF_CACHE: dict = {}


def zipf_cdf(vocab: int, s: float = ZIPF_S) -> np.ndarray:
    key = (vocab, s)
    if key not in _ZIPF_CDF_CACHE:
        w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        _ZIPF_CDF_CACHE[key] = c / c[-1]
    return _ZIPF_CDF_CACHE[key]


def zipf_ids(vocab: int, seed: int, start: int, count: int, s: float = ZIPF_S) -> np.ndarray:
    u = uniform01(splitmix64(seed, start, count))
    ids = np.searchsorted(zipf_cdf(vocab, s), u, side="left")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def zipf_batch(vocab: int, B: int, T: int, micro_step: int, seed: int = DATA_SEED):
    """(tokens [B,T] int32, targets [B,T] int32) for one micro-step."""
    n = B * T + 1
    ids = zipf_ids(vocab, seed, micro_step * n, n)
    return ids[:-1].reshape(B, T).copy(), ids[1:].reshape(B, T).copy()


def toy_batch():
    """The 12 BabyGPT examples: tokens [12,3], targets [12,3] (-1 except the last position)."""
    bits = np.array([int(c) for c in TOY_BITS], np.int32)
    n = len(bits) - 3
    tok = np.stack([bits[i:i + 3] for i in range(n)])
    tgt = np.full((n, 3), -1, np.int32)
    tgt[:, 2] = bits[3:3 + n]
    return tok, tgt


def toy_states():
    """All 8 context-3 binary states, state k = bits of k (most significant first)."""
    return np.array([[(k >> 2) & 1, (k >> 1) & 1, k & 1] for k in range(8)], np.int32)
