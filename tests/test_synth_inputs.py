"""The seeded input generators: counter-based slicing, distribution sanity, toy data."""
import math

import numpy as np

from gpt_transformer_step_train_amd import synth


def test_streams_are_counter_based():
    a = synth.splitmix64(7, 0, 100)
    assert np.array_equal(a[37:61], synth.splitmix64(7, 37, 24))
    z = synth.normals(7, 0, 101)
    assert np.array_equal(z[13:80], synth.normals(7, 13, 67))
    assert np.array_equal(z[1:2], synth.normals(7, 1, 1))


def test_normals_and_uniforms_look_right():
    u = synth.uniform01(synth.splitmix64(1, 0, 1 << 18))
    assert 0.0 < u.min() and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 3e-3
    z = synth.normals(1337, 0, 1 << 18)
    assert abs(z.mean()) < 1e-2 and abs(z.std() - 1.0) < 1e-2


def test_zipf_stream_frequencies():
    V = 50257
    ids = synth.zipf_ids(V, 42, 0, 1 << 20)
    assert ids.min() >= 0 and ids.max() < V
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    p = w / w.sum()
    assert abs((ids == 0).mean() - p[0]) < 3e-3          # ~0.139
    H = -(p * np.log(p)).sum()
    assert abs(H - 6.4647) < 1e-3                        # entropy of the source, nats


def test_zipf_batch_shift():
    tok, tgt = synth.zipf_batch(50257, 2, 8, micro_step=3)
    ids = synth.zipf_ids(50257, synth.DATA_SEED, 3 * 17, 17)
    assert np.array_equal(tok.reshape(-1), ids[:-1]) and np.array_equal(tgt.reshape(-1), ids[1:])


def test_toy_batch():
    tok, tgt = synth.toy_batch()
    bits = synth.TOY_BITS
    assert tok.shape == (12, 3)
    for i in range(12):
        assert "".join(map(str, tok[i])) == bits[i:i + 3]
        assert tgt[i, 2] == int(bits[i + 3]) and tgt[i, 0] == tgt[i, 1] == -1


def test_init_params_recipe():
    p = synth.init_params(1, 8, 16, 4, True, True, seed=5)
    shapes = synth.param_tensor_shapes(1, 8, 16, 4)
    off, idx = 0, 0
    for name, shape in shapes:
        n = int(np.prod(shape))
        seg = p[off:off + n]
        if len(shape) == 2:
            ref = (0.02 * synth.normals(5, idx, n)).astype(np.float32)
            assert np.array_equal(seg, ref)
            idx += n
        elif name.endswith("w"):
            assert np.all(seg == 1.0)
        else:
            assert np.all(seg == 0.0)
        off += n
    assert off == p.size and math.isclose(float(np.std(p[:128])), 0.02, rel_tol=0.3)
