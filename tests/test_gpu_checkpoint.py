"""Checkpoint + bitwise resume: N straight updates equal k updates, gpt2_save, a new process,
gpt2_load, and N - k updates, bit for bit (parameters and every loss). Each part runs in its own
process, one after the other."""
import os
import subprocess
import sys

import numpy as np
import pytest

from gpt_transformer_step_train_amd import binding as bd

pytestmark = pytest.mark.gpu

WORKER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workers", "ckpt_worker.py")


def worker(*args, no_master=0):
    env = dict(os.environ, CKPT_NO_MASTER=str(no_master))
    r = subprocess.run([sys.executable, "-u", WORKER, *map(str, args)], capture_output=True, text=True, timeout=300,
                       env=env)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("no_master", [0, 1])
def test_resume_is_bitwise_identical(tmp_path, no_master):
    """(no_master 1: the stochastic rounding's counters restart from the saved update count, so
    the resumed run draws the same bits.)"""
    n, k = 7, 3
    straight = tmp_path / "straight.npy"
    resumed = tmp_path / "resumed.npy"
    ckpt = tmp_path / "model.ckpt"
    worker("straight", n, straight, no_master=no_master)
    worker("first", k, n, ckpt, no_master=no_master)
    worker("second", n, ckpt, resumed, no_master=no_master)
    a, b = np.load(straight), np.load(resumed)
    assert np.array_equal(a, b)
    la = np.load(str(straight) + ".losses.npy")
    lb = np.load(str(resumed) + ".losses.npy")
    assert np.array_equal(la[k:], lb)


def test_load_rejects_other_architecture_and_bad_files(tmp_path, gpu_lib):
    m = bd.Model(1, 2, 128, 500, 512, 64, 2, 32, bd.GPT2_BF16)
    path = tmp_path / "a.ckpt"
    bd.check(bd.gpt2_save(path, 5, 11), "gpt2_save")
    rc, t, cur = bd.gpt2_load(path)
    assert (rc, t, cur) == (bd.GPT2_OK, 5, 11)
    (tmp_path / "junk.ckpt").write_bytes(b"not a checkpoint")
    assert bd.gpt2_load(tmp_path / "junk.ckpt")[0] == bd.GPT2_EIO
    assert bd.gpt2_load(tmp_path / "missing.ckpt")[0] == bd.GPT2_EIO
    short = tmp_path / "short.ckpt"
    short.write_bytes(path.read_bytes()[:1000])
    assert bd.gpt2_load(short)[0] == bd.GPT2_EIO
    m2 = bd.Model(1, 2, 128, 500, 512, 128, 2, 32, bd.GPT2_BF16)  # other max_seq: other wpe
    assert bd.gpt2_load(path)[0] == bd.GPT2_EIO
    del m, m2
