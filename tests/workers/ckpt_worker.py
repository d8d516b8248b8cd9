"""Runs part of a bf16 training run in its own process for the checkpoint-resume test.

python ckpt_worker.py straight N out.npy          N updates from the seeded host init
python ckpt_worker.py first k N ckpt              k updates, then gpt2_save (cursor = k)
python ckpt_worker.py second N ckpt out.npy       gpt2_load into a differently seeded model,
                                                  then the remaining updates up to N
Each update: one forward/backward on seeded batch `step`, AdamW with the scheduled rate.
Writes the final fp32 parameters and the per-update losses.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from gpt_transformer_step_train_amd import binding as bd  # noqa: E402
from gpt_transformer_step_train_amd import synth  # noqa: E402

L, H, C, V, VP, MAXT, B, T = 2, 2, 128, 1000, 1024, 128, 4, 128


NO_MASTER = int(os.environ.get("CKPT_NO_MASTER", "0"))  # 1: bf16 parameters, stochastic rounding


def make(seed, from_inputs=False):
    m = bd.Model(L, H, C, V, VP, MAXT, B, T, bd.GPT2_BF16, grad_clip=1.0, seed=seed, no_master=NO_MASTER)
    if from_inputs:  # the seeded host init the oracle starts from (the stochastic-rounding seed stays `seed`)
        m.set_params(synth.init_params(L, C, VP, MAXT))
    return m


def run(m, first, last, losses):
    for step in range(first, last):
        tok, tgt = synth.zipf_batch(V, B, T, 1000 + step)
        losses.append(m.forward(torch.tensor(tok, dtype=torch.int32, device="cuda"),
                                torch.tensor(tgt, dtype=torch.int32, device="cuda")))
        m.backward()
        lr = bd.gpt2_lr_schedule(step + 1, 6e-4, 3, 40, 0.1)
        m.step(lr, 0.9, 0.95, 1e-8, 0.1, step + 1)


def main():
    mode = sys.argv[1]
    losses = []
    if mode == "straight":
        n, out = int(sys.argv[2]), sys.argv[3]
        m = make(synth.PARAM_SEED, from_inputs=True)
        run(m, 0, n, losses)
    elif mode == "first":
        k, path = int(sys.argv[2]), sys.argv[4]
        m = make(synth.PARAM_SEED, from_inputs=True)
        run(m, 0, k, losses)
        bd.check(bd.gpt2_save(path, k, k), "gpt2_save")
        print("saved", k, flush=True)
        return
    else:
        n, path, out = int(sys.argv[2]), sys.argv[3], sys.argv[4]
        m = make(synth.PARAM_SEED + 99)  # different init: everything must come from the file
        rc, t, cursor = bd.gpt2_load(path)
        bd.check(rc, "gpt2_load")
        assert t == cursor, (t, cursor)
        run(m, cursor, n, losses)
    np.save(out, m.params())
    np.save(out + ".losses.npy", np.asarray(losses, np.float64))
    print("done", mode, flush=True)


if __name__ == "__main__":
    main()
