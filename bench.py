#!/usr/bin/env python3
"""Throughput of the GPT-2 training step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2-124m|gpt2-350m|gpt2-1558m]

A step is one full training step through the C ABI: forward + backward (times grad_accum
micro-batches) + the AdamW update, on synthetic Zipf(1.1) token batches that are already resident
in HBM. The default workload is GPT-2 124M, B=16, T=1024, bf16 mixed precision (fp32 master
weights, grads and AdamW state), AdamW lr 6e-4, betas (0.9, 0.95), wd 0.1, clip 1.0.

Prints one JSON line: tokens/s, ms/step and model-FLOPs utilisation (6N + 6LCT FLOPs per token,
the formula that reproduces the MFU column of the llm.c GPT-2 reproduction post), the roofline of
the kernel class that takes the most time (timed with HIP events on the library's stream over the
timed steps) and the CPU oracle timed on a bounded sample of the same workload. `calibration` holds
rates of this part measured live next to the published peaks: the MFMA rate of the GEMM main loop
on random and on zero operand bits, and a plain HBM copy; the roofline object also gives the
dominant class's fraction of the matching sustained rate.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s (published)
PEAK_HBM = 8.0e12       # MI355X HBM3E, bytes/s (published)
WORKLOADS = {
    "gpt2-124m": dict(name="124M", L=12, H=12, C=768, V=50257, Vp=50304, T=1024, B=16, accum=1),
    "gpt2-350m": dict(name="350M", L=24, H=16, C=1024, V=50257, Vp=50304, T=1024, B=16, accum=1),
    "gpt2-1558m": dict(name="1558M", L=48, H=25, C=1600, V=50257, Vp=50304, T=1024, B=16, accum=64),
}


def metric_name(w):
    return f"training tokens/sec + bf16 MFU, GPT-2 {w['name']} B={w['B']} T={w['T']} on 1 MI355X"
HP = dict(lr=6e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)


def num_params(w):
    C = w["C"]
    return w["Vp"] * C + w["T"] * C + w["L"] * (12 * C * C + 13 * C) + 2 * C


def class_work(name, w):
    """(bound, algorithmic flops or bytes per launch) of one launch of a kernel class."""
    B, T, C, H, Vp, L = w["B"], w["T"], w["C"], w["H"], w["Vp"], w["L"]
    BT, hs = B * T, C // H
    gemm = {"gemm_qkv": (BT, 3 * C, C), "gemm_attproj": (BT, C, C), "gemm_fc": (BT, 4 * C, C),
            "gemm_fcproj": (BT, C, 4 * C), "gemm_classifier": (BT, Vp, C), "gemm_classifier_dx": (BT, C, Vp),
            "gemm_classifier_dw": (Vp, C, BT), "gemm_fcproj_dx": (BT, 4 * C, C), "gemm_fcproj_dw": (C, 4 * C, BT),
            "gemm_fc_dx": (BT, C, 4 * C), "gemm_fc_dw": (4 * C, C, BT), "gemm_attproj_dx": (BT, C, C),
            "gemm_attproj_dw": (C, C, BT), "gemm_qkv_dx": (BT, C, 3 * C), "gemm_qkv_dw": (4 * C, C, BT)}  # qkv_dw: qkv and attproj dW
    if name in gemm:
        M, N, K = gemm[name]
        return "mfma", 2.0 * M * N * K
    if name == "attention_fwd":      # QK^T and PV over the causal half
        return "mfma", 2.0 * B * H * T * T * hs
    if name == "attention_bwd":      # dK/dV kernel: dP, dV, dK (the recompute of P is not credited)
        return "mfma", 3.0 * B * H * T * T * hs
    if name == "attention_bwd_q":    # dQ kernel: dQ (the recomputes of P and dP are not credited)
        return "mfma", 1.0 * B * H * T * T * hs
    e = 2  # bf16 activations
    N = num_params(w)
    bytes_ = {
        "encoder_fwd": BT * C * e * 2 + T * C * e + BT * 4,          # gather rows + wpe + write
        "attention_bwd_pre": BT * C * e * 2 + BT * H * 4,            # read O and dO, write D
        "layernorm_fwd": BT * C * e * 2 + BT * 8 + 2 * C * e,
        "cross_entropy": BT * Vp * e * 2 + BT * 8,                   # read logits, write dlogits in place
        "layernorm_bwd": BT * C * e * 4 + BT * 8 + 2 * C * 4,         # dy, x, dres read+write
        "bias_grad": BT * C * e,                                      # average row width ~C
        "encoder_bwd": BT * C * e + BT * C * 4 + T * C * 4,
        "grad_norm": N * 4,
        # p, m, v rw + g read + bf16 write, + the transposed bf16 copies of the matrices
        "adamw": N * (4 * 3 * 2 + 4 + 2) + (Vp * C + 12 * C * C * L) * e,
        "weight_transpose": (Vp * C + 12 * C * C * L) * e * 2,        # bf16 matrices read + written
        # the column-sum partial rows it reads: 2L + 1 LayerNorm backwards (256 blocks x 3C), the fc
        # bias sums of the fcproj input gradient (two rows per 256-row tile x 4C) and the qkv bias sums
        # of the attention backward (one row per 128-query tile x 3C)
        "grad_finish": 4 * ((2 * L + 1) * 256 * 3 * C + L * (BT // 128) * 4 * C + L * B * (T // 128) * 3 * C),
    }
    return "hbm", float(bytes_.get(name, 0))


def sources_sha256():
    """Digest of the HIP sources and headers the library is built from."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "gpt_transformer_step_train_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cls, workload):
    """HBM bytes per launch of kernel class `cls` in `workload` from the counter summaries under
    profiles/ (lines 'TRAFFIC workload=... class=... fetch_bytes=... write_bytes=...
    sources_sha256=...'), or None when there is none for this class and workload or the sources
    changed since the counters were taken."""
    import glob
    digest = None
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(f):
            if not line.startswith("TRAFFIC "):
                continue
            kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
            if kv.get("class") != cls or kv.get("workload") != workload:
                continue
            digest = digest or sources_sha256()
            if kv.get("sources_sha256") != digest:
                return None
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w):
    """The oracle (plain fp64 numpy, test infrastructure, as it stands) timed on the host.

    Bounded sample of the workload: one whole training step of the same GPT-2 at B=4 (the fp32
    parity configuration), timed by phase on every BLAS thread
    (forward = the logits of the batch; backward = forward + backward minus that; update = AdamW
    over all parameters); plus the forward of one T-long sequence on one thread for a scaling point.
    `value` is tokens/s of the whole step on all threads."""
    import numpy as np
    import oracle as O
    from gpt_transformer_step_train_amd import synth
    from threadpoolctl import threadpool_info, threadpool_limits
    cfg = O.Config(w["L"], w["H"], w["C"], w["V"], w["Vp"], w["T"])
    B = 4
    p = synth.init_params(cfg.n_layer, cfg.n_embd, cfg.padded_vocab, cfg.max_seq).astype(np.float64)
    tok, tgt = synth.zipf_batch(w["V"], B, w["T"], 0)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    t0 = time.perf_counter()
    O.forward_logits(cfg, p, tok)
    t1 = time.perf_counter()
    _, g = O.forward_backward(cfg, p, tok, tgt)
    t2 = time.perf_counter()
    O.adamw_update(cfg, p, g, np.zeros_like(p), np.zeros_like(p), 3e-4, 0.9, 0.999, 1e-8, 0.0, 1)
    t3 = time.perf_counter()
    fwd, fb, upd = t1 - t0, t2 - t1, t3 - t2
    ntok = B * w["T"]
    with threadpool_limits(1):
        t4 = time.perf_counter()
        O.forward_logits(cfg, p, tok[:1])
        one = time.perf_counter() - t4
    return {"value": round(ntok / (fb + upd), 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"one fp64 oracle training step of the same model at B={B}, T={w['T']} (forward + backward + "
                      f"AdamW, {fb + upd:.1f} s) on {threads} BLAS threads; one-thread point: forward of one "
                      f"sequence",
            "phases_s": {"forward": round(fwd, 2), "backward": round(fb - fwd, 2), "update": round(upd, 2)},
            "single_thread_forward_tokens_per_s": round(w["T"] / one, 3),
            "all_threads_forward_tokens_per_s": round(ntok / fwd, 3)}


def calibrate(bd, torch, np):
    """Sustained rates of this part, measured live: the GEMM main loop's MFMA work on random operand
    bits and on zeros (gpt2op_mfma_rate: the matrix cores draw more power on random bits and the
    clock follows the power), and a plain 16-byte streaming copy (gpt2op_copy), read + write."""
    lib = bd.load()
    st = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(7)
    # bf16 bits: random sign and mantissa, exponent 2^-7 (values of the size a trained layer sees)
    rnd = (rng.integers(0, 1 << 16, 32768, dtype=np.uint32) & 0x807F | 0x3C00).astype(np.uint16)
    blocks, iters = 1024, 2000
    out = torch.empty(blocks, dtype=torch.float32, device="cuda")
    res = {}
    for name, host in (("random_operands", rnd), ("zero_operands", np.zeros(32768, np.uint16))):
        ops = torch.tensor(host.view(np.int16), device="cuda")
        ms = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bd.check(lib.gpt2op_mfma_rate(ops.data_ptr(), out.data_ptr(), blocks, iters, st), "mfma_rate")
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        res[name] = round(blocks * 8 * iters * 32 * 32768 / (min(ms[1:]) / 1e3) / 1e12, 1)
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    ms = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bd.check(lib.gpt2op_copy(dst.data_ptr(), src.data_ptr(), n, st), "copy")
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    return {"mfma_bf16_tflops": res, "hbm_copy_tbs": round(2 * n / (min(ms[1:]) / 1e3) / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2-124m", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-master", type=int, default=0, choices=(0, 1),
                    help="1: bf16 parameters without an fp32 master copy (stochastic rounding)")
    ap.add_argument("--recompute", type=int, default=0, choices=(0, 1, 2),
                    help="activation recompute: 1 GELU, 2 also the LayerNorm outputs (less memory)")
    ap.add_argument("--kernel-table", action="store_true", help="print the per-class kernel times to stderr")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the training step here has no multi-GPU path); got --gpus "
              f"{args.gpus}, WORLD_SIZE {world}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from gpt_transformer_step_train_amd import binding as bd
    from gpt_transformer_step_train_amd import synth

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    m = bd.Model(w["L"], w["H"], w["C"], w["V"], w["Vp"], w["T"], w["B"], w["T"], bd.GPT2_BF16,
                 grad_accum=w["accum"], grad_clip=1.0, seed=synth.PARAM_SEED, recompute=args.recompute,
                 no_master=args.no_master)
    n_micro = (args.warmup + args.steps + 1) * w["accum"]
    n_distinct = min(n_micro, 8)           # batches are reused cyclically beyond 8 micro-steps
    batches = []
    for s in range(n_distinct):
        tok, tgt = synth.zipf_batch(w["V"], w["B"], w["T"], s)
        batches.append((torch.tensor(tok.reshape(-1), device="cuda"), torch.tensor(tgt.reshape(-1), device="cuda")))
    torch.cuda.synchronize()

    state = {"t": 0, "micro": 0}
    losses = []

    def step():
        for _ in range(w["accum"]):
            tok, tgt = batches[state["micro"] % n_distinct]
            state["micro"] += 1
            losses.append(m.forward(tok, tgt))
            m.backward()
        state["t"] += 1
        m.step(HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], state["t"])

    for _ in range(args.warmup):
        step()
    # one profiled step (outside the timed region) picks the class that takes the most time
    ncls = len(bd.KERNEL_CLASSES)
    ms = np.zeros(ncls, np.float32)
    cnt = np.zeros(ncls, np.int32)
    bd.check(bd.gpt2_profile_enable((1 << ncls) - 1), "profile")
    step()
    bd.check(bd.gpt2_profile_read(ms, cnt), "profile")
    dom = int(np.argmax(ms))
    if args.kernel_table:
        for i in np.argsort(-ms):
            if cnt[i]:
                print(f"  {bd.KERNEL_CLASSES[i]:20s} {ms[i]:8.3f} ms  x{cnt[i]:3d}  avg {ms[i] / cnt[i] * 1e3:8.1f} us",
                      file=sys.stderr)

    # timed region: only the dominant class carries events
    bd.check(bd.gpt2_profile_enable(1 << dom), "profile")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bd.check(bd.gpt2_profile_read(ms, cnt), "profile")
    bd.gpt2_profile_enable(0)

    sec = (t1 - t0) / args.steps
    tokens_per_step = w["B"] * w["T"] * w["accum"]
    tps = tokens_per_step / sec
    flops_tok = 6 * num_params(w) + 6 * w["L"] * w["C"] * w["T"]
    mfu = tps * flops_tok / PEAK_BF16
    name = bd.KERNEL_CLASSES[dom]
    bound, work = class_work(name, w)
    avg_s = ms[dom] / 1e3 / max(cnt[dom], 1)
    achieved = work / avg_s
    peak = PEAK_BF16 if bound == "mfma" else PEAK_HBM
    unit = "TFLOP/s" if bound == "mfma" else "GB/s"
    scale = 1e12 if bound == "mfma" else 1e9
    roof = {"bound": bound, "kernel": name, "launches_per_step": int(cnt[dom] // args.steps),
            "avg_launch_us": round(avg_s * 1e6, 2), "achieved": round(achieved / scale, 2),
            "peak": peak / scale, "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(name, args.workload)}
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        bd.check(bd.load().gpt2op_copy(dst.data_ptr(), src.data_ptr(), n, torch.cuda.current_stream().cuda_stream),
                 "copy")
        torch.cuda.synchronize()

    cal = calibrate(bd, torch, np)
    sustained = cal["mfma_bf16_tflops"]["random_operands"] * 1e12 if bound == "mfma" else cal["hbm_copy_tbs"] * 1e12
    roof["sustained_peak"] = round(sustained / scale, 2)
    roof["frac_of_sustained"] = round(achieved / sustained, 4)
    out = {
        "metric": metric_name(w), "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} train step, B={w['B']} T={w['T']} grad_accum={w['accum']}, "
                               f"bf16 mixed (fp32 master/grads/AdamW), Zipf(1.1) tokens"
                               + (f", activation recompute {args.recompute}" if args.recompute else "")
                               + (", no fp32 master (stochastic rounding)" if args.no_master else ""),
                   "global_batch": w["B"] * w["accum"], "seq_len": w["T"], "parallelism": "single GPU"},
        "mfu": round(mfu, 4),
        "flops_per_token": flops_tok,
        "final_loss": round(float(losses[-1]), 5),
        "roofline": roof,
        "workspace_bytes": int(m.cfg.workspace_bytes),
        "calibration": cal,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
