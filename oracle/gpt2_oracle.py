"""Plain fp64 CPU oracle of one GPT-2 training step. TEST INFRASTRUCTURE ONLY.

What it computes follows the pages on llm.c:
  * layer order of the forward pass (encoder, LayerNorm, QKV projection, attention, ...) and
    the hand-ordered backward that starts from the gradient of the loss w.r.t. the logits:
    "Karpathy 的 llm.c：从零理解大模型训练的 C/CUDA 实现", section 代码解剖 (code walk-through);
  * scaled dot-product attention softmax(Q K^T / sqrt(d_k)) V: the LLM primer page
    ("从Andrej Karpathy《深入了解ChatGPT之类的大语言模型》入门LLMs"), attention formula;
    GPT-2 is a decoder, so the softmax runs over keys u <= t only;
  * a vocabulary padded from 50257 to 50304 for efficiency only, tied token embedding and
    classifier (the parameter count printed in "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672",
    section 训练 (training), holds exactly with tying and every bias present), AdamW with m and
    v and an fp32 master copy (same section), weight decay on 2-D tensors only (section 参数
    指南, flag -c), gradient accumulation to a total batch (section 参数指南, flag -d);
  * BabyGPT ("无需写代码能力，手搓最简单BabyGPT模型"): 2 tokens, context 3.

Readings where the pages are silent: GELU is the tanh form of
GPT-2; LayerNorm uses eps = 1e-5 and the biased variance; logits of padded rows v >= V are
not part of the softmax and get zero gradient; weight decay is decoupled and uses the
pre-update parameter; gradient clipping scales all gradients by clip/||g|| when ||g|| > clip;
the loss is the mean over valid targets (target < 0 is ignored).

Every floating-point quantity is float64. Matrix products use numpy's matmul as a library
primitive. No blocking, fusion or reordering beyond the definitions is done; the batch is
processed one sequence at a time because the loss is a sum over sequences and so is its
gradient (this bounds memory, it does not change the result beyond rounding order).

Pins (tests/test_oracle_*.py): HF transformers GPT2LMHeadModel + torch autograd in fp64
(forward logits and every gradient), central finite differences, torch's layer_norm / gelu /
scaled_dot_product_attention / cross_entropy / AdamW / clip_grad_norm_, parameter counts
printed on the pages, causality, probabilities summing to one, the BabyGPT loss floor; the
learning-rate schedule against the lr column printed on the pages and its closed forms
(tests/test_host_helpers.py); the stochastic rounding against the properties that define it and
its generator against an independent implementation (tests/test_oracle_stochastic_rounding.py).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

LN_EPS = 1e-5
GELU_K = math.sqrt(2.0 / math.pi)
GELU_C = 0.044715

__all__ = [
    "Config", "param_layout", "num_params", "views", "decay_mask",
    "layernorm_forward", "layernorm_backward", "gelu", "gelu_grad",
    "attention_forward", "attention_backward", "cross_entropy_forward_backward",
    "encoder_forward", "encoder_backward",
    "forward_backward", "forward_logits", "next_token_probs",
    "grad_norm", "clip_scale", "adamw_update", "train", "matmul_nt", "lr_schedule", "OutlierDetector",
    "splitmix64", "stochastic_round_bf16", "bf16_bits_to_float", "adamw_update_no_master", "SR_SEED_XOR",
    "CFG_TOY", "CFG_124M", "CFG_350M", "CFG_1558M",
]


@dataclass(frozen=True)
class Config:
    n_layer: int
    n_head: int
    n_embd: int
    vocab: int
    padded_vocab: int
    max_seq: int
    linear_bias: bool = True
    ln_bias: bool = True

    @property
    def head_size(self) -> int:
        return self.n_embd // self.n_head


# BabyGPT: 2 tokens, context 3 (BabyGPT page). n_layer/n_head/n_embd and the bias reading
# (linear layers without bias, LayerNorm with weight and bias) are the ones that give the
# page's 12,656 parameters.
CFG_TOY = Config(4, 4, 16, 2, 2, 3, linear_bias=False, ln_bias=True)
CFG_124M = Config(12, 12, 768, 50257, 50304, 1024)
CFG_350M = Config(24, 16, 1024, 50257, 50304, 1024)
CFG_1558M = Config(48, 25, 1600, 50257, 50304, 1024)


def param_layout(cfg: Config):
    """List of (name, shape) in flat-layout order; weights are [out, in]."""
    C = cfg.n_embd
    lay = [("wte", (cfg.padded_vocab, C)), ("wpe", (cfg.max_seq, C))]
    for l in range(cfg.n_layer):
        p = f"h{l}."
        lay += [(p + "ln1w", (C,))]
        lay += [(p + "ln1b", (C,))] if cfg.ln_bias else []
        lay += [(p + "qkvw", (3 * C, C))]
        lay += [(p + "qkvb", (3 * C,))] if cfg.linear_bias else []
        lay += [(p + "attprojw", (C, C))]
        lay += [(p + "attprojb", (C,))] if cfg.linear_bias else []
        lay += [(p + "ln2w", (C,))]
        lay += [(p + "ln2b", (C,))] if cfg.ln_bias else []
        lay += [(p + "fcw", (4 * C, C))]
        lay += [(p + "fcb", (4 * C,))] if cfg.linear_bias else []
        lay += [(p + "fcprojw", (C, 4 * C))]
        lay += [(p + "fcprojb", (C,))] if cfg.linear_bias else []
    lay += [("lnfw", (C,))]
    lay += [("lnfb", (C,))] if cfg.ln_bias else []
    return lay


def num_params(cfg: Config) -> int:
    return sum(int(np.prod(s)) for _, s in param_layout(cfg))


def views(cfg: Config, flat: np.ndarray) -> dict:
    """Name -> reshaped view into a flat parameter (or gradient) vector."""
    out, off = {}, 0
    for name, shape in param_layout(cfg):
        n = int(np.prod(shape))
        out[name] = flat[off:off + n].reshape(shape)
        off += n
    assert off == flat.size, (off, flat.size)
    return out


def decay_mask(cfg: Config) -> np.ndarray:
    """1.0 on elements of 2-D tensors (weight decay applies), 0.0 elsewhere."""
    parts = [np.full(int(np.prod(s)), 1.0 if len(s) == 2 else 0.0) for _, s in param_layout(cfg)]
    return np.concatenate(parts)


# ----------------------------------------------------------------------------------------
# Layers (each one a plain definition)
# ----------------------------------------------------------------------------------------

def layernorm_forward(x, w, b):
    """y = (x - mean) / sqrt(var + eps) * w + b over the last axis; var is the biased one."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = (x - mu) * rstd
    y = xhat * w + (b if b is not None else 0.0)
    return y, (mu[..., 0], rstd[..., 0], xhat)


def layernorm_backward(dy, xhat, rstd, w):
    """Gradients of LayerNorm: (dx, dw, db) for rows of x with the saved xhat and rstd."""
    dw = (dy * xhat).reshape(-1, dy.shape[-1]).sum(axis=0)
    db = dy.reshape(-1, dy.shape[-1]).sum(axis=0)
    g = dy * w
    dx = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True)
                            - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    return dx, dw, db


def gelu(f):
    """GELU, tanh form: 0.5 f (1 + tanh(sqrt(2/pi) (f + 0.044715 f^3)))."""
    return 0.5 * f * (1.0 + np.tanh(GELU_K * (f + GELU_C * f * f * f)))


def gelu_grad(f):
    """d gelu / d f for the tanh form."""
    t = np.tanh(GELU_K * (f + GELU_C * f * f * f))
    return 0.5 * (1.0 + t) + 0.5 * f * (1.0 - t * t) * GELU_K * (1.0 + 3.0 * GELU_C * f * f)


def attention_forward(qkv, n_head):
    """Causal multi-head attention of one sequence.

    qkv: [T, 3C], columns Q | K | V, head h owning columns h*hs .. (h+1)*hs-1 of each third.
    Returns out [T, C], probs [H, T, T] (zero above the diagonal) and lse [H, T].
    """
    T, C3 = qkv.shape
    C = C3 // 3
    hs = C // n_head
    out = np.zeros((T, C))
    probs = np.zeros((n_head, T, T))
    lse = np.zeros((n_head, T))
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    for h in range(n_head):
        q = qkv[:, h * hs:(h + 1) * hs]
        k = qkv[:, C + h * hs:C + (h + 1) * hs]
        v = qkv[:, 2 * C + h * hs:2 * C + (h + 1) * hs]
        s = (q @ k.T) / math.sqrt(hs)
        s[future] = -np.inf
        smax = s.max(axis=-1, keepdims=True)
        e = np.exp(s - smax)
        den = e.sum(axis=-1, keepdims=True)
        p = e / den
        out[:, h * hs:(h + 1) * hs] = p @ v
        probs[h] = p
        lse[h] = (smax + np.log(den))[:, 0]
    return out, probs, lse


def attention_backward(dout, qkv, probs, n_head):
    """Gradient of attention_forward w.r.t. qkv, through the softmax Jacobian."""
    T, C3 = qkv.shape
    C = C3 // 3
    hs = C // n_head
    dqkv = np.zeros_like(qkv)
    scale = 1.0 / math.sqrt(hs)
    for h in range(n_head):
        sl = slice(h * hs, (h + 1) * hs)
        q = qkv[:, sl]
        k = qkv[:, C + h * hs:C + (h + 1) * hs]
        v = qkv[:, 2 * C + h * hs:2 * C + (h + 1) * hs]
        p = probs[h]
        do = dout[:, sl]
        dv = p.T @ do
        dp = do @ v.T
        ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
        dqkv[:, sl] = (ds @ k) * scale
        dqkv[:, C + h * hs:C + (h + 1) * hs] = (ds.T @ q) * scale
        dqkv[:, 2 * C + h * hs:2 * C + (h + 1) * hs] = dv
    return dqkv


def cross_entropy_forward_backward(logits, targets, dloss):
    """Softmax cross-entropy over the V real classes of each row.

    logits [N, V], targets [N] (< 0 = ignored), dloss = d(total loss)/d(loss of a valid row).
    Returns (losses [N] with 0 on ignored rows, dlogits [N, V]).
    """
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(den))[:, 0]
    valid = targets >= 0
    rows = np.nonzero(valid)[0]
    losses = np.zeros(logits.shape[0])
    losses[rows] = lse[rows] - logits[rows, targets[rows]]
    d = e / den
    d[rows, targets[rows]] -= 1.0
    d *= np.where(valid, dloss, 0.0)[:, None]
    return losses, d


def encoder_forward(wte, wpe, tokens):
    """h0[t] = wte[tokens[t]] + wpe[t]."""
    return wte[tokens] + wpe[:tokens.shape[-1]]


def encoder_backward(dwte, dwpe, dh0, tokens):
    """Scatter-add dh0 rows into the token rows of dwte and the position rows of dwpe."""
    np.add.at(dwte, tokens, dh0)
    dwpe[:tokens.shape[-1]] += dh0


# ----------------------------------------------------------------------------------------
# Model
# ----------------------------------------------------------------------------------------

def _linear(x, w, b):
    y = x @ w.T
    return y + b if b is not None else y


def _sequence_forward(cfg, P, tok):
    """Forward of one sequence; returns logits [T, V] and the cache for the backward pass."""
    C, V = cfg.n_embd, cfg.vocab
    h = encoder_forward(P["wte"], P["wpe"], tok)
    cache = {"layers": []}
    for l in range(cfg.n_layer):
        p = f"h{l}."
        a, (_, rs1, xh1) = layernorm_forward(h, P[p + "ln1w"], P.get(p + "ln1b"))
        qkv = _linear(a, P[p + "qkvw"], P.get(p + "qkvb"))
        att, probs, _ = attention_forward(qkv, cfg.n_head)
        h = h + _linear(att, P[p + "attprojw"], P.get(p + "attprojb"))
        m, (_, rs2, xh2) = layernorm_forward(h, P[p + "ln2w"], P.get(p + "ln2b"))
        f = _linear(m, P[p + "fcw"], P.get(p + "fcb"))
        g = gelu(f)
        h = h + _linear(g, P[p + "fcprojw"], P.get(p + "fcprojb"))
        cache["layers"].append(dict(a=a, rs1=rs1, xh1=xh1, qkv=qkv, att=att, probs=probs,
                                    m=m, rs2=rs2, xh2=xh2, f=f, g=g))
    z, (_, rsf, xhf) = layernorm_forward(h, P["lnfw"], P.get("lnfb"))
    logits = z @ P["wte"][:V].T
    cache.update(z=z, rsf=rsf, xhf=xhf)
    return logits, cache


def _sequence_backward(cfg, P, G, tok, cache, dlogits):
    """Accumulate the gradients of one sequence into the gradient views G."""
    V = cfg.vocab
    z = cache["z"]
    dz = dlogits @ P["wte"][:V]
    G["wte"][:V] += dlogits.T @ z
    dh, dw, db = layernorm_backward(dz, cache["xhf"], cache["rsf"], P["lnfw"])
    G["lnfw"] += dw
    if cfg.ln_bias:
        G["lnfb"] += db
    for l in reversed(range(cfg.n_layer)):
        p = f"h{l}."
        c = cache["layers"][l]
        # MLP: h_out = h_mid + gelu(LN2(h_mid) Wfc^T + bfc) Wfcproj^T + bfcproj
        dg = dh @ P[p + "fcprojw"]
        G[p + "fcprojw"] += dh.T @ c["g"]
        if cfg.linear_bias:
            G[p + "fcprojb"] += dh.sum(axis=0)
        df = dg * gelu_grad(c["f"])
        dm = df @ P[p + "fcw"]
        G[p + "fcw"] += df.T @ c["m"]
        if cfg.linear_bias:
            G[p + "fcb"] += df.sum(axis=0)
        dx, dw, db = layernorm_backward(dm, c["xh2"], c["rs2"], P[p + "ln2w"])
        dh = dh + dx
        G[p + "ln2w"] += dw
        if cfg.ln_bias:
            G[p + "ln2b"] += db
        # attention: h_mid = h_in + attn(LN1(h_in)) Wproj^T + bproj
        datt = dh @ P[p + "attprojw"]
        G[p + "attprojw"] += dh.T @ c["att"]
        if cfg.linear_bias:
            G[p + "attprojb"] += dh.sum(axis=0)
        dqkv = attention_backward(datt, c["qkv"], c["probs"], cfg.n_head)
        da = dqkv @ P[p + "qkvw"]
        G[p + "qkvw"] += dqkv.T @ c["a"]
        if cfg.linear_bias:
            G[p + "qkvb"] += dqkv.sum(axis=0)
        dx, dw, db = layernorm_backward(da, c["xh1"], c["rs1"], P[p + "ln1w"])
        dh = dh + dx
        G[p + "ln1w"] += dw
        if cfg.ln_bias:
            G[p + "ln1b"] += db
    encoder_backward(G["wte"], G["wpe"], dh, tok)


def forward_backward(cfg: Config, params, tokens, targets, grad_accum: int = 1,
                     need_grads: bool = True):
    """Mean loss over valid targets and its gradient (flat float64, layout order).

    tokens, targets: [B, T] int. The gradient is of loss / grad_accum, so that summing the
    gradients of grad_accum micro-steps gives the gradient of their mean loss.
    With no valid target the loss is 0 and the gradient is 0.
    """
    params = np.asarray(params, np.float64)
    P = views(cfg, params)
    grads = np.zeros_like(params) if need_grads else None
    G = views(cfg, grads) if need_grads else None
    tokens = np.asarray(tokens)
    targets = np.asarray(targets)
    n_valid = int((targets >= 0).sum())
    if n_valid == 0:
        return 0.0, grads
    dloss = 1.0 / (n_valid * grad_accum)
    total = 0.0
    for b in range(tokens.shape[0]):
        logits, cache = _sequence_forward(cfg, P, tokens[b])
        losses, dlogits = cross_entropy_forward_backward(logits, targets[b], dloss)
        total += losses.sum()
        if need_grads:
            _sequence_backward(cfg, P, G, tokens[b], cache, dlogits)
    return total / n_valid, grads


def forward_logits(cfg: Config, params, tokens):
    """Logits [B, T, V] over the real vocabulary."""
    P = views(cfg, np.asarray(params, np.float64))
    return np.stack([_sequence_forward(cfg, P, np.asarray(t))[0] for t in tokens])


def next_token_probs(cfg: Config, params, tokens):
    """softmax of the last position's logits, [B, V]."""
    lg = forward_logits(cfg, params, tokens)[:, -1, :]
    e = np.exp(lg - lg.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------------------
# Update
# ----------------------------------------------------------------------------------------

def grad_norm(grads) -> float:
    """Global L2 norm over every gradient element."""
    g = np.asarray(grads, np.float64)
    return float(np.sqrt(np.dot(g, g)))


def clip_scale(norm: float, clip: float) -> float:
    """clip / ||g|| when clipping is on and ||g|| exceeds it, else 1."""
    return clip / norm if (clip > 0.0 and norm > clip) else 1.0


def adamw_update(cfg: Config, params, grads, m, v, lr, b1, b2, eps, wd, t, clip=0.0):
    """One AdamW step with decoupled weight decay on 2-D tensors; returns (p, m, v, norm).

    g <- s g with s from clip_scale; m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
    p <- p - lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd_i p), wd_i = wd on 2-D tensors.
    """
    p = np.asarray(params, np.float64)
    g = np.asarray(grads, np.float64)
    norm = grad_norm(g)
    g = g * clip_scale(norm, clip)
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    lam = wd * decay_mask(cfg)
    p = p - lr * (mhat / (np.sqrt(vhat) + eps) + lam * p)
    return p, m, v, norm


def train(cfg: Config, params, batches, lr, b1, b2, eps, wd, clip=0.0, grad_accum=1):
    """Run len(batches) // grad_accum updates; batches is a list of (tokens, targets).

    Returns (final params, m, v, list of per-update mean losses, list of pre-clip norms).
    """
    p = np.asarray(params, np.float64).copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    losses, norms = [], []
    n_up = len(batches) // grad_accum
    for u in range(n_up):
        g = np.zeros_like(p)
        lsum = 0.0
        for a in range(grad_accum):
            tok, tgt = batches[u * grad_accum + a]
            loss, ga = forward_backward(cfg, p, tok, tgt, grad_accum=grad_accum)
            g += ga
            lsum += loss
        p, m, v, nrm = adamw_update(cfg, p, g, m, v, lr, b1, b2, eps, wd, u + 1, clip)
        losses.append(lsum / grad_accum)
        norms.append(nrm)
    return p, m, v, losses, norms


# ----------------------------------------------------------------------------------------
# Update without an fp32 master copy
# ----------------------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> int:
    """Output number n (0-based) of SplitMix64 seeded with `seed` (Steele, Lea & Flood 2014):
    state_n = seed + (n + 1) * 0x9E3779B97F4A7C15, then the three xor-shift-multiply steps."""
    z = (seed + (n + 1) * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


SR_SEED_XOR = 0xD1B54A32D192ED03


def _splitmix64_np(seed: int, n: np.ndarray) -> np.ndarray:
    """splitmix64 for an array of output numbers (uint64 arithmetic wraps mod 2^64)."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (n.astype(np.uint64) + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def stochastic_round_bf16(x, seed: int, t: int, index0: int = 0) -> np.ndarray:
    """fp32 -> bf16 bits with stochastic rounding ("Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672",
    section 参数指南: -w 0 keeps no fp32 master and relies on stochastic rounding).

    Element i takes r = the low 16 bits of SplitMix64 output (t << 32 | (index0 + i)); the
    magnitude rounds up to the next bf16 value when r + (its 16 discarded bits) >= 2^16, i.e.
    with probability discarded / 2^16, so the rounding is unbiased. Inf stays inf, NaN stays NaN.
    """
    x = np.ascontiguousarray(x, np.float32)
    u = x.reshape(-1).view(np.uint32).astype(np.uint64)
    idx = (np.uint64(t) << np.uint64(32)) | (np.uint64(index0) + np.arange(u.size, dtype=np.uint64))
    r = _splitmix64_np(seed, idx) & np.uint64(0xFFFF)
    out = ((u + r) >> np.uint64(16)).astype(np.uint16)
    special = (u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)
    nan = special & ((u & np.uint64(0x7FFFFF)) != 0)
    out[special] = (u[special] >> np.uint64(16)).astype(np.uint16)
    out[nan] |= np.uint16(0x40)
    return out.reshape(x.shape)


def bf16_bits_to_float(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def adamw_update_no_master(cfg: Config, params_bf16_bits, grads, m, v, lr, b1, b2, eps, wd, t, seed, clip=0.0):
    """AdamW on bf16 parameters: the update of adamw_update from the bf16 values, then the result
    rounded to fp32 and stochastically to bf16 (stream seed XOR SR_SEED_XOR, counters by flat
    index). Returns (new bf16 bits, m, v, norm, the fp64 updated values before rounding)."""
    p = bf16_bits_to_float(params_bf16_bits).astype(np.float64)
    p1, m1, v1, norm = adamw_update(cfg, p, grads, m, v, lr, b1, b2, eps, wd, t, clip)
    bits = stochastic_round_bf16(p1.astype(np.float32), seed ^ SR_SEED_XOR, t, 0)
    return bits, m1, v1, norm, p1


# ----------------------------------------------------------------------------------------
# Training-loop helpers around the update
# ----------------------------------------------------------------------------------------

def lr_schedule(step: int, lr_max: float, warmup: int, total: int, final_frac: float) -> float:
    """Learning rate of update `step` (1-based).

    "Karpathy 用 C 复现 GPT-2：单卡 24 小时 $672", section 参数指南: -u warms the rate up linearly
    from 0 to the maximum (-l) over the first updates; -k cosine with -q decays it to that
    fraction of the maximum over the whole run (-x updates). Section 训练 prints the first ten
    rates of such a run. Between warmup and the end the decay is half a cosine period (the
    plain reading of "cosine"); after the end it stays at the final value.
    """
    if step <= warmup:
        return lr_max * step / warmup
    lr_min = final_frac * lr_max
    if step >= total:
        return lr_min
    frac = (step - warmup) / (total - warmup)
    return lr_min + 0.5 * (1.0 + math.cos(math.pi * frac)) * (lr_max - lr_min)


class OutlierDetector:
    """z-score of each new value against the previous `window` values (population standard
    deviation); None until `window` values have been seen or when they are all equal.

    The update-skip of the same post (section 400B token 运行, flags -sl 5.0 -sg 5.0) compares the
    loss and the gradient norm this way; the window length is not printed (128 here).
    """

    def __init__(self, window: int = 128):
        self.window = window
        self.values = []

    def update(self, x: float):
        z = None
        if len(self.values) == self.window:
            mean = sum(self.values) / self.window
            var = sum((v - mean) ** 2 for v in self.values) / self.window
            if var > 0.0:
                z = (x - mean) / math.sqrt(var)
            self.values.pop(0)
        self.values.append(x)
        return z


def matmul_nt(a, b):
    """a @ b^T in float64: the product every Linear layer (y = x W^T) and its gradients use."""
    return np.asarray(a, np.float64) @ np.asarray(b, np.float64).T
