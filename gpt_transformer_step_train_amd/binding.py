"""ctypes binding of libgpt2.so: the C ABI of include/gpt2.h and include/gpt2_ops.h, same names.

Argument marshalling only. Device buffers are torch tensors (or raw device addresses); every step
of the training step runs in the library's HIP kernels. Loading fails loudly when the library has
not been built (python -m gpt_transformer_step_train_amd.build).
"""
import ctypes
import math
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpt2.so")

GPT2_OK, GPT2_EINVAL, GPT2_ENOMEM, GPT2_EHIP, GPT2_ESTATE, GPT2_ERANGE, GPT2_ENONFINITE = 0, -1, -2, -3, -4, -5, -6
GPT2_EIO = -7
GPT2_FP32, GPT2_BF16 = 0, 1
EPI_BIAS, EPI_GELU, EPI_RESID, EPI_GELU_BWD, EPI_F32, EPI_GELU_GRAD, EPI_MUL = 0, 1, 2, 3, 4, 5, 6

# every symbol the headers declare (checked by the CPU tests against include/*.h)
EXPORTS = [
    "gpt2_workspace_bytes", "gpt2_init", "gpt2_forward", "gpt2_backward", "gpt2_adamw_step", "gpt2_grad_norm",
    "gpt2_last_status", "gpt2_last_error", "gpt2_num_params", "gpt2_get_params", "gpt2_set_params",
    "gpt2_get_grads", "gpt2_get_adam_state", "gpt2_get_logits", "gpt2_free", "gpt2_profile_enable",
    "gpt2_profile_read", "gpt2_skip_update", "gpt2_save", "gpt2_load", "gpt2_lr_schedule", "gpt2_outlier_reset", "gpt2_outlier_update",
    "gpt2_grad_sumsq_range", "gpt2_adamw_step_range",
    "gpt2op_gemm", "gpt2op_layernorm_forward", "gpt2op_layernorm_backward", "gpt2op_layernorm_backward_scratch",
    "gpt2op_attention_forward", "gpt2op_attention_backward", "gpt2op_cross_entropy", "gpt2op_encoder_forward",
    "gpt2op_encoder_backward", "gpt2op_encoder_backward_scratch", "gpt2op_copy", "gpt2op_gemm_colsum",
    "gpt2op_attention_backward_colsum", "gpt2op_stochastic_round", "gpt2op_attention_backward_noalloc",
    "gpt2op_mfma_rate",
]
GPT2_NOALLOC_ATTN_SCRATCH_FLOATS = 1 << 20


class gpt2_config(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_embd", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("padded_vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("linear_bias", ctypes.c_int32), ("ln_bias", ctypes.c_int32), ("grad_accum", ctypes.c_int32),
                ("grad_clip", ctypes.c_float), ("recompute", ctypes.c_int32), ("no_master", ctypes.c_int32),
                ("stream", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_uint64)]


GPT2_OUTLIER_WINDOW = 128


class gpt2_outlier(ctypes.Structure):
    _fields_ = [("values", ctypes.c_double * GPT2_OUTLIER_WINDOW), ("count", ctypes.c_int32),
                ("next", ctypes.c_int32)]


_lib = None
_vp, _i32, _i64, _u64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_FP = ctypes.POINTER(ctypes.c_float)


def load(path=LIB_PATH):
    """Load libgpt2.so and declare every signature. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with python -m gpt_transformer_step_train_amd.build")
    lib = ctypes.CDLL(path)
    sig = {
        "gpt2_workspace_bytes": (_u64, [ctypes.POINTER(gpt2_config)]),
        "gpt2_init": (ctypes.c_int, [ctypes.POINTER(gpt2_config), _u64]),
        "gpt2_forward": (_f32, [_vp, _vp]),
        "gpt2_backward": (ctypes.c_int, []),
        "gpt2_adamw_step": (ctypes.c_int, [_f32, _f32, _f32, _f32, _f32, _i32]),
        "gpt2_grad_norm": (_f32, []),
        "gpt2_last_status": (ctypes.c_int, []),
        "gpt2_last_error": (ctypes.c_char_p, []),
        "gpt2_num_params": (_u64, []),
        "gpt2_get_params": (ctypes.c_int, [_vp, _u64]),
        "gpt2_set_params": (ctypes.c_int, [_vp, _u64]),
        "gpt2_get_grads": (ctypes.c_int, [_vp, _u64]),
        "gpt2_get_adam_state": (ctypes.c_int, [_vp, _vp, _u64]),
        "gpt2_get_logits": (ctypes.c_int, [_vp, _u64]),
        "gpt2_free": (None, []),
        "gpt2_profile_enable": (ctypes.c_int, [ctypes.c_uint32]),
        "gpt2_profile_read": (ctypes.c_int, [_vp, _vp, _i32]),
        "gpt2_skip_update": (ctypes.c_int, []),
        "gpt2_grad_sumsq_range": (ctypes.c_int, [_u64, _u64, ctypes.POINTER(ctypes.c_double)]),
        "gpt2_adamw_step_range": (ctypes.c_int, [_f32, _f32, _f32, _f32, _f32, _i32, _u64, _u64, ctypes.c_double,
                                                 ctypes.c_int]),
        "gpt2_save": (ctypes.c_int, [ctypes.c_char_p, _i32, _u64]),
        "gpt2_load": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(_i32), ctypes.POINTER(_u64)]),
        "gpt2_lr_schedule": (_f32, [_i32, _f32, _i32, _i32, _f32]),
        "gpt2_outlier_reset": (None, [ctypes.POINTER(gpt2_outlier)]),
        "gpt2_outlier_update": (ctypes.c_double, [ctypes.POINTER(gpt2_outlier), ctypes.c_double]),
        "gpt2op_gemm": (ctypes.c_int, [ctypes.c_int] * 7 + [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp,
                                                            ctypes.c_int, _vp, _u64, _vp]),
        "gpt2op_gemm_colsum": (ctypes.c_int, [ctypes.c_int] * 7 + [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64,
                                                                   _vp, _vp, ctypes.c_int, _vp, _u64, _vp]),
        "gpt2op_layernorm_forward": (ctypes.c_int, [ctypes.c_int] * 3 + [_vp] * 7),
        "gpt2op_layernorm_backward": (ctypes.c_int, [ctypes.c_int] * 3 + [_vp] * 9 + [ctypes.c_int, _vp, _vp]),
        "gpt2op_layernorm_backward_scratch": (_u64, [ctypes.c_int, ctypes.c_int]),
        "gpt2op_attention_forward": (ctypes.c_int, [ctypes.c_int] * 5 + [_vp] * 4),
        "gpt2op_attention_backward": (ctypes.c_int, [ctypes.c_int] * 5 + [_vp] * 7),
        "gpt2op_attention_backward_noalloc": (ctypes.c_int, [ctypes.c_int] * 5 + [_vp] * 6),
        "gpt2op_mfma_rate": (ctypes.c_int, [_vp, _vp, ctypes.c_int, ctypes.c_int, _vp]),
        "gpt2op_stochastic_round": (ctypes.c_int, [_vp, _vp, _u64, _u64, _i32, _u64, _vp]),
        "gpt2op_attention_backward_colsum": (ctypes.c_int, [ctypes.c_int] * 5 + [_vp] * 7 + [ctypes.c_int, _vp, _u64,
                                                                                          _vp]),
        "gpt2op_cross_entropy": (ctypes.c_int, [ctypes.c_int] * 4 + [_vp] * 5),
        "gpt2op_encoder_forward": (ctypes.c_int, [ctypes.c_int] * 5 + [_vp] * 6),
        "gpt2op_encoder_backward": (ctypes.c_int, [ctypes.c_int] * 6 + [_vp] * 4 + [ctypes.c_int, _vp, _vp, _vp]),
        "gpt2op_encoder_backward_scratch": (_u64, [ctypes.c_int, ctypes.c_int]),
        "gpt2op_copy": (ctypes.c_int, [_vp, _vp, _u64, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x):
    """Device/host address of a torch tensor, a numpy array, an int address or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    assert x.is_contiguous()
    return x.data_ptr()


def last_error():
    return load().gpt2_last_error().decode()


class GPT2Error(RuntimeError):
    pass


def check(rc, what=""):
    if rc != GPT2_OK:
        raise GPT2Error(f"{what}: status {rc}: {last_error()}")
    return rc


# ---------------------------------------------------------------- C ABI, same names

def make_config(n_layer, n_head, n_embd, vocab, padded_vocab, max_seq, batch, seq, precision=GPT2_BF16,
                linear_bias=1, ln_bias=1, grad_accum=1, grad_clip=0.0, stream=None, workspace=None,
                workspace_bytes=0, recompute=0, no_master=0):
    return gpt2_config(n_layer, n_head, n_embd, vocab, padded_vocab, max_seq, batch, seq, precision, linear_bias,
                       ln_bias, grad_accum, grad_clip, recompute, no_master,
                       _ptr(stream) if stream is not None else None, _ptr(workspace), workspace_bytes)


def gpt2_workspace_bytes(cfg):
    return load().gpt2_workspace_bytes(ctypes.byref(cfg))


def gpt2_init(cfg, seed):
    return load().gpt2_init(ctypes.byref(cfg), seed)


def gpt2_forward(tokens, targets=None):
    return load().gpt2_forward(_ptr(tokens), _ptr(targets))


def gpt2_backward():
    return load().gpt2_backward()


def gpt2_adamw_step(lr, b1, b2, eps, wd, t):
    return load().gpt2_adamw_step(lr, b1, b2, eps, wd, t)


def gpt2_grad_norm():
    return load().gpt2_grad_norm()


def gpt2_skip_update():
    return load().gpt2_skip_update()


def gpt2_grad_sumsq_range(begin, end):
    """Returns (status, sum of g^2 over [begin, end))."""
    out = ctypes.c_double(0.0)
    rc = load().gpt2_grad_sumsq_range(begin, end, ctypes.byref(out))
    return rc, out.value


def gpt2_adamw_step_range(lr, b1, b2, eps, wd, t, begin, end, global_sumsq, finish):
    return load().gpt2_adamw_step_range(lr, b1, b2, eps, wd, t, begin, end, global_sumsq, int(finish))


def gpt2_save(path, t, cursor):
    return load().gpt2_save(os.fsencode(path), t, cursor)


def gpt2_load(path):
    """Returns (status, t, cursor)."""
    t, cur = _i32(0), _u64(0)
    rc = load().gpt2_load(os.fsencode(path), ctypes.byref(t), ctypes.byref(cur))
    return rc, t.value, cur.value


def gpt2_lr_schedule(step, lr_max, warmup, total, final_frac):
    return load().gpt2_lr_schedule(step, lr_max, warmup, total, final_frac)


def gpt2_outlier_reset(d):
    load().gpt2_outlier_reset(ctypes.byref(d))


def gpt2_outlier_update(d, x):
    return load().gpt2_outlier_update(ctypes.byref(d), x)


def gpt2_last_status():
    return load().gpt2_last_status()


def gpt2_num_params():
    return load().gpt2_num_params()


def gpt2_get_params(dst):
    return load().gpt2_get_params(_ptr(dst), dst.size)


def gpt2_set_params(src):
    src = np.ascontiguousarray(src, dtype=np.float32)
    return load().gpt2_set_params(_ptr(src), src.size)


def gpt2_get_grads(dst):
    return load().gpt2_get_grads(_ptr(dst), dst.size)


def gpt2_get_adam_state(m, v):
    return load().gpt2_get_adam_state(_ptr(m), _ptr(v), m.size)


def gpt2_get_logits(dst):
    return load().gpt2_get_logits(_ptr(dst), dst.size)


def gpt2_free():
    load().gpt2_free()


KERNEL_CLASSES = ["encoder_fwd", "layernorm_fwd", "gemm_qkv", "attention_fwd", "gemm_attproj", "gemm_fc",
                  "gemm_fcproj", "gemm_classifier", "cross_entropy", "gemm_classifier_dx", "gemm_classifier_dw",
                  "layernorm_bwd", "gemm_fcproj_dx", "gemm_fcproj_dw", "bias_grad", "gemm_fc_dx", "gemm_fc_dw",
                  "gemm_attproj_dx", "gemm_attproj_dw", "attention_bwd", "gemm_qkv_dx", "gemm_qkv_dw",
                  "encoder_bwd", "grad_norm", "adamw", "attention_bwd_q", "attention_bwd_pre",
                  "weight_transpose", "recompute", "grad_finish"]


def gpt2_profile_enable(mask):
    return load().gpt2_profile_enable(mask)


def gpt2_profile_read(ms, launches):
    return load().gpt2_profile_read(_ptr(ms), _ptr(launches), ms.size)


# ---------------------------------------------------------------- convenience

class Model:
    """Owns the torch workspace and stream pointer of one gpt2_init'ed model."""

    def __init__(self, n_layer, n_head, n_embd, vocab, padded_vocab, max_seq, batch, seq, precision=GPT2_BF16,
                 linear_bias=1, ln_bias=1, grad_accum=1, grad_clip=0.0, seed=1337, device="cuda", recompute=0,
                 no_master=0):
        import torch
        self.torch = torch
        self.stream = torch.cuda.current_stream(device)
        cfg = make_config(n_layer, n_head, n_embd, vocab, padded_vocab, max_seq, batch, seq, precision,
                          linear_bias, ln_bias, grad_accum, grad_clip, recompute=recompute, no_master=no_master)
        nbytes = gpt2_workspace_bytes(cfg)
        if nbytes == 0:
            raise GPT2Error(f"bad config: {last_error()}")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        cfg.stream = self.stream.cuda_stream
        cfg.workspace = self.workspace.data_ptr()
        cfg.workspace_bytes = nbytes
        self.cfg = cfg
        self.B, self.T, self.V = batch, seq, vocab
        check(gpt2_init(cfg, seed), "gpt2_init")
        self.n = gpt2_num_params()

    def forward(self, tokens, targets=None):
        loss = gpt2_forward(tokens, targets)
        if math.isnan(loss) and targets is not None or gpt2_last_status() != GPT2_OK:
            check(gpt2_last_status(), "gpt2_forward")
        return loss

    def backward(self):
        check(gpt2_backward(), "gpt2_backward")

    def step(self, lr, b1, b2, eps, wd, t):
        check(gpt2_adamw_step(lr, b1, b2, eps, wd, t), "gpt2_adamw_step")

    def params(self):
        out = np.empty(self.n, np.float32)
        check(gpt2_get_params(out), "gpt2_get_params")
        return out

    def set_params(self, p):
        check(gpt2_set_params(p), "gpt2_set_params")

    def grads(self):
        out = np.empty(self.n, np.float32)
        check(gpt2_get_grads(out), "gpt2_get_grads")
        return out

    def adam_state(self):
        m = np.empty(self.n, np.float32)
        v = np.empty(self.n, np.float32)
        check(gpt2_get_adam_state(m, v), "gpt2_get_adam_state")
        return m, v

    def logits(self):
        out = np.empty(self.B * self.T * self.V, np.float32)
        check(gpt2_get_logits(out), "gpt2_get_logits")
        return out.reshape(self.B, self.T, self.V)
