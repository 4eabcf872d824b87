"""ctypes binding of libgpt2.so (include/gpt2.h): argument marshalling only.

Every step of the training step runs in the library's HIP kernels; PyTorch only provides the
device arena (one uint8 tensor), the token/target/loss buffers and the stream. If the library is
missing this module raises: there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpt2.so")

GPT2_OK, GPT2_E_INVALID, GPT2_E_NOMEM, GPT2_E_HIP, GPT2_E_STATE, GPT2_E_UNSUPPORTED, \
    GPT2_E_DEVICE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "OK", -1: "INVALID", -2: "NOMEM", -3: "HIP", -4: "STATE", -5: "UNSUPPORTED",
                -6: "DEVICE"}
FP32, BF16 = 0, 1
TIMING_FAMILIES = {"lm_head_gemm": 0, "gemm": 1, "attention_fwd": 2, "xent": 3, "adamw": 4,
                   "gemm_dw": 5, "attention_bwd": 6, "ln_fwd": 7, "ln_bwd": 8, "splitk_sum": 9,
                   "colsum": 10, "embedding": 11, "gemm_fwd": 12, "gemm_dx": 13}


class Config(ctypes.Structure):
    _fields_ = [("n_layer", c_int32), ("d_model", c_int32), ("n_head", c_int32),
                ("seq_len", c_int32), ("vocab", c_int32), ("vocab_padded", c_int32),
                ("batch", c_int32), ("precision", c_int32), ("seed", c_uint64),
                ("init_std", c_float), ("reserved", c_int32)]

    @classmethod
    def make(cls, n_layer, d_model, n_head, seq_len, vocab, vocab_padded, batch,
             precision="bf16", seed=1234, init_std=0.02):
        p = {"fp32": FP32, "bf16": BF16}.get(precision, precision)
        return cls(n_layer, d_model, n_head, seq_len, vocab, vocab_padded, batch, p, seed,
                   init_std, 0)

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class GPT2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gpt2 status {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load libgpt2.so (after torch, so that both share one HIP runtime) and declare signatures.
    The library is the in-tree build unless GPT2_LIBRARY names another build of it."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("GPT2_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run: python -m transformer_lm_pretraining_gpt_amd.build")
    try:
        import torch  # noqa: F401  (binds the HIP runtime torch ships before ours is loaded)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    st = c_int32
    sig = {
        "gpt2_workspace_bytes": (c_size_t, [POINTER(Config)]),
        "gpt2_param_count": (st, [POINTER(Config), POINTER(c_size_t)]),
        "gpt2_init": (st, [POINTER(Config), c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
        "gpt2_forward_loss": (st, [c_void_p, c_void_p, c_void_p, c_void_p]),
        "gpt2_backward": (st, [c_void_p, c_float, c_int32]),
        "gpt2_adamw_step": (st, [c_void_p, c_float, c_float, c_float, c_float, c_float]),
        "gpt2_clip_grad_norm": (st, [c_void_p, c_float, c_void_p]),
        "gpt2_check": (st, [c_void_p]),
        "gpt2_join": (st, [c_void_p]),
        "gpt2_destroy": (st, [c_void_p]),
        "gpt2_copy_params": (st, [c_void_p, c_int32, c_void_p, c_size_t]),
        "gpt2_copy_grads": (st, [c_void_p, c_int32, c_void_p, c_size_t]),
        "gpt2_copy_adam_state": (st, [c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                      POINTER(c_int64)]),
        "gpt2_copy_row_loss": (st, [c_void_p, c_void_p, c_size_t]),
        "gpt2_timing_begin": (st, [c_void_p, c_int32]),
        "gpt2_timing_end": (st, [c_void_p, POINTER(c_double), POINTER(c_int64), POINTER(c_double)]),
        "gpt2_last_error": (ctypes.c_char_p, []),
        "gpt2_op_gemm": (st, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                              c_int64, c_void_p, c_int64, c_void_p, c_int64, c_float, c_float,
                              c_void_p]),
        "gpt2_op_gemm_epilogue": (st, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                       c_int64, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
                                       c_int64, c_void_p, c_void_p, c_float, c_void_p]),
        "gpt2_op_attention_forward": (st, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                           c_void_p, c_void_p, c_void_p]),
        "gpt2_op_attention_backward": (st, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p]),
        "gpt2_op_attention_backward_noalloc": (st, [c_int32, c_int32, c_int32, c_int32, c_int32,
                                                    c_void_p, c_void_p, c_void_p, c_void_p,
                                                    c_void_p, c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != GPT2_OK:
        raise GPT2Error(status, _lib.gpt2_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(cfg: Config) -> int:
    return load_library().gpt2_workspace_bytes(ctypes.byref(cfg))


def param_count(cfg: Config) -> int:
    lib = load_library()
    n = c_size_t(0)
    _check(lib.gpt2_param_count(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


class GPT2:
    """One training context: parameters, AdamW state and activations in a torch-owned arena."""

    def __init__(self, cfg: Config, device: str = "cuda"):
        import torch
        self.lib = load_library()
        self.cfg = cfg
        ws = self.lib.gpt2_workspace_bytes(ctypes.byref(cfg))
        if ws == 0:
            raise GPT2Error(GPT2_E_INVALID, "invalid or unsupported configuration")
        self.arena = torch.empty(ws, dtype=torch.uint8, device=device)
        self.n = param_count(cfg)
        self.rows = cfg.batch * cfg.seq_len
        ctx = c_void_p()
        _check(self.lib.gpt2_init(ctypes.byref(cfg), c_void_p(self.arena.data_ptr()), ws,
                                  c_void_p(_stream()), ctypes.byref(ctx)))
        self.ctx = ctx

    # ---- the four step calls (asynchronous on torch's current stream at init) ----
    def forward_loss(self, tokens, targets, loss=None):
        _check(self.lib.gpt2_forward_loss(self.ctx, _ptr(tokens), _ptr(targets), _ptr(loss)))

    def backward(self, grad_scale: float = 1.0, accumulate: bool = False):
        _check(self.lib.gpt2_backward(self.ctx, grad_scale, 1 if accumulate else 0))

    def adamw_step(self, lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
        _check(self.lib.gpt2_adamw_step(self.ctx, lr, beta1, beta2, eps, weight_decay))

    def clip_grad_norm(self, max_norm: float, norm=None):
        """Clip the gradients to global norm max_norm; the norm before clipping goes to the
        device float tensor ``norm`` when given."""
        _check(self.lib.gpt2_clip_grad_norm(self.ctx, max_norm, _ptr(norm)))

    def check(self):
        _check(self.lib.gpt2_check(self.ctx))

    def join(self):
        """Order torch's current stream after everything the context queued on its internal
        stream (AdamW, weight gradients), without a host wait."""
        _check(self.lib.gpt2_join(self.ctx))

    # ---- synchronous host copies ----
    def params(self) -> np.ndarray:
        out = np.empty(self.n, dtype=np.float32)
        _check(self.lib.gpt2_copy_params(self.ctx, 0, out.ctypes.data, self.n))
        return out

    def set_params(self, p: np.ndarray):
        p = np.ascontiguousarray(p, dtype=np.float32)
        _check(self.lib.gpt2_copy_params(self.ctx, 1, p.ctypes.data, self.n))

    def grads(self) -> np.ndarray:
        out = np.empty(self.n, dtype=np.float32)
        _check(self.lib.gpt2_copy_grads(self.ctx, 0, out.ctypes.data, self.n))
        return out

    def set_grads(self, g: np.ndarray):
        g = np.ascontiguousarray(g, dtype=np.float32)
        _check(self.lib.gpt2_copy_grads(self.ctx, 1, g.ctypes.data, self.n))

    def adam_state(self):
        m = np.empty(self.n, dtype=np.float32)
        v = np.empty(self.n, dtype=np.float32)
        t = c_int64(0)
        _check(self.lib.gpt2_copy_adam_state(self.ctx, 0, m.ctypes.data, v.ctypes.data, self.n,
                                             ctypes.byref(t)))
        return m, v, t.value

    def set_adam_state(self, m, v, t: int):
        m = np.ascontiguousarray(m, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        tt = c_int64(t)
        _check(self.lib.gpt2_copy_adam_state(self.ctx, 1, m.ctypes.data, v.ctypes.data, self.n,
                                             ctypes.byref(tt)))

    def row_loss(self) -> np.ndarray:
        out = np.empty(self.rows, dtype=np.float32)
        _check(self.lib.gpt2_copy_row_loss(self.ctx, out.ctypes.data, self.rows))
        return out

    # ---- per-kernel timing with HIP events on the context's stream ----
    def timing_begin(self, family: str):
        _check(self.lib.gpt2_timing_begin(self.ctx, TIMING_FAMILIES[family]))

    def timing_end(self):
        ms, n, work = c_double(0), c_int64(0), c_double(0)
        _check(self.lib.gpt2_timing_end(self.ctx, ctypes.byref(ms), ctypes.byref(n),
                                        ctypes.byref(work)))
        return ms.value, n.value, work.value

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.gpt2_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- single-kernel entry points (torch tensors in, marshalled to device pointers) ----
def op_gemm(a, b, c, *, a_kmajor: bool, b_kmajor: bool, m: int, n: int, k: int, alpha=1.0,
            beta=0.0, precision="bf16"):
    import torch
    lib = load_library()
    prec = BF16 if precision == "bf16" else FP32
    lda = a.shape[-1]
    ldb = b.shape[-1]
    _check(lib.gpt2_op_gemm(prec, int(a_kmajor), int(b_kmajor), m, n, k, a.data_ptr(), lda,
                            b.data_ptr(), ldb, c.data_ptr(), c.shape[-1], alpha, beta,
                            torch.cuda.current_stream().cuda_stream))


EPI_STORE, EPI_BIAS_GELU, EPI_BIAS_RESID, EPI_GELU_BWD = 0, 1, 2, 3


def op_gemm_epilogue(a, b, c, *, a_kmajor: bool, b_kmajor: bool, m: int, n: int, k: int,
                     epilogue: int, c2=None, bias=None, aux=None, alpha=1.0):
    import torch
    lib = load_library()
    _check(lib.gpt2_op_gemm_epilogue(int(a_kmajor), int(b_kmajor), m, n, k, a.data_ptr(),
                                     a.shape[-1], b.data_ptr(), b.shape[-1], epilogue,
                                     c.data_ptr(), _ptr(c2), c.shape[-1], _ptr(bias), _ptr(aux),
                                     alpha, torch.cuda.current_stream().cuda_stream))


def op_attention_forward(qkv, out, lse, batch, seq_len, n_head, head_dim, precision="bf16"):
    import torch
    lib = load_library()
    prec = BF16 if precision == "bf16" else FP32
    _check(lib.gpt2_op_attention_forward(prec, batch, seq_len, n_head, head_dim, qkv.data_ptr(),
                                         out.data_ptr(), lse.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream))


def op_attention_backward(qkv, out, lse, dout, dqkv, scratch, batch, seq_len, n_head, head_dim,
                          precision="bf16"):
    import torch
    lib = load_library()
    prec = BF16 if precision == "bf16" else FP32
    _check(lib.gpt2_op_attention_backward(prec, batch, seq_len, n_head, head_dim, qkv.data_ptr(),
                                          out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                          dqkv.data_ptr(), scratch.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream))


def op_attention_backward_noalloc(qkv, out, lse, dout, dqkv, batch, seq_len, n_head, head_dim,
                                  precision="bf16"):
    """The attention backward with the library's fixed scratch instead of a caller workspace."""
    import torch
    lib = load_library()
    prec = BF16 if precision == "bf16" else FP32
    _check(lib.gpt2_op_attention_backward_noalloc(prec, batch, seq_len, n_head, head_dim,
                                                  _ptr(qkv), _ptr(out), _ptr(lse), _ptr(dout),
                                                  _ptr(dqkv),
                                                  torch.cuda.current_stream().cuda_stream))
