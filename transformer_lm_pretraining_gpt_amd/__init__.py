"""GPT-2 pretraining step (forward, backward, AdamW) as hand-written HIP kernels for MI355X.

The compute lives in libgpt2.so (C ABI declared in include/gpt2.h); ``gpt2`` is its ctypes
binding, ``configs`` the named workloads, ``synthetic`` the seeded input generators.
"""
from .configs import PEAK_BF16_FLOPS, PRESETS, flops_per_token, param_count  # noqa: F401


def __getattr__(name):
    # the binding (and torch) load only when asked for
    if name in ("GPT2", "Config", "GPT2Error", "load_library", "op_gemm", "op_attention_forward",
                "op_attention_backward", "workspace_bytes"):
        from . import gpt2
        return getattr(gpt2, name)
    raise AttributeError(name)
