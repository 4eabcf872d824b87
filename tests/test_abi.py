"""Host-side tests of the C ABI: the library loads and exports every symbol include/gpt2.h
declares, the config struct matches the C layout, the parameter count matches the oracle's
layout, and every host-checkable misuse returns its status before any GPU work (no GPU needed)."""
import ctypes
import os
import re

import pytest

import oracle as O
from transformer_lm_pretraining_gpt_amd import PRESETS, configs
from transformer_lm_pretraining_gpt_amd import gpt2 as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gpt2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(G.LIB_PATH):
        pytest.fail("libgpt2.so is not built: run python -m transformer_lm_pretraining_gpt_amd.build")
    return G.load_library()


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert len(syms) >= 18
    for s in syms:
        assert hasattr(lib, s), s


def test_config_struct_layout():
    assert ctypes.sizeof(G.Config) == 48
    assert G.Config.seed.offset == 32 and G.Config.init_std.offset == 40


def cfg_of(name, **kw):
    L, d, H, T, V, Vp, B, prec, _ = PRESETS[name]
    c = G.Config.make(L, d, H, T, V, Vp, B, prec)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("name", sorted(PRESETS))
def test_param_count_matches_oracle_layout(lib, name):
    L, d, H, T, V, Vp, B, prec, _ = PRESETS[name]
    ocfg = O.Config(L, d, H, T, V, Vp, B)
    assert G.param_count(cfg_of(name)) == O.param_count(ocfg) == configs.param_count(L, d, Vp, T)
    assert G.workspace_bytes(cfg_of(name)) > 16 * O.param_count(ocfg)


def test_flops_per_token_matches_oracle_tally_form():
    """6N + 6LTd equals 3 x (Kaplan forward 2N + 2 L T d) per token."""
    L, d, H, T, V, Vp, B, _, _ = PRESETS["gpt2_124m"]
    n = configs.param_count(L, d, Vp, T)
    assert configs.flops_per_token(L, d, Vp, T) == 3 * (2 * n + 2 * L * T * d) == 803_478_528


@pytest.mark.parametrize("field,value,status", [
    ("n_head", 5, G.GPT2_E_INVALID),         # 64 % 5 != 0
    ("vocab_padded", 100, G.GPT2_E_INVALID),  # < vocab
    ("n_layer", 0, G.GPT2_E_INVALID),
    ("precision", 7, G.GPT2_E_INVALID),
    ("reserved", 1, G.GPT2_E_INVALID),
    ("vocab_padded", 70000, G.GPT2_E_INVALID),
    ("n_head", 8, G.GPT2_E_UNSUPPORTED),     # head_dim 8
    ("batch", 1100, G.GPT2_E_UNSUPPORTED),   # batch * seq_len > 65536
])
def test_init_rejects_bad_config(lib, field, value, status):
    c = cfg_of("tiny", **{field: value})
    ctx = ctypes.c_void_p()
    st = lib.gpt2_init(ctypes.byref(c), ctypes.c_void_p(4096), 1 << 40, None, ctypes.byref(ctx))
    assert st == status, lib.gpt2_last_error()
    assert ctx.value is None
    assert lib.gpt2_last_error()
    if status == G.GPT2_E_INVALID:
        assert lib.gpt2_workspace_bytes(ctypes.byref(c)) == 0


def test_init_rejects_small_or_null_arena(lib):
    c = cfg_of("tiny")
    ws = lib.gpt2_workspace_bytes(ctypes.byref(c))
    ctx = ctypes.c_void_p()
    assert lib.gpt2_init(ctypes.byref(c), ctypes.c_void_p(4096), ws - 1, None,
                         ctypes.byref(ctx)) == G.GPT2_E_NOMEM
    assert lib.gpt2_init(ctypes.byref(c), None, ws, None, ctypes.byref(ctx)) == G.GPT2_E_INVALID
    assert lib.gpt2_init(ctypes.byref(c), ctypes.c_void_p(4100), ws, None,
                         ctypes.byref(ctx)) == G.GPT2_E_INVALID  # misaligned
    assert lib.gpt2_init(None, ctypes.c_void_p(4096), ws, None, ctypes.byref(ctx)) == G.GPT2_E_INVALID
    assert lib.gpt2_init(ctypes.byref(c), ctypes.c_void_p(4096), ws, None, None) == G.GPT2_E_INVALID


def test_null_context_and_ops_are_rejected(lib):
    assert lib.gpt2_forward_loss(None, None, None, None) == G.GPT2_E_INVALID
    assert lib.gpt2_backward(None, 1.0, 0) == G.GPT2_E_INVALID
    assert lib.gpt2_adamw_step(None, 1e-3, 0.9, 0.95, 1e-8, 0.1) == G.GPT2_E_INVALID
    assert lib.gpt2_clip_grad_norm(None, 1.0, None) == G.GPT2_E_INVALID
    assert lib.gpt2_check(None) == G.GPT2_E_INVALID
    assert lib.gpt2_destroy(None) == G.GPT2_E_INVALID
    assert lib.gpt2_op_gemm(1, 1, 1, 8, 8, 8, None, 8, None, 8, None, 8, 1.0, 0.0, None) == G.GPT2_E_INVALID
    assert lib.gpt2_op_gemm(1, 1, 1, 8, 8, 12, 16, 12, 16, 12, 16, 8, 1.0, 0.0, None) == G.GPT2_E_UNSUPPORTED
    epi = lib.gpt2_op_gemm_epilogue
    assert epi(1, 1, 8, 8, 8, None, 8, None, 8, 0, None, None, 8, None, None, 1.0, None) == G.GPT2_E_INVALID
    assert epi(1, 1, 8, 8, 8, 16, 8, 16, 8, 7, 16, None, 8, None, None, 1.0, None) == G.GPT2_E_INVALID
    assert epi(1, 1, 8, 8, 8, 16, 8, 16, 8, 1, 16, None, 8, None, None, 1.0, None) == G.GPT2_E_INVALID
    assert epi(1, 1, 8, 8, 8, 16, 8, 16, 8, 2, 16, None, 8, None, None, 1.0, None) == G.GPT2_E_INVALID
    assert epi(1, 1, 8, 12, 8, 16, 8, 16, 8, 0, 16, None, 16, None, None, 1.0, None) == G.GPT2_E_UNSUPPORTED
    assert epi(1, 1, 8, 8, 8, 16, 8, 24, 8, 0, 16, None, 8, None, None, 1.0, None) == G.GPT2_E_UNSUPPORTED
    assert lib.gpt2_op_attention_forward(1, 1, 8, 1, 48, 16, 16, 16, None) == G.GPT2_E_UNSUPPORTED
    # the fixed-scratch attention backward: NULL buffers, and sizes beyond its array, are refused
    # before any GPU work
    noalloc = lib.gpt2_op_attention_backward_noalloc
    assert noalloc(1, 1, 64, 1, 64, None, 16, 16, 16, 16, None) == G.GPT2_E_INVALID
    assert noalloc(1, 1, 64, 1, 48, 16, 16, 16, 16, 16, None) == G.GPT2_E_UNSUPPORTED
    assert noalloc(1, 512, 1025, 1, 64, 16, 16, 16, 16, 16, None) == G.GPT2_E_UNSUPPORTED
    assert b"exceed" in lib.gpt2_last_error()
    assert lib.gpt2_join(None) == G.GPT2_E_INVALID
    pc = ctypes.c_size_t()
    assert lib.gpt2_param_count(None, ctypes.byref(pc)) == G.GPT2_E_INVALID
