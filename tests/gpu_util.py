"""Shared helpers of the GPU parity tests (imported by test modules only)."""
import numpy as np

import oracle as O
from transformer_lm_pretraining_gpt_amd import synthetic as S

# fp32 path bars and bf16 path bars of the step
FP32_LOSS_REL, FP32_GRAD_REL = 1e-5, 1e-4
BF16_LOSS_REL, BF16_GRAD_COS = 1e-2, 0.999


def torch_cuda():
    import pytest
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make(G, spec, seed=1234):
    L, d, H, T, V, Vp, B, prec, kind = spec
    cfg = G.Config.make(L, d, H, T, V, Vp, B, prec, seed=seed)
    ocfg = O.Config(L, d, H, T, V, Vp, B)
    return G.GPT2(cfg), ocfg, kind


def tokens(kind, ocfg, seed):
    s = S.tokens_for(kind, ocfg.batch, ocfg.seq_len, ocfg.vocab, seed)
    return S.batch_from_stream(s, ocfg.batch, ocfg.seq_len)


def gpu_forward_backward(torch, model, x, y, grad_scale=1.0, accumulate=False):
    xt = torch.from_numpy(x).cuda()
    yt = torch.from_numpy(y).cuda()
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    model.forward_loss(xt, yt, loss)
    model.backward(grad_scale, accumulate)
    model.check()
    return float(loss.item()), model.row_loss(), model.grads()


def per_tensor(ocfg, flat):
    return {name: flat[off:off + int(np.prod(shape))]
            for name, shape, off, _ in O.param_layout(ocfg)}


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def normwise_rel(a, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.abs(np.asarray(a, np.float64) - ref).max() / max(np.abs(ref).max(), 1e-300))


def truncate_params(p, ocfg, t_cut):
    """The same parameters for a model whose position table has only t_cut rows."""
    small = O.Config(ocfg.n_layer, ocfg.d_model, ocfg.n_head, t_cut, ocfg.vocab,
                     ocfg.vocab_padded, 1)
    out = np.empty(O.param_count(small), dtype=p.dtype)
    big = per_tensor(ocfg, p)
    for name, shape, off, _ in O.param_layout(small):
        n = int(np.prod(shape))
        src = big[name]
        out[off:off + n] = src[:n]  # wpe rows are a prefix; every other tensor has equal size
    return out, small
