"""Pins of the float64 oracle against things other than itself: numbers the pages print, closed
forms, invariants, brute force (finite differences) and independent library routines (torch's
functional ops and torch.optim.AdamW, in float64 on the CPU)."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from transformer_lm_pretraining_gpt_amd import synthetic as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))

TINY = O.Config(n_layer=2, d_model=64, n_head=4, seq_len=64, vocab=512, vocab_padded=512, batch=2)
TINY_PAD = O.Config(n_layer=2, d_model=64, n_head=4, seq_len=64, vocab=500, vocab_padded=512,
                    batch=2)
SMALL_HD64 = O.Config(n_layer=1, d_model=128, n_head=2, seq_len=24, vocab=200, vocab_padded=256,
                      batch=2)


def gpt2_like(cfg, seed=0, std=0.02):
    """GPT-2 style init: matrices N(0, std), biases 0, LayerNorm gain 1 / bias 0."""
    p = np.zeros(O.param_count(cfg))
    P = O.unpack(p, cfg)
    rng = np.random.default_rng(seed)
    for name, shape, off, decays in O.param_layout(cfg):
        if decays:
            P[name][...] = rng.standard_normal(shape) * std
        elif name.endswith(".g"):
            P[name][...] = 1.0
    return p


def random_params(cfg, seed=0, std=0.3):
    """Every parameter random (LN gains and biases too) so that no term can hide behind a 0 or 1."""
    p = S.normal_vector(O.param_count(cfg), seed, std, dtype=np.float64)
    P = O.unpack(p, cfg)
    for name, shape, off, decays in O.param_layout(cfg):
        if name.endswith(".g"):
            P[name][...] += 1.0
    return p


def tokens(cfg, seed=1):
    s = S.uniform_tokens(cfg.rows + 1, seed, cfg.vocab)
    return S.batch_from_stream(s, cfg.batch, cfg.seq_len)


# ------------------------------------------------------------------------------ page values

def test_param_counts_match_pages():
    small = O.Config(12, 768, 12, 1024, 50257, 50257, 1)
    assert O.param_count(small) == 124_439_808
    g = GOLD["params_gpt2_small"]
    assert abs(O.param_count(small) - g["value"]) <= g["tolerance"]
    assert O.param_count(O.Config(12, 768, 12, 1024, 50257, 50304, 16)) == 124_475_904
    xl = O.Config(48, 1600, 25, 1024, 50257, 50257, 1)
    g = GOLD["params_gpt2_1p6b_llmc"]
    assert abs(O.param_count(xl) - g["value"]) <= g["tolerance"]
    # without the linear/LN biases the count would round to 1.557 B: the biases are pinned
    n_bias = 48 * (2 + 3 + 1 + 2 + 4 + 1) * 1600 + 2 * 1600
    assert abs(O.param_count(xl) - n_bias - g["value"]) > g["tolerance"]
    assert O.param_count(TINY) == 136_960


def test_state_bytes_match_pages():
    assert O.state_bytes_fp32_adamw(1) == GOLD["bytes_per_param_fp32_adamw"]["value"]
    xl = O.Config(48, 1600, 25, 1024, 50257, 50257, 1)
    assert O.state_bytes_fp32_adamw(O.param_count(xl)) >= GOLD["zero_1p5b_model_states_min_bytes"]["value"]
    g = GOLD["zero_70b_model_states_bytes"]
    assert abs(O.state_bytes_fp32_adamw(70_000_000_000) - g["value"]) <= g["tolerance"]
    g = GOLD["persistent_state_5p8M_MB"]
    assert abs(O.state_bytes_fp32_adamw(5_800_000) / 2**20 - g["value"]) <= g["tolerance"]


@pytest.mark.parametrize("cfg", [TINY, TINY_PAD, SMALL_HD64])
def test_flop_tally_identity(cfg):
    """The tally the oracle keeps while it runs equals the closed form, and bwd = 2 fwd exactly."""
    x, y = tokens(cfg)
    t = O.Tally()
    O.loss_and_grad(random_params(cfg), x, y, cfg, tally=t)
    assert t.fwd == O.flops_forward(cfg)
    assert (t.fwd + t.bwd) / t.fwd == GOLD["fwd_plus_bwd_over_fwd"]["value"]
    assert t.bwd == 2 * t.fwd
    if cfg is TINY:
        assert t.fwd == 35_684_352


def test_flop_ratios_match_pages():
    """Counted work (dense T^2 attention, as a dispatch-level counter sees it) over 6ND with N
    counting the embeddings: the pages print 1.145 (d=768) and 1.100 (d=1600) at T=1024."""
    def ratio(L, d, H):
        cfg = O.Config(L, d, H, 1024, 50257, 50257, 1)
        return O.flops_step(cfg, "full") / (6 * O.param_count(cfg) * cfg.rows)
    g = GOLD["counted_over_6ND_T1024_d768"]
    assert abs(ratio(12, 768, 12) - g["value"]) <= g["tolerance"]
    g = GOLD["counted_over_6ND_T1024_d1600"]
    assert abs(ratio(48, 1600, 25) - g["value"]) <= g["tolerance"]
    band = GOLD["counted_over_6ND_band"]
    for L, d, H in [(12, 768, 12), (24, 1024, 16), (48, 1600, 25)]:
        assert band["low"] <= ratio(L, d, H) <= band["high"]


def test_initial_loss_matches_page_and_closed_form():
    """GPT-2 small at a GPT-2 init on Zipf tokens: loss ~= ln V + d*std^2/2 (iid Gaussian logits of
    variance d*std^2), and the page's initial validation loss of 10.95."""
    cfg = O.Config(12, 768, 12, 1024, 50257, 50304, 1)
    x, y = S.batch_from_stream(S.zipf_tokens(cfg.rows + 1, 7), 1, 1024)
    loss, rows = O.forward(gpt2_like(cfg, seed=3), x, y, cfg)
    closed = math.log(50257) + 768 * 0.02 ** 2 / 2
    assert abs(loss - closed) < 0.03
    g = GOLD["initial_val_loss_gpt2_small"]
    assert abs(loss - g["value"]) <= g["tolerance"]
    g = GOLD["ln_50304"]
    assert abs(math.log(50304) - g["value"]) <= g["tolerance"]


# ------------------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("cfg", [TINY, TINY_PAD])
def test_zero_embedding_gives_ln_v(cfg):
    """wte = 0 makes every logit 0, so the loss is ln(vocab) exactly: the real vocabulary, not the
    padded width (the padded columns are masked)."""
    p = random_params(cfg)
    O.unpack(p, cfg)["wte"][...] = 0.0
    x, y = tokens(cfg)
    loss, rows = O.forward(p, x, y, cfg)
    assert abs(loss - math.log(cfg.vocab)) < 1e-12
    assert np.allclose(rows, math.log(cfg.vocab), atol=1e-12, rtol=0)


def test_layernorm_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3 + 1.5
    y, xhat, rstd = O.layernorm(x, np.ones(33), np.zeros(33))
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-13)
    assert np.allclose(y.var(axis=1), var / (var + O.gpt2_oracle.LN_EPS), rtol=1e-12)
    g, b = rng.standard_normal(33), rng.standard_normal(33)
    y2, _, _ = O.layernorm(x, g, b)
    assert np.allclose(y2, xhat * g + b, rtol=1e-13)


def test_gelu_special_values():
    assert O.gelu(np.array([0.0]))[0] == 0.0
    big = np.array([30.0, -30.0])
    assert np.allclose(O.gelu(big), [30.0, 0.0], atol=1e-12)
    # tanh form at u = 1: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert abs(O.gelu(np.array([1.0]))[0] - 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) < 1e-15
    u = np.linspace(-4, 4, 41)
    h = 1e-6
    assert np.allclose(O.gelu_grad(u), (O.gelu(u + h) - O.gelu(u - h)) / (2 * h), atol=1e-9)


def test_adamw_closed_form_first_step():
    """At t = 1 the bias-corrected moments are g and g^2: dp = -lr (g / (|g| + eps) + wd p)."""
    rng = np.random.default_rng(0)
    p, g = rng.standard_normal(1000), rng.standard_normal(1000)
    m = v = np.zeros(1000)
    decay = (rng.random(1000) < 0.5).astype(np.float64)
    lr, eps, wd = 6e-4, 1e-8, 0.1
    p1, m1, v1 = O.adamw_update(p, g, m, v, 1, lr, 0.9, 0.95, eps, wd, decay)
    assert np.allclose(p1 - p, -lr * (g / (np.abs(g) + eps) + wd * decay * p), rtol=1e-12, atol=1e-18)
    assert np.allclose(m1, 0.1 * g, rtol=1e-15) and np.allclose(v1, 0.05 * g * g, rtol=1e-15)


def test_adamw_matches_torch_optim():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    n = 257
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) for _ in range(6)]
    decay = np.zeros(n)
    decay[:150] = 1.0
    a = torch.tensor(p0[:150].copy(), dtype=torch.float64, requires_grad=True)
    b = torch.tensor(p0[150:].copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([{"params": [a], "weight_decay": 0.1},
                             {"params": [b], "weight_decay": 0.0}],
                            lr=6e-4, betas=(0.9, 0.95), eps=1e-8)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        a.grad = torch.tensor(g[:150].copy())
        b.grad = torch.tensor(g[150:].copy())
        opt.step()
        p, m, v = O.adamw_update(p, g, m, v, t, 6e-4, 0.9, 0.95, 1e-8, 0.1, decay)
    ref = np.concatenate([a.detach().numpy(), b.detach().numpy()])
    assert np.allclose(p, ref, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------------------ invariants

def test_causal_softmax_rows():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal((37, 16)), rng.standard_normal((37, 16))
    p = O.causal_softmax(q, k)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[np.triu_indices(37, k=1)] == 0.0)
    assert p[0, 0] == 1.0


def test_ce_grad_rows_sum_to_zero_and_pad_is_zero():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((9, 64)) * 4
    y = rng.integers(0, 50, 9)
    dz = O.ce_grad_rows(z, y, vocab=50)
    assert np.allclose(dz.sum(axis=1), 0.0, atol=1e-14)
    assert np.all(dz[:, 50:] == 0.0)


def test_attention_with_one_position_returns_v():
    cfg = O.Config(1, 32, 2, 1, 40, 48, 3)
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((3, 32)) for _ in range(3))
    assert np.array_equal(O.gpt2_oracle.attention_forward(q, k, v, cfg), v)


def test_causality_of_the_loss():
    """Changing token x[b, t] leaves the loss rows of positions < t of row b, and every other row,
    bitwise unchanged, and does change position t."""
    cfg = TINY_PAD
    p = random_params(cfg)
    x, y = tokens(cfg)
    _, r0 = O.forward(p, x, y, cfg)
    b, t = 1, 37
    x2 = x.copy()
    x2[b, t] = (x2[b, t] + 17) % cfg.vocab
    _, r1 = O.forward(p, x2, y, cfg)
    r0, r1 = r0.reshape(cfg.batch, cfg.seq_len), r1.reshape(cfg.batch, cfg.seq_len)
    assert np.array_equal(r0[b, :t], r1[b, :t])
    assert np.array_equal(r0[0], r1[0])
    assert np.all(r0[b, t:] != r1[b, t:])


# ------------------------------------------------------------------------------ brute force

def _fd_check(cfg, seed, masked=False):
    p = random_params(cfg, seed=seed)
    x, y = tokens(cfg, seed=seed + 1)
    if masked:
        y = S.chat_mask(y, seed + 3, prompt_mean=8, answer_mean=8)
    loss, _, g = O.loss_and_grad(p, x, y, cfg)
    rng = np.random.default_rng(seed + 2)
    h = 1e-5
    for name, shape, off, _ in O.param_layout(cfg):
        n = int(np.prod(shape))
        gt = g[off:off + n]
        idx = set(rng.integers(0, n, 8).tolist()) | {int(np.argmax(np.abs(gt)))}
        for i in idx:
            pp, pm = p.copy(), p.copy()
            pp[off + i] += h
            pm[off + i] -= h
            fd = (O.forward(pp, x, y, cfg)[0] - O.forward(pm, x, y, cfg)[0]) / (2 * h)
            assert abs(fd - gt[i]) <= 1e-7 + 1e-5 * abs(gt[i]), (name, i, fd, gt[i])


def test_finite_differences_tiny():
    _fd_check(TINY, 10)


def test_finite_differences_padded_vocab():
    """Pad rows of wte receive exactly zero gradient from the masked head and from the embedding."""
    _fd_check(TINY_PAD, 20)
    cfg = TINY_PAD
    x, y = tokens(cfg)
    _, _, g = O.loss_and_grad(random_params(cfg), x, y, cfg)
    assert np.all(O.unpack(g, cfg)["wte"][cfg.vocab:] == 0.0)


# ------------------------------------------------------------------------------ library routine

def _torch_step(p_np, x, y, cfg):
    """The same model written with torch's own functional ops (float64, CPU), differentiated by
    autograd. Independent of the oracle's formulas."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    p = torch.tensor(p_np, dtype=torch.float64, requires_grad=True)
    P = {name: p[off:off + int(np.prod(shape))].view(*shape)
         for name, shape, off, _ in O.param_layout(cfg)}
    B, T, d, H = cfg.batch, cfg.seq_len, cfg.d_model, cfg.n_head
    xt, yt = torch.tensor(x, dtype=torch.long), torch.tensor(y, dtype=torch.long)
    h = P["wte"][xt] + P["wpe"][:T]
    for l in range(cfg.n_layer):
        pre = f"h{l}."
        a = F.layer_norm(h, (d,), P[pre + "ln1.g"], P[pre + "ln1.b"], eps=1e-5)
        qkv = a @ P[pre + "w_qkv"] + P[pre + "b_qkv"]
        q, k, v = (t.reshape(B, T, H, d // H).transpose(1, 2).contiguous() for t in qkv.split(d, -1))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        o = o.transpose(1, 2).reshape(B, T, d)
        h = h + o @ P[pre + "w_o"] + P[pre + "b_o"]
        c = F.layer_norm(h, (d,), P[pre + "ln2.g"], P[pre + "ln2.b"], eps=1e-5)
        u = c @ P[pre + "w_fc"] + P[pre + "b_fc"]
        h = h + F.gelu(u, approximate="tanh") @ P[pre + "w_proj"] + P[pre + "b_proj"]
    f = F.layer_norm(h, (d,), P["lnf.g"], P["lnf.b"], eps=1e-5)
    z = f @ P["wte"].T
    mask = torch.arange(cfg.vocab_padded) >= cfg.vocab
    z = z.masked_fill(mask, float("-inf"))
    loss = F.cross_entropy(z.reshape(-1, cfg.vocab_padded), yt.reshape(-1), ignore_index=-1)
    loss.backward()
    return loss.item(), p.grad.numpy()


@pytest.mark.parametrize("cfg", [TINY, TINY_PAD, SMALL_HD64])
def test_matches_torch_functional_autograd(cfg):
    p = random_params(cfg, seed=5, std=0.2)
    x, y = tokens(cfg, seed=6)
    loss, _, g = O.loss_and_grad(p, x, y, cfg)
    tl, tg = _torch_step(p, x, y, cfg)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    for name, shape, off, _ in O.param_layout(cfg):
        n = int(np.prod(shape))
        ref = tg[off:off + n]
        err = np.abs(g[off:off + n] - ref).max()
        assert err <= 1e-10 * max(np.abs(ref).max(), 1e-30), name


# ------------------------------------------------------------------------------ untrained positions

def _chat(cfg, seed):
    x, y = tokens(cfg, seed=seed)
    return x, y, S.chat_mask(y, seed + 100, prompt_mean=8, answer_mean=8)


def test_masked_loss_is_mean_over_trained_rows():
    """The forward never reads the targets except to pick z[y]: with some targets at -1 the other
    rows keep exactly their losses, the ignored rows report 0 and the loss is the mean over the
    trained rows."""
    cfg = TINY_PAD
    p = random_params(cfg, seed=7)
    x, y, ym = _chat(cfg, 8)
    keep = ym.reshape(-1) != O.IGNORE
    assert 0 < keep.sum() < keep.size
    _, rows = O.forward(p, x, y, cfg)
    loss_m, rows_m = O.forward(p, x, ym, cfg)
    assert np.array_equal(rows_m[keep], rows[keep]) and np.all(rows_m[~keep] == 0.0)
    assert loss_m == pytest.approx(rows[keep].mean(), rel=1e-13)


def test_finite_differences_masked_targets():
    _fd_check(TINY_PAD, 30, masked=True)


@pytest.mark.parametrize("cfg", [TINY_PAD, SMALL_HD64])
def test_masked_targets_match_torch_ignore_index(cfg):
    """torch's cross_entropy with ignore_index = -1 averages over the other positions."""
    p = random_params(cfg, seed=15, std=0.2)
    x, _, ym = _chat(cfg, 16)
    loss, _, g = O.loss_and_grad(p, x, ym, cfg)
    tl, tg = _torch_step(p, x, ym, cfg)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    assert np.abs(g - tg).max() <= 1e-10 * np.abs(tg).max()


def test_every_position_ignored():
    """No trained position: loss 0 and an all-zero gradient (the reading taken where a mean over
    nothing is undefined)."""
    cfg = TINY_PAD
    p = random_params(cfg, seed=17)
    x, y = tokens(cfg, seed=18)
    loss, rows, g = O.loss_and_grad(p, x, np.full_like(y, O.IGNORE), cfg)
    assert loss == 0.0 and np.all(rows == 0.0) and np.all(g == 0.0)


def test_chat_mask_spans():
    """The synthetic chat mask starts each sequence with a prompt and alternates spans."""
    y = np.arange(4 * 300, dtype=np.int32).reshape(4, 300)
    m = S.chat_mask(y, 3, prompt_mean=10, answer_mean=20)
    assert np.all(m[:, 0] == -1)
    kept = m != -1
    assert np.array_equal(m[kept], y[kept])
    frac = 1.0 - kept.mean()
    assert 0.2 < frac < 0.5


def test_full_step_consistency():
    """step() = loss_and_grad() followed by adamw_update() with the 2-D decay mask."""
    cfg = TINY_PAD
    p = random_params(cfg)
    x, y = tokens(cfg)
    m = S.normal_vector(p.size, 3, 0.01, np.float64)
    v = np.abs(S.normal_vector(p.size, 4, 0.01, np.float64))
    loss, rows, g, p1, m1, v1 = O.step(p, m, v, 4, x, y, cfg)
    mask = O.decay_mask(cfg)
    P = O.unpack(mask, cfg)
    assert np.all(P["wte"] == 1) and np.all(P["h0.w_qkv"] == 1) and np.all(P["h1.b_fc"] == 0)
    assert np.all(P["lnf.g"] == 0) and np.all(P["wpe"] == 1)
    e1, e2 = O.adamw_update(p, g, m, v, 4, 6e-4, 0.9, 0.95, 1e-8, 0.1, mask)[:2]
    assert np.array_equal(p1, e1) and np.array_equal(m1, e2)


# ------------------------------------------------------------------------------ inputs

def test_zipf_stream_mass():
    """Mass of id 0 is 1 / H(V, 1.1); ids stay inside the real vocabulary."""
    s = S.zipf_tokens(400_000, 1234)
    H = np.sum(np.arange(1, 50258, dtype=np.float64) ** -1.1)
    assert abs((s == 0).mean() - 1 / H) < 0.003
    assert s.min() >= 0 and s.max() < 50257
    x, y = S.batch_from_stream(s, 4, 1000)
    assert np.array_equal(x.reshape(-1)[1:], y.reshape(-1)[:-1])
