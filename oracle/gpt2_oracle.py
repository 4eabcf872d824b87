"""Float64 CPU oracle for one GPT-2 pretraining step: forward, backward and AdamW.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything under ``oracle/``. The HIP library never does, and this
module imports nothing from it: the two share no code. The only shared input is the flat parameter
vector in the canonical order written out in :func:`param_layout`.

What is computed, and where the pages state it
----------------------------------------------
* Objective. Pretraining keeps the next-token objective: the target of position t is the token at
  t+1, the loss is cross-entropy and the optimiser is AdamW ("Pré-treinar um LLM: dados, compute,
  leis de escala e custo", opening paragraph on the objective).
* Model. GPT-2 small is 12 layers of width 768, built the nanoGPT/build-nanogpt way ("Criei GPT-2
  do zero com uma RTX 4090", sections "Ambiente" and "Configuração do treinamento"). The pages do
  not spell the block out; the plainest reading, used here, is GPT-2's pre-LN block:
  h += attn(LN1(h)); h += mlp(LN2(h)); final LN; tied token embedding / LM head; learned absolute
  positions; biases in every linear layer and LayerNorm; LayerNorm eps 1e-5 with biased variance;
  GELU in its tanh form; causal attention scaled by 1/sqrt(head_dim); no dropout.
* Vocabulary padding. The embedding/LM-head matrix has ``vocab_padded`` rows (50257 -> 50304, a
  multiple of 128, same page, section "Configuração do treinamento"). The padded columns of the
  logits are masked to -inf, so they get probability 0 and gradient 0.
* Backward. Each layer yields a gradient for its input and one for its weights ("Pré-treinar um
  LLM", paragraph deriving the 6ND count). Everything below is plain reverse-mode differentiation
  of the forward, written out formula by formula.
* Positions that are not trained. A target of -1 marks a position whose next token is only read:
  it gets no loss and no gradient, and the loss is the mean over the other positions (0, with zero
  gradient, when there are none). The instruction-tuning run on the first page trains only the
  assistant's answer and its end marker ("Criei GPT-2 do zero com uma RTX 4090", section on SFT,
  list item on training only the answer); its chat markers reuse the spare ids of the padded
  vocabulary (same list), which a configuration with vocab = vocab_padded makes real columns.
* AdamW. Moments m and v per parameter (same page, paragraph on memory), bias-corrected, with
  decay decoupled from the gradient and scaled by the learning rate; decay applies to 2-D tensors
  only.
* FLOP tally. Every matmul this module performs adds 2*m*n*k to the phase it runs in; the two
  attention products count only the unmasked (causal) pairs; backward counts dX, dW, dP, dV, dQ, dK
  and never the forward recomputation it does to save memory. Forward is 2N per token plus the
  attention term, backward twice the forward ("Pré-treinar um LLM", paragraphs on the 6ND
  derivation, on FlopCounterMode and on Kaplan's Eq. (2.2)).

Memory: only each layer's input is kept between the forward and the backward; each layer is
recomputed from it inside its own backward, and attention runs one (batch, head) pair at a time,
so the largest configurations fit in host memory. The LM head runs over row chunks when the logits
would be large; each row's loss is independent of the others, so chunking changes only the order
of the sums that accumulate the tied embedding's gradient.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

LN_EPS = 1e-5
GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


@dataclass(frozen=True)
class Config:
    n_layer: int
    d_model: int
    n_head: int
    seq_len: int
    vocab: int
    vocab_padded: int
    batch: int

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_head

    @property
    def rows(self) -> int:
        return self.batch * self.seq_len


# --------------------------------------------------------------------------------------------
# Parameter layout (canonical flat order; weights stored (in, out) so that y = x @ W + b)
# --------------------------------------------------------------------------------------------

def param_layout(cfg: Config):
    """List of (name, shape, offset, decays) in canonical order."""
    d, Vp, T = cfg.d_model, cfg.vocab_padded, cfg.seq_len
    shapes = [("wte", (Vp, d)), ("wpe", (T, d))]
    for l in range(cfg.n_layer):
        p = f"h{l}."
        shapes += [
            (p + "ln1.g", (d,)), (p + "ln1.b", (d,)),
            (p + "w_qkv", (d, 3 * d)), (p + "b_qkv", (3 * d,)),
            (p + "w_o", (d, d)), (p + "b_o", (d,)),
            (p + "ln2.g", (d,)), (p + "ln2.b", (d,)),
            (p + "w_fc", (d, 4 * d)), (p + "b_fc", (4 * d,)),
            (p + "w_proj", (4 * d, d)), (p + "b_proj", (d,)),
        ]
    shapes += [("lnf.g", (d,)), ("lnf.b", (d,))]
    out, off = [], 0
    for name, shape in shapes:
        out.append((name, shape, off, len(shape) == 2))
        off += int(np.prod(shape))
    return out


def param_count(cfg: Config) -> int:
    name, shape, off, _ = param_layout(cfg)[-1]
    return off + int(np.prod(shape))


def decay_mask(cfg: Config) -> np.ndarray:
    """1.0 for elements of 2-D tensors (decayed by AdamW), 0.0 for biases and LayerNorm params."""
    mask = np.zeros(param_count(cfg), dtype=np.float64)
    for _, shape, off, decays in param_layout(cfg):
        if decays:
            mask[off:off + int(np.prod(shape))] = 1.0
    return mask


def unpack(flat: np.ndarray, cfg: Config) -> dict:
    """Name -> view of ``flat`` with the tensor's shape (no copy, dtype kept)."""
    return {name: flat[off:off + int(np.prod(shape))].reshape(shape)
            for name, shape, off, _ in param_layout(cfg)}


def state_bytes_fp32_adamw(n_params: int) -> int:
    """Persistent bytes of plain fp32 AdamW training: weight, gradient, m and v, 4 bytes each."""
    return 16 * n_params


# --------------------------------------------------------------------------------------------
# FLOP tally
# --------------------------------------------------------------------------------------------

@dataclass
class Tally:
    fwd: int = 0
    bwd: int = 0
    by_phase: dict = field(default_factory=dict)

    def add(self, phase: str, flops: int):
        if phase == "fwd":
            self.fwd += int(flops)
        elif phase == "bwd":
            self.bwd += int(flops)
        else:
            raise ValueError(phase)


def _mm(a: np.ndarray, b: np.ndarray, tally, phase) -> np.ndarray:
    """a @ b, counting 2*m*n*k."""
    if tally is not None:
        tally.add(phase, 2 * a.shape[0] * a.shape[1] * b.shape[1])
    return a @ b


def _causal_pairs(T: int) -> int:
    return T * (T + 1) // 2


def flops_forward(cfg: Config, attention: str = "causal") -> int:
    """Closed form of the forward tally: linear layers + LM head, plus the attention products.

    attention='causal' counts the unmasked pairs (what the oracle tallies); 'full' counts all T^2
    pairs of both products, the way a counter that sees two dense (T, T) matmuls would.
    """
    L, d, T, B, Vp = cfg.n_layer, cfg.d_model, cfg.seq_len, cfg.batch, cfg.vocab_padded
    M = B * T
    dense = 2 * M * (12 * L * d * d + Vp * d)
    pairs = _causal_pairs(T) if attention == "causal" else T * T
    if attention not in ("causal", "full"):
        raise ValueError(attention)
    attn = L * B * cfg.n_head * 2 * (2 * pairs * cfg.head_dim)
    return dense + attn


def flops_step(cfg: Config, attention: str = "causal") -> int:
    """Forward + backward, with backward = 2 x forward."""
    return 3 * flops_forward(cfg, attention)


# --------------------------------------------------------------------------------------------
# Building blocks (forward and backward written out)
# --------------------------------------------------------------------------------------------

def layernorm(x: np.ndarray, g: np.ndarray, b: np.ndarray):
    """Row-wise: mean, biased variance, (x - mean) / sqrt(var + eps) * g + b."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = (x - mu) * rstd
    return xhat * g + b, xhat, rstd


def layernorm_backward(dy: np.ndarray, xhat: np.ndarray, rstd: np.ndarray, g: np.ndarray):
    """dx = rstd * (dxh - mean(dxh) - xhat * mean(dxh * xhat)) with dxh = dy * g."""
    dxh = dy * g
    dx = rstd * (dxh - dxh.mean(axis=-1, keepdims=True)
                 - xhat * (dxh * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def gelu(u: np.ndarray) -> np.ndarray:
    """Tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """Derivative of the tanh form."""
    t = np.tanh(GELU_C * (u + GELU_A * u ** 3))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * u * u)


def causal_softmax(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """P = softmax over j of q_i . k_j / sqrt(hd), with j > i masked to -inf. q, k: (T, hd)."""
    T, hd = q.shape
    s = (q @ k.T) / math.sqrt(hd)
    s[np.triu_indices(T, k=1)] = -np.inf
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def _heads(x: np.ndarray, cfg: Config, b: int, h: int) -> np.ndarray:
    """Rows of batch element b, columns of head h, from an (M, d) matrix."""
    T, hd = cfg.seq_len, cfg.head_dim
    return x[b * T:(b + 1) * T, h * hd:(h + 1) * hd]


def attention_forward(q, k, v, cfg: Config, tally=None, phase="fwd"):
    """Per (batch, head): o = P v with P = causal_softmax(q, k). q, k, v, o: (M, d), heads merged."""
    o = np.empty_like(q)
    T, hd = cfg.seq_len, cfg.head_dim
    for b in range(cfg.batch):
        for h in range(cfg.n_head):
            qb, kb, vb = _heads(q, cfg, b, h), _heads(k, cfg, b, h), _heads(v, cfg, b, h)
            p = causal_softmax(qb, kb)
            _heads(o, cfg, b, h)[...] = p @ vb
            if tally is not None:
                tally.add(phase, 2 * 2 * _causal_pairs(T) * hd)
    return o


def attention_backward(do, q, k, v, cfg: Config, tally=None):
    """dv = P^T do; dP = do v^T; dS = P (dP - rowsum(dP P)); dq = dS k / sqrt(hd); dk = dS^T q / sqrt(hd)."""
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    T, hd = cfg.seq_len, cfg.head_dim
    scale = 1.0 / math.sqrt(hd)
    for b in range(cfg.batch):
        for h in range(cfg.n_head):
            qb, kb, vb = _heads(q, cfg, b, h), _heads(k, cfg, b, h), _heads(v, cfg, b, h)
            dob = _heads(do, cfg, b, h)
            p = causal_softmax(qb, kb)
            _heads(dv, cfg, b, h)[...] = p.T @ dob
            dp = dob @ vb.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            _heads(dq, cfg, b, h)[...] = (ds @ kb) * scale
            _heads(dk, cfg, b, h)[...] = (ds.T @ qb) * scale
            if tally is not None:
                tally.add("bwd", 4 * 2 * _causal_pairs(T) * hd)
    return dq, dk, dv


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def block_forward(h: np.ndarray, P: dict, l: int, cfg: Config, tally=None, phase="fwd"):
    """One pre-LN transformer block. Returns (h_out, cache of everything the backward needs)."""
    pre = f"h{l}."
    d = cfg.d_model
    a, xhat1, rstd1 = layernorm(h, _f64(P[pre + "ln1.g"]), _f64(P[pre + "ln1.b"]))
    qkv = _mm(a, _f64(P[pre + "w_qkv"]), tally, phase) + _f64(P[pre + "b_qkv"])
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = attention_forward(q, k, v, cfg, tally, phase)
    h_mid = h + _mm(o, _f64(P[pre + "w_o"]), tally, phase) + _f64(P[pre + "b_o"])
    c, xhat2, rstd2 = layernorm(h_mid, _f64(P[pre + "ln2.g"]), _f64(P[pre + "ln2.b"]))
    u = _mm(c, _f64(P[pre + "w_fc"]), tally, phase) + _f64(P[pre + "b_fc"])
    g = gelu(u)
    h_out = h_mid + _mm(g, _f64(P[pre + "w_proj"]), tally, phase) + _f64(P[pre + "b_proj"])
    cache = dict(a=a, xhat1=xhat1, rstd1=rstd1, q=q, k=k, v=v, o=o,
                 xhat2=xhat2, rstd2=rstd2, c=c, u=u, g=g)
    return h_out, cache


def block_backward(dh_out: np.ndarray, h_in: np.ndarray, P: dict, l: int, cfg: Config,
                   G: dict, tally=None):
    """Backward of :func:`block_forward`, recomputing its forward from the layer input h_in.

    Adds the layer's parameter gradients into ``G`` (name -> float64 array) and returns dh_in.
    """
    pre = f"h{l}."
    _, C = block_forward(h_in, P, l, cfg, tally=None)
    # h_out = h_mid + g @ W_proj + b_proj
    G[pre + "w_proj"] += _mm(C["g"].T, dh_out, tally, "bwd")
    G[pre + "b_proj"] += dh_out.sum(axis=0)
    dg = _mm(dh_out, _f64(P[pre + "w_proj"]).T, tally, "bwd")
    du = dg * gelu_grad(C["u"])
    # u = c @ W_fc + b_fc
    G[pre + "w_fc"] += _mm(C["c"].T, du, tally, "bwd")
    G[pre + "b_fc"] += du.sum(axis=0)
    dc = _mm(du, _f64(P[pre + "w_fc"]).T, tally, "bwd")
    dx2, dg2, db2 = layernorm_backward(dc, C["xhat2"], C["rstd2"], _f64(P[pre + "ln2.g"]))
    G[pre + "ln2.g"] += dg2
    G[pre + "ln2.b"] += db2
    dh_mid = dh_out + dx2
    # h_mid = h_in + o @ W_o + b_o
    G[pre + "w_o"] += _mm(C["o"].T, dh_mid, tally, "bwd")
    G[pre + "b_o"] += dh_mid.sum(axis=0)
    do = _mm(dh_mid, _f64(P[pre + "w_o"]).T, tally, "bwd")
    dq, dk, dv = attention_backward(do, C["q"], C["k"], C["v"], cfg, tally)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    # qkv = a @ W_qkv + b_qkv
    G[pre + "w_qkv"] += _mm(C["a"].T, dqkv, tally, "bwd")
    G[pre + "b_qkv"] += dqkv.sum(axis=0)
    da = _mm(dqkv, _f64(P[pre + "w_qkv"]).T, tally, "bwd")
    dx1, dg1, db1 = layernorm_backward(da, C["xhat1"], C["rstd1"], _f64(P[pre + "ln1.g"]))
    G[pre + "ln1.g"] += dg1
    G[pre + "ln1.b"] += db1
    return dh_mid + dx1


def embed(x: np.ndarray, P: dict, cfg: Config) -> np.ndarray:
    """h0[b, t] = wte[x[b, t]] + wpe[t]; returns (M, d)."""
    wte, wpe = _f64(P["wte"]), _f64(P["wpe"])
    return (wte[x] + wpe[np.arange(cfg.seq_len)][None, :, :]).reshape(cfg.rows, cfg.d_model)


def _lm_chunk_rows(cfg: Config, max_elems: int = 1 << 25) -> int:
    return max(1, min(cfg.rows, max_elems // cfg.vocab_padded))


IGNORE = -1  # target of a position that is not trained


def trained_count(y: np.ndarray) -> int:
    """Number of positions whose target is not IGNORE."""
    return int(np.count_nonzero(np.asarray(y).reshape(-1) != IGNORE))


def mean_loss(rows: np.ndarray, y: np.ndarray) -> float:
    """Mean of the per-row losses over the trained positions; 0 when there are none."""
    keep = np.asarray(y).reshape(-1) != IGNORE
    n = int(np.count_nonzero(keep))
    return float(rows[keep].sum() / n) if n else 0.0


def lm_head_loss(f: np.ndarray, wte: np.ndarray, y: np.ndarray, cfg: Config, tally=None,
                 want_grad: bool = True):
    """Logits z = f @ wte^T with the padded columns at -inf; per-row loss = logsumexp(z) - z[y],
    and 0 on rows whose target is IGNORE.

    Returns (row_losses (M,), df (M, d) or None, dwte (Vp, d) or None), where the gradients are
    those of the MEAN loss over the n trained rows: dz = (softmax(z) - onehot(y)) / n on those rows
    and 0 on the others, df = dz @ wte, dwte = dz^T @ f.
    """
    M, V = cfg.rows, cfg.vocab
    yf = y.reshape(-1)
    n = trained_count(yf)
    rows = np.empty(M)
    df = np.empty_like(f) if want_grad else None
    dwte = np.zeros_like(wte) if want_grad else None
    step = _lm_chunk_rows(cfg)
    for lo in range(0, M, step):
        hi = min(M, lo + step)
        z = _mm(f[lo:hi], wte.T, tally, "fwd")
        z[:, V:] = -np.inf
        zmax = z.max(axis=1, keepdims=True)
        lse = zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))
        yc = yf[lo:hi]
        keep = yc != IGNORE
        r = np.arange(hi - lo)
        rows[lo:hi] = np.where(keep, lse - z[r, np.where(keep, yc, 0)], 0.0)
        if want_grad:
            dz = np.exp(z - lse[:, None])
            dz[r[keep], yc[keep]] -= 1.0
            dz[~keep] = 0.0
            dz /= max(n, 1)
            df[lo:hi] = _mm(dz, wte, tally, "bwd")
            dwte += _mm(dz.T, f[lo:hi], tally, "bwd")
    return rows, df, dwte


def ce_grad_rows(z: np.ndarray, y: np.ndarray, vocab: int) -> np.ndarray:
    """(softmax(z) - onehot(y)) of an (R, Vp) block of logits with columns >= vocab masked."""
    z = np.array(z, dtype=np.float64)
    z[:, vocab:] = -np.inf
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(z.shape[0]), y] -= 1.0
    return p


# --------------------------------------------------------------------------------------------
# Whole step
# --------------------------------------------------------------------------------------------

def forward(params: np.ndarray, x: np.ndarray, y: np.ndarray, cfg: Config, tally=None):
    """Mean loss and per-row losses, shape (M,), of the model at ``params`` (flat, any float dtype)."""
    P = unpack(params, cfg)
    h = embed(x, P, cfg)
    for l in range(cfg.n_layer):
        h, _ = block_forward(h, P, l, cfg, tally, "fwd")
    f, _, _ = layernorm(h, _f64(P["lnf.g"]), _f64(P["lnf.b"]))
    rows, _, _ = lm_head_loss(f, _f64(P["wte"]), y, cfg, tally, want_grad=False)
    return mean_loss(rows, y), rows


def loss_and_grad(params: np.ndarray, x: np.ndarray, y: np.ndarray, cfg: Config, tally=None):
    """Mean loss (over the trained positions), per-row losses and the float64 flat gradient of the
    mean loss."""
    P = unpack(params, cfg)
    grad = np.zeros(param_count(cfg), dtype=np.float64)
    G = unpack(grad, cfg)
    h = embed(x, P, cfg)
    inputs = []
    for l in range(cfg.n_layer):
        inputs.append(h)
        h, _ = block_forward(h, P, l, cfg, tally, "fwd")
    f, xhatf, rstdf = layernorm(h, _f64(P["lnf.g"]), _f64(P["lnf.b"]))
    rows, df, dwte = lm_head_loss(f, _f64(P["wte"]), y, cfg, tally, want_grad=True)
    G["wte"] += dwte
    dh, dgf, dbf = layernorm_backward(df, xhatf, rstdf, _f64(P["lnf.g"]))
    G["lnf.g"] += dgf
    G["lnf.b"] += dbf
    for l in reversed(range(cfg.n_layer)):
        dh = block_backward(dh, inputs[l], P, l, cfg, G, tally)
        inputs[l] = None
    # h0 = wte[x] + wpe[t]: scatter-add into the tied embedding, sum over the batch for positions
    dh3 = dh.reshape(cfg.batch, cfg.seq_len, cfg.d_model)
    np.add.at(G["wte"], x.reshape(-1), dh)
    G["wpe"] += dh3.sum(axis=0)
    return mean_loss(rows, y), rows, grad


def clip_grad_norm(g: np.ndarray, max_norm: float):
    """Global-norm clipping of a flat gradient: norm = sqrt(sum g^2); the gradient times
    max_norm / (norm + 1e-6) when that factor is below 1, else unchanged. Returns (norm, g').
    The pages set no clipping; a training loop may ask for it."""
    g = np.asarray(g, dtype=np.float64)
    norm = math.sqrt(float(np.dot(g, g)))
    coef = max_norm / (norm + 1e-6)
    return norm, (g * coef if coef < 1.0 else g.copy())


def cosine_lr(step: int, total_steps: int, max_lr: float, warmup_steps: int = 0,
              min_lr: float = 0.0) -> float:
    """Learning rate of optimiser step ``step`` (0-based) under a cosine schedule sized to the run:
    linear warm-up over warmup_steps, then max_lr -> min_lr along half a cosine that ends at
    total_steps ("Pré-treinar um LLM", paragraph on Chinchilla's method and learning-rate
    schedules: the cosine must reach its end at the token budget)."""
    if step < warmup_steps:
        return max_lr * (step + 1) / warmup_steps
    if step >= total_steps:
        return min_lr
    x = (step - warmup_steps) / max(1, total_steps - warmup_steps)
    return min_lr + 0.5 * (max_lr - min_lr) * (1.0 + math.cos(math.pi * x))


def adamw_update(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float,
                 weight_decay, decay=None):
    """One AdamW step at step number t (t = 1 on the first step). Returns new (p, m, v) in float64.

    m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
    p = p - lr * ( (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + wd * p ),
    with wd = weight_decay where ``decay`` is 1 and 0 where it is 0 (all ones if None).
    """
    p, g, m, v = _f64(p), _f64(g), _f64(m), _f64(v)
    wd = weight_decay * (np.ones_like(p) if decay is None else _f64(decay))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = p - lr * (mhat / (np.sqrt(vhat) + eps) + wd * p)
    return p, m, v


def step(params, m, v, t: int, x, y, cfg: Config, lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8,
         weight_decay=0.1, tally=None):
    """One full training step: loss and gradient at ``params``, then AdamW at step number t."""
    loss, rows, grad = loss_and_grad(params, x, y, cfg, tally)
    p, m, v = adamw_update(params, grad, m, v, t, lr, beta1, beta2, eps, weight_decay,
                           decay_mask(cfg))
    return loss, rows, grad, p, m, v
