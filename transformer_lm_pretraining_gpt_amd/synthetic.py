"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle's tests.

This module holds no arithmetic of the training step. It only draws random numbers:

* token streams that stand in for the pages' pretraining corpus (FineWeb-Edu, tokenised with the
  50257-id GPT-2 BPE; neither is available here, see "Criei GPT-2 do zero com uma RTX 4090",
  section "Preparação dos dados"). A Zipf(s) law over the real vocabulary gives the skew that
  natural text has on the embedding scatter and on the cross-entropy targets;
* flat normal vectors, used by oracle-only tests as parameters.

Targets follow the next-token objective ("Pré-treinar um LLM", opening paragraph on the
objective): one stream of M+1 ids is cut into x = s[0:M] and y = s[1:M+1], each viewed (B, T).
"""
from __future__ import annotations

import numpy as np


def zipf_tokens(n: int, seed: int, vocab: int = 50257, s: float = 1.1) -> np.ndarray:
    """n ids in [0, vocab) with P(id = k-1) proportional to k**-s, k = 1..vocab.

    Sampled by inverse CDF: float64 cumulative sum of the unnormalised weights, uniform draws
    from ``numpy.random.default_rng(seed)`` scaled by the total, ``searchsorted(side='right')``.
    """
    if n < 0 or vocab <= 0:
        raise ValueError("n must be >= 0 and vocab > 0")
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-float(s)))
    u = np.random.default_rng(seed).random(n) * cdf[-1]
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def uniform_tokens(n: int, seed: int, vocab: int) -> np.ndarray:
    """n ids uniform over [0, vocab) from ``numpy.random.default_rng(seed)``."""
    return np.random.default_rng(seed).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def batch_from_stream(stream: np.ndarray, batch: int, seq_len: int, index: int = 0):
    """Window ``index`` of a stream of at least (index+1)*B*T + 1 ids -> (x, y), each (B, T) int32."""
    m = batch * seq_len
    lo = index * m
    if stream.shape[0] < lo + m + 1:
        raise ValueError("stream too short for this window")
    x = np.ascontiguousarray(stream[lo:lo + m].reshape(batch, seq_len), dtype=np.int32)
    y = np.ascontiguousarray(stream[lo + 1:lo + m + 1].reshape(batch, seq_len), dtype=np.int32)
    return x, y


def tokens_for(kind: str, batch: int, seq_len: int, vocab: int, seed: int, windows: int = 1):
    """Stream of windows*B*T+1 ids: kind 'zipf' (s=1.1 over ``vocab``) or 'uniform'."""
    n = windows * batch * seq_len + 1
    if kind == "zipf":
        return zipf_tokens(n, seed, vocab)
    if kind == "uniform":
        return uniform_tokens(n, seed, vocab)
    raise ValueError(f"unknown token kind {kind!r}")


def normal_vector(n: int, seed: int, std: float = 0.02, dtype=np.float32) -> np.ndarray:
    """n draws of N(0, std^2) from ``numpy.random.default_rng(seed)``."""
    return (np.random.default_rng(seed).standard_normal(n) * std).astype(dtype)


def chat_mask(y: np.ndarray, seed: int, prompt_mean: int = 48, answer_mean: int = 96) -> np.ndarray:
    """A copy of the targets y (B, T) with the positions of synthetic prompts set to -1.

    Stands in for chat data in which only the assistant's answers are trained ("Criei GPT-2 do zero
    com uma RTX 4090", section on SFT; the chat corpus it uses is not available here): each
    sequence alternates prompt and answer spans, starting with a prompt, with span lengths drawn
    uniformly from [1, 2 * mean - 1] by ``numpy.random.default_rng(seed)``.
    """
    rng = np.random.default_rng(seed)
    out = np.array(y, dtype=np.int32, copy=True)
    B, T = out.shape
    for b in range(B):
        t, prompt = 0, True
        while t < T:
            mean = prompt_mean if prompt else answer_mean
            n = int(rng.integers(1, 2 * mean))
            if prompt:
                out[b, t:t + n] = -1
            t += n
            prompt = not prompt
    return out
