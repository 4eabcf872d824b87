"""The five named workloads of the step (and the 124M model at micro-batch 32) and the FLOP
accounting used for MFU.

Geometry of GPT-2 small/medium/XL; micro-batch and sequence length per workload. The 124M
workload is the one the pages train ("Criei GPT-2 do zero com uma RTX 4090", section
"Configuração do treinamento": 12 layers, width 768, micro-batch 16 x 1024, vocabulary 50257
padded to 50304).
"""
from __future__ import annotations

PRESETS = {
    # name: (n_layer, d_model, n_head, seq_len, vocab, vocab_padded, batch, precision, tokens)
    "tiny": (2, 64, 4, 64, 512, 512, 2, "fp32", "uniform"),
    "gpt2_124m": (12, 768, 12, 1024, 50257, 50304, 16, "bf16", "zipf"),
    "gpt2_350m": (24, 1024, 16, 1024, 50257, 50304, 8, "bf16", "zipf"),
    "gpt2_1p5b": (48, 1600, 25, 1024, 50257, 50304, 4, "bf16", "zipf"),
    "gpt2_124m_t8192": (12, 768, 12, 8192, 50257, 50304, 2, "bf16", "zipf"),
    # not one of the five: the 124M model at twice the micro-batch (32768 rows per step), which
    # one GPU's HBM holds with room to spare
    "gpt2_124m_mb32": (12, 768, 12, 1024, 50257, 50304, 32, "bf16", "zipf"),
}

# MI355X dense bf16 matrix peak: 256 CUs x 2.4 GHz x 4096 FLOP/clock/CU
PEAK_BF16_FLOPS = 256 * 2.4e9 * 4096


def param_count(n_layer, d_model, vocab_padded, seq_len):
    """All parameters as built: tied (Vp, d) embedding, (T, d) positions, 12d^2+13d per layer,
    final LayerNorm."""
    d = d_model
    return vocab_padded * d + seq_len * d + n_layer * (12 * d * d + 13 * d) + 2 * d


def flops_per_token(n_layer, d_model, vocab_padded, seq_len):
    """6N + 6 L T d: three times Kaplan's forward 2N + 2 n_layer n_ctx d_model ("Pré-treinar um
    LLM", paragraphs on the 6ND derivation and on Eq. (2.2)), with N counting the embeddings."""
    n = param_count(n_layer, d_model, vocab_padded, seq_len)
    return 6 * n + 6 * n_layer * seq_len * d_model
