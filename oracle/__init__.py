"""Float64 CPU oracle of one GPT-2 pretraining step. Test infrastructure only: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the HIP library's path."""
from .gpt2_oracle import (IGNORE, Config, Tally, adamw_update, clip_grad_norm, cosine_lr, block_forward, causal_softmax,
                          ce_grad_rows, decay_mask, flops_forward, flops_step, forward, gelu,
                          gelu_grad, layernorm, layernorm_backward, lm_head_loss, loss_and_grad,
                          mean_loss, param_count, param_layout, state_bytes_fp32_adamw, step,
                          trained_count, unpack)

__all__ = ["IGNORE", "Config", "Tally", "adamw_update", "clip_grad_norm", "cosine_lr", "block_forward", "causal_softmax", "ce_grad_rows",
           "decay_mask", "flops_forward", "flops_step", "forward", "gelu", "gelu_grad",
           "layernorm", "layernorm_backward", "lm_head_loss", "loss_and_grad", "mean_loss",
           "param_count", "param_layout", "state_bytes_fp32_adamw", "step", "trained_count",
           "unpack"]
