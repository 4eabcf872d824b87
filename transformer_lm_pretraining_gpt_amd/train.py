"""Training-loop shell around the step: learning-rate schedule, gradient accumulation, optional
global-norm clipping, periodic checkpoints with bit-exact resume, and evaluation that cannot stop
the run.

What the pages ask of such a loop:
* checkpoints every 500 optimiser steps and a resume from the last one after the run stopped
  ("Criei GPT-2 do zero com uma RTX 4090", section on the incident that stopped training after
  2.5 hours);
* evaluation wrapped so that its failure does not stop training (same section: a failure outside
  the core, evaluation or logging, must not bring the run down);
* a cosine learning-rate schedule whose end is the token budget of the run ("Pré-treinar um LLM",
  paragraph on Chinchilla's method and learning-rate schedules);
* 32 micro-batches of 16 x 1024 tokens per optimiser step, about 520k tokens ("Criei GPT-2 do
  zero", table of the training configuration).

The step itself is the C ABI (``gpt2.GPT2``); this module only sequences calls. Any object with the
methods of :class:`StepModel` can be driven, which lets the failure and resume logic be tested on
the CPU. A checkpoint holds the fp32 parameters, both AdamW moments, the AdamW step count and the
next optimiser step; the data of a step is a pure function of its index, so a run resumed from a
checkpoint repeats the uninterrupted run bit for bit.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import asdict, dataclass
from typing import Callable, Optional, Protocol

import numpy as np


def cosine_lr(step: int, total_steps: int, max_lr: float, warmup_steps: int = 0,
              min_lr: float = 0.0) -> float:
    """Learning rate of optimiser step ``step`` (0-based): a linear warm-up over warmup_steps, then
    half a cosine from max_lr down to min_lr that ends exactly at total_steps (and stays there)."""
    if step < warmup_steps:
        return max_lr * (step + 1) / warmup_steps
    if step >= total_steps:
        return min_lr
    frac = (step - warmup_steps) / max(1, total_steps - warmup_steps)
    return min_lr + (max_lr - min_lr) * 0.5 * (1.0 + math.cos(math.pi * frac))


def steps_for_budget(token_budget: int, tokens_per_step: int) -> int:
    """Optimiser steps that a token budget buys (the schedule ends with the budget)."""
    if token_budget <= 0 or tokens_per_step <= 0:
        raise ValueError("token_budget and tokens_per_step must be positive")
    return -(-token_budget // tokens_per_step)


@dataclass
class LoopConfig:
    total_steps: int                 # optimiser steps of the whole run (the schedule's length)
    grad_accum: int = 1              # micro-batches per optimiser step
    max_lr: float = 6e-4
    min_lr: float = 0.0              # the schedule decays to zero at the end of the budget
    warmup_steps: int = 0
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    clip_norm: Optional[float] = None   # global-norm clipping threshold; None = no clipping
    checkpoint_every: int = 500
    checkpoint_dir: Optional[str] = None
    eval_every: int = 0              # 0 = never

    def validate(self):
        if self.total_steps < 1 or self.grad_accum < 1:
            raise ValueError("total_steps and grad_accum must be >= 1")
        if self.checkpoint_every < 1:
            raise ValueError("checkpoint_every must be >= 1")
        if self.clip_norm is not None and not self.clip_norm > 0:
            raise ValueError("clip_norm must be positive")


class StepModel(Protocol):
    """What the loop needs from a model (``GPT2Steps`` adapts the C ABI binding)."""

    def micro_step(self, tokens, targets, grad_scale: float, accumulate: bool) -> None: ...
    def clip(self, max_norm: float) -> None: ...
    def optimizer_step(self, lr: float, beta1: float, beta2: float, eps: float,
                       weight_decay: float) -> None: ...
    def last_loss(self) -> float: ...
    def get_state(self) -> dict: ...
    def set_state(self, state: dict) -> None: ...


class GPT2Steps:
    """StepModel over ``gpt2.GPT2``: the loss of each micro-batch goes to a device float; reading
    it (``last_loss``) synchronises, so the loop reads it only when it logs."""

    def __init__(self, model):
        import torch
        self.model = model
        self.loss = torch.zeros(1, dtype=torch.float32, device="cuda")

    def micro_step(self, tokens, targets, grad_scale, accumulate):
        self.model.forward_loss(tokens, targets, self.loss)
        self.model.backward(grad_scale, accumulate)

    def clip(self, max_norm):
        self.model.clip_grad_norm(max_norm)

    def optimizer_step(self, lr, beta1, beta2, eps, weight_decay):
        self.model.adamw_step(lr, beta1, beta2, eps, weight_decay)

    def last_loss(self):
        return float(self.loss.item())

    def get_state(self):
        m, v, t = self.model.adam_state()
        return {"params": self.model.params(), "m": m, "v": v, "t": int(t)}

    def set_state(self, state):
        self.model.set_params(np.asarray(state["params"], dtype=np.float32))
        self.model.set_adam_state(np.asarray(state["m"], dtype=np.float32),
                                  np.asarray(state["v"], dtype=np.float32), int(state["t"]))


def save_checkpoint(path: str, state: dict, next_step: int, cfg: LoopConfig):
    """Write the state atomically: a temporary file in the same folder, then a rename, so that a
    crash mid-write leaves the previous checkpoint intact."""
    folder = os.path.dirname(os.path.abspath(path))
    os.makedirs(folder, exist_ok=True)
    tmp = path + ".tmp"
    with open(tmp, "wb") as f:
        np.savez(f, params=state["params"], m=state["m"], v=state["v"],
                 t=np.int64(state["t"]), next_step=np.int64(next_step),
                 config=np.frombuffer(json.dumps(asdict(cfg)).encode(), dtype=np.uint8))
        f.flush()
        os.fsync(f.fileno())
    os.replace(tmp, path)


def load_checkpoint(path: str):
    """(state, next_step, loop config as a dict); arrays only, nothing is unpickled."""
    with np.load(path, allow_pickle=False) as z:
        state = {"params": z["params"], "m": z["m"], "v": z["v"], "t": int(z["t"])}
        next_step = int(z["next_step"])
        cfg = json.loads(bytes(z["config"]).decode())
    return state, next_step, cfg


def latest_checkpoint(folder: str) -> Optional[str]:
    """The checkpoint of the highest step in folder (names step_XXXXXXXX.npz), or None."""
    if not folder or not os.path.isdir(folder):
        return None
    names = sorted(n for n in os.listdir(folder) if n.startswith("step_") and n.endswith(".npz"))
    return os.path.join(folder, names[-1]) if names else None


class Trainer:
    """Runs optimiser steps [start, total_steps) of a LoopConfig.

    ``batch(step, micro)`` returns the (tokens, targets) of micro-batch ``micro`` of optimiser step
    ``step``; it must depend on nothing else for a resumed run to repeat the original. ``evaluate``
    (optional) is called as evaluate(step) every eval_every steps; an exception from it is recorded
    in ``eval_failures`` and the run goes on. An exception from the step itself stops the run: the
    caller resumes from the last checkpoint.
    """

    def __init__(self, model: StepModel, cfg: LoopConfig, batch: Callable[[int, int], tuple],
                 evaluate: Optional[Callable[[int], object]] = None,
                 log: Optional[Callable[[str], None]] = None, log_every: int = 0):
        cfg.validate()
        self.model, self.cfg, self.batch, self.evaluate = model, cfg, batch, evaluate
        self.log = log or (lambda s: None)
        self.log_every = log_every
        self.step = 0
        self.history: list[tuple[int, float, float]] = []   # (step, lr, loss) where logged
        self.eval_results: list[tuple[int, object]] = []
        self.eval_failures: list[tuple[int, str]] = []

    def lr(self, step: int) -> float:
        c = self.cfg
        return cosine_lr(step, c.total_steps, c.max_lr, c.warmup_steps, c.min_lr)

    def checkpoint_path(self, next_step: int) -> str:
        return os.path.join(self.cfg.checkpoint_dir, f"step_{next_step:08d}.npz")

    def save(self, path: Optional[str] = None) -> str:
        path = path or self.checkpoint_path(self.step)
        save_checkpoint(path, self.model.get_state(), self.step, self.cfg)
        return path

    def resume(self, path: Optional[str] = None) -> bool:
        """Load the given checkpoint, or the latest one in checkpoint_dir; False if there is none."""
        path = path or latest_checkpoint(self.cfg.checkpoint_dir)
        if path is None:
            return False
        state, next_step, _ = load_checkpoint(path)
        self.model.set_state(state)
        self.step = next_step
        self.log(f"resumed from {path} at step {next_step}")
        return True

    def run_step(self):
        c, s = self.cfg, self.step
        for k in range(c.grad_accum):
            tokens, targets = self.batch(s, k)
            self.model.micro_step(tokens, targets, 1.0 / c.grad_accum, k > 0)
        if c.clip_norm is not None:
            self.model.clip(c.clip_norm)
        lr = self.lr(s)
        self.model.optimizer_step(lr, c.beta1, c.beta2, c.eps, c.weight_decay)
        self.step = s + 1
        return lr

    def run(self, until: Optional[int] = None):
        c = self.cfg
        end = c.total_steps if until is None else min(until, c.total_steps)
        while self.step < end:
            lr = self.run_step()
            done = self.step
            if self.log_every and done % self.log_every == 0:
                loss = self.model.last_loss()
                self.history.append((done - 1, lr, loss))
                self.log(f"step {done - 1} lr {lr:.3e} loss {loss:.4f}")
            if c.eval_every and self.evaluate is not None and done % c.eval_every == 0:
                try:
                    self.eval_results.append((done, self.evaluate(done)))
                except Exception as e:  # evaluation is outside the core: it must not stop the run
                    self.eval_failures.append((done, f"{type(e).__name__}: {e}"))
                    self.log(f"evaluation at step {done} failed ({type(e).__name__}: {e}); "
                             "training goes on")
            if c.checkpoint_dir and done % c.checkpoint_every == 0:
                self.log(f"checkpoint {self.save()}")
        return self
