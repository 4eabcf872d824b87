"""Benchmark of one GPT-2 pretraining step (forward + loss, backward, AdamW) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_124m] [--no-cpu]

A step is the whole hot path over one micro-batch of seeded synthetic tokens already resident in
HBM: gpt2_forward_loss + gpt2_backward + gpt2_adamw_step. value = tokens per second over the K
timed steps of the headline workload (GPT-2 124M, T = 1024, micro-batch 16). MFU counts
6N + 6 L T d FLOPs per token ("Pré-treinar um LLM", paragraphs on the 6ND derivation and on
Kaplan's Eq. (2.2), with N counting the embeddings) against the MI355X dense bf16 peak. The other
large workloads (350M, 1.5B, 124M at T = 8192) are timed after it, each in a sub-object. One JSON
line is printed on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

# BLAS threads of the oracle leg, fixed before NumPy is first imported: the machine's CPU share as the
# environment states it (OMP_NUM_THREADS), else every core this process may run on
HOST_THREADS = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(HOST_THREADS))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PAGES_TOKENS_PER_S = 120_000.0  # GPT-2 124M on one RTX 4090 (context only)
HBM_PEAK_GBS = 8000.0
OTHER_WORKLOADS = ("gpt2_350m", "gpt2_1p5b", "gpt2_124m_t8192", "gpt2_124m_mb32")

# families timed per launch by the library: (name, unit of its work figure, roofline)
FAMILIES = (
    ("gemm_fwd", "flop", "mfma"), ("gemm_dx", "flop", "mfma"), ("gemm_dw", "flop", "mfma"),
    ("attention_fwd", "flop", "mfma"), ("attention_bwd", "flop", "mfma"),
    ("ln_fwd", "byte", "hbm"), ("ln_bwd", "byte", "hbm"), ("xent", "byte", "hbm"),
    ("adamw", "byte", "hbm"), ("splitk_sum", "byte", "hbm"), ("colsum", "byte", "hbm"),
    ("embedding", None, "hbm"),
)
FAMILY_KERNELS = {
    "gemm_dw": "gemm_dma_kernel<0,0,256,256,64,3,1,0,8> (weight gradients X^T dY, split-K, and "
               "the tied LM head's dz^T f)",
    "gemm_fwd": "gemm_dma_kernel<1,0,...> forward products and the LM head",
    "gemm_dx": "gemm_dma_kernel<1,1,...> input-gradient products",
    "attention_bwd": "attn_bwd_dkdv64_kernel + attn_bwd_dq64_kernel",
    "ln_bwd": "ln_bwd_kernel", "xent": "xent_kernel", "adamw": "adamw_kernel",
}
GEMM_SOURCES = ("gemm.hip", "lds_dma.h", "common.h", "kernels.h")


def _source_hash(files=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "transformer_lm_pretraining_gpt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(family: str, workload: str):
    """HBM bytes per launch of a family from the committed rocprofv3 counter summary
    (profiles/<family>_traffic.json), or None when it is absent or was taken on another version
    of the kernel sources or another workload."""
    path = os.path.join(ROOT, "profiles", f"{family}_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    files = tuple(t.get("source_files") or GEMM_SOURCES)
    try:
        same = t.get("source_hash") == _source_hash(files)
    except OSError:
        same = False
    if not same or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def device_facts():
    """Compute-unit count and peak engine clock of the gfx950 agent, as rocminfo states them."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return {"source": "rocminfo unavailable"}
    for agent in out.split("*******")[1:]:
        if re.search(r"Name:\s+gfx950", agent):
            cu = re.search(r"Compute Unit:\s+(\d+)", agent)
            clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
            return {"source": "rocminfo", "agent": "gfx950",
                    "compute_units": int(cu.group(1)) if cu else None,
                    "max_sclk_mhz": int(clk.group(1)) if clk else None}
    return {"source": "rocminfo", "agent": "no gfx950 agent listed"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return HOST_THREADS


def cpu_baseline(model, ocfg, x, y):
    """The float64 oracle, untuned, on one sequence of the bench batch: forward, backward and
    AdamW for the full model at seq_len T; plus the tiny configuration single-threaded."""
    import numpy as np

    import oracle as O
    from transformer_lm_pretraining_gpt_amd import PRESETS
    from transformer_lm_pretraining_gpt_amd import synthetic as S
    threads = blas_threads()
    p = model.params()
    one = O.Config(ocfg.n_layer, ocfg.d_model, ocfg.n_head, ocfg.seq_len, ocfg.vocab,
                   ocfg.vocab_padded, 1)
    m = np.zeros(p.size)
    v = np.zeros(p.size)
    t0 = time.perf_counter()
    O.step(p, m, v, 1, x[:1], y[:1], one)
    dt = time.perf_counter() - t0
    out = {"value": round(ocfg.seq_len / dt, 2), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"one full step (float64 forward, backward, AdamW over all {p.size} "
                     f"parameters) on 1 of the {ocfg.batch} sequences ({ocfg.seq_len} tokens) of "
                     f"the bench batch; {dt:.1f} s with {threads} BLAS threads"}
    # the tiny configuration (2 layers, width 64, T 64, batch 2) on one thread
    L, d, H, T, V, Vp, B, _, kind = PRESETS["tiny"]
    tc = O.Config(L, d, H, T, V, Vp, B)
    xt, yt = S.batch_from_stream(S.tokens_for(kind, B, T, V, seed=3), B, T)
    pt = (np.random.default_rng(7).standard_normal(O.param_count(tc)) * 0.02).astype(np.float32)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        O.step(pt, np.zeros(pt.size), np.zeros(pt.size), 1, xt, yt, tc)
    dt1 = (time.perf_counter() - t0) / reps
    if limit is not None:
        limit.unregister() if hasattr(limit, "unregister") else limit.__exit__(None, None, None)
    out["tiny_single_thread"] = {"value": round(B * T / dt1, 1), "unit": "tokens/s", "cores": 1,
                                 "sample": f"tiny config (L=2 d=64 T=64 B=2), mean of {reps} "
                                           f"full steps, {1e3 * dt1:.2f} ms each"}
    return out


class Workload:
    """One model and its seeded token windows, resident in HBM."""

    def __init__(self, name, steps, warmup):
        import torch

        from transformer_lm_pretraining_gpt_amd import PRESETS
        from transformer_lm_pretraining_gpt_amd import gpt2 as G
        from transformer_lm_pretraining_gpt_amd import synthetic as S
        self.torch, self.S = torch, S
        self.name = name
        self.spec = PRESETS[name]
        L, d, H, T, V, Vp, B, prec, kind = self.spec
        self.model = G.GPT2(G.Config.make(L, d, H, T, V, Vp, B, prec, seed=1234))
        self.M = B * T
        self.nwin = warmup + steps
        self.stream = S.tokens_for(kind, B, T, V, seed=1234, windows=self.nwin)
        self.xs, self.ys = [], []
        for i in range(self.nwin):
            x, y = S.batch_from_stream(self.stream, B, T, i)
            self.xs.append(torch.from_numpy(x).cuda())
            self.ys.append(torch.from_numpy(y).cuda())
        self.loss = torch.zeros(1, dtype=torch.float32, device="cuda")

    def step(self, i):
        m = self.model
        m.forward_loss(self.xs[i], self.ys[i], self.loss)
        m.backward(1.0, False)
        m.adamw_step(6e-4, 0.9, 0.95, 1e-8, 0.1)

    def timed(self, first, count):
        """count whole steps from window `first`, an event on the caller's stream before each
        step and one after the last (which waits for that step's AdamW on the library's internal
        stream). Returns per-step milliseconds and the total."""
        torch = self.torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
        torch.cuda.synchronize()
        for k in range(count):
            evs[k].record()
            self.step(first + (k % (self.nwin - first)))
        self.model.join()
        evs[count].record()
        torch.cuda.synchronize()
        per = [evs[k].elapsed_time(evs[k + 1]) for k in range(count)]
        return per, evs[0].elapsed_time(evs[count])

    def family(self, fam, first, count):
        """Per-launch HIP-event timing of one kernel family over `count` steps."""
        self.model.timing_begin(fam)
        for k in range(count):
            self.step(first + (k % (self.nwin - first)))
        self.model.join()
        return self.model.timing_end()

    def close(self):
        self.model.close()
        del self.xs, self.ys
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def _median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def rate_entry(ms, n, work, unit, bound, steps, peak_flops):
    e = {"ms_per_step": round(ms / steps, 4), "launches_per_step": round(n / steps, 2),
         "avg_launch_ms": round(ms / max(n, 1), 5)}
    if unit == "flop" and work > 0:
        r = work / (ms / 1e3)
        e.update({"bound": bound, "achieved": round(r / 1e12, 1), "unit": "TFLOP/s",
                  "peak": round(peak_flops / 1e12, 1), "frac": round(r / peak_flops, 4),
                  "work_per_launch": work / max(n, 1), "work_unit": "FLOP"})
    elif unit == "byte" and work > 0:
        r = work / (ms / 1e3)
        e.update({"bound": bound, "achieved": round(r / 1e9, 1), "unit": "GB/s",
                  "peak": HBM_PEAK_GBS, "frac": round(r / 1e9 / HBM_PEAK_GBS, 4),
                  "work_per_launch": work / max(n, 1), "work_unit": "byte"})
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle's cpu_baseline leg")
    ap.add_argument("--no-breakdown", action="store_true", help="skip per-family kernel timing")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the forward+backward-only, masked-target and 32x gradient-accumulation variants")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 350M, 1.5B and T=8192 workloads")
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB): "
                         "the reference dispatch that scales HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the step on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np  # noqa: F401  (after the thread pinning above)
    import torch

    import oracle as O
    from transformer_lm_pretraining_gpt_amd import PEAK_BF16_FLOPS, flops_per_token

    torch.cuda.set_device(0)
    W = Workload(args.workload, args.steps, args.warmup)
    L, d, H, T, V, Vp, B, prec, kind = W.spec
    M = W.M
    for i in range(args.warmup):
        W.step(i)
    W.model.check()

    # ---- timed region: K whole steps, nothing else on the streams ----
    t0 = time.perf_counter()
    per, ms_total = W.timed(args.warmup, args.steps)
    wall = time.perf_counter() - t0
    W.model.check()
    final_loss = float(W.loss.item())
    ms_per_step = ms_total / args.steps
    tok_s = M * args.steps / (ms_total / 1e3)
    ftok = flops_per_token(L, d, Vp, T)
    mfu = tok_s * ftok / PEAK_BF16_FLOPS

    out = {
        "metric": "train tokens/sec + MFU (6ND+attn FLOPs) for GPT-2 124M, T=1024, 1 GPU",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_median": round(_median(per), 3), "ms_per_step_mean": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(tok_s / PAGES_TOKENS_PER_S, 3),
        "baseline_context": "pages: ~120k tokens/s for GPT-2 124M, micro-batch 16x1024, on one "
                            "RTX 4090 (other hardware, not a target)",
        "mfu": round(mfu, 4), "flops_per_token": ftok, "dtype": prec,
        "data": "synthetic: seeded Zipf(1.1) token stream over 50257 ids; random-init weights",
        "config": {"workload": f"{args.workload}: L={L} d={d} H={H} T={T} vocab={V}->{Vp} "
                               f"micro-batch={B}, forward+backward+AdamW per step",
                   "tokens_per_step": M, "seq_len": T, "micro_batch": B, "parallelism": "none"},
        "device": device_facts(),
        "peak_bf16_tflops": round(PEAK_BF16_FLOPS / 1e12, 1),
        "final_loss": round(final_loss, 4), "wall_s_timed": round(wall, 3),
    }

    # ---- per-family kernel timing, then the roofline of the family that takes the most time ----
    fam_steps = 3
    kernels = {}
    for fam, unit, bound in (() if args.no_breakdown else FAMILIES):
        ms, n, work = W.family(fam, args.warmup, fam_steps)
        if n:
            kernels[fam] = rate_entry(ms, n, work, unit, bound, fam_steps, PEAK_BF16_FLOPS)
    out["kernels"] = kernels
    out["kernels_note"] = ("per family: each launch timed with HIP events on its own stream over "
                           f"{fam_steps} steps of separate passes; the weight-gradient products, "
                           "their split-K sums, the QKV bias sums and AdamW run on the library's "
                           "second stream beside the main stream's chain, so these in-step "
                           "durations include time spent sharing CUs and their sum exceeds the "
                           "step")
    # without the breakdown the weight-gradient family (the largest in every measurement so far)
    dom = max((f for f in kernels if "frac" in kernels[f]), key=lambda f: kernels[f]["ms_per_step"],
              default="gemm_dw")
    unit = dict((f, u) for f, u, _ in FAMILIES)[dom]
    bound = dict((f, b) for f, _, b in FAMILIES)[dom]
    ms, n, work = W.family(dom, args.warmup, args.steps)
    e = rate_entry(ms, n, work, unit, bound, args.steps, PEAK_BF16_FLOPS)
    out["roofline"] = {
        "bound": e["bound"], "achieved": e["achieved"], "peak": e["peak"], "unit": e["unit"],
        "frac": e["frac"], "traffic": _traffic(dom, args.workload),
        "family": dom, "kernel": FAMILY_KERNELS.get(dom, dom),
        "work_per_launch": e["work_per_launch"], "work_unit": e["work_unit"],
        "avg_launch_ms": e["avg_launch_ms"], "launches_timed": n,
        "measured": "HIP events around every launch of the family on the stream it runs on, "
                    f"over a second pass of the {args.steps} timed steps (the headline pass "
                    "carries no per-kernel events)"}

    # ---- the other large workloads ----
    if not args.no_configs:
        cfgs = {}
        W_head = W
        W = None
        for name in OTHER_WORKLOADS:
            if name == args.workload:
                continue
            w = Workload(name, args.config_steps, 5)
            for i in range(5):
                w.step(i)
            w.model.check()
            per_c, tot = w.timed(5, args.config_steps)
            w.model.check()
            Lc, dc, Hc, Tc, Vc, Vpc, Bc, precc, _ = w.spec
            ts = w.M * args.config_steps / (tot / 1e3)
            f = flops_per_token(Lc, dc, Vpc, Tc)
            cfgs[name] = {"tokens_per_s": round(ts, 1), "mfu": round(ts * f / PEAK_BF16_FLOPS, 4),
                          "ms_per_step_mean": round(tot / args.config_steps, 3),
                          "ms_per_step_median": round(_median(per_c), 3),
                          "steps": args.config_steps, "warmup": 5, "flops_per_token": f,
                          "config": f"L={Lc} d={dc} H={Hc} T={Tc} vocab={Vc}->{Vpc} "
                                    f"micro-batch={Bc} {precc}",
                          "final_loss": round(float(w.loss.item()), 4)}
            w.close()
            del w
        out["configs"] = cfgs
        W = W_head

    # ---- variants of the step (separate timings, not part of value) ----
    if not args.no_variants:
        out["variants"] = variants(W, torch)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30}
        del src, dst

    if not args.no_cpu:
        ocfg = O.Config(L, d, H, T, V, Vp, B)
        x0, y0 = W.S.batch_from_stream(W.stream, B, T, 0)
        out["cpu_baseline"] = cpu_baseline(W.model, ocfg, x0, y0)
    W.close()
    print(json.dumps(out))


def variants(W, torch):
    """Three variants of the timed step on the same windows:
    * forward_backward_only: forward_loss + backward without the AdamW step (the optimizer's
      share of the step is the difference to the headline);
    * sft_masked_targets: targets of synthetic prompt spans set to -1 (not trained), the rest as
      in the headline step; tokens/s counts every position processed;
    * grad_accum_32: one AdamW step per 32 micro-batches (forward + backward with accumulate = 1
      and grad_scale = 1/32), the pages' regime of about 0.5M tokens per optimiser step."""
    S, model, M = W.S, W.model, W.M
    first = min(len(W.xs) - 1, 10)
    res = {}
    loss = W.loss
    yms = [torch.from_numpy(S.chat_mask(y.cpu().numpy(), 100 + i)).cuda()
           for i, y in enumerate(W.ys)]
    frac = float(sum((y == -1).sum().item() for y in yms)) / (M * len(yms))
    n = len(W.xs)

    def timed(fn, reps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for r in range(reps):
            fn(r)
        model.join()  # the last AdamW runs on the library's internal stream
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    def masked(r):
        i = first + r % (n - first)
        model.forward_loss(W.xs[i], yms[i], loss)
        model.backward(1.0, False)
        model.adamw_step(6e-4, 0.9, 0.95, 1e-8, 0.1)

    def fwd_bwd(r):
        i = first + r % (n - first)
        model.forward_loss(W.xs[i], W.ys[i], loss)
        model.backward(1.0, False)

    fwd_bwd(0)
    ms = timed(fwd_bwd, 20)
    model.check()
    res["forward_backward_only"] = {"ms_per_step": round(ms, 3),
                                    "tokens_per_s": round(M / (ms / 1e3), 1)}

    masked(0)
    ms = timed(masked, 10)
    model.check()
    res["sft_masked_targets"] = {"ms_per_step": round(ms, 3),
                                 "tokens_per_s": round(M / (ms / 1e3), 1),
                                 "ignored_fraction": round(frac, 4)}
    acc = 32

    def accum(r):
        for k in range(acc):
            i = (r * acc + k) % n
            model.forward_loss(W.xs[i], W.ys[i], loss)
            model.backward(1.0 / acc, k > 0)
        model.adamw_step(6e-4, 0.9, 0.95, 1e-8, 0.1)

    accum(0)
    ms = timed(accum, 2)
    model.check()
    res["grad_accum_32"] = {"ms_per_optimizer_step": round(ms, 2),
                            "tokens_per_optimizer_step": acc * M,
                            "tokens_per_s": round(acc * M / (ms / 1e3), 1)}
    return res


if __name__ == "__main__":
    main()
