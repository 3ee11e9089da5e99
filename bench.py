"""Benchmark: fp32 GPT-2 training step (forward + backward + AdamW) on one MI355X.

python bench.py [--steps K] [--warmup W] [--config 124m] [--gpus 1]

One step = gpt2_forward (ids resident in HBM) + gpt2_zero_grad +
gpt2_backward + gpt2_update, all enqueued on one HIP stream.  W untimed
steps, then K timed steps between two device synchronizations.  Prints one
JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="124m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "see the sharding design notes.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from transformer_lm_step_flat_amd import gpt2, synth

    cfg = synth.config(args.config)
    B, T = cfg["B"], cfg["T"]
    M = gpt2.Model(cfg, B, T, init_params=gpt2.pack_params(cfg, synth.init_params(cfg), B, T))
    nb = 4
    batches = []
    for i in range(nb):
        inp, tgt = synth.batch(cfg, step=i)
        batches.append((torch.from_numpy(inp.ravel()).cuda(), torch.from_numpy(tgt.ravel()).cuda()))
    torch.cuda.synchronize()

    def step(i):
        di, dt = batches[i % nb]
        M.forward(di, dt, want_loss=False)
        M.zero_grad()
        M.backward()
        M.update(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=i + 1)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    dt_s = time.perf_counter() - t0
    M.sync()
    loss = float(M.act("loss")[0].item())
    ms = dt_s / args.steps * 1e3
    tok_s = B * T * args.steps / dt_s
    out = {
        "metric": "train tokens/sec (fwd+bwd+AdamW) GPT-2 124M B=4 T=1024 fp32",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"gpt2 {args.config}: L={cfg['L']} C={cfg['C']} NH={cfg['NH']} "
                               f"V={cfg['V']} (Vp={cfg['Vp']}) B={B} T={T}, seeded N(0,0.02) init, "
                               f"Zipf(1.1) ids" if cfg.get("tokens") == "zipf" else "uniform ids",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "last_loss": loss,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
