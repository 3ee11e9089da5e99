"""Seeded synthetic workloads: model shapes, initial weights and token batches.

This module holds no arithmetic of the training step.  It only draws numbers:
it is the one piece that both the GPU path and the CPU oracle consume, so that
the two see the same bytes.  Each tensor is returned by name; each side places
the named tensors into its own flat layout.

No public dataset is used.  The pages' workloads (a 65-character text, a
vocabulary-1000 subword corpus, GPT-2's 50257-token vocabulary) are stood in
for by uniform character-level tokens (V=65) and Zipf(s=1.1) tokens over V,
which mimic the rank-frequency shape of subword text.
"""
from __future__ import annotations

import math

import numpy as np

# Model/batch shapes.  maxT is the number of position-embedding rows.
CONFIGS = {
    # L=2, C=64, 4 heads, T=64, B=4, V=65 (character level), uniform tokens, 1 step
    "tiny": dict(L=2, C=64, NH=4, T=64, B=4, V=65, maxT=64, tokens="uniform"),
    # L=8, C=128, 8 heads, T=256, B=32, V=1000, Zipf tokens, 10 steps
    "small": dict(L=8, C=128, NH=8, T=256, B=32, V=1000, maxT=256, tokens="zipf"),
    # GPT-2 124M shape: L=12, C=768, 12 heads, T=1024, B=4, V=50257 (head padded to 50304)
    "124m": dict(L=12, C=768, NH=12, T=1024, B=4, V=50257, maxT=1024, tokens="zipf"),
    # the same model at B=16
    "124m_b16": dict(L=12, C=768, NH=12, T=1024, B=16, V=50257, maxT=1024, tokens="zipf"),
    # GPT-2 XL shape: L=48, C=1600, 25 heads (head dim 64), T=1024, B=4
    "xl": dict(L=48, C=1600, NH=25, T=1024, B=4, V=50257, maxT=1024, tokens="zipf"),
}

INIT_SEED = 1337
DATA_SEED = 42
ZIPF_S = 1.1

PARAM_NAMES = ("wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb")


def padded_vocab(V: int) -> int:
    """The head's column count: V rounded up to a multiple of 128."""
    return (V + 127) // 128 * 128


def config(name_or_dict, **overrides) -> dict:
    """A full config dict (adds Vp) from a preset name or a dict."""
    cfg = dict(CONFIGS[name_or_dict]) if isinstance(name_or_dict, str) else dict(name_or_dict)
    cfg.update(overrides)
    cfg.setdefault("maxT", cfg["T"])
    cfg.setdefault("tokens", "uniform")
    cfg["Vp"] = cfg.get("Vp") or padded_vocab(cfg["V"])
    return cfg


def param_shapes(cfg) -> dict:
    C, L = cfg["C"], cfg["L"]
    return {
        "wte": (cfg["Vp"], C), "wpe": (cfg["maxT"], C),
        "ln1w": (L, C), "ln1b": (L, C), "qkvw": (L, 3 * C, C), "qkvb": (L, 3 * C),
        "attprojw": (L, C, C), "attprojb": (L, C), "ln2w": (L, C), "ln2b": (L, C),
        "fcw": (L, 4 * C, C), "fcb": (L, 4 * C), "fcprojw": (L, C, 4 * C), "fcprojb": (L, C),
        "lnfw": (C,), "lnfb": (C,),
    }


def init_params(cfg, seed: int = INIT_SEED, std: float = 0.02) -> dict:
    """Named float32 tensors: matrices N(0, std) (the two residual projections
    N(0, std/sqrt(2L))), biases 0, LayerNorm gains 1 and shifts 0, and the
    padded rows of wte (index >= V) exactly 0.  Each tensor has its own
    stream, so the draw does not depend on any packing order."""
    shapes = param_shapes(cfg)
    out = {}
    for i, name in enumerate(PARAM_NAMES):
        shp = shapes[name]
        if name in ("ln1w", "ln2w", "lnfw"):
            a = np.ones(shp, dtype=np.float32)
        elif name.endswith("b"):
            a = np.zeros(shp, dtype=np.float32)
        else:
            s = std / math.sqrt(2 * cfg["L"]) if name in ("attprojw", "fcprojw") else std
            rng = np.random.default_rng([seed, i])
            a = (rng.standard_normal(shp) * s).astype(np.float32)
            if name == "wte":
                a[cfg["V"]:] = 0.0
        out[name] = a
    return out


def zipf_cdf(V: int, s: float = ZIPF_S) -> np.ndarray:
    """Cumulative distribution of P(k) ~ (k+1)^-s over k in [0, V), in float64."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def token_stream(cfg, n: int, seed: int = DATA_SEED, step: int = 0) -> np.ndarray:
    """n int32 token ids for one step: uniform over [0, V) or Zipf(1.1)."""
    rng = np.random.default_rng([seed, step])
    V = cfg["V"]
    if cfg.get("tokens", "uniform") == "uniform":
        return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    u = rng.random(n)
    idx = np.searchsorted(zipf_cdf(V), u, side="right")
    return np.minimum(idx, V - 1).astype(np.int32)


def batch(cfg, step: int = 0, seed: int = DATA_SEED, B: int | None = None, T: int | None = None):
    """(inputs, targets), each int32 [B, T]: one stream of B*T+1 ids, targets
    being the inputs shifted by one position."""
    B = cfg["B"] if B is None else B
    T = cfg["T"] if T is None else T
    s = token_stream(cfg, B * T + 1, seed=seed, step=step)
    return s[:-1].reshape(B, T).copy(), s[1:].reshape(B, T).copy()
