"""An independent float64 GPT-2 forward built from torch library routines
(embedding, layer_norm, linear, scaled_dot_product_attention, gelu,
cross_entropy), with torch autograd for the backward.  It is a referee for
the oracle's definitions on the CPU only; it is not used by the GPU path.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def params_to_torch(tensors: dict) -> dict:
    return {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
            for k, v in tensors.items()}


def forward(cfg, P: dict, inputs: np.ndarray, targets: np.ndarray | None):
    B, T = inputs.shape
    C, NH, L, V = cfg["C"], cfg["NH"], cfg["L"], cfg["V"]
    hd = C // NH
    tok = torch.tensor(inputs, dtype=torch.long)
    x = F.embedding(tok, P["wte"]) + P["wpe"][:T].unsqueeze(0)
    for l in range(L):
        h = F.layer_norm(x, (C,), P["ln1w"][l], P["ln1b"][l], eps=1e-5)
        qkv = F.linear(h, P["qkvw"][l], P["qkvb"][l])
        q, k, v = qkv.split(C, dim=-1)
        q = q.view(B, T, NH, hd).transpose(1, 2)
        k = k.view(B, T, NH, hd).transpose(1, 2)
        v = v.view(B, T, NH, hd).transpose(1, 2)
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        y = y.transpose(1, 2).reshape(B, T, C)
        x = x + F.linear(y, P["attprojw"][l], P["attprojb"][l])
        h = F.layer_norm(x, (C,), P["ln2w"][l], P["ln2b"][l], eps=1e-5)
        h = F.gelu(F.linear(h, P["fcw"][l], P["fcb"][l]), approximate="tanh")
        x = x + F.linear(h, P["fcprojw"][l], P["fcprojb"][l])
    x = F.layer_norm(x, (C,), P["lnfw"], P["lnfb"], eps=1e-5)
    logits = F.linear(x, P["wte"][:V])
    if targets is None:
        return logits, None
    loss = F.cross_entropy(logits.reshape(B * T, V), torch.tensor(targets, dtype=torch.long).reshape(-1))
    return logits, loss
