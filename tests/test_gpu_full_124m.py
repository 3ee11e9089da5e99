"""Parity at the full GPT-2 124M shape (L=12, C=768, 12 heads, V=50257 -> 50304,
B=4, T=1024), in the launch configuration bench.py times, on outputs the
oracle can compute on their own:

- forward: attention is causal, so the loss and logits of position t depend
  only on ids 0..t of its own sequence.  The oracle runs the same 124M
  weights on the first 32 ids of every sequence; the GPU's full-batch
  per-position losses and logit rows at t < 32 must match it.
- backward: the head's two split-K / large-K products at their full shapes
  (dlnf = dlogits wte, dwte += dlogits^T lnf) on sampled rows; the other
  backward kernels are checked at full shapes in test_gpu_kernels.py.
- properties of the whole step at full size: gradients finite, padded wte
  rows untouched, bitwise reproducible, and one small AdamW step lowers the
  loss of the same batch by what the gradients predict to first order.
"""
import math

import numpy as np
import pytest

from transformer_lm_step_flat_amd import synth

from .step_checks import check_first_order_step

pytestmark = pytest.mark.gpu

T0 = 32  # prefix the oracle recomputes


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


@pytest.fixture(scope="module")
def full(g):
    import torch
    cfg = synth.config("124m")
    B, T = cfg["B"], cfg["T"]
    tensors = synth.init_params(cfg)
    M = g.Model(cfg, B, T, init_params=g.pack_params(cfg, tensors, B, T))
    inp, tgt = synth.batch(cfg)
    di = torch.from_numpy(inp.ravel()).cuda()
    dt = torch.from_numpy(tgt.ravel()).cuda()
    M.forward(di, None)
    torch.cuda.synchronize()
    logits_prefix = M.act("logits").view(B, T, cfg["Vp"])[:, :T0, :cfg["V"]].cpu().numpy().astype(np.float64)
    loss = M.forward(di, dt)
    losses = M.act("losses").view(B, T).cpu().numpy().astype(np.float64)
    yield dict(cfg=cfg, tensors=tensors, M=M, inp=inp, tgt=tgt, di=di, dt=dt, loss=loss, losses=losses,
               logits_prefix=logits_prefix)
    M.close()


def test_prefix_losses_and_logits_match_oracle(full, oracle_lib):
    cfg, B = full["cfg"], full["cfg"]["B"]
    R = oracle_lib.RefModel(cfg, B, T0)
    p = oracle_lib.pack(cfg, full["tensors"])
    R.forward(p, full["inp"][:, :T0].copy(), full["tgt"][:, :T0].copy())
    rl = R.get("losses").reshape(B, T0)
    rz = R.get("logits").reshape(B, T0, cfg["V"])
    gl = full["losses"][:, :T0]
    assert np.abs(gl - rl).max() <= 1e-5 * np.abs(rl).max()
    z = full["logits_prefix"]
    per_row = np.abs(z - rz).max(-1) / np.abs(rz).max(-1)
    assert per_row.max() <= 1e-4
    R.close()


def test_full_loss_is_near_ln_v(full):
    # seeded N(0, 0.02) weights: logits are small, the loss is ln V plus a little
    V, C = full["cfg"]["V"], full["cfg"]["C"]
    expect = math.log(V) + C * 0.02 ** 2 / 2
    assert abs(full["loss"] - expect) <= 0.02 * expect
    assert abs(full["loss"] - full["losses"].mean()) <= 1e-5 * full["loss"]


def test_head_backward_products_at_full_shape(g, oracle_lib):
    """dlnf = dlogits wte (K = 50304, split K) and dwte += dlogits^T lnf
    (K = 4096), exactly as the step launches them, on sampled rows."""
    import torch
    N, K, OC = 4096, 768, 50304
    rng = np.random.default_rng(21)
    dout = (rng.standard_normal((N, OC)) * 1e-4).astype(np.float32)
    lnf = rng.standard_normal((N, K)).astype(np.float32)
    wte = (rng.standard_normal((OC, K)) * 0.02).astype(np.float32)
    dinp = torch.empty(N * K, device="cuda")
    dW = torch.zeros(OC * K, device="cuda")
    g.linear_backward(dinp, dW, None, torch.from_numpy(dout).cuda(), torch.from_numpy(lnf).cuda(),
                      torch.from_numpy(wte).cuda(), N, K, OC)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(N, 16, replace=False))
    rd = np.zeros(len(rows) * K)
    oracle_lib.matmul_backward(rd, np.zeros(OC * K), None, np.ascontiguousarray(dout[rows]).astype(np.float64).ravel(),
                               np.ascontiguousarray(lnf[rows]).astype(np.float64).ravel(),
                               wte.astype(np.float64).ravel(), len(rows), K, OC)
    got = dinp.view(N, K)[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64).ravel()
    assert np.abs(got - rd).max() <= 1e-5 * np.abs(rd).max()
    cols = np.sort(rng.choice(OC, 16, replace=False))
    rW = np.zeros(len(cols) * K)
    oracle_lib.matmul_backward(np.zeros(N * K), rW, None, np.ascontiguousarray(dout[:, cols]).astype(np.float64).ravel(),
                               lnf.astype(np.float64).ravel(), np.zeros(len(cols) * K), N, K, len(cols))
    gotW = dW.view(OC, K)[torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64).ravel()
    assert np.abs(gotW - rW).max() <= 1e-5 * np.abs(rW).max()


def test_full_step_properties(full):
    import torch
    M, cfg = full["M"], full["cfg"]
    V, Vp, C = cfg["V"], cfg["Vp"], cfg["C"]
    M.zero_grad()
    M.backward()
    torch.cuda.synchronize()
    g1 = M.grads.clone()
    assert bool(torch.isfinite(g1).all())
    wte_g = g1[:Vp * C].view(Vp, C)
    assert bool((wte_g[V:] == 0).all())
    assert float(wte_g[:V].abs().max()) > 0
    # bitwise reproducible
    M.zero_grad()
    M.backward()
    torch.cuda.synchronize()
    assert bool(torch.equal(M.grads, g1))
    # one small AdamW step lowers the loss by what the gradients predict
    check_first_order_step(M, full["di"], full["dt"], full["loss"])
