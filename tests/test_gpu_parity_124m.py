"""Element-wise parity of one whole training step at the headline workload,
GPT-2 124M (L=12, C=768, 12 heads, V=50257 -> 50304), B=4, T=1024, in the
launch configuration bench.py times (forward with targets, zero_grad,
backward, AdamW at t = 1 over the same flat buffers).

Oracle side: the mean loss of a batch is the mean of its sequences' mean
losses (every sequence has T positions), and sequences do not interact, so
the oracle runs one sequence at a time (B=1, T=1024: about 12 GB of float64
activations instead of 48) and accumulates the four gradients, then scales
them by 1/4 and applies its own AdamW.  Every tensor of the parameter layout
is compared, element by element, with the bars of the whole-step test:
  loss: |L - L_ref| / |L_ref| <= 1e-5 (and per position)
  logits (v < V), per row: max|z - z_ref| / max|z_ref| <= 1e-4
  grads, m, v per tensor: max|x - x_ref| / max|x_ref| <= 2e-3
  update and updated parameters per tensor <= 2e-3 normwise over elements
  with |g_ref| >= 1e-5 max|g_ref|; the others within lr (AdamW's first step
  turns fp32 rounding noise of a gradient that is zero in exact arithmetic
  into a move of up to lr).
"""
import time

import numpy as np
import pytest

from transformer_lm_step_flat_amd import synth

pytestmark = pytest.mark.gpu

TOL_LOSS, TOL_LOGITS, TOL_GRAD = 1e-5, 1e-4, 2e-3
LR, B1, B2, EPS, WD = (float(np.float32(x)) for x in (1e-4, 0.9, 0.999, 1e-8, 0.0))


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def nrel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.timeout(900)
def test_headline_step_matches_oracle_per_tensor(g, oracle_lib):
    import torch
    cfg = synth.config("124m")
    B, T, V, Vp = cfg["B"], cfg["T"], cfg["V"], cfg["Vp"]
    tensors = synth.init_params(cfg)
    inp, tgt = synth.batch(cfg)  # the first batch bench.py steps on
    M = g.Model(cfg, B, T, init_params=g.pack_params(cfg, tensors, B, T))
    di = torch.from_numpy(inp.ravel()).cuda()
    dt = torch.from_numpy(tgt.ravel()).cuda()
    M.forward(di, None)
    torch.cuda.synchronize()
    logits = M.act("logits").view(B, T, Vp)[:, :, :V].cpu().numpy()
    t0 = time.time()
    loss = M.forward(di, dt)
    losses = M.act("losses").view(B, T).cpu().numpy().astype(np.float64)
    M.zero_grad()
    M.backward()
    M.update(lr=LR, beta1=B1, beta2=B2, eps=EPS, weight_decay=WD, t=1)
    M.sync()
    print(f"GPU step done in {time.time() - t0:.2f} s (loss {loss:.6f})", flush=True)
    grads, params1 = M.grads.cpu().numpy(), M.params.cpu().numpy()
    m1, v1 = M.adam_m.cpu().numpy(), M.adam_v.cpu().numpy()
    M.close()
    del M
    torch.cuda.empty_cache()

    p0 = oracle_lib.pack(cfg, tensors)
    R = oracle_lib.RefModel(cfg, 1, T)
    rg = np.zeros_like(p0)
    rlosses = np.empty((B, T))
    worst_row = 0.0
    for b in range(B):
        t1 = time.time()
        R.forward(p0, inp[b:b + 1], tgt[b:b + 1])
        rlosses[b] = R.get("losses")
        rz = R.get("logits").reshape(T, V)
        per_row = np.abs(logits[b].astype(np.float64) - rz).max(1) / np.abs(rz).max(1)
        worst_row = max(worst_row, float(per_row.max()))
        del rz
        R.backward(p0, rg)  # accumulates this sequence's gradient
        print(f"oracle sequence {b}: {time.time() - t1:.1f} s, worst logit row so far {worst_row:.2e}", flush=True)
    R.close()
    del logits
    rg *= 1.0 / B
    rloss = float(rlosses.mean())
    print(f"loss {loss:.7f} oracle {rloss:.7f} rel {abs(loss - rloss) / rloss:.2e}", flush=True)
    assert abs(loss - rloss) <= TOL_LOSS * abs(rloss)
    assert np.abs(losses - rlosses).max() <= TOL_LOSS * np.abs(rlosses).max()
    assert worst_row <= TOL_LOGITS

    rp, rm, rv = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    oracle_lib.adamw(rp, rg, rm, rv, LR, B1, B2, EPS, WD, 1)

    failures = []
    print(f"{'tensor':<10s} {'grad':>9s} {'p99.9':>9s} {'m':>9s} {'v':>9s} {'update':>9s} {'theta':>9s} excluded",
          flush=True)
    for name, off, cnt in oracle_lib.param_layout(cfg):
        sl = slice(off, off + cnt)
        gg, gr = grads[sl].astype(np.float64), rg[sl]
        gmax = max(np.abs(gr).max(), 1e-30)
        e_g = nrel(gg, gr)
        p999 = float(np.percentile(np.abs(gg - gr) / np.maximum(np.abs(gr), 1e-6 * gmax), 99.9))
        e_m = nrel(m1[sl].astype(np.float64), rm[sl])
        e_v = nrel(v1[sl].astype(np.float64), rv[sl])
        keep = np.abs(gr) >= 1e-5 * gmax
        p1, pr, pz = params1[sl].astype(np.float64), rp[sl], p0[sl]
        e_u = nrel((p1 - pz)[keep], (pr - pz)[keep]) if keep.any() else 0.0
        e_p = float(np.abs(p1 - pr)[keep].max() / max(np.abs(pr).max(), 1e-30)) if keep.any() else 0.0
        off_keep = float(np.abs(p1 - pr)[~keep].max()) if (~keep).any() else 0.0
        print(f"{name:<10s} {e_g:9.2e} {p999:9.2e} {e_m:9.2e} {e_v:9.2e} {e_u:9.2e} {e_p:9.2e} "
              f"{int((~keep).sum())} of {cnt}", flush=True)
        for what, err, bar in (("grad", e_g, TOL_GRAD), ("m", e_m, TOL_GRAD), ("v", e_v, TOL_GRAD),
                               ("update", e_u, TOL_GRAD), ("theta", e_p, TOL_GRAD),
                               ("theta (excluded elements)", off_keep, LR * (1 + 1e-5))):
            if not err <= bar:
                failures.append(f"{name} {what}: {err:.3e} > {bar:.1e}")
    # padded rows of wte take no gradient and stay zero
    C = cfg["C"]
    assert np.all(grads[:Vp * C].reshape(Vp, C)[V:] == 0.0)
    assert np.all(params1[:Vp * C].reshape(Vp, C)[V:] == 0.0)
    assert not failures, failures
