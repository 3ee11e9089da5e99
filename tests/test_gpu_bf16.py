"""bfloat16 products (gpt2_set_matmul_precision / gpt2k_linear_*_prec)
against the oracle in its bfloat16 mode, in which every linear-layer product
multiplies the bfloat16 roundings of its operands at full precision.

Kernel level: the operands are exact fp32 values, so both sides round them
identically and only the fp32 accumulation order differs: the fp32 bar
(1e-5 of the largest magnitude) applies.

Whole step: the GPU's fp32 activations differ from the oracle's float64 ones
by fp32 rounding, so an activation within that distance of a bfloat16
rounding boundary can round the other way: one bfloat16 unit in the last
place (up to 2^-7 relative) on that element.  Such flips are rare (of order
one element in 2^16) and each moves one term of a product by up to 2^-7 of
itself; with C = 64 a term of the head product is about a tenth of a row's
largest logit, so one flip is about 1e-3 of that row, and the tiny model's
16k head inputs make a flip or two likely.  Bars: loss 1e-4 relative,
logits 5e-3 per row (a few flips), gradients, m and v 1e-2 normwise per
tensor; the test prints the measured errors."""
import numpy as np
import pytest

from transformer_lm_step_flat_amd import synth

pytestmark = pytest.mark.gpu

LINEAR_SHAPES = [(64, 64, 64), (100, 44, 36), (256, 128, 512), (512, 768, 2304), (4096, 768, 3072),
                 (4036, 300, 2260)]


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def f32(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("N,K,OC", LINEAR_SHAPES)
def test_bf16_linear_forward_and_backward(g, oracle_lib, N, K, OC):
    import torch
    rng = np.random.default_rng(N + K + OC)
    x, W, b, dout = f32(rng, N, K), f32(rng, OC, K, scale=0.05), f32(rng, OC), f32(rng, N, OC, scale=0.01)
    out = torch.empty(N * OC, device="cuda")
    g.linear_forward(out, dev(x), dev(W), dev(b), N, K, OC, precision=g.GPT2_BF16)
    dW0, db0 = f32(rng, OC, K, scale=0.01), f32(rng, OC, scale=0.01)
    dinp, dW, db = torch.empty(N * K, device="cuda"), dev(dW0.ravel()), dev(db0)
    g.linear_backward(dinp, dW, db, dev(dout), dev(x), dev(W), N, K, OC, precision=g.GPT2_BF16)
    with oracle_lib.bf16_products():
        ro = oracle_lib.matmul_forward(x.astype(np.float64).ravel(), W.astype(np.float64).ravel(),
                                       b.astype(np.float64), N, K, OC)
        rdx, rdW, rdb = np.zeros(N * K), dW0.astype(np.float64).ravel(), db0.astype(np.float64)
        oracle_lib.matmul_backward(rdx, rdW, rdb, dout.astype(np.float64).ravel(), x.astype(np.float64).ravel(),
                                   W.astype(np.float64).ravel(), N, K, OC)
    assert rel(host(out), ro) <= 1e-5
    assert rel(host(dinp), rdx) <= 1e-5
    assert rel(host(dW), rdW) <= 1e-5
    assert rel(host(db), rdb) <= 1e-5
    # the same inputs with fp32 products differ by the operand rounding
    out32 = torch.empty(N * OC, device="cuda")
    g.linear_forward(out32, dev(x), dev(W), dev(b), N, K, OC)
    assert rel(host(out32), ro) > 1e-4


def test_bf16_head_product_at_full_shape(g, oracle_lib):
    """logits = lnf wte^T at 4096 x 50304 x 768 in bfloat16, sampled rows."""
    import torch
    N, K, OC = 4096, 768, 50304
    rng = np.random.default_rng(77)
    x, W = f32(rng, N, K), f32(rng, OC, K, scale=0.02)
    out = torch.empty(N * OC, device="cuda")
    g.linear_forward(out, dev(x), dev(W), None, N, K, OC, precision=g.GPT2_BF16)
    rows = np.sort(rng.choice(N, 8, replace=False))
    with oracle_lib.bf16_products():
        ro = oracle_lib.matmul_forward(np.ascontiguousarray(x[rows]).astype(np.float64).ravel(),
                                       W.astype(np.float64).ravel(), None, len(rows), K, OC)
    got = out.view(N, OC)[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64).ravel()
    assert rel(got, ro) <= 1e-5


CASES = {
    "tiny": synth.config("tiny"),
    "ragged": synth.config(dict(L=1, C=48, NH=3, T=20, B=3, V=36, Vp=36, maxT=24)),
    "small_b4": synth.config("small", B=4),
    "hd64": synth.config(dict(L=2, C=128, NH=2, T=132, B=2, V=300, maxT=132, tokens="zipf")),
}


@pytest.mark.parametrize("case", list(CASES))
def test_bf16_step_matches_oracle_bf16_mode(g, oracle_lib, case):
    import torch
    cfg = CASES[case]
    B, T, V = cfg["B"], cfg["T"], cfg["V"]
    tensors = synth.init_params(cfg)
    inp, tgt = synth.batch(cfg)
    M = g.Model(cfg, B, T, init_params=g.pack_params(cfg, tensors, B, T))
    M.set_matmul_precision(g.GPT2_BF16)
    di, dt = dev(inp.ravel()), dev(tgt.ravel())
    M.forward(di, None)
    logits = host(M.act("logits")).reshape(B * T, cfg["Vp"])[:, :V]
    loss = M.forward(di, dt)
    M.zero_grad()
    M.backward()
    M.update(lr=1e-4, t=1)
    grads, m1, v1 = host(M.grads), host(M.adam_m), host(M.adam_v)
    M.close()
    R = oracle_lib.RefModel(cfg, B, T)
    p = oracle_lib.pack(cfg, tensors)
    with oracle_lib.bf16_products():
        rloss = R.forward(p, inp, tgt)
        rlogits = R.get("logits").reshape(B * T, V)
        rg = np.zeros_like(p)
        R.backward(p, rg)
    R.close()
    rm, rv = np.zeros_like(p), np.zeros_like(p)
    rp = p.copy()
    oracle_lib.adamw(rp, rg, rm, rv, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1)
    e_loss = abs(loss - rloss) / abs(rloss)
    e_logits = float((np.abs(logits - rlogits).max(1) / np.abs(rlogits).max(1)).max())
    worst = {}
    for name, off, cnt in oracle_lib.param_layout(cfg):
        sl = slice(off, off + cnt)
        worst[name] = max(rel(grads[sl], rg[sl]), rel(m1[sl], rm[sl]), rel(v1[sl], rv[sl]))
    print(f"{case}: loss {e_loss:.2e} logits {e_logits:.2e} worst grad/m/v "
          f"{max(worst.values()):.2e} ({max(worst, key=worst.get)})", flush=True)
    assert e_loss <= 1e-4
    assert e_logits <= 5e-3
    for name, e in worst.items():
        assert e <= 1e-2, (name, e)
