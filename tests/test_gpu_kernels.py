"""Per-kernel parity on the GPU: each kernel-level entry point of the C ABI
against the oracle's function for the same layer, on the same seeded inputs.
Shapes span several tiles with ragged tails; the full GPT-2 124M shapes are
checked on sampled outputs (rows the oracle computes on its own)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

rel = lambda a, b: float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.astype(dtype) if dtype else a)
    return t.cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def f32(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- linear layers

LINEAR_SHAPES = [(64, 64, 192), (37, 20, 44), (130, 96, 200), (256, 128, 512), (300, 516, 132), (1024, 768, 3072),
                 # the planner takes the 64 x 192 tile here; ragged in M, N and K
                 (4036, 300, 2260)]


@pytest.mark.parametrize("N,K,OC", LINEAR_SHAPES)
def test_linear_forward(g, oracle_lib, N, K, OC):
    import torch
    rng = np.random.default_rng(N * 7 + K)
    x, W, b = f32(rng, N, K), f32(rng, OC, K, scale=0.05), f32(rng, OC)
    out = torch.empty(N * OC, device="cuda")
    g.linear_forward(out, dev(x), dev(W), dev(b), N, K, OC)
    ref = oracle_lib.matmul_forward(x.astype(np.float64).ravel(), W.astype(np.float64).ravel(),
                                    b.astype(np.float64), N, K, OC)
    assert rel(host(out), ref) < 1e-5


@pytest.mark.parametrize("N,K,OC", LINEAR_SHAPES)
def test_linear_backward(g, oracle_lib, N, K, OC):
    import torch
    rng = np.random.default_rng(N * 11 + OC)
    x, W, dout = f32(rng, N, K), f32(rng, OC, K, scale=0.05), f32(rng, N, OC)
    dW0, db0 = f32(rng, OC, K), f32(rng, OC)
    dinp = torch.empty(N * K, device="cuda")
    dW, db = dev(dW0), dev(db0)
    g.linear_backward(dinp, dW, db, dev(dout), dev(x), dev(W), N, K, OC)
    rdinp, rdW, rdb = np.zeros(N * K), dW0.astype(np.float64).ravel(), db0.astype(np.float64)
    oracle_lib.matmul_backward(rdinp, rdW, rdb, dout.astype(np.float64).ravel(), x.astype(np.float64).ravel(),
                               W.astype(np.float64).ravel(), N, K, OC)
    assert rel(host(dinp), rdinp) < 1e-5
    assert rel(host(dW).ravel(), rdW) < 1e-5
    assert rel(host(db), rdb) < 1e-5


def test_linear_full_head_shape_sampled_rows(g, oracle_lib):
    """logits = lnf wte^T at 4096 x 50304 x 768; 24 sampled rows vs the oracle."""
    import torch
    rng = np.random.default_rng(3)
    N, K, OC = 4096, 768, 50304
    x = f32(rng, N, K)
    W = f32(rng, OC, K, scale=0.02)
    out = torch.empty(N * OC, device="cuda")
    g.linear_forward(out, dev(x), dev(W), None, N, K, OC)
    rows = np.sort(rng.choice(N, 24, replace=False))
    got = out.view(N, OC)[torch.from_numpy(rows).cuda()]
    ref = oracle_lib.matmul_forward(x[rows].astype(np.float64).ravel(), W.astype(np.float64).ravel(), None,
                                    len(rows), K, OC)
    assert rel(host(got).ravel(), ref) < 1e-5


# ---------------------------------------------------------------- layernorm

@pytest.mark.parametrize("N,C", [(64, 64), (37, 20), (200, 768), (33, 1600), (4096, 768), (1000, 1600), (129, 1540),
                                 (300, 2048)])
def test_layernorm(g, oracle_lib, N, C):
    import torch
    rng = np.random.default_rng(N + C)
    x = (rng.standard_normal((N, C)) * rng.uniform(0.1, 3, (N, 1)) + rng.uniform(-2, 2, (N, 1))).astype(np.float32)
    w, b = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32), f32(rng, C, scale=0.1)
    out, mean, rstd = (torch.empty(n, device="cuda") for n in (N * C, N, N))
    g.layernorm_forward(out, mean, rstd, dev(x), dev(w), dev(b), N, C)
    ro, rm, rr = oracle_lib.layernorm_forward(x.astype(np.float64).ravel(), w.astype(np.float64),
                                              b.astype(np.float64), N, C)
    assert rel(host(out), ro) < 1e-5
    assert rel(host(mean), rm) < 1e-5
    assert rel(host(rstd), rr) < 1e-5
    # backward, accumulating into dinp
    dy, dx0 = f32(rng, N, C), f32(rng, N, C)
    dw0, db0 = f32(rng, C), f32(rng, C)
    dx, dw, db = dev(dx0), dev(dw0), dev(db0)
    g.layernorm_backward(dx, dw, db, dev(dy), dev(x), dev(w), mean, rstd, N, C, True)
    rdx, rdw, rdb = dx0.astype(np.float64).ravel(), dw0.astype(np.float64), db0.astype(np.float64)
    oracle_lib.layernorm_backward(rdx, rdw, rdb, dy.astype(np.float64).ravel(), x.astype(np.float64).ravel(),
                                  w.astype(np.float64), rm, rr, N, C)
    assert rel(host(dx).ravel(), rdx) < 1e-5
    assert rel(host(dw), rdw) < 1e-5
    assert rel(host(db), rdb) < 1e-5


# ---------------------------------------------------------------- attention

ATT_SHAPES = [(2, 64, 64, 4), (1, 100, 48, 3), (3, 20, 24, 2), (2, 256, 128, 2), (1, 132, 128, 8)]


@pytest.mark.parametrize("B,T,C,NH", ATT_SHAPES)
def test_attention(g, oracle_lib, B, T, C, NH):
    import torch
    rng = np.random.default_rng(B * T + C)
    qkv = f32(rng, B, T, 3 * C)
    att = torch.empty(B * NH * T * T, device="cuda")
    atty = torch.empty(B * T * C, device="cuda")
    dq = dev(qkv)
    g.attention_forward(atty, att, dq, B, T, C, NH)
    ry, rpre, ratt = oracle_lib.attention_forward(qkv.astype(np.float64).ravel(), B, T, C, NH)
    assert rel(host(atty), ry) < 1e-5
    ga = host(att).reshape(B, NH, T, T)
    ra = ratt.reshape(B, NH, T, T)
    low = np.tril(np.ones((T, T), dtype=bool))
    assert rel(ga[:, :, low], ra[:, :, low]) < 1e-5
    # zeros above the diagonal up to the next multiple of 128 columns
    for t in range(T):
        e = min(T, (t // 128 + 1) * 128)
        assert np.all(ga[:, :, t, t + 1:e] == 0.0)
    datty = f32(rng, B, T, C)
    dqkv = torch.empty(B * T * 3 * C, device="cuda")
    g.attention_backward(dqkv, dev(datty), dq, att, B, T, C, NH)
    rdqkv = np.zeros(B * T * 3 * C)
    oracle_lib.attention_backward(rdqkv, datty.astype(np.float64).ravel(), qkv.astype(np.float64).ravel(), ratt,
                                  B, T, C, NH)
    gd = host(dqkv).reshape(B, T, 3, C)
    rd = rdqkv.reshape(B, T, 3, C)
    for i in range(3):
        assert rel(gd[:, :, i], rd[:, :, i]) < 1e-4, "qkv"[i]


FLASH_SHAPES = [(2, 64, 64, 4), (1, 100, 48, 3), (2, 256, 128, 2), (1, 132, 128, 8), (3, 20, 96, 3),
                (1, 260, 128, 2), (2, 4, 64, 1), (1, 700, 128, 2), (1, 1024, 64, 1),
                # more dk/dv iterations than resident workgroups: ranges that cross
                # key blocks and (batch, head) boundaries
                (2, 520, 768, 12)]


@pytest.mark.parametrize("B,T,C,NH", FLASH_SHAPES)
def test_flash_attention(g, oracle_lib, B, T, C, NH):
    """The fused kernels: output, log-sum-exp and all three input gradients."""
    import torch
    rng = np.random.default_rng(B * T + C + 1)
    qkv = f32(rng, B, T, 3 * C, scale=1.5)
    atty = torch.empty(B * T * C, device="cuda")
    lse = torch.empty(B * NH * T, device="cuda")
    dq = dev(qkv)
    g.flash_attention_forward(atty, lse, dq, B, T, C, NH)
    ry, rpre, ratt = oracle_lib.attention_forward(qkv.astype(np.float64).ravel(), B, T, C, NH)
    assert rel(host(atty), ry) < 1e-5
    pre = rpre.reshape(B, NH, T, T)
    low = np.tril(np.ones((T, T), dtype=bool))
    mx = np.where(low, pre, -np.inf).max(-1)
    rlse = mx + np.log(np.where(low, np.exp(pre - mx[..., None]), 0.0).sum(-1))
    assert np.abs(host(lse).reshape(B, NH, T) - rlse).max() < 1e-5 * max(1.0, np.abs(rlse).max())
    datty = f32(rng, B, T, C)
    dqkv = torch.full((B * T * 3 * C,), float("nan"), device="cuda")
    g.flash_attention_backward(dqkv, dev(datty), dq, atty, lse, B, T, C, NH)
    rdqkv = np.zeros(B * T * 3 * C)
    oracle_lib.attention_backward(rdqkv, datty.astype(np.float64).ravel(), qkv.astype(np.float64).ravel(), ratt,
                                  B, T, C, NH)
    gd = host(dqkv).reshape(B, T, 3, C)
    rd = rdqkv.reshape(B, T, 3, C)
    for i in range(3):
        assert rel(gd[:, :, i], rd[:, :, i]) < 1e-4, "qkv"[i]


def test_flash_attention_rejects_other_head_dims(g):
    import torch
    B, T, C, NH = 1, 8, 24, 2
    x = torch.zeros(B * T * 3 * C, device="cuda")
    with pytest.raises(g.Gpt2Error) as e:
        g.flash_attention_forward(torch.empty(B * T * C, device="cuda"), torch.empty(B * NH * T, device="cuda"), x,
                                  B, T, C, NH)
    assert e.value.status == g.GPT2_EINVAL


def test_attention_full_shape_sampled_heads(g, oracle_lib):
    """B=4, T=1024, C=768, 12 heads; the oracle recomputes 2 (b, h) pairs."""
    import torch
    B, T, C, NH = 4, 1024, 768, 12
    hd = C // NH
    rng = np.random.default_rng(5)
    qkv = f32(rng, B, T, 3 * C)
    att = torch.empty(B * NH * T * T, device="cuda")
    atty = torch.empty(B * T * C, device="cuda")
    dq = dev(qkv)
    g.attention_forward(atty, att, dq, B, T, C, NH)
    datty = f32(rng, B, T, C)
    dqkv = torch.empty(B * T * 3 * C, device="cuda")
    g.attention_backward(dqkv, dev(datty), dq, att, B, T, C, NH)
    # the fused path at the same shape, on the same inputs
    fy = torch.empty(B * T * C, device="cuda")
    flse = torch.empty(B * NH * T, device="cuda")
    g.flash_attention_forward(fy, flse, dq, B, T, C, NH)
    fd = torch.empty(B * T * 3 * C, device="cuda")
    g.flash_attention_backward(fd, dev(datty), dq, fy, flse, B, T, C, NH)
    for gy, gd in [(host(atty).reshape(B, T, C), host(dqkv).reshape(B, T, 3, C)),
                   (host(fy).reshape(B, T, C), host(fd).reshape(B, T, 3, C))]:
        check_sampled_heads(oracle_lib, qkv, datty, gy, gd, B, T, C, NH)


def check_sampled_heads(oracle_lib, qkv, datty, gy, gd, B, T, C, NH):
    hd = C // NH
    for b, h in [(0, 0), (3, 11)]:
        sl = slice(h * hd, (h + 1) * hd)
        sub = np.ascontiguousarray(qkv[b:b + 1].reshape(1, T, 3, C)[:, :, :, sl]).astype(np.float64)
        ry, _, ratt = oracle_lib.attention_forward(sub.ravel(), 1, T, hd, 1)
        assert rel(gy[b, :, sl].ravel(), ry) < 1e-5
        rd = np.zeros(T * 3 * hd)
        oracle_lib.attention_backward(rd, np.ascontiguousarray(datty[b, :, sl]).astype(np.float64).ravel(),
                                      sub.ravel(), ratt, 1, T, hd, 1)
        rd = rd.reshape(T, 3, hd)
        for i in range(3):
            assert rel(gd[b, :, i, sl], rd[:, i]) < 1e-4


# ---------------------------------------------------------------- gelu, cross-entropy, encoder, adamw

def test_gelu(g, oracle_lib):
    import torch
    rng = np.random.default_rng(9)
    x = np.concatenate([np.linspace(-10, 10, 4000), rng.standard_normal(4000) * 3]).astype(np.float32)
    out = torch.empty(x.size, device="cuda")
    g.gelu_forward(out, dev(x))
    ref = oracle_lib.gelu_forward(x.astype(np.float64))
    assert np.abs(host(out) - ref).max() < 1e-5 * np.abs(ref).max()
    d = f32(rng, x.size)
    din = torch.empty(x.size, device="cuda")
    g.gelu_backward(din, dev(x), dev(d))
    rdin = np.zeros(x.size)
    oracle_lib.gelu_backward(rdin, x.astype(np.float64), d.astype(np.float64))
    assert rel(host(din), rdin) < 1e-5


@pytest.mark.parametrize("BT,V,Vp", [(64, 65, 128), (33, 1000, 1024), (8, 7, 8), (4096, 50257, 50304)])
def test_crossentropy(g, oracle_lib, BT, V, Vp):
    import torch
    rng = np.random.default_rng(BT + V)
    z = f32(rng, BT, Vp, scale=2.0)
    tg = rng.integers(0, V, BT).astype(np.int32)
    zl = dev(z)
    losses, loss = torch.empty(BT, device="cuda"), torch.empty(1, device="cuda")
    g.crossentropy(zl, losses, loss, dev(tg), BT, V, Vp)
    rows = np.arange(BT) if BT <= 64 else np.sort(rng.choice(BT, 64, replace=False))
    zr = np.ascontiguousarray(z[rows]).astype(np.float64)
    rl, rp = oracle_lib.softmax_crossentropy_forward(zr.ravel(), tg[rows], len(rows), V, Vp)
    gl = host(losses)
    assert rel(gl[rows], rl) < 1e-5
    full_l, _ = oracle_lib.softmax_crossentropy_forward(z.astype(np.float64).ravel(), tg, BT, V, Vp) \
        if BT <= 64 else (None, None)
    if full_l is not None:
        assert abs(host(loss)[0] - full_l.mean()) <= 1e-5 * abs(full_l.mean())
    rd = oracle_lib.crossentropy_softmax_backward(rp, tg[rows], len(rows), V, Vp).reshape(len(rows), Vp)
    gd = host(zl).reshape(BT, Vp)[rows]
    # the oracle scales by 1/len(rows); the kernel by 1/BT
    rd *= len(rows) / BT
    assert rel(gd, rd) < 1e-5
    assert np.all(gd[:, V:] == 0.0)


@pytest.mark.parametrize("B,T,C", [(3, 100, 64), (1, 68, 32), (2, 512, 96)])
def test_encoder_backward_long_runs(g, oracle_lib, B, T, C):
    """Runs of one id longer than the 64-entry segments of the scatter-add,
    crossing several segment boundaries, with B*T not a multiple of 64."""
    import torch
    V = 50
    rng = np.random.default_rng(B * T + C)
    ids = rng.integers(0, V, (B, T)).astype(np.int32)
    ids[rng.random((B, T)) < 0.7] = 7  # one id takes ~70 % of the positions
    ids[0, 0], ids[-1, -1] = 0, V - 1
    dids = dev(ids)
    order = torch.empty(B * T, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.token_order(order, err, dids, None, B * T, V)
    dout = f32(rng, B, T, C)
    dwte0, dwpe0 = f32(rng, V, C), f32(rng, T, C)
    dwte, dwpe = dev(dwte0), dev(dwpe0)
    g.encoder_backward(dwte, dwpe, dev(dout), dids, order, B, T, C, V)
    rw, rp = dwte0.astype(np.float64).ravel(), dwpe0.astype(np.float64).ravel()
    oracle_lib.encoder_backward(rw, rp, dout.astype(np.float64).ravel(), ids.ravel().astype(np.int32), B, T, C)
    assert rel(host(dwte).ravel(), rw) < 1e-5
    assert rel(host(dwpe).ravel(), rp) < 1e-5
    assert int(err.item()) == 0


def test_encoder_and_token_order(g, oracle_lib):
    import torch
    from transformer_lm_step_flat_amd import synth
    cfg = synth.config("small")
    B, T, C, V = 8, 256, 128, 1000
    ids, tg = synth.batch(cfg, B=B, T=T)
    rng = np.random.default_rng(1)
    wte, wpe = f32(rng, 1024, C), f32(rng, T, C)
    out = torch.empty(B * T * C, device="cuda")
    dids = dev(ids)
    g.encoder_forward(out, dids, dev(wte), dev(wpe), B, T, C, V)
    ref = oracle_lib.encoder_forward(ids.ravel().astype(np.int32), wte.astype(np.float64), wpe.astype(np.float64),
                                     B, T, C)
    # one fp32 add: bit-exact against the same add done in fp32
    assert np.array_equal(host(out).astype(np.float32), ref.astype(np.float32))
    order = torch.empty(B * T, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.token_order(order, err, dids, dev(tg), B * T, V)
    torch.cuda.synchronize()
    expect = np.lexsort((np.arange(B * T), ids.ravel()))
    assert np.array_equal(order.cpu().numpy(), expect)
    assert int(err.item()) == 0
    dout = f32(rng, B, T, C)
    dwte0, dwpe0 = f32(rng, 1024, C), f32(rng, T, C)
    dwte, dwpe = dev(dwte0), dev(dwpe0)
    g.encoder_backward(dwte, dwpe, dev(dout), dids, order, B, T, C, V)
    rw, rp = dwte0.astype(np.float64).ravel(), dwpe0.astype(np.float64).ravel()
    oracle_lib.encoder_backward(rw, rp, dout.astype(np.float64).ravel(), ids.ravel().astype(np.int32), B, T, C)
    assert rel(host(dwte).ravel(), rw) < 1e-5
    assert rel(host(dwpe).ravel(), rp) < 1e-5
    # an out-of-range id raises the flag and stays memory-safe
    bad = ids.copy()
    bad[0, 3] = V + 5
    bad[1, 0] = -1
    err.zero_()
    g.token_order(order, err, dev(bad), dev(tg), B * T, V)
    torch.cuda.synchronize()
    assert int(err.item()) & 1


@pytest.mark.parametrize("BT,V,ids", [(1, 7, "zipf"), (3, 50257, "zipf"), (1000, 50257, "zipf"),
                                      (4096, 50257, "zipf"), (8191, 50257, "zipf"), (8192, 50257, "zipf"),
                                      (8193, 50257, "zipf"), (16384, 50257, "zipf"), (16384, 50257, "one"),
                                      (16384, 2000000, "uniform"), (33000, 50257, "zipf")])
def test_token_order_sizes(g, BT, V, ids):
    """The position order of the embedding backward on both sides of the
    switch from the counting kernel to chunk sort + binary search (8192
    positions), with ragged last chunks, Zipf ids with long runs of repeats,
    a single repeated id and ids spread over a large vocabulary, against
    numpy's stable sort by id."""
    import torch
    rng = np.random.default_rng(BT)
    if ids == "zipf":
        a = np.minimum(rng.zipf(1.1, BT) - 1, V - 1)
    elif ids == "one":
        a = np.full(BT, 17)
    else:
        a = rng.integers(0, V, BT)
    a = a.astype(np.int32)
    order = torch.empty(BT, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.token_order(order, err, dev(a), None, BT, V)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), np.argsort(a, kind="stable"))
    assert int(err.item()) == 0
    bad = a.copy()
    bad[BT // 2] = V
    g.token_order(order, err, dev(bad), None, BT, V)
    torch.cuda.synchronize()
    assert int(err.item()) == 1


def test_adamw(g, oracle_lib):
    import torch
    rng = np.random.default_rng(2)
    n = 1 << 16
    p, gr = f32(rng, n), (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)).astype(np.float32)
    m, v = f32(rng, n, scale=1e-3), np.abs(f32(rng, n, scale=1e-6))
    dp, dm, dv = dev(p), dev(m), dev(v)
    # the C ABI takes fp32 hyperparameters: give the oracle the same values
    hp = [float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8, 0.01)]
    g.adamw(dp, dev(gr), dm, dv, *hp, 7)
    rp, rm, rv = (a.astype(np.float64) for a in (p, m, v))
    oracle_lib.adamw(rp, gr.astype(np.float64), rm, rv, *hp, 7)
    assert rel(host(dm), rm) < 1e-6
    assert rel(host(dv), rv) < 1e-6
    assert rel(host(dp) - p, rp - p) < 1e-5
    assert rel(host(dp), rp) < 1e-6


# ---------------------------------------------------------------- calibration kernels of the measurement

def test_probes(g):
    """The copy probe copies exactly (ragged tail of the last workgroup); the
    matrix-core probe runs and reports its work; bad sizes are rejected."""
    import torch
    rng = np.random.default_rng(11)
    n = 4 * 1000 + 4 * 257
    src = f32(rng, n)
    dst = torch.zeros(n, device="cuda")
    g.probe_copy(dst, dev(src))
    assert np.array_equal(host(dst), src)
    out = torch.zeros(1, device="cuda")
    flops = g.probe_mfma(out, 3)
    torch.cuda.synchronize()
    assert flops > 0 and float(out.item()) == 0.0
    with pytest.raises(g.Gpt2Error):
        g.probe_mfma(out, 0)
    with pytest.raises(g.Gpt2Error):
        g.probe_copy(dst[:6], dev(src)[:6])
