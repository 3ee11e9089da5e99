"""The LayerNorm backward entry point that allocates nothing
(gpt2k_layernorm_backward_noalloc, static device scratch) against the one
that takes a workspace (gpt2k_layernorm_backward): the same kernels in the
same order, so the results must be bitwise equal; and both within the
oracle's bars.  Two calls in a row on the same stream, the second with a
smaller input, then a shape beyond the static scratch, which must be
refused without launching anything."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def _case(rng, N, C):
    x = rng.standard_normal((N, C)) * 1.5 + 0.3
    w = 1.0 + 0.1 * rng.standard_normal(C)
    dy = rng.standard_normal((N, C))
    mean = x.mean(1)
    rstd = 1.0 / np.sqrt(((x - mean[:, None]) ** 2).mean(1) + 1e-5)
    dx0 = 0.1 * rng.standard_normal((N, C))
    dw0 = 0.05 * rng.standard_normal(C)
    db0 = 0.05 * rng.standard_normal(C)
    return [a.astype(np.float32) for a in (x, w, dy, mean, rstd, dx0, dw0, db0)]


def test_noalloc_matches_workspace_entry_and_oracle(g, oracle_lib):
    import torch
    rng = np.random.default_rng(2024)
    for N, C in ((4096, 768), (1000, 768)):  # second call smaller
        x, w, dy, mean, rstd, dx0, dw0, db0 = _case(rng, N, C)
        dev = {k: torch.from_numpy(v).cuda() for k, v in
               dict(x=x, w=w, dy=dy, mean=mean, rstd=rstd).items()}
        outs = []
        for which in ("workspace", "noalloc"):
            dinp = torch.from_numpy(dx0).cuda()
            dw = torch.from_numpy(dw0).cuda()
            db = torch.from_numpy(db0).cuda()
            args = (dinp, dw, db, dev["dy"], dev["x"], dev["w"], dev["mean"], dev["rstd"], N, C, True)
            if which == "workspace":
                g.layernorm_backward(*args)
            else:
                g.layernorm_backward_noalloc(*args)
            torch.cuda.synchronize()
            outs.append([t.cpu().numpy() for t in (dinp, dw, db)])
        for a, b in zip(*outs):
            assert np.array_equal(a, b), (N, C)
        rdx, rdw, rdb = (dx0.astype(np.float64).ravel(), dw0.astype(np.float64), db0.astype(np.float64))
        oracle_lib.layernorm_backward(rdx, rdw, rdb, dy.astype(np.float64).ravel(), x.astype(np.float64).ravel(),
                                      w.astype(np.float64), mean.astype(np.float64), rstd.astype(np.float64), N, C)
        for got, ref in zip(outs[1], (rdx, rdw, rdb)):
            got = got.astype(np.float64).ravel()
            assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max(), (N, C)


def test_noalloc_refuses_shapes_beyond_its_scratch(g):
    import torch
    C = 2048
    N = 8192 + 16  # ceil(N / 16) * 2C partial floats
    need = -(-N // 16) * 2 * C
    assert need > 2 ** 21, need  # beyond the static scratch, checked here on the host
    # every buffer has the full size of the shape, so that even a launch the
    # entry point wrongly accepted would stay inside them
    big = torch.zeros(N * C, device="cuda")
    row = torch.zeros(N, device="cuda")
    col = torch.zeros(C, device="cuda")
    with pytest.raises(g.Gpt2Error) as e:
        g.layernorm_backward_noalloc(big, col, col.clone(), big.clone(), big.clone(), col.clone(), row, row.clone(),
                                     N, C, True)
    assert e.value.status == g.GPT2_EINVAL
    assert b"scratch" in g.lib().gpt2_last_error(None)
    # the largest accepted shape at this C runs (rows 8192: 512 partial rows)
    N2 = 8192
    g.layernorm_backward_noalloc(big, col, col.clone(), big.clone(), big.clone(), col.clone(), row, row.clone(),
                                 N2, C, True)
    torch.cuda.synchronize()
