"""Checkpoint and resume of the training state (gpt2_save_checkpoint /
gpt2_load_checkpoint): five AdamW steps, save, load into a fresh model,
five more steps.  The ten losses must follow the oracle's uninterrupted
ten-step curve (each within 1e-5 relative), the loaded params, m and v must
equal the saved ones bit for bit, and the resumed run must be bitwise the
same as the run that never stopped.  Damaged or mismatched files are refused
and leave the model unchanged."""
import os

import numpy as np
import pytest

from transformer_lm_step_flat_amd import synth

pytestmark = pytest.mark.gpu

LR = float(np.float32(1e-4))


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def dev_ids(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32).ravel()).cuda()


def step(M, cfg, s):
    inp, tgt = synth.batch(cfg, step=s)
    loss = M.forward(dev_ids(inp), dev_ids(tgt))
    M.zero_grad()
    M.backward()
    M.update(lr=LR, t=s + 1)
    return loss


def state(M):
    import torch
    torch.cuda.synchronize()
    return [t.clone() for t in (M.params, M.adam_m, M.adam_v)]


def test_resume_follows_the_uninterrupted_curve(g, oracle_lib, tmp_path):
    import torch
    cfg = synth.config("small", B=8)
    B, T = cfg["B"], cfg["T"]
    tensors = synth.init_params(cfg)
    flat = g.pack_params(cfg, tensors, B, T)
    A = g.Model(cfg, B, T, init_params=flat)
    losses = [step(A, cfg, s) for s in range(5)]
    path = str(tmp_path / "state.ck")
    A.save(path, t=5)
    saved = state(A)
    assert os.path.getsize(path) == 576 + 3 * 4 * A.sizes.params

    # a fresh model with other weights, then the checkpoint
    Bm = g.Model(cfg, B, T, init_params=g.pack_params(cfg, synth.init_params(cfg, seed=7), B, T))
    assert Bm.load(path) == 5
    for a, b in zip(saved, state(Bm)):
        assert torch.equal(a, b)
    resumed = [step(Bm, cfg, s) for s in range(5, 10)]
    straight = [step(A, cfg, s) for s in range(5, 10)]
    assert resumed == straight  # bitwise: the same kernels on the same state
    for a, b in zip(state(A), state(Bm)):
        assert torch.equal(a, b)
    losses += resumed

    R = oracle_lib.RefModel(cfg, B, T)
    p = oracle_lib.pack(cfg, tensors)
    m, v = np.zeros_like(p), np.zeros_like(p)
    for s in range(10):
        inp, tgt = synth.batch(cfg, step=s)
        rl = R.forward(p, inp, tgt)
        gr = np.zeros_like(p)
        R.backward(p, gr)
        oracle_lib.adamw(p, gr, m, v, LR, 0.9, 0.999, 1e-8, 0.0, s + 1)
        print(f"step {s}: loss {losses[s]:.6f} oracle {rl:.6f}", flush=True)
        assert abs(losses[s] - rl) <= 1e-5 * abs(rl), (s, losses[s], rl)
    R.close()
    A.close()
    Bm.close()


def test_damaged_or_mismatched_checkpoints_are_refused(g, tmp_path):
    cfg = synth.config("tiny")
    B, T = cfg["B"], cfg["T"]
    M = g.Model(cfg, B, T, init_params=g.pack_params(cfg, synth.init_params(cfg), B, T))
    step(M, cfg, 0)
    good = str(tmp_path / "good.ck")
    M.save(good, t=1)
    blob = open(good, "rb").read()
    M2 = g.Model(cfg, B, T, init_params=g.pack_params(cfg, synth.init_params(cfg, seed=3), B, T))
    before = state(M2)

    def refused(data, status, name):
        import torch
        p = str(tmp_path / name)
        with open(p, "wb") as fh:
            fh.write(data)
        with pytest.raises(g.Gpt2Error) as e:
            M2.load(p)
        assert e.value.status == status, name
        for a, b in zip(before, state(M2)):
            assert torch.equal(a, b), name

    refused(blob[:-4], g.GPT2_EIO, "truncated.ck")
    flipped = bytearray(blob)
    flipped[600] ^= 0x40
    refused(bytes(flipped), g.GPT2_EIO, "corrupted.ck")
    refused(b"not a checkpoint" * 40, g.GPT2_EIO, "garbage.ck")
    other = synth.config(dict(cfg, L=cfg["L"] + 1))
    M3 = g.Model(other, B, T, init_params=g.pack_params(other, synth.init_params(other), B, T))
    p3 = str(tmp_path / "other.ck")
    M3.save(p3, t=0)
    refused(open(p3, "rb").read(), g.GPT2_EINVAL, "other_config.ck")
    with pytest.raises(g.Gpt2Error) as e:
        M2.load(str(tmp_path / "missing.ck"))
    assert e.value.status == g.GPT2_EIO
    # a good file still loads (into a model built for another B and T of the same config)
    M4 = g.Model(cfg, 2, 32)
    assert M4.load(good) == 1
    for x in (M, M2, M3, M4):
        x.close()
