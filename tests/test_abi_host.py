"""The C-ABI library on the CPU: it loads, exports every symbol the headers
declare, and its host-only calls (sizes, layout, argument checks) behave.
No kernel is launched here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from transformer_lm_step_flat_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_printed.json")


@pytest.fixture(scope="module")
def g():
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    return gpt2


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(gpt2k?_[a-z0-9_]+)\s*\(", txt, re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported(g):
    names = header_functions()
    assert len(names) >= 25
    L = g.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert names == set(g.EXPORTS)


def test_param_count_pin_and_padding(g):
    h = json.load(open(GOLDEN))["model_header"]
    cfg = dict(maxT=h["max_seq_len"], V=h["vocab_size"], Vp=h["vocab_size"] + 3, L=h["num_layers"],
               NH=h["num_heads"], C=h["channels"])
    # Vp must be a multiple of 4, so check the unpadded count through the layout table
    cfg["Vp"] = 50260
    lay = g.layout(cfg, 4, 64, g.GPT2_PARAMS)
    n = lay[-1][1] + lay[-1][2]
    assert n - (50260 - 50257) * 768 == h["num_parameters"]
    cfg["Vp"] = 50304
    assert g.query_sizes(cfg, 4, 1024).params == h["num_parameters"] + 47 * 768


@pytest.mark.parametrize("name", ["tiny", "small", "124m", "xl"])
def test_layout_agrees_with_oracle_and_shapes(g, oracle_lib, name):
    cfg = synth.config(name)
    lay = g.layout(cfg, cfg["B"], cfg["T"], g.GPT2_PARAMS)
    assert [n for n, _, _ in lay] == list(synth.PARAM_NAMES)
    assert [(n, o, c) for n, o, c in lay] == oracle_lib.param_layout(cfg)
    shapes = synth.param_shapes(cfg)
    for n, o, c in lay:
        assert c == int(np.prod(shapes[n]))


def test_activation_table_is_aligned_and_disjoint(g):
    cfg = synth.config("small")
    acts = g.layout(cfg, 32, 256, g.GPT2_ACTS)
    names = [a[0] for a in acts]
    assert names[:3] == ["encoded", "ln1", "ln1_mean"] and names[-4:] == ["logits", "losses", "loss", "lse"]
    sizes = {n: c for n, _, c in acts}
    # head dim 16: fused attention keeps lse, not the T x T probabilities
    assert sizes["att"] == 0 and sizes["lse"] == cfg["L"] * 32 * cfg["NH"] * 256
    cfg12 = synth.config(dict(L=1, C=48, NH=4, T=8, B=2, V=10))
    sizes12 = {n: c for n, _, c in g.layout(cfg12, 2, 8, g.GPT2_ACTS)}
    assert sizes12["att"] == 2 * 4 * 8 * 8 and sizes12["lse"] == 0
    end = 0
    for n, o, c in acts:
        assert o % 64 == 0 and o >= end, n
        end = o + c
    assert g.query_sizes(cfg, 32, 256).acts >= end


@pytest.mark.parametrize("bad", [
    dict(C=66), dict(NH=5), dict(Vp=999), dict(T=300), dict(T=62, C=48, NH=4), dict(C=4096, NH=64), dict(L=0)])
def test_invalid_shapes_are_rejected(g, bad):
    cfg = synth.config("small")
    cfg.update(bad)
    T = cfg["T"]
    with pytest.raises(g.Gpt2Error) as e:
        g.query_sizes(cfg, 2, T)
    assert e.value.status == g.GPT2_EINVAL
    assert g.lib().gpt2_last_error(None)


@pytest.mark.parametrize("T", [1, 7, 62])
def test_any_T_with_fused_attention_head_dims(g, T):
    """T need not be a multiple of 4 when the head dimension (16 here) takes
    the fused attention; the score-gradient rows are then padded."""
    cfg = synth.config("small")
    cfg.update(T=T)
    s = g.query_sizes(cfg, 2, T)
    assert s.work > 0 and s.acts > 0


def test_xl_state_fits_in_hbm(g):
    cfg = synth.config("xl")
    s = g.query_sizes(cfg, 4, 1024)
    assert s.params == 1557611200 + 47 * 1600
    total_bytes = 4 * (4 * s.params + s.acts + s.work) + 4 * s.iwork
    assert total_bytes < 200e9
