"""Python access to the CPU oracle (``gpt2_ref.c``) through ctypes.

This is test infrastructure: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.  It imports nothing from the GPU library
and the GPU library imports nothing from here.  Every array crossing this
boundary is float64 (values) or int32 (tokens), C-contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gpt2_ref.c")
_LIB = os.path.join(_HERE, "libgpt2ref.so")
# A test may point this module at another build of the oracle (a planted
# mistake, compiled on the CPU) through this variable; it is then loaded as is.
_LIB_OVERRIDE = os.environ.get("GPT2_ORACLE_LIB")

_i64 = ctypes.c_longlong
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libgpt2ref.so`` (gcc, OpenMP, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-D_GNU_SOURCE",
             "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        L.ref_param_tensor.restype = _i64
        L.ref_param_tensor.argtypes = [ctypes.c_int] * 7 + [
            ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_char_p)]
        L.ref_num_param_tensors.restype = ctypes.c_int
        L.ref_num_activations.restype = _i64
        L.ref_num_activations.argtypes = [ctypes.c_int] * 8
        L.ref_create.restype = ctypes.c_void_p
        L.ref_create.argtypes = [ctypes.c_int] * 8
        L.ref_destroy.argtypes = [ctypes.c_void_p]
        L.ref_forward.restype = ctypes.c_double
        L.ref_forward.argtypes = [ctypes.c_void_p, _dp, _ip, _ip]
        L.ref_backward.restype = ctypes.c_int
        L.ref_backward.argtypes = [ctypes.c_void_p, _dp, _dp]
        L.ref_get.restype = _i64
        L.ref_get.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int, _dp, _i64]
        L.ref_act_count.restype = _i64
        L.ref_act_count.argtypes = [ctypes.c_void_p, ctypes.c_char_p]
        L.ref_num_threads.restype = ctypes.c_int
        L.ref_decode_step.restype = ctypes.c_int
        L.ref_decode_step.argtypes = [ctypes.c_void_p, _dp, _ip, ctypes.c_int, _dp, _ip]
        L.ref_round_bf16.restype = ctypes.c_double
        L.ref_round_bf16.argtypes = [ctypes.c_double]
        L.ref_set_bf16_products.restype = None
        L.ref_set_bf16_products.argtypes = [ctypes.c_int]
        L.ref_sample.restype = ctypes.c_int
        L.ref_sample.argtypes = [_dp, ctypes.c_int, ctypes.c_double]
        for name, args in {
            "ref_encoder_forward": [_dp, _ip, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int],
            "ref_encoder_backward": [_dp, _dp, _dp, _ip, ctypes.c_int, ctypes.c_int, ctypes.c_int],
            "ref_layernorm_forward": [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int],
            "ref_layernorm_backward": [_dp] * 8 + [ctypes.c_int, ctypes.c_int],
            "ref_matmul_forward": [_dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int],
            "ref_matmul_backward": [_dp] * 6 + [ctypes.c_int] * 3,
            "ref_attention_forward": [_dp, _dp, _dp, _dp] + [ctypes.c_int] * 4,
            "ref_attention_backward": [_dp] * 6 + [ctypes.c_int] * 4,
            "ref_gelu_forward": [_dp, _dp, _i64],
            "ref_gelu_backward": [_dp, _dp, _dp, _i64],
            "ref_residual_forward": [_dp, _dp, _dp, _i64],
            "ref_softmax_crossentropy_forward": [_dp, _dp, _dp, _ip] + [ctypes.c_int] * 3,
            "ref_crossentropy_softmax_backward": [_dp, _dp, _ip] + [ctypes.c_int] * 3,
            "ref_adamw": [_dp, _dp, _dp, _dp, _i64] + [ctypes.c_double] * 5 + [ctypes.c_int],
        }.items():
            f = getattr(L, name)
            f.restype = None
            f.argtypes = args
        _lib = L
    return _lib


def _d(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous, "oracle arrays are C-contiguous float64"
    return a.ctypes.data_as(_dp)


def _i(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous, "oracle token arrays are C-contiguous int32"
    return a.ctypes.data_as(_ip)


def num_threads() -> int:
    return lib().ref_num_threads()


# ---------------------------------------------------------------- layout

def shape_args(cfg) -> tuple:
    """(maxT, V, Vp, L, NH, C) from a config mapping."""
    return (cfg["maxT"], cfg["V"], cfg["Vp"], cfg["L"], cfg["NH"], cfg["C"])


def param_layout(cfg):
    """The oracle's own parameter layout: [(name, offset, count)] in order."""
    L = lib()
    out = []
    for i in range(L.ref_num_param_tensors()):
        off, cnt, nm = _i64(), _i64(), ctypes.c_char_p()
        L.ref_param_tensor(*shape_args(cfg), i, ctypes.byref(off), ctypes.byref(cnt), ctypes.byref(nm))
        out.append((nm.value.decode(), off.value, cnt.value))
    return out


def num_parameters(cfg) -> int:
    return lib().ref_param_tensor(*shape_args(cfg), -1, None, None, None)


def num_activations(cfg, B: int, T: int) -> int:
    return lib().ref_num_activations(*shape_args(cfg), B, T)


def pack(cfg, tensors: dict) -> np.ndarray:
    """Place named tensors (any float dtype) into one flat float64 array."""
    flat = np.zeros(num_parameters(cfg), dtype=np.float64)
    for name, off, cnt in param_layout(cfg):
        a = np.asarray(tensors[name], dtype=np.float64).reshape(-1)
        assert a.size == cnt, (name, a.size, cnt)
        flat[off:off + cnt] = a
    return flat


def unpack(cfg, flat: np.ndarray) -> dict:
    return {name: flat[off:off + cnt] for name, off, cnt in param_layout(cfg)}


# ---------------------------------------------------------------- model

class RefModel:
    """The oracle's whole model at a fixed (B, T): forward, backward."""

    def __init__(self, cfg, B: int, T: int):
        self.cfg, self.B, self.T = cfg, B, T
        self._h = lib().ref_create(*shape_args(cfg), B, T)
        if not self._h:
            raise ValueError("oracle rejected the configuration or ran out of memory")

    def close(self):
        if self._h:
            lib().ref_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, params: np.ndarray, inputs: np.ndarray, targets: np.ndarray | None = None) -> float:
        inputs = np.ascontiguousarray(inputs, dtype=np.int32).reshape(-1)
        tg = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
        return lib().ref_forward(self._h, _d(params), _i(inputs), _i(tg))

    def backward(self, params: np.ndarray, grads: np.ndarray) -> None:
        if lib().ref_backward(self._h, _d(params), _d(grads)) != 0:
            raise RuntimeError("oracle backward needs a forward with targets first")

    def decode_step(self, params: np.ndarray, tokens: np.ndarray, pos: int, coins: np.ndarray | None = None):
        """Row (b, pos) of every sequence through the model with the cached
        keys and values of the earlier positions; returns the next ids."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        nxt = np.empty(self.B, dtype=np.int32)
        c = None if coins is None else np.ascontiguousarray(coins, dtype=np.float64).reshape(-1)
        if lib().ref_decode_step(self._h, _d(params), _i(tokens), pos, _d(c), _i(nxt)) != 0:
            raise ValueError("oracle decode: bad position or token")
        return nxt

    def get(self, name: str, grad: bool = False) -> np.ndarray:
        n = lib().ref_act_count(self._h, name.encode())
        if n < 0:
            raise KeyError(name)
        out = np.empty(n, dtype=np.float64)
        lib().ref_get(self._h, name.encode(), int(grad), _d(out), n)
        return out


# ---------------------------------------------------------------- layers

def encoder_forward(tok, wte, wpe, B, T, C):
    out = np.empty(B * T * C)
    lib().ref_encoder_forward(_d(out), _i(tok), _d(wte), _d(wpe), B, T, C)
    return out


def encoder_backward(dwte, dwpe, dout, tok, B, T, C):
    lib().ref_encoder_backward(_d(dwte), _d(dwpe), _d(dout), _i(tok), B, T, C)


def layernorm_forward(inp, w, b, N, C):
    out, mean, rstd = np.empty(N * C), np.empty(N), np.empty(N)
    lib().ref_layernorm_forward(_d(out), _d(mean), _d(rstd), _d(inp), _d(w), _d(b), N, C)
    return out, mean, rstd


def layernorm_backward(dinp, dw, db, dout, inp, w, mean, rstd, N, C):
    lib().ref_layernorm_backward(_d(dinp), _d(dw), _d(db), _d(dout), _d(inp), _d(w), _d(mean),
                                 _d(rstd), N, C)


def matmul_forward(inp, W, bias, N, K, OC):
    out = np.empty(N * OC)
    lib().ref_matmul_forward(_d(out), _d(inp), _d(W), _d(bias), N, K, OC)
    return out


def matmul_backward(dinp, dW, db, dout, inp, W, N, K, OC):
    lib().ref_matmul_backward(_d(dinp), _d(dW), _d(db), _d(dout), _d(inp), _d(W), N, K, OC)


def attention_forward(qkv, B, T, C, NH):
    out = np.empty(B * T * C)
    pre = np.empty(B * NH * T * T)
    att = np.empty(B * NH * T * T)
    lib().ref_attention_forward(_d(out), _d(pre), _d(att), _d(qkv), B, T, C, NH)
    return out, pre, att


def attention_backward(dqkv, dout, qkv, att, B, T, C, NH):
    dpre = np.empty(B * NH * T * T)
    datt = np.empty(B * NH * T * T)
    lib().ref_attention_backward(_d(dqkv), _d(dpre), _d(datt), _d(dout), _d(qkv), _d(att), B, T, C, NH)
    return dpre, datt


def gelu_forward(x):
    out = np.empty_like(x)
    lib().ref_gelu_forward(_d(out), _d(x), x.size)
    return out


def gelu_backward(dinp, x, dout):
    lib().ref_gelu_backward(_d(dinp), _d(x), _d(dout), x.size)


def residual_forward(a, b):
    out = np.empty_like(a)
    lib().ref_residual_forward(_d(out), _d(a), _d(b), a.size)
    return out


def softmax_crossentropy_forward(logits, targets, N, V, ld):
    losses, probs = np.empty(N), np.empty(N * V)
    lib().ref_softmax_crossentropy_forward(_d(losses), _d(probs), _d(logits), _i(targets), N, V, ld)
    return losses, probs


def crossentropy_softmax_backward(probs, targets, N, V, ld):
    d = np.empty(N * ld)
    lib().ref_crossentropy_softmax_backward(_d(d), _d(probs), _i(targets), N, V, ld)
    return d


def round_bf16(x: float) -> float:
    """x rounded to bfloat16 (8 significant bits, ties to even), as a float."""
    return lib().ref_round_bf16(float(x))


class bf16_products:
    """Within this context the oracle's linear-layer products (forward and
    backward, the head included) use bfloat16 roundings of their operands."""

    def __enter__(self):
        lib().ref_set_bf16_products(1)
        return self

    def __exit__(self, *exc):
        lib().ref_set_bf16_products(0)
        return False


def sample(z: np.ndarray, coin: float = -1.0) -> int:
    """The oracle's next-token choice from one row of logits (coin < 0: argmax)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    return lib().ref_sample(_d(z), z.size, coin)


def adamw(params, grads, m, v, lr, b1, b2, eps, wd, t):
    lib().ref_adamw(_d(params), _d(grads), _d(m), _d(v), params.size, lr, b1, b2, eps, wd, t)
