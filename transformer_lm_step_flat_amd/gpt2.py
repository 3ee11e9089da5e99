"""ctypes binding of ``libgpt2mi.so`` (include/gpt2.h, include/gpt2_kernels.h,
include/gpt2_audit.h).

Argument marshalling only: PyTorch provides device memory (``torch.empty``)
and the current HIP stream; every step of the training path runs in the
library's HIP kernels.  There is no fallback: if the library is missing or
no GPU is present, construction raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime the library then shares)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2mi.so")

GPT2_OK, GPT2_EINVAL, GPT2_ERANGE, GPT2_ESTATE, GPT2_EDEVICE, GPT2_EIO = 0, -1, -2, -3, -4, -5
GPT2_PARAMS, GPT2_ACTS = 0, 1
GPT2_FP32, GPT2_BF16 = 0, 1
_STATUS = {0: "GPT2_OK", -1: "GPT2_EINVAL", -2: "GPT2_ERANGE", -3: "GPT2_ESTATE", -4: "GPT2_EDEVICE",
           -5: "GPT2_EIO"}


class Gpt2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("max_seq_len", ctypes.c_int), ("vocab_size", ctypes.c_int), ("padded_vocab_size", ctypes.c_int),
                ("num_layers", ctypes.c_int), ("num_heads", ctypes.c_int), ("channels", ctypes.c_int)]


class Sizes(ctypes.Structure):
    _fields_ = [("params", ctypes.c_size_t), ("acts", ctypes.c_size_t), ("work", ctypes.c_size_t),
                ("iwork", ctypes.c_size_t)]


class Buffers(ctypes.Structure):
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("adam_m", ctypes.c_void_p),
                ("adam_v", ctypes.c_void_p), ("acts", ctypes.c_void_p), ("work", ctypes.c_void_p),
                ("iwork", ctypes.c_void_p)]


class ProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 128), ("launches", ctypes.c_longlong), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGS = {
    "gpt2_query_sizes": [ctypes.POINTER(Config), _I, _I, ctypes.POINTER(Sizes)],
    "gpt2_layout": [ctypes.POINTER(Config), _I, _I, _I, _I, ctypes.POINTER(ctypes.c_char_p),
                    ctypes.POINTER(_Z), ctypes.POINTER(_Z)],
    "gpt2_build": [ctypes.POINTER(Config), _I, _I, ctypes.POINTER(Buffers), _P, _P, ctypes.POINTER(_P)],
    "gpt2_forward": [_P, _P, _P, ctypes.POINTER(_F)],
    "gpt2_zero_grad": [_P],
    "gpt2_backward": [_P],
    "gpt2_update": [_P, _F, _F, _F, _F, _F, _I],
    "gpt2_sync": [_P],
    "gpt2_set_matmul_precision": [_P, _I],
    "gpt2_decode_step": [_P, _P, _I, _P, _P],
    "gpt2_save_checkpoint": [_P, ctypes.c_char_p, _I],
    "gpt2_audit_step": [ctypes.POINTER(Config), _I, _I, ctypes.c_char_p, _Z, ctypes.c_char_p, _Z,
                        ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_longlong)],
    "gpt2_load_checkpoint": [_P, ctypes.c_char_p, ctypes.POINTER(_I)],
    "gpt2_profile_enable": [_P, _I],
    "gpt2_profile_read": [_P, ctypes.POINTER(ProfileEntry), _I, ctypes.POINTER(_I)],
    "gpt2k_linear_forward": [_P, _P, _P, _P, _I, _I, _I, _P],
    "gpt2k_linear_backward": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P],
    "gpt2k_linear_forward_prec": [_P, _P, _P, _P, _I, _I, _I, _I, _P],
    "gpt2k_linear_backward_prec": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P],
    "gpt2k_layernorm_forward": [_P, _P, _P, _P, _P, _P, _I, _I, _P],
    "gpt2k_layernorm_backward": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P],
    "gpt2k_layernorm_backward_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "gpt2k_attention_forward": [_P, _P, _P, _I, _I, _I, _I, _P],
    "gpt2k_attention_backward": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
    "gpt2k_flash_attention_forward": [_P, _P, _P, _I, _I, _I, _I, _P, _P],
    "gpt2k_flash_attention_backward": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
    "gpt2k_gelu_forward": [_P, _P, _Z, _P],
    "gpt2k_gelu_backward": [_P, _P, _P, _Z, _P],
    "gpt2k_crossentropy": [_P, _P, _P, _P, _I, _I, _I, _P],
    "gpt2k_encoder_forward": [_P, _P, _P, _P, _I, _I, _I, _I, _P],
    "gpt2k_token_order": [_P, _P, _P, _P, _I, _I, _P, _P],
    "gpt2k_encoder_backward": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P],
    "gpt2k_adamw": [_P, _P, _P, _P, _Z, _F, _F, _F, _F, _F, _I, _P],
    "gpt2k_probe_mfma": [_P, _I, ctypes.POINTER(ctypes.c_double), _P],
    "gpt2k_probe_copy": [_P, _P, _Z, _P],
}
_SIZE_FNS = {
    "gpt2k_token_order_work": [_I],
    "gpt2k_linear_backward_work": [_I, _I, _I],
    "gpt2k_layernorm_backward_work": [_I, _I],
    "gpt2k_attention_backward_work": [_I, _I, _I, _I],
    "gpt2k_flash_attention_work": [_I, _I, _I, _I],
    "gpt2k_encoder_backward_work": [_I, _I, _I],
}

# every symbol the headers declare
EXPORTS = sorted(list(_SIGS) + list(_SIZE_FNS) + ["gpt2_free", "gpt2_last_error"])


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m transformer_lm_step_flat_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        for name, args in _SIZE_FNS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _Z
        L.gpt2_free.argtypes = [_P]
        L.gpt2_free.restype = None
        L.gpt2_last_error.argtypes = [_P]
        L.gpt2_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, handle=None):
    if status != GPT2_OK:
        msg = lib().gpt2_last_error(handle)
        raise Gpt2Error(status, (msg or b"").decode())


def make_config(cfg) -> Config:
    return Config(cfg["maxT"], cfg["V"], cfg["Vp"], cfg["L"], cfg["NH"], cfg["C"])


def query_sizes(cfg, B: int, T: int) -> Sizes:
    s = Sizes()
    c = make_config(cfg)
    _check(lib().gpt2_query_sizes(ctypes.byref(c), B, T, ctypes.byref(s)))
    return s


def layout(cfg, B: int, T: int, which: int):
    """[(name, offset, count)] of the parameter (GPT2_PARAMS) or activation table."""
    c = make_config(cfg)
    out = []
    i = 0
    while True:
        nm, off, cnt = ctypes.c_char_p(), _Z(), _Z()
        st = lib().gpt2_layout(ctypes.byref(c), B, T, which, i, ctypes.byref(nm), ctypes.byref(off),
                               ctypes.byref(cnt))
        if st != GPT2_OK:
            break
        out.append((nm.value.decode(), off.value, cnt.value))
        i += 1
    return out


def pack_params(cfg, tensors: dict, B: int = 1, T: int = 4) -> np.ndarray:
    """Named host tensors -> one flat float32 array in the library's layout."""
    lay = layout(cfg, B, T, GPT2_PARAMS)
    n = lay[-1][1] + lay[-1][2]
    flat = np.empty(n, dtype=np.float32)
    for name, off, cnt in lay:
        a = np.asarray(tensors[name], dtype=np.float32).reshape(-1)
        if a.size != cnt:
            raise ValueError(f"{name}: {a.size} values, layout wants {cnt}")
        flat[off:off + cnt] = a
    return flat


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def audit_step(cfg, B: int, T: int, shrink: str | None = None, shrink_floats: int = 0):
    """Host-only replay of one training step's launches against the layout
    (no GPU): (ranges declared, ranges outside their tensor, report text)."""
    c = make_config(cfg)
    buf = ctypes.create_string_buffer(1 << 16)
    nr, nv = ctypes.c_longlong(), ctypes.c_longlong()
    _check(lib().gpt2_audit_step(ctypes.byref(c), B, T, shrink.encode() if shrink else None, shrink_floats, buf,
                                 len(buf), ctypes.byref(nr), ctypes.byref(nv)))
    return nr.value, nv.value, buf.value.decode()


class Model:
    """One fp32 GPT-2 at fixed (B, T) over flat device buffers owned here
    (allocated once with torch.empty) and borrowed by the library."""

    def __init__(self, cfg, B: int, T: int, init_params: np.ndarray | None = None, device: str = "cuda"):
        if not torch.cuda.is_available():
            raise RuntimeError("libgpt2mi needs a GPU; none is visible")
        self.cfg, self.B, self.T = dict(cfg), B, T
        self.device = torch.device(device)
        sz = query_sizes(cfg, B, T)
        self.sizes = sz
        f32 = dict(dtype=torch.float32, device=self.device)
        self.params = torch.empty(sz.params, **f32)
        self.grads = torch.empty(sz.params, **f32)
        self.adam_m = torch.empty(sz.params, **f32)
        self.adam_v = torch.empty(sz.params, **f32)
        self.acts = torch.empty(sz.acts, **f32)
        self.work = torch.empty(max(sz.work, 1), **f32)
        self.iwork = torch.empty(sz.iwork, dtype=torch.int32, device=self.device)
        self._bufs = Buffers(*[t.data_ptr() for t in (self.params, self.grads, self.adam_m, self.adam_v, self.acts,
                                                       self.work, self.iwork)])
        host = None
        if init_params is not None:
            host = np.ascontiguousarray(init_params, dtype=np.float32)
            if host.size != sz.params:
                raise ValueError(f"init_params has {host.size} values, the layout has {sz.params}")
        c = make_config(cfg)
        h = _P()
        st = lib().gpt2_build(ctypes.byref(c), B, T, ctypes.byref(self._bufs),
                              None if host is None else host.ctypes.data, _stream(self.device), ctypes.byref(h))
        _check(st)
        self._h = h
        self.param_layout = {n: (o, k) for n, o, k in layout(cfg, B, T, GPT2_PARAMS)}
        self.act_layout = {n: (o, k) for n, o, k in layout(cfg, B, T, GPT2_ACTS)}

    def close(self):
        if getattr(self, "_h", None):
            lib().gpt2_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # --- views into the flat buffers
    def param(self, name):
        o, k = self.param_layout[name]
        return self.params[o:o + k]

    def grad(self, name):
        o, k = self.param_layout[name]
        return self.grads[o:o + k]

    def act(self, name):
        o, k = self.act_layout[name]
        return self.acts[o:o + k]

    # --- the step
    def forward(self, inputs, targets=None, want_loss: bool = True):
        """inputs/targets: int32 device tensors of B*T ids.  Returns the mean
        loss (waits for the GPU) when targets are given and want_loss."""
        for t in (inputs, targets):
            if t is not None and (t.dtype != torch.int32 or not t.is_cuda or t.numel() != self.B * self.T
                                  or not t.is_contiguous()):
                raise ValueError("ids must be contiguous int32 device tensors of B*T elements")
        loss = ctypes.c_float()
        st = lib().gpt2_forward(self._h, _ptr(inputs), _ptr(targets),
                                ctypes.byref(loss) if (targets is not None and want_loss) else None)
        _check(st, self._h)
        return loss.value if (targets is not None and want_loss) else None

    def zero_grad(self):
        _check(lib().gpt2_zero_grad(self._h), self._h)

    def backward(self):
        _check(lib().gpt2_backward(self._h), self._h)

    def update(self, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=1):
        _check(lib().gpt2_update(self._h, lr, beta1, beta2, eps, weight_decay, t), self._h)

    def sync(self):
        _check(lib().gpt2_sync(self._h), self._h)

    def set_matmul_precision(self, precision: int):
        """GPT2_FP32 or GPT2_BF16 for the linear-layer products of later calls."""
        _check(lib().gpt2_set_matmul_precision(self._h, precision), self._h)

    # --- evaluation and decoding
    def eval_loss(self, batches) -> float:
        """Mean of the mean losses of (inputs, targets) device batches: forward
        passes only (the pages' validation loss)."""
        losses = [self.forward(i, t) for i, t in batches]
        return sum(losses) / len(losses)

    def decode_step(self, tokens, pos: int, coins=None, next_ids=None):
        """Row pos of every sequence through the model with the cached keys and
        values of positions < pos; returns the device int32[B] next ids."""
        for t, dt in ((tokens, torch.int32), (coins, torch.float32)):
            if t is not None and (t.dtype != dt or not t.is_cuda or t.numel() != self.B or not t.is_contiguous()):
                raise ValueError("tokens (int32) and coins (float32) must be contiguous device tensors of B elements")
        if next_ids is None:
            next_ids = torch.empty(self.B, dtype=torch.int32, device=self.device)
        _check(lib().gpt2_decode_step(self._h, _ptr(tokens), pos, _ptr(coins), _ptr(next_ids)), self._h)
        return next_ids

    # --- checkpoints
    def save(self, path: str, t: int):
        """Write params, m, v and the step count t (optimizer steps taken) to path."""
        _check(lib().gpt2_save_checkpoint(self._h, os.fsencode(path), t), self._h)

    def load(self, path: str) -> int:
        """Read a checkpoint of the same config into params, m, v; returns its step count."""
        t = _I()
        _check(lib().gpt2_load_checkpoint(self._h, os.fsencode(path), ctypes.byref(t)), self._h)
        return t.value

    # --- per-launch timing
    def profile_enable(self, on: bool = True):
        _check(lib().gpt2_profile_enable(self._h, int(on)), self._h)

    def profile_read(self):
        """[{name, launches, ms, flops, bytes}] since the last read (waits for the GPU)."""
        n = ctypes.c_int()
        buf = (ProfileEntry * 256)()
        _check(lib().gpt2_profile_read(self._h, buf, 256, ctypes.byref(n)), self._h)
        return [dict(name=buf[i].name.decode(), launches=buf[i].launches, ms=buf[i].ms, flops=buf[i].flops,
                     bytes=buf[i].bytes) for i in range(min(n.value, 256))]


# ---------------------------------------------------------------- kernel-level calls
#
# Each wrapper checks, before the call, that every tensor holds at least the
# elements the kernels will touch for the given sizes (the C ABI takes raw
# device pointers and cannot), so a size mistake raises here instead of
# reaching the GPU as an out-of-bounds access.

def _s():
    return _stream()


def _need(**tensors):
    """tensors: name=(tensor or None, element count it must hold)."""
    for name, (t, n) in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements, the call touches {n}")


def linear_forward(out, inp, W, bias, N, K, OC, precision=GPT2_FP32):
    _need(out=(out, N * OC), inp=(inp, N * K), W=(W, OC * K), bias=(bias, OC))
    _check(lib().gpt2k_linear_forward_prec(_ptr(out), _ptr(inp), _ptr(W), _ptr(bias), N, K, OC, precision, _s()))


def linear_backward(dinp, dW, dbias, dout, inp, W, N, K, OC, precision=GPT2_FP32):
    _need(dinp=(dinp, N * K), dW=(dW, OC * K), dbias=(dbias, OC), dout=(dout, N * OC), inp=(inp, N * K),
          W=(W, OC * K))
    work = torch.empty(max(1, lib().gpt2k_linear_backward_work(N, K, OC)), dtype=torch.float32, device=dout.device)
    _check(lib().gpt2k_linear_backward_prec(_ptr(dinp), _ptr(dW), _ptr(dbias), _ptr(dout), _ptr(inp), _ptr(W), N,
                                            K, OC, _ptr(work), precision, _s()))
    return work


def layernorm_forward(out, mean, rstd, inp, w, b, N, C):
    _need(out=(out, N * C), mean=(mean, N), rstd=(rstd, N), inp=(inp, N * C), w=(w, C), b=(b, C))
    _check(lib().gpt2k_layernorm_forward(_ptr(out), _ptr(mean), _ptr(rstd), _ptr(inp), _ptr(w), _ptr(b), N, C,
                                         _s()))


def _ln_bwd_need(dinp, dw, db, dout, inp, w, mean, rstd, N, C):
    _need(dinp=(dinp, N * C), dw=(dw, C), db=(db, C), dout=(dout, N * C), inp=(inp, N * C), w=(w, C),
          mean=(mean, N), rstd=(rstd, N))


def layernorm_backward(dinp, dw, db, dout, inp, w, mean, rstd, N, C, accumulate):
    _ln_bwd_need(dinp, dw, db, dout, inp, w, mean, rstd, N, C)
    work = torch.empty(max(1, lib().gpt2k_layernorm_backward_work(N, C)), dtype=torch.float32, device=dout.device)
    _check(lib().gpt2k_layernorm_backward(_ptr(dinp), _ptr(dw), _ptr(db), _ptr(dout), _ptr(inp), _ptr(w),
                                          _ptr(mean), _ptr(rstd), N, C, int(accumulate), _ptr(work), _s()))
    return work


def layernorm_backward_noalloc(dinp, dw, db, dout, inp, w, mean, rstd, N, C, accumulate):
    """The same as layernorm_backward, with the library's static scratch (no allocation)."""
    _ln_bwd_need(dinp, dw, db, dout, inp, w, mean, rstd, N, C)
    _check(lib().gpt2k_layernorm_backward_noalloc(_ptr(dinp), _ptr(dw), _ptr(db), _ptr(dout), _ptr(inp), _ptr(w),
                                                  _ptr(mean), _ptr(rstd), N, C, int(accumulate), _s()))


def attention_forward(atty, att, qkv, B, T, C, NH):
    _need(atty=(atty, B * T * C), att=(att, B * NH * T * T), qkv=(qkv, B * T * 3 * C))
    _check(lib().gpt2k_attention_forward(_ptr(atty), _ptr(att), _ptr(qkv), B, T, C, NH, _s()))


def attention_backward(dqkv, datty, qkv, att, B, T, C, NH):
    _need(dqkv=(dqkv, B * T * 3 * C), datty=(datty, B * T * C), qkv=(qkv, B * T * 3 * C), att=(att, B * NH * T * T))
    work = torch.empty(max(1, lib().gpt2k_attention_backward_work(B, T, C, NH)), dtype=torch.float32,
                       device=qkv.device)
    _check(lib().gpt2k_attention_backward(_ptr(dqkv), _ptr(datty), _ptr(qkv), _ptr(att), B, T, C, NH, _ptr(work),
                                          _s()))
    return work


def _flash_work(B, T, C, NH, device):
    return torch.empty(max(1, lib().gpt2k_flash_attention_work(B, T, C, NH)), dtype=torch.float32, device=device)


def flash_attention_forward(atty, lse, qkv, B, T, C, NH):
    _need(atty=(atty, B * T * C), lse=(lse, B * NH * T), qkv=(qkv, B * T * 3 * C))
    work = _flash_work(B, T, C, NH, qkv.device)
    _check(lib().gpt2k_flash_attention_forward(_ptr(atty), _ptr(lse), _ptr(qkv), B, T, C, NH, _ptr(work), _s()))
    return work


def flash_attention_backward(dqkv, datty, qkv, atty, lse, B, T, C, NH):
    _need(dqkv=(dqkv, B * T * 3 * C), datty=(datty, B * T * C), qkv=(qkv, B * T * 3 * C), atty=(atty, B * T * C),
          lse=(lse, B * NH * T))
    work = _flash_work(B, T, C, NH, qkv.device)
    _check(lib().gpt2k_flash_attention_backward(_ptr(dqkv), _ptr(datty), _ptr(qkv), _ptr(atty), _ptr(lse), B, T, C,
                                                NH, _ptr(work), _s()))
    return work


def gelu_forward(out, inp):
    _need(out=(out, inp.numel()))
    _check(lib().gpt2k_gelu_forward(_ptr(out), _ptr(inp), inp.numel(), _s()))


def gelu_backward(dinp, inp, dout):
    _need(dinp=(dinp, inp.numel()), dout=(dout, inp.numel()))
    _check(lib().gpt2k_gelu_backward(_ptr(dinp), _ptr(inp), _ptr(dout), inp.numel(), _s()))


def crossentropy(logits, losses, loss, targets, BT, V, Vp):
    _need(logits=(logits, BT * Vp), losses=(losses, BT), loss=(loss, 1), targets=(targets, BT))
    _check(lib().gpt2k_crossentropy(_ptr(logits), _ptr(losses), _ptr(loss), _ptr(targets), BT, V, Vp, _s()))


def encoder_forward(out, ids, wte, wpe, B, T, C, V):
    _need(out=(out, B * T * C), ids=(ids, B * T), wte=(wte, V * C), wpe=(wpe, T * C))
    _check(lib().gpt2k_encoder_forward(_ptr(out), _ptr(ids), _ptr(wte), _ptr(wpe), B, T, C, V, _s()))


def token_order(order, err, ids, targets, BT, V):
    _need(order=(order, BT), err=(err, 1), ids=(ids, BT), targets=(targets, BT))
    nw = lib().gpt2k_token_order_work(BT)
    work = torch.empty(nw, dtype=torch.int32, device=ids.device) if nw else None
    _check(lib().gpt2k_token_order(_ptr(order), _ptr(err), _ptr(ids), _ptr(targets), BT, V, _ptr(work), _s()))


def encoder_backward(dwte, dwpe, dout, ids, order, B, T, C, V):
    _need(dwte=(dwte, V * C), dwpe=(dwpe, T * C), dout=(dout, B * T * C), ids=(ids, B * T), order=(order, B * T))
    work = torch.empty(max(1, lib().gpt2k_encoder_backward_work(B, T, C)), dtype=torch.float32, device=dout.device)
    _check(lib().gpt2k_encoder_backward(_ptr(dwte), _ptr(dwpe), _ptr(dout), _ptr(ids), _ptr(order), B, T, C, V,
                                        _ptr(work), _s()))
    return work


def adamw(params, grads, m, v, lr, b1, b2, eps, wd, t):
    n = params.numel()
    _need(grads=(grads, n), m=(m, n), v=(v, n))
    _check(lib().gpt2k_adamw(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), n, lr, b1, b2, eps, wd, t, _s()))


def probe_mfma(out, iters):
    """Launch the matrix-core calibration kernel; returns the FLOPs it does."""
    _need(out=(out, 1))
    flops = ctypes.c_double(0.0)
    _check(lib().gpt2k_probe_mfma(_ptr(out), iters, ctypes.byref(flops), _s()))
    return flops.value


def probe_copy(dst, src):
    _need(dst=(dst, src.numel()))
    _check(lib().gpt2k_probe_copy(_ptr(dst), _ptr(src), src.numel(), _s()))
