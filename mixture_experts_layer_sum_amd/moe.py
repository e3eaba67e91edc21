"""Thin ctypes binding over libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the layer runs in the library's HIP kernels.  There
is no fallback: if the library is missing or fails to load, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_COMBINE, MOE_OP_AUX_LOSS,
 MOE_OP_EXPERT_DOWN, MOE_OP_PERMUTE_REROUTE, MOE_OP_EXPERT_BACKWARD,
 MOE_OP_ROUTER_BACKWARD, MOE_OP_EXPERT_BACKWARD_SAVED) = range(10)

# Every symbol include/moe.h declares, with (restype, argtypes).
_P, _I, _F, _D, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_capacity": (_I, [_I, _I, _I, _D]),
    "moe_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_route": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_permute": (_I, [_P, _P, _I, _I, _I, _I, _D, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_permute_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _D, _I, _P, _P, _P, _P, _P, _P]),
    "moe_permute_reroute": (_I, [_P, _P, _P, _I, _I, _I, _I, _D, _I, _P, _P, _P, _P, _P, _P, _Z,
                                 _P]),
    "moe_expert_ffn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "moe_expert_up": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_expert_up_save": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_expert_down": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "moe_quantize_fp8": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_expert_up_fp8": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_expert_down_fp8": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_aux_loss": (_I, [_P, _P, _I, _I, _I, _P, _P, _Z, _P]),
    "moe_combine_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_expert_backward": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                 _Z, _P]),
    "moe_expert_backward_saved": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P,
                                       _P, _P, _P, _Z, _P]),
    "moe_router_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _F, _I, _I, _I, _I,
                                 _I, _P, _P, _P, _P, _Z, _P]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(or python -m mixture_experts_layer_sum_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = load_library()


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode()}")


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(op: int, T: int, d: int, N: int, k: int, f: int, dtype: torch.dtype) -> int:
    return int(_lib.moe_workspace_size(op, T, d, N, k, f,
                                       MOE_BF16 if dtype == torch.bfloat16 else MOE_F32))


def _empty(shape, dtype, device, out):
    return torch.empty(shape, dtype=dtype, device=device) if out is None else out


def moe_route(hidden, w_router, k, bias=None, logits=None, topk_idx=None, topk_w=None,
              counts=None, ws=None, stream=None):
    T, d = hidden.shape
    N = w_router.shape[1]
    dev = hidden.device
    logits = _empty((T, N), torch.float32, dev, logits)
    topk_idx = _empty((T, k), torch.int32, dev, topk_idx)
    topk_w = _empty((T, k), torch.float32, dev, topk_w)
    counts = _empty((N,), torch.int32, dev, counts)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_ROUTE, T, d, N, k, 1, hidden.dtype)),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_route(_ptr(hidden), _ptr(w_router), _ptr(bias), T, d, N, k, _dt(hidden),
                          _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(ws),
                          ws.numel(), _stream(stream)), "moe_route")
    return logits, topk_idx, topk_w, counts


def moe_permute(hidden, topk_idx, N, capacity_factor=0.0, x_perm=None, perm_src=None,
                slot_row=None, kept=None, offsets=None, ws=None, stream=None):
    T, d = hidden.shape
    k = topk_idx.shape[1]
    dev = hidden.device
    x_perm = _empty((T * k, d), hidden.dtype, dev, x_perm)
    perm_src = _empty((T * k,), torch.int32, dev, perm_src)
    slot_row = _empty((T, k), torch.int32, dev, slot_row)
    kept = _empty((N,), torch.int32, dev, kept)
    offsets = _empty((N + 1,), torch.int32, dev, offsets)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_PERMUTE, T, d, N, k, 1, hidden.dtype)),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_permute(_ptr(hidden), _ptr(topk_idx), T, d, N, k, float(capacity_factor),
                            _dt(hidden), _ptr(x_perm), _ptr(perm_src), _ptr(slot_row), _ptr(kept),
                            _ptr(offsets), _ptr(ws), ws.numel(), _stream(stream)), "moe_permute")
    return x_perm, perm_src, slot_row, kept, offsets


def moe_permute_noalloc(hidden, topk_idx, N, capacity_factor=0.0, x_perm=None, perm_src=None,
                        slot_row=None, kept=None, offsets=None, stream=None):
    """moe_permute with the library's static scratch instead of a workspace (outputs are
    allocated here only when not given)."""
    T, d = hidden.shape
    k = topk_idx.shape[1]
    dev = hidden.device
    x_perm = _empty((T * k, d), hidden.dtype, dev, x_perm)
    perm_src = _empty((T * k,), torch.int32, dev, perm_src)
    slot_row = _empty((T, k), torch.int32, dev, slot_row)
    kept = _empty((N,), torch.int32, dev, kept)
    offsets = _empty((N + 1,), torch.int32, dev, offsets)
    _check(_lib.moe_permute_noalloc(_ptr(hidden), _ptr(topk_idx), T, d, N, k,
                                    float(capacity_factor), _dt(hidden), _ptr(x_perm),
                                    _ptr(perm_src), _ptr(slot_row), _ptr(kept), _ptr(offsets),
                                    _stream(stream)), "moe_permute_noalloc")
    return x_perm, perm_src, slot_row, kept, offsets


def moe_permute_reroute(hidden, topk_idx, logits, N, capacity_factor=0.0, x_perm=None,
                        perm_src=None, slot_row=None, kept=None, offsets=None, ws=None,
                        stream=None):
    T, d = hidden.shape
    k = topk_idx.shape[1]
    dev = hidden.device
    x_perm = _empty((T * k, d), hidden.dtype, dev, x_perm)
    perm_src = _empty((T * k,), torch.int32, dev, perm_src)
    slot_row = _empty((T, k), torch.int32, dev, slot_row)
    kept = _empty((N,), torch.int32, dev, kept)
    offsets = _empty((N + 1,), torch.int32, dev, offsets)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_PERMUTE_REROUTE, T, d, N, k, 1, hidden.dtype)),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_permute_reroute(_ptr(hidden), _ptr(topk_idx), _ptr(logits), T, d, N, k,
                                    float(capacity_factor), _dt(hidden), _ptr(x_perm),
                                    _ptr(perm_src), _ptr(slot_row), _ptr(kept), _ptr(offsets),
                                    _ptr(ws), ws.numel(), _stream(stream)), "moe_permute_reroute")
    return x_perm, perm_src, slot_row, kept, offsets


def moe_expert_up(x_perm, offsets, w1, w3, act=None, stream=None):
    max_rows, d = x_perm.shape
    N, _, f = w1.shape
    act = _empty((max_rows, f), x_perm.dtype, x_perm.device, act)
    _check(_lib.moe_expert_up(_ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), N, d, f, max_rows,
                              _dt(x_perm), _ptr(act), _stream(stream)), "moe_expert_up")
    return act


def moe_expert_up_save(x_perm, offsets, w1, w3, act=None, h13=None, stream=None):
    """moe_expert_up that also stores h13 = [x W1 | x W3] per row for the backward."""
    max_rows, d = x_perm.shape
    N, _, f = w1.shape
    act = _empty((max_rows, f), x_perm.dtype, x_perm.device, act)
    h13 = _empty((max_rows, 2 * f), x_perm.dtype, x_perm.device, h13)
    _check(_lib.moe_expert_up_save(_ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), N, d, f,
                                   max_rows, _dt(x_perm), _ptr(act), _ptr(h13), _stream(stream)),
           "moe_expert_up_save")
    return act, h13


def moe_expert_down(act, offsets, w2, y_perm=None, ws=None, stream=None):
    max_rows, f = act.shape
    N, _, d = w2.shape
    y_perm = _empty((max_rows, d), torch.float32, act.device, y_perm)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_EXPERT_DOWN, max_rows, d, N, 1, f, act.dtype)),
                         dtype=torch.uint8, device=act.device)
    _check(_lib.moe_expert_down(_ptr(act), _ptr(offsets), _ptr(w2), N, d, f, max_rows, _dt(act),
                                _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_down")
    return y_perm


def moe_expert_ffn(x_perm, offsets, w1, w3, w2, y_perm=None, ws=None, stream=None):
    max_rows, d = x_perm.shape
    N, _, f = w1.shape
    dev = x_perm.device
    y_perm = _empty((max_rows, d), torch.float32, dev, y_perm)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_EXPERT_FFN, max_rows, d, N, 1, f, x_perm.dtype)),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_expert_ffn(_ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2), N, d, f,
                               max_rows, _dt(x_perm), _ptr(y_perm), _ptr(ws), ws.numel(),
                               _stream(stream)), "moe_expert_ffn")
    return y_perm


def moe_quantize_fp8(w, q=None, scale=None, stream=None):
    """Per-column OCP FP8 E4M3 codes and fp32 scales of w [N, K, M] (bf16 or fp32)."""
    N, K, M = w.shape
    q = _empty((N, K, M), torch.uint8, w.device, q)
    scale = _empty((N, M), torch.float32, w.device, scale)
    _check(_lib.moe_quantize_fp8(_ptr(w), _dt(w), N, K, M, _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_fp8")
    return q, scale


def moe_expert_up_fp8(x_perm, offsets, w1q, w3q, s1, s3, act=None, stream=None):
    max_rows, d = x_perm.shape
    N, _, f = w1q.shape
    act = _empty((max_rows, f), torch.bfloat16, x_perm.device, act)
    _check(_lib.moe_expert_up_fp8(_ptr(x_perm), _ptr(offsets), _ptr(w1q), _ptr(w3q), _ptr(s1),
                                  _ptr(s3), N, d, f, max_rows, _ptr(act), _stream(stream)),
           "moe_expert_up_fp8")
    return act


def moe_expert_down_fp8(act, offsets, w2q, s2, y_perm=None, stream=None):
    max_rows, f = act.shape
    N, _, d = w2q.shape
    y_perm = _empty((max_rows, d), torch.float32, act.device, y_perm)
    _check(_lib.moe_expert_down_fp8(_ptr(act), _ptr(offsets), _ptr(w2q), _ptr(s2), N, d, f,
                                    max_rows, _ptr(y_perm), _stream(stream)), "moe_expert_down_fp8")
    return y_perm


def moe_combine(y_perm, slot_row, topk_w, dtype, y=None, y_shared=None, stream=None):
    """y_shared: None or fp32 [n_shared, T, d] (the shared experts' outputs)."""
    T, k = slot_row.shape
    d = y_perm.shape[1]
    y = _empty((T, d), dtype, y_perm.device, y)
    n_shared = 0 if y_shared is None else y_shared.shape[0]
    _check(_lib.moe_combine(_ptr(y_perm), _ptr(slot_row), _ptr(topk_w), _ptr(y_shared), n_shared,
                            T, d, k, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32, _ptr(y),
                            _stream(stream)), "moe_combine")
    return y


def moe_aux_loss(logits, counts, k, aux=None, ws=None, stream=None):
    T, N = logits.shape
    dev = logits.device
    aux = _empty((1,), torch.float32, dev, aux)
    if ws is None:
        ws = torch.empty(workspace_size(MOE_OP_AUX_LOSS, T, 1, N, k, 1, torch.float32),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_aux_loss(_ptr(logits), _ptr(counts), T, N, k, _ptr(aux), _ptr(ws), ws.numel(),
                             _stream(stream)), "moe_aux_loss")
    return aux


class MoEBuffers:
    """Every output and workspace of one layer forward, allocated once."""

    def __init__(self, T, d, N, k, f, dtype, device="cuda", n_shared=0, f_shared=None,
                 save_for_backward=False):
        self.T, self.d, self.N, self.k, self.f, self.dtype = T, d, N, k, f, dtype
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
        self.logits = e((T, N), torch.float32)
        self.topk_idx = e((T, k), torch.int32)
        self.topk_w = e((T, k), torch.float32)
        self.counts = e((N,), torch.int32)
        self.x_perm = e((T * k, d), dtype)
        self.perm_src = e((T * k,), torch.int32)
        self.slot_row = e((T, k), torch.int32)
        self.kept = e((N,), torch.int32)
        self.offsets = e((N + 1,), torch.int32)
        self.act = e((T * k, f), dtype)
        # training: [x W1 | x W3] per routed row, kept for moe_expert_backward_saved
        self.h13 = e((T * k, 2 * f), dtype) if save_for_backward else None
        self.y_perm = e((T * k, d), torch.float32)
        self.y = e((T, d), dtype)
        self.aux = e((1,), torch.float32)
        self.ws_route = e((max(1, workspace_size(MOE_OP_ROUTE, T, d, N, k, f, dtype)),), torch.uint8)
        self.ws_permute = e((max(1, workspace_size(MOE_OP_PERMUTE, T, d, N, k, f, dtype),
                                 workspace_size(MOE_OP_PERMUTE_REROUTE, T, d, N, k, f, dtype)),),
                            torch.uint8)
        self.ws_aux = e((max(1, workspace_size(MOE_OP_AUX_LOSS, T, d, N, k, f, dtype)),), torch.uint8)
        self.ws_down = e((max(1, workspace_size(MOE_OP_EXPERT_DOWN, T, d, N, k, f, dtype)),),
                         torch.uint8)
        self.n_shared = n_shared
        if n_shared:
            fs = f if f_shared is None else f_shared
            self.shared_offsets = torch.tensor([0, T], dtype=torch.int32, device=device)
            self.y_shared = e((n_shared, T, d), torch.float32)
            self.ws_shared = e((max(1, workspace_size(MOE_OP_EXPERT_FFN, T, d, 1, 1, fs, dtype)),),
                               torch.uint8)


def moe_forward(hidden, w_router, w1, w3, w2, k, capacity_factor=0.0, bias=None,
                bufs: Optional[MoEBuffers] = None, stream=None, overflow="drop", shared=None,
                fp8=None, save_for_backward=False):
    """Run the five steps on the current stream.  Returns the MoEBuffers holding every result.

    ``y`` excludes the residual: the layer output with residual is hidden + y.
    ``overflow`` is "drop" (moe_permute) or "reroute" (moe_permute_reroute).
    ``shared`` is None or (w1s [Ns, d, fs], w3s, w2s [Ns, fs, d]): shared experts every
    token passes through, added with weight 1.
    ``fp8`` is None or (w1q, w3q, w2q, s1, s3, s2) from moe_quantize_fp8: the expert GEMMs
    then read the FP8 codes (w1, w3, w2 are only used for their shapes).
    ``save_for_backward`` (bf16 / fp32 weights): the up projection also keeps
    h13 = [x W1 | x W3] (moe_expert_up_save), which moe_backward then uses instead of
    recomputing it; with ``bufs`` given, they must have been built with it.
    """
    if overflow not in ("drop", "reroute"):
        raise ValueError(f"unknown overflow policy {overflow!r}")
    T, d = hidden.shape
    N, _, f = w1.shape
    ns = 0 if shared is None else shared[0].shape[0]
    if save_for_backward and fp8 is not None:
        raise ValueError("save_for_backward needs bf16 / fp32 expert weights")
    if bufs is None:
        bufs = MoEBuffers(T, d, N, k, f, hidden.dtype, hidden.device, ns,
                          None if shared is None else shared[0].shape[2], save_for_backward)
    b = bufs
    if save_for_backward and b.h13 is None:
        raise ValueError("bufs were built without save_for_backward")
    moe_route(hidden, w_router, k, bias, b.logits, b.topk_idx, b.topk_w, b.counts, b.ws_route,
              stream)
    if overflow == "drop":
        moe_permute(hidden, b.topk_idx, N, capacity_factor, b.x_perm, b.perm_src, b.slot_row,
                    b.kept, b.offsets, b.ws_permute, stream)
    else:
        moe_permute_reroute(hidden, b.topk_idx, b.logits, N, capacity_factor, b.x_perm, b.perm_src,
                            b.slot_row, b.kept, b.offsets, b.ws_permute, stream)
    b.saved = bool(save_for_backward)
    if fp8 is None:
        if save_for_backward:
            moe_expert_up_save(b.x_perm, b.offsets, w1, w3, b.act, b.h13, stream)
        else:
            moe_expert_up(b.x_perm, b.offsets, w1, w3, b.act, stream)
        moe_expert_down(b.act, b.offsets, w2, b.y_perm, b.ws_down, stream)
    else:
        w1q, w3q, w2q, s1, s3, s2 = fp8
        moe_expert_up_fp8(b.x_perm, b.offsets, w1q, w3q, s1, s3, b.act, stream)
        moe_expert_down_fp8(b.act, b.offsets, w2q, s2, b.y_perm, stream)
    y_shared = None
    if ns:
        for q in range(ns):
            moe_expert_ffn(hidden, b.shared_offsets, shared[0][q:q + 1], shared[1][q:q + 1],
                           shared[2][q:q + 1], b.y_shared[q], b.ws_shared, stream)
        y_shared = b.y_shared
    moe_combine(b.y_perm, b.slot_row, b.topk_w, hidden.dtype, b.y, y_shared, stream)
    moe_aux_loss(b.logits, b.counts, k, b.aux, b.ws_aux, stream)
    return b


# ---------------------------------------------------------------- backward
def moe_combine_backward(dy, y_perm, slot_row, topk_w, g_perm=None, dgate=None, stream=None):
    T, d = dy.shape
    k = slot_row.shape[1]
    g_perm = _empty((y_perm.shape[0], d), dy.dtype, dy.device, g_perm)
    dgate = _empty((T, k), torch.float32, dy.device, dgate)
    _check(_lib.moe_combine_backward(_ptr(dy), _ptr(y_perm), _ptr(slot_row), _ptr(topk_w), T, d, k,
                                     _dt(dy), _ptr(g_perm), _ptr(dgate), _stream(stream)),
           "moe_combine_backward")
    return g_perm, dgate


def moe_expert_backward(x_perm, g_perm, offsets, w1, w3, w2, dx_perm=None, dw1=None, dw3=None,
                        dw2=None, ws=None, stream=None):
    max_rows, d = x_perm.shape
    N, _, f = w1.shape
    dev = x_perm.device
    dx_perm = _empty((max_rows, d), torch.float32, dev, dx_perm)
    dw1 = _empty((N, d, f), torch.float32, dev, dw1)
    dw3 = _empty((N, d, f), torch.float32, dev, dw3)
    dw2 = _empty((N, f, d), torch.float32, dev, dw2)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_EXPERT_BACKWARD, max_rows, d, N, 1, f,
                                               x_perm.dtype)), dtype=torch.uint8, device=dev)
    _check(_lib.moe_expert_backward(_ptr(x_perm), _ptr(g_perm), _ptr(offsets), _ptr(w1), _ptr(w3),
                                    _ptr(w2), N, d, f, max_rows, _dt(x_perm), _ptr(dx_perm),
                                    _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(ws), ws.numel(),
                                    _stream(stream)), "moe_expert_backward")
    return dx_perm, dw1, dw3, dw2


def moe_expert_backward_saved(x_perm, g_perm, h13, offsets, w1, w3, w2, dx_perm=None, dw1=None,
                              dw3=None, dw2=None, ws=None, stream=None, act=None):
    """``act``: the forward's activations [max_rows, f] (None: recomputed from h13)."""
    max_rows, d = x_perm.shape
    N, _, f = w1.shape
    dev = x_perm.device
    dx_perm = _empty((max_rows, d), torch.float32, dev, dx_perm)
    dw1 = _empty((N, d, f), torch.float32, dev, dw1)
    dw3 = _empty((N, d, f), torch.float32, dev, dw3)
    dw2 = _empty((N, f, d), torch.float32, dev, dw2)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_EXPERT_BACKWARD_SAVED, max_rows, d, N, 1, f,
                                               x_perm.dtype)), dtype=torch.uint8, device=dev)
    _check(_lib.moe_expert_backward_saved(_ptr(x_perm), _ptr(g_perm), _ptr(h13), _ptr(act),
                                          _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2), N, d, f,
                                          max_rows,
                                          _dt(x_perm), _ptr(dx_perm), _ptr(dw1), _ptr(dw3),
                                          _ptr(dw2), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_backward_saved")
    return dx_perm, dw1, dw3, dw2


def moe_router_backward(hidden, w_router, logits, topk_idx, topk_w, counts, dgate, dx_perm,
                        slot_row, aux_coef=0.0, dhidden=None, dw_router=None, dbias=None,
                        want_dbias=True, ws=None, stream=None, dx_shared=None):
    T, d = hidden.shape
    N = w_router.shape[1]
    k = topk_idx.shape[1]
    dev = hidden.device
    dhidden = _empty((T, d), torch.float32, dev, dhidden)
    dw_router = _empty((d, N), torch.float32, dev, dw_router)
    if want_dbias:
        dbias = _empty((N,), torch.float32, dev, dbias)
    if ws is None:
        ws = torch.empty(max(1, workspace_size(MOE_OP_ROUTER_BACKWARD, T, d, N, k, 1,
                                               hidden.dtype)), dtype=torch.uint8, device=dev)
    ns = 0 if dx_shared is None else dx_shared.shape[0]
    _check(_lib.moe_router_backward(_ptr(hidden), _ptr(w_router), _ptr(logits), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(counts), _ptr(dgate), _ptr(dx_perm),
                                    _ptr(slot_row), _ptr(dx_shared), ns, float(aux_coef), T, d, N,
                                    k, _dt(hidden),
                                    _ptr(dhidden), _ptr(dw_router),
                                    _ptr(dbias) if want_dbias else None, _ptr(ws), ws.numel(),
                                    _stream(stream)), "moe_router_backward")
    return dhidden, dw_router, (dbias if want_dbias else None)


class MoEGradBuffers:
    """Every gradient and workspace of one layer backward, allocated once (fp32 gradients)."""

    def __init__(self, T, d, N, k, f, dtype, device="cuda", n_shared=0, f_shared=None):
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
        self.g_perm = e((T * k, d), dtype)
        self.dgate = e((T, k), torch.float32)
        self.dx_perm = e((T * k, d), torch.float32)
        self.dw1 = e((N, d, f), torch.float32)
        self.dw3 = e((N, d, f), torch.float32)
        self.dw2 = e((N, f, d), torch.float32)
        self.dhidden = e((T, d), torch.float32)
        self.dw_router = e((d, N), torch.float32)
        self.dbias = e((N,), torch.float32)
        self.ws_expert = e((max(1, workspace_size(MOE_OP_EXPERT_BACKWARD, T, d, N, k, f, dtype)),),
                           torch.uint8)
        self.ws_router = e((max(1, workspace_size(MOE_OP_ROUTER_BACKWARD, T, d, N, k, f, dtype)),),
                           torch.uint8)
        self.n_shared = n_shared
        if n_shared:
            fs = f if f_shared is None else f_shared
            self.dx_shared = e((n_shared, T, d), torch.float32)
            self.dw1s = e((n_shared, d, fs), torch.float32)
            self.dw3s = e((n_shared, d, fs), torch.float32)
            self.dw2s = e((n_shared, fs, d), torch.float32)
            self.ws_shared = e((max(1, workspace_size(MOE_OP_EXPERT_BACKWARD, T, d, 1, 1, fs,
                                                      dtype)),), torch.uint8)


def moe_backward(hidden, w_router, w1, w3, w2, dy, fwd: MoEBuffers, aux_coef=0.0,
                 grads: Optional[MoEGradBuffers] = None, want_dbias=True, stream=None,
                 shared=None):
    """Gradients of <dy, y> + aux_coef * aux for the batch `fwd` holds (moe_forward's
    buffers of the same call; when that forward saved h13, the expert backward uses it).  Returns the MoEGradBuffers (dhidden, dw_router, dbias,
    dw1, dw3, dw2 in fp32; with ``shared`` = (w1s, w3s, w2s) also dw1s, dw3s, dw2s)."""
    T, d = hidden.shape
    N, _, f = w1.shape
    k = fwd.topk_idx.shape[1]
    ns = 0 if shared is None else shared[0].shape[0]
    if grads is None:
        grads = MoEGradBuffers(T, d, N, k, f, hidden.dtype, hidden.device, ns,
                               None if shared is None else shared[0].shape[2])
    g = grads
    dx_shared = None
    if ns:
        # each shared expert: the expert backward over all T rows with weight 1 (g = dy)
        for q in range(ns):
            moe_expert_backward(hidden, dy, fwd.shared_offsets, shared[0][q:q + 1],
                                shared[1][q:q + 1], shared[2][q:q + 1], g.dx_shared[q],
                                g.dw1s[q:q + 1], g.dw3s[q:q + 1], g.dw2s[q:q + 1], g.ws_shared,
                                stream)
        dx_shared = g.dx_shared
    moe_combine_backward(dy, fwd.y_perm, fwd.slot_row, fwd.topk_w, g.g_perm, g.dgate, stream)
    if getattr(fwd, "saved", False):
        moe_expert_backward_saved(fwd.x_perm, g.g_perm, fwd.h13, fwd.offsets, w1, w3, w2,
                                  g.dx_perm, g.dw1, g.dw3, g.dw2, g.ws_expert, stream,
                                  act=fwd.act)
    else:
        moe_expert_backward(fwd.x_perm, g.g_perm, fwd.offsets, w1, w3, w2, g.dx_perm, g.dw1,
                            g.dw3, g.dw2, g.ws_expert, stream)
    moe_router_backward(hidden, w_router, fwd.logits, fwd.topk_idx, fwd.topk_w, fwd.counts,
                        g.dgate, g.dx_perm, fwd.slot_row, aux_coef, g.dhidden, g.dw_router,
                        g.dbias, want_dbias, g.ws_router, stream, dx_shared)
    return g
