"""ctypes binding of libqspec.so (C-ABI in include/qspec.h).

Argument marshalling only: every function checks dtype, device, contiguity and
shape of the torch tensors it is handed, passes their device pointers and the
current HIP stream to the C function of the same name, and raises QSpecError on
a nonzero status.  All arithmetic runs in the library's HIP kernels; there is
no fallback.  Importing this module raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libqspec.so")

QS_W4A16 = 0
QS_W4A4 = 1
QS_W4A8 = 2
GROUP = 128
MAX_M = 256

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqspec.so not found at {LIB_PATH}; build it with "
        "`python -m quantized_speculative_decoding_int4_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "qs_status_string": ([_i], ctypes.c_char_p),
    "qs_packed_weight_bytes": ([_i, _i], _sz),
    "qs_packed_scale_bytes": ([_i, _i], _sz),
    "qs_pack_weights": ([_p, _p, _i, _i, _p, _p, _p], _i),
    "qs_linear_w4a16": ([_p, _p, _p, _p, _i, _i, _i, _p], _i),
    "qs_linear_workspace_bytes": ([_i, _i, _i, _i], _sz),
    "qs_linear_w4a4": ([_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _sz, _p], _i),
    "qs_linear_w4a8": ([_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _sz, _p], _i),
    "qs_lmhead": ([_i, _p, _p, _p, _p, _i, _i, _i, _p, _sz, _p], _i),
    "qs_lmhead_top1_workspace_bytes": ([_i, _i, _i, _i], _sz),
    "qs_lmhead_top1": ([_i, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "qs_verify_workspace_bytes": ([_i, _i, _i], _sz),
    "qs_chain_workspace_bytes": ([_i, _i, _p, _i], _sz),
    "qs_chain_forward": ([_i, _p, _i, _p, _i, _p, _p, _sz, _p], _i),
    "qs_chain_top1_workspace_bytes": ([_i, _i, _p, _i], _sz),
    "qs_chain_forward_top1": ([_i, _p, _i, _p, _i, _p, _p, _p, _p, _sz, _p], _i),
    "qs_accept_greedy": ([_p, _p, _i, _i, _p, _p, _p], _i),
    "qs_chain_pass_launches": ([_i, _i, _p, _i], _i),
    "qs_set_barrier_timeout_us": ([_i], _i),
    "qs_chain_pass_status": ([_i, _i, _p, _i, _p, _sz, _p, _p], _i),
    "qs_chain_trace_bytes": ([_i, _i, _p, _i], _sz),
    "qs_chain_forward_trace": ([_i, _p, _i, _p, _i, _p, _p, _sz, _p, _sz, _p], _i),
    "qs_verify_greedy": ([_p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p], _i),
    "qs_verify_greedy_noalloc": ([_p, _p, _i, _i, _i, _p, _p, _p, _p, _p], _i),
    "qs_verify_greedy_noalloc_max_bytes": ([], _sz),
    "qs_verify_tree_greedy": ([_p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p], _i),
    "qs_verify_sample": ([_p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p], _i),
}
for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _ret


class QSpecError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status} ({_lib.qs_status_string(status).decode()})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QSpecError(fn, status)


def _ptr(t, dtype, shape=None, name="tensor", nullable=False):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def status_string(status: int) -> str:
    return _lib.qs_status_string(status).decode()


def packed_weight_bytes(n: int, k: int) -> int:
    return _lib.qs_packed_weight_bytes(n, k)


def packed_scale_bytes(n: int, k: int) -> int:
    return _lib.qs_packed_scale_bytes(n, k)


def linear_workspace_bytes(mode: int, m: int, n: int, k: int) -> int:
    return _lib.qs_linear_workspace_bytes(mode, m, n, k)


def verify_workspace_bytes(b: int, gamma: int, v: int) -> int:
    return _lib.qs_verify_workspace_bytes(b, gamma, v)


def qs_pack_weights(q: torch.Tensor, s: torch.Tensor, w_packed=None, s_packed=None):
    """q int8 [N, K], s fp16 [N, K/128] -> (w_packed uint8, s_packed fp16)."""
    n, k = q.shape
    dev = q.device
    if w_packed is None:
        w_packed = torch.empty(packed_weight_bytes(n, k), dtype=torch.uint8, device=dev)
    if s_packed is None:
        s_packed = torch.empty(packed_scale_bytes(n, k) // 2, dtype=torch.float16, device=dev)
    _check("qs_pack_weights", _lib.qs_pack_weights(
        _ptr(q, torch.int8, (n, k), "q"), _ptr(s, torch.float16, (n, k // GROUP), "s"), n, k,
        _ptr(w_packed, torch.uint8, (packed_weight_bytes(n, k),), "w_packed"),
        _ptr(s_packed, torch.float16, (packed_scale_bytes(n, k) // 2,), "s_packed"), _stream()))
    return w_packed, s_packed


def _wcheck(w_packed, s_packed, n, k):
    return (_ptr(w_packed, torch.uint8, (packed_weight_bytes(n, k),), "w_packed"),
            _ptr(s_packed, torch.float16, (packed_scale_bytes(n, k) // 2,), "s_packed"))


def qs_linear_w4a16(x, w_packed, s_packed, n: int, y=None):
    """x fp16 [M, K] -> y fp32 [M, N]."""
    m, k = x.shape
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    wp, sp = _wcheck(w_packed, s_packed, n, k)
    _check("qs_linear_w4a16", _lib.qs_linear_w4a16(
        _ptr(x, torch.float16, (m, k), "x"), wp, sp, _ptr(y, torch.float32, (m, n), "y"), m, n, k,
        _stream()))
    return y


def _linear_int(name, mode, x, w_packed, s_packed, n, y, xq_out, sx_out, acc_out, ws):
    m, k = x.shape
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    need = linear_workspace_bytes(mode, m, n, k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp, sp = _wcheck(w_packed, s_packed, n, k)
    _check(name, getattr(_lib, name)(
        _ptr(x, torch.float16, (m, k), "x"), wp, sp, _ptr(y, torch.float32, (m, n), "y"), m, n, k,
        _ptr(xq_out, torch.int8, (m, k), "xq_out", nullable=True),
        _ptr(sx_out, torch.float16, (m,), "sx_out", nullable=True),
        _ptr(acc_out, torch.int32, (m, n, k // GROUP), "acc_out", nullable=True),
        _ptr(ws, torch.uint8, None, "ws", nullable=True), 0 if ws is None else ws.numel(), _stream()))
    return y


def qs_linear_w4a4(x, w_packed, s_packed, n: int, y=None, xq_out=None, sx_out=None, acc_out=None,
                   ws=None):
    """x fp16 [M, K] -> y fp32 [M, N] with INT4 activations; optional xq int8 [M, K],
    sx fp16 [M], acc int32 [M, N, K/128] outputs; ws uint8 workspace (allocated if needed)."""
    return _linear_int("qs_linear_w4a4", QS_W4A4, x, w_packed, s_packed, n, y, xq_out, sx_out, acc_out, ws)


def qs_linear_w4a8(x, w_packed, s_packed, n: int, y=None, xq_out=None, sx_out=None, acc_out=None,
                   ws=None):
    """As qs_linear_w4a4 with INT8 activations (scale max|x| / 127)."""
    return _linear_int("qs_linear_w4a8", QS_W4A8, x, w_packed, s_packed, n, y, xq_out, sx_out, acc_out, ws)


def qs_lmhead(mode: int, x, w_packed, s_packed, v: int, logits=None, ws=None):
    """x fp16 [M, K] -> logits fp32 [M, V] in mode QS_W4A16, QS_W4A4 or QS_W4A8."""
    m, k = x.shape
    if logits is None:
        logits = torch.empty((m, v), dtype=torch.float32, device=x.device)
    need = linear_workspace_bytes(mode, m, v, k)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp, sp = _wcheck(w_packed, s_packed, v, k)
    _check("qs_lmhead", _lib.qs_lmhead(
        mode, _ptr(x, torch.float16, (m, k), "x"), wp, sp, _ptr(logits, torch.float32, (m, v), "logits"),
        m, v, k, _ptr(ws, torch.uint8, None, "ws", nullable=True), 0 if ws is None else ws.numel(),
        _stream()))
    return logits


def lmhead_top1_workspace_bytes(mode: int, m: int, v: int, k: int) -> int:
    return _lib.qs_lmhead_top1_workspace_bytes(mode, m, v, k)


def qs_lmhead_top1(mode: int, x, w_packed, s_packed, v: int, logits=None, want_logits=True, top1=None,
                   top1_prob=None, ws=None):
    """x fp16 [M, K] -> dict(logits fp32 [M, V] or None, top1 int32 [M], top1_prob fp32 [M]).
    ws: uint8 workspace, zero-filled before its first use (allocated zeroed if None)."""
    m, k = x.shape
    dev = x.device
    if logits is None and want_logits:
        logits = torch.empty((m, v), dtype=torch.float32, device=dev)
    if top1 is None:
        top1 = torch.empty((m,), dtype=torch.int32, device=dev)
    if top1_prob is None:
        top1_prob = torch.empty((m,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.zeros(lmhead_top1_workspace_bytes(mode, m, v, k), dtype=torch.uint8, device=dev)
    wp, sp = _wcheck(w_packed, s_packed, v, k)
    _check("qs_lmhead_top1", _lib.qs_lmhead_top1(
        mode, _ptr(x, torch.float16, (m, k), "x"), wp, sp,
        _ptr(logits, torch.float32, (m, v), "logits", nullable=True), m, v, k,
        _ptr(top1, torch.int32, (m,), "top1"), _ptr(top1_prob, torch.float32, (m,), "top1_prob", nullable=True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()))
    return {"logits": logits, "top1": top1, "top1_prob": top1_prob}


def _ws_for(b, gamma, v, ws, device):
    need = verify_workspace_bytes(b, gamma, v)
    if ws is None:  # zero-filled: the first bytes are arrival counters that start at zero
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
    return ws


def qs_verify_greedy(tgt_logits, draft_ids, out=None, ws=None, want_prob=True):
    """tgt_logits fp32 [B, gamma+1, V], draft_ids int32 [B, gamma] ->
    dict(tgt_top1, top1_prob, n_accept, out_tokens)."""
    b, gp1, v = tgt_logits.shape
    gamma = gp1 - 1
    dev = tgt_logits.device
    if out is None:
        out = {
            "tgt_top1": torch.empty((b, gp1), dtype=torch.int32, device=dev),
            "top1_prob": torch.empty((b, gp1), dtype=torch.float32, device=dev) if want_prob else None,
            "n_accept": torch.empty((b,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((b, gp1), dtype=torch.int32, device=dev),
        }
    ws = _ws_for(b, gamma, v, ws, dev)
    _check("qs_verify_greedy", _lib.qs_verify_greedy(
        _ptr(tgt_logits, torch.float32, (b, gp1, v), "tgt_logits"),
        _ptr(draft_ids, torch.int32, (b, gamma), "draft_ids", nullable=gamma == 0),
        b, gamma, v,
        _ptr(out["tgt_top1"], torch.int32, (b, gp1), "tgt_top1"),
        _ptr(out["top1_prob"], torch.float32, (b, gp1), "top1_prob", nullable=True),
        _ptr(out["n_accept"], torch.int32, (b,), "n_accept"),
        _ptr(out["out_tokens"], torch.int32, (b, gp1), "out_tokens"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()))
    return out


def verify_greedy_noalloc_max_bytes() -> int:
    return _lib.qs_verify_greedy_noalloc_max_bytes()


def qs_verify_greedy_noalloc(tgt_logits, draft_ids, out=None, want_prob=True):
    """qs_verify_greedy without a workspace argument: its scratch is the library's own fixed device
    array (calls that overlap in time on one GPU race).  Same arguments and outputs."""
    b, gp1, v = tgt_logits.shape
    gamma = gp1 - 1
    dev = tgt_logits.device
    if out is None:
        out = {
            "tgt_top1": torch.empty((b, gp1), dtype=torch.int32, device=dev),
            "top1_prob": torch.empty((b, gp1), dtype=torch.float32, device=dev) if want_prob else None,
            "n_accept": torch.empty((b,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((b, gp1), dtype=torch.int32, device=dev),
        }
    _check("qs_verify_greedy_noalloc", _lib.qs_verify_greedy_noalloc(
        _ptr(tgt_logits, torch.float32, (b, gp1, v), "tgt_logits"),
        _ptr(draft_ids, torch.int32, (b, gamma), "draft_ids", nullable=gamma == 0),
        b, gamma, v,
        _ptr(out["tgt_top1"], torch.int32, (b, gp1), "tgt_top1"),
        _ptr(out["top1_prob"], torch.float32, (b, gp1), "top1_prob", nullable=True),
        _ptr(out["n_accept"], torch.int32, (b,), "n_accept"),
        _ptr(out["out_tokens"], torch.int32, (b, gp1), "out_tokens"),
        _stream()))
    return out


def qs_verify_tree_greedy(tgt_logits, tokens, parent, out=None, ws=None):
    """tgt_logits fp32 [B, T, V] (row t: target scores after node t, node 0 the root), tokens and
    parent int32 [B, T] -> dict(tgt_top1, n_accept, out_tokens, out_nodes)."""
    b, t, v = tgt_logits.shape
    dev = tgt_logits.device
    if out is None:
        out = {
            "tgt_top1": torch.empty((b, t), dtype=torch.int32, device=dev),
            "n_accept": torch.empty((b,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((b, t), dtype=torch.int32, device=dev),
            "out_nodes": torch.empty((b, t), dtype=torch.int32, device=dev),
        }
    ws = _ws_for(b, t - 1, v, ws, dev)
    _check("qs_verify_tree_greedy", _lib.qs_verify_tree_greedy(
        _ptr(tgt_logits, torch.float32, (b, t, v), "tgt_logits"),
        _ptr(tokens, torch.int32, (b, t), "tokens", nullable=t == 1),
        _ptr(parent, torch.int32, (b, t), "parent", nullable=t == 1),
        b, t, v,
        _ptr(out["tgt_top1"], torch.int32, (b, t), "tgt_top1"),
        _ptr(out["n_accept"], torch.int32, (b,), "n_accept"),
        _ptr(out["out_tokens"], torch.int32, (b, t), "out_tokens"),
        _ptr(out.get("out_nodes"), torch.int32, (b, t), "out_nodes", nullable=True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()))
    return out


def qs_verify_sample(tgt_logits, drf_logits, draft_ids, u_accept, u_final, out=None, ws=None,
                     want_final_dist=False):
    """tgt_logits fp32 [B, gamma+1, V], drf_logits fp32 [B, gamma, V], draft_ids int32 [B, gamma],
    u_accept fp32 [B, gamma], u_final fp32 [B] -> dict(accept_prob, n_accept, out_tokens, final_dist)."""
    b, gp1, v = tgt_logits.shape
    gamma = gp1 - 1
    dev = tgt_logits.device
    if out is None:
        out = {
            "accept_prob": torch.empty((b, gamma), dtype=torch.float32, device=dev),
            "n_accept": torch.empty((b,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((b, gp1), dtype=torch.int32, device=dev),
            "final_dist": torch.empty((b, v), dtype=torch.float32, device=dev) if want_final_dist else None,
        }
    ws = _ws_for(b, gamma, v, ws, dev)
    g0 = gamma == 0
    _check("qs_verify_sample", _lib.qs_verify_sample(
        _ptr(tgt_logits, torch.float32, (b, gp1, v), "tgt_logits"),
        _ptr(drf_logits, torch.float32, (b, gamma, v), "drf_logits", nullable=g0),
        _ptr(draft_ids, torch.int32, (b, gamma), "draft_ids", nullable=g0),
        _ptr(u_accept, torch.float32, (b, gamma), "u_accept", nullable=g0),
        _ptr(u_final, torch.float32, (b,), "u_final"),
        b, gamma, v,
        _ptr(out["accept_prob"], torch.float32, (b, gamma), "accept_prob", nullable=g0),
        _ptr(out["n_accept"], torch.int32, (b,), "n_accept"),
        _ptr(out["out_tokens"], torch.int32, (b, gp1), "out_tokens"),
        _ptr(out["final_dist"], torch.float32, (b, v), "final_dist", nullable=True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()))
    return out


class LinearDesc(ctypes.Structure):
    """Mirror of qs_linear_desc."""
    _fields_ = [("w_packed", ctypes.c_void_p), ("s_packed", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]


class Chain:
    """A host array of qs_linear_desc plus references that keep the packed
    weight tensors alive.  `layers` is a sequence of (w_packed, s_packed, N, K)."""

    def __init__(self, layers):
        self.tensors = []
        self.n = len(layers)
        self.array = (LinearDesc * self.n)()
        for i, (wp, sp, n, k) in enumerate(layers):
            _wcheck(wp, sp, n, k)
            self.tensors.append((wp, sp))
            self.array[i] = LinearDesc(wp.data_ptr(), sp.data_ptr(), n, k)
        self.out_features = layers[-1][2]
        self.in_features = layers[0][3]

    def workspace_bytes(self, mode: int, m: int) -> int:
        return _lib.qs_chain_workspace_bytes(mode, m, ctypes.cast(self.array, ctypes.c_void_p), self.n)

    def top1_workspace_bytes(self, mode: int, m: int) -> int:
        """Workspace of qs_chain_forward_top1."""
        return _lib.qs_chain_top1_workspace_bytes(mode, m, ctypes.cast(self.array, ctypes.c_void_p), self.n)

    def trace_bytes(self, mode: int, m: int) -> int:
        """Timestamp buffer of qs_chain_forward_trace (0: the row count runs one launch per linear)."""
        return _lib.qs_chain_trace_bytes(mode, m, ctypes.cast(self.array, ctypes.c_void_p), self.n)

    def pass_launches(self, mode: int, m: int) -> int:
        """Persistent pass-kernel launches of qs_chain_forward (0: one launch per linear)."""
        rc = _lib.qs_chain_pass_launches(mode, m, ctypes.cast(self.array, ctypes.c_void_p), self.n)
        if rc < 0:
            _check("qs_chain_pass_launches", rc)
        return rc


def qs_set_barrier_timeout_us(us: int) -> None:
    """Wall-clock limit of each grid-barrier wait of the persistent pass (0: fail at once)."""
    _check("qs_set_barrier_timeout_us", _lib.qs_set_barrier_timeout_us(int(us)))


def qs_chain_pass_status(mode: int, m: int, chain: "Chain", ws) -> bool:
    """True if the last persistent chain call on `ws` had a grid-barrier wait time out."""
    flag = ctypes.c_int(0)
    _check("qs_chain_pass_status", _lib.qs_chain_pass_status(
        mode, m, ctypes.cast(chain.array, ctypes.c_void_p), chain.n, _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), ctypes.byref(flag), _stream()))
    return bool(flag.value)


def qs_chain_forward(mode: int, x, chain: Chain, out=None, ws=None):
    """x fp16 [M, chain.in_features] -> out fp32 [M, chain.out_features]."""
    m, k = x.shape
    if k != chain.in_features:
        raise ValueError("x width does not match the first linear")
    if out is None:
        out = torch.empty((m, chain.out_features), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(chain.workspace_bytes(mode, m), dtype=torch.uint8, device=x.device)
    _check("qs_chain_forward", _lib.qs_chain_forward(
        mode, _ptr(x, torch.float16, (m, k), "x"), m, ctypes.cast(chain.array, ctypes.c_void_p), chain.n,
        _ptr(out, torch.float32, (m, chain.out_features), "out"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _stream()))
    return out


def qs_chain_forward_trace(mode: int, x, chain: Chain, trace, out=None, ws=None):
    """qs_chain_forward that also records the persistent pass's boundary timestamps into trace
    (int64 tensor of chain.trace_bytes(mode, M) / 8 elements, viewed as [entries][workgroups][4])."""
    m, k = x.shape
    if k != chain.in_features:
        raise ValueError("x width does not match the first linear")
    if out is None:
        out = torch.empty((m, chain.out_features), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(chain.workspace_bytes(mode, m), dtype=torch.uint8, device=x.device)
    _check("qs_chain_forward_trace", _lib.qs_chain_forward_trace(
        mode, _ptr(x, torch.float16, (m, k), "x"), m, ctypes.cast(chain.array, ctypes.c_void_p), chain.n,
        _ptr(out, torch.float32, (m, chain.out_features), "out"), _ptr(ws, torch.uint8, None, "ws"),
        ws.numel(), _ptr(trace, torch.int64, None, "trace"), trace.numel() * 8, _stream()))
    return out


def qs_chain_forward_top1(mode: int, x, chain: Chain, out=None, want_logits=True, top1=None, top1_prob=None,
                          want_prob=True, ws=None):
    """x fp16 [M, chain.in_features] -> (out fp32 [M, chain.out_features] or None, top1 int32 [M],
    top1_prob fp32 [M] or None): the chain with the LM-head's Top-1 fused into its last stage."""
    m, k = x.shape
    if k != chain.in_features:
        raise ValueError("x width does not match the first linear")
    dev = x.device
    if out is None and want_logits:
        out = torch.empty((m, chain.out_features), dtype=torch.float32, device=dev)
    if top1 is None:
        top1 = torch.empty((m,), dtype=torch.int32, device=dev)
    if top1_prob is None and want_prob:
        top1_prob = torch.empty((m,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(chain.top1_workspace_bytes(mode, m), dtype=torch.uint8, device=dev)
    _check("qs_chain_forward_top1", _lib.qs_chain_forward_top1(
        mode, _ptr(x, torch.float16, (m, k), "x"), m, ctypes.cast(chain.array, ctypes.c_void_p), chain.n,
        _ptr(out, torch.float32, (m, chain.out_features), "out", nullable=True),
        _ptr(top1, torch.int32, (m,), "top1"),
        _ptr(top1_prob, torch.float32, (m,), "top1_prob", nullable=True),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream()))
    return out, top1, top1_prob


def qs_accept_greedy(tgt_top1, draft_ids, out=None):
    """tgt_top1 int32 [B, gamma+1], draft_ids int32 [B, gamma] -> dict(n_accept, out_tokens)."""
    b, gp1 = tgt_top1.shape
    gamma = gp1 - 1
    dev = tgt_top1.device
    if out is None:
        out = {
            "n_accept": torch.empty((b,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((b, gp1), dtype=torch.int32, device=dev),
        }
    _check("qs_accept_greedy", _lib.qs_accept_greedy(
        _ptr(tgt_top1, torch.int32, (b, gp1), "tgt_top1"),
        _ptr(draft_ids, torch.int32, (b, gamma), "draft_ids", nullable=gamma == 0),
        b, gamma,
        _ptr(out["n_accept"], torch.int32, (b,), "n_accept"),
        _ptr(out["out_tokens"], torch.int32, (b, gp1), "out_tokens"), _stream()))
    return out
