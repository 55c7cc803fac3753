"""ctypes binding of libmoe_mi355x.so (the gfx950 MoE layer library).

Argument marshalling only: torch tensors supply device memory and the current stream; every step
of the layer runs in the library's HIP kernels. The library must have been built
(``python -m sparse_moe_layer_05_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8 = 0, 1, 2, 3, 4
_EXPERT_DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4,
                  "mxfp8": MOE_MXFP8}
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
PATH_AUTO, PATH_GROUPED, PATH_STREAM, ROUTING_GIVEN, SAVED_IN_WORKSPACE = 0, 1, 2, 4, 8
WGRAD_BF16 = 16
_PATHS = {"auto": PATH_AUTO, "grouped": PATH_GROUPED, "stream": PATH_STREAM}

EXPORTS = ("moe_workspace_size", "moe_layer_forward", "latent_moe_forward", "moe_route",
           "moe_dispatch_workspace_size", "moe_dispatch", "moe_bias_update",
           "moe_backward_workspace_size", "moe_layer_forward_train", "moe_layer_backward",
           "moe_layer_forward_static", "moe_status_str",
           "moe_trace_enable",
           "moe_trace_count", "moe_trace_read", "moe_trace_reset")


class MoeDesc(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("I", C.c_int32), ("I_shared", C.c_int32), ("latent", C.c_int32),
                ("act_dtype", C.c_int32), ("expert_dtype", C.c_int32), ("flags", C.c_uint32)]


class MoeWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("x", "W_r", "b", "W_up", "W_down", "s_up", "s_down",
                                          "Ws_up", "Ws_down", "W_in", "W_out")]


class MoeRouting(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("idx", "gates", "counts", "offsets", "perm", "pos",
                                          "logits")]


class MoeGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dx", "dW_r", "dW_up", "dW_down", "dWs_up",
                                          "dWs_down", "dW_in", "dW_out")]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_str(code)} ({code})")
        self.code = code


_lock = threading.Lock()
_lib = None


def lib() -> C.CDLL:
    """Load the library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                                   "(run python -m sparse_moe_layer_05_amd.build)")
            L = C.CDLL(LIB_PATH)
            vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
            L.moe_workspace_size.argtypes = [C.POINTER(MoeDesc), C.POINTER(sz)]
            for fn in (L.moe_layer_forward, L.latent_moe_forward):
                fn.argtypes = [C.POINTER(MoeDesc), C.POINTER(MoeWeights), vp, vp, sz,
                               C.POINTER(MoeRouting), vp]
            L.moe_layer_forward_static.argtypes = [C.POINTER(MoeDesc), C.POINTER(MoeWeights),
                                                   vp, C.POINTER(MoeRouting), vp]
            L.moe_route.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
            L.moe_dispatch_workspace_size.argtypes = [i32, i32, i32, C.POINTER(sz)]
            L.moe_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
            L.moe_bias_update.argtypes = [vp, vp, i32, C.c_float, vp, vp]
            L.moe_backward_workspace_size.argtypes = [C.POINTER(MoeDesc), C.POINTER(sz)]
            L.moe_layer_backward.argtypes = [C.POINTER(MoeDesc), C.POINTER(MoeWeights), vp,
                                             C.POINTER(MoeGrads), vp, sz, vp]
            L.moe_layer_forward_train.argtypes = [C.POINTER(MoeDesc), C.POINTER(MoeWeights), vp,
                                                  vp, sz, vp]
            L.moe_status_str.argtypes = [i32]
            L.moe_trace_enable.argtypes = [i32, C.c_char_p]
            L.moe_trace_count.argtypes = []
            L.moe_trace_read.argtypes = [i32, C.POINTER(C.c_char_p), C.POINTER(C.c_float)]
            L.moe_trace_reset.argtypes = []
            for name in EXPORTS:
                getattr(L, name).restype = C.c_int32
            L.moe_status_str.restype = C.c_char_p
            L.moe_trace_reset.restype = None
            _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().moe_status_str(code).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _used_on(stream, *tensors):
    """Tell the caching allocator that `tensors` (allocated on the current stream) are in use on
    `stream` too, so that their memory is not handed out again before that stream's work ends."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def expert_dtype_code(x, W_up, s_up=None, W_in=None, expert_dtype=None) -> int:
    """moe_dtype_t of the expert weights: given by name, or read off the tensors (float / bf16
    weights: their dtype; uint8 codes with fp32 scales: e4m3; with uint8 block scales: MXFP8,
    or MXFP4 when a row holds half as many bytes as the expert input width)."""
    if expert_dtype is not None:
        return _EXPERT_DTYPES[expert_dtype]
    if W_up.dtype in (torch.uint8, torch.float8_e4m3fn) and s_up is not None \
            and s_up.dtype == torch.uint8:
        D = W_in.shape[0] if W_in is not None else x.shape[1]
        return MOE_MXFP4 if 2 * W_up.shape[-1] == D else MOE_MXFP8
    return _dtype_code(W_up)


def _need(t, shape, what, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{what} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")


def check_shapes(desc, x, W_r, b, W_up, W_down, s_up=None, s_down=None, Ws_up=None,
                 Ws_down=None, W_in=None, W_out=None):
    """Every tensor must have the shape, dtype and device the descriptor implies: the library
    only sees pointers, so a mismatch would make it read outside a buffer."""
    T, H, E, I, Is, L = desc.T, desc.H, desc.E, desc.I, desc.I_shared, desc.latent
    D = L or H
    act = x.dtype
    dev = x.device
    _need(W_r, (E, H), "W_r", act, dev)
    _need(b, (E,), "b", torch.float32, dev)
    ed = desc.expert_dtype
    if ed in (MOE_F32, MOE_BF16):
        _need(W_up, (E, I, D), "W_up", act, dev)
        _need(W_down, (E, D, I), "W_down", act, dev)
    elif ed == MOE_FP8_E4M3:
        _need(W_up, (E, I, D), "W_up", W_up.dtype, dev)
        _need(W_down, (E, D, I), "W_down", W_down.dtype, dev)
        _need(s_up, (E, I), "s_up", torch.float32, dev)
        _need(s_down, (E, D), "s_down", torch.float32, dev)
    else:  # MXFP4 packs two elements per byte, MXFP8 one; one uint8 scale per 32 along K
        per = 2 if ed == MOE_MXFP4 else 1
        _need(W_up, (E, I, D // per), "W_up", W_up.dtype, dev)
        _need(W_down, (E, D, I // per), "W_down", W_down.dtype, dev)
        _need(s_up, (E, I, D // 32), "s_up", torch.uint8, dev)
        _need(s_down, (E, D, I // 32), "s_down", torch.uint8, dev)
    if ed not in (MOE_F32, MOE_BF16) and W_up.element_size() != 1:
        raise ValueError("8- and 4-bit expert weights are passed as 1-byte tensors")
    if Is:
        _need(Ws_up, (Is, H), "Ws_up", act, dev)
        _need(Ws_down, (H, Is), "Ws_down", act, dev)
    if L:
        _need(W_in, (L, H), "W_in", act, dev)
        _need(W_out, (H, L), "W_out", act, dev)


def make_desc(x, W_r, W_up, k, Ws_up=None, W_in=None, path="auto", routing_given=False,
              s_up=None, expert_dtype=None):
    T, H = x.shape
    E, I = W_up.shape[0], W_up.shape[1]
    d = MoeDesc()
    d.T, d.H, d.E, d.k, d.I = T, H, E, k, I
    d.I_shared = Ws_up.shape[0] if Ws_up is not None else 0
    d.latent = W_in.shape[0] if W_in is not None else 0
    d.act_dtype = _dtype_code(x)
    d.expert_dtype = expert_dtype_code(x, W_up, s_up, W_in, expert_dtype)
    d.flags = _PATHS[path] | (ROUTING_GIVEN if routing_given else 0)
    return d


def workspace_size(desc: MoeDesc) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_workspace_size(C.byref(desc), C.byref(n)), "moe_workspace_size")
    return n.value


def alloc_routing(T: int, E: int, k: int, device) -> dict:
    i32 = dict(dtype=torch.int32, device=device)
    return dict(idx=torch.empty((T, k), **i32), gates=torch.empty((T, k), dtype=torch.float32,
                                                                  device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                perm=torch.empty(T * k, **i32), pos=torch.empty((T, k), **i32),
                logits=torch.empty((T, E), dtype=torch.float32, device=device))


class Layer:
    """One layer call prepared once (descriptor, weights struct, workspace, outputs), so that a
    benchmark loop or a graph capture can replay ``__call__`` without any allocation."""

    def __init__(self, x, W_r, b, W_up, W_down, k, *, s_up=None, s_down=None, Ws_up=None,
                 Ws_down=None, W_in=None, W_out=None, path="auto", routing=None,
                 routing_given=False, out=None, expert_dtype=None, no_alloc=False):
        self.desc = make_desc(x, W_r, W_up, k, Ws_up, W_in, path, routing_given, s_up,
                              expert_dtype)
        check_shapes(self.desc, x, W_r, b, W_up, W_down, s_up, s_down, Ws_up, Ws_down, W_in,
                     W_out)
        if out is not None:
            _need(out, x.shape, "out", x.dtype, x.device)
        w = MoeWeights()
        w.x, w.W_r, w.b, w.W_up, w.W_down = _p(x), _p(W_r), _p(b), _p(W_up), _p(W_down)
        w.s_up, w.s_down = _p(s_up), _p(s_down)
        w.Ws_up, w.Ws_down, w.W_in, w.W_out = _p(Ws_up), _p(Ws_down), _p(W_in), _p(W_out)
        self.w = w
        self._keep = [x, W_r, b, W_up, W_down, s_up, s_down, Ws_up, Ws_down, W_in, W_out]
        self.y = out if out is not None else torch.empty_like(x)
        self.no_alloc = no_alloc
        if no_alloc:          # moe_layer_forward_static: the library's own per-GPU scratch
            self.ws_bytes, self.ws = 0, None
        else:
            self.ws_bytes = workspace_size(self.desc)
            self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=x.device)
        self.routing = routing
        self.r = None
        if routing is not None:
            r = MoeRouting()
            for name, _ in MoeRouting._fields_:
                setattr(r, name, _p(routing.get(name)))
            self.r = r
        self.fn = lib().latent_moe_forward if self.desc.latent else lib().moe_layer_forward

    def __call__(self, stream=None):
        r = C.byref(self.r) if self.r is not None else None
        if self.no_alloc:
            rc = lib().moe_layer_forward_static(C.byref(self.desc), C.byref(self.w), _p(self.y),
                                                r, _stream(stream))
            _check(rc, "moe_layer_forward_static")
            return self.y
        rc = self.fn(C.byref(self.desc), C.byref(self.w), _p(self.y), _p(self.ws), self.ws_bytes,
                     r, _stream(stream))
        _check(rc, "latent_moe_forward" if self.desc.latent else "moe_layer_forward")
        return self.y


class Backward:
    """One backward call prepared once (descriptor, weights, gradient outputs in fp32,
    workspace): ``__call__(dy)`` writes the gradients of sum(dy * y) into ``self.grads``.
    ``wgrad_bf16``: the expert weight gradients (dW_up, dW_down, dWs_up, dWs_down) in bf16."""

    def __init__(self, x, W_r, b, W_up, W_down, k, *, Ws_up=None, Ws_down=None, W_in=None,
                 W_out=None, wgrad_bf16=False):
        self.desc = make_desc(x, W_r, W_up, k, Ws_up, W_in)
        check_shapes(self.desc, x, W_r, b, W_up, W_down, Ws_up=Ws_up, Ws_down=Ws_down,
                     W_in=W_in, W_out=W_out)
        w = MoeWeights()
        w.x, w.W_r, w.b, w.W_up, w.W_down = _p(x), _p(W_r), _p(b), _p(W_up), _p(W_down)
        w.Ws_up, w.Ws_down, w.W_in, w.W_out = _p(Ws_up), _p(Ws_down), _p(W_in), _p(W_out)
        self.w = w
        self._keep = [x, W_r, b, W_up, W_down, Ws_up, Ws_down, W_in, W_out]
        f32 = dict(dtype=torch.float32, device=x.device)
        wg = dict(dtype=torch.bfloat16 if wgrad_bf16 else torch.float32, device=x.device)
        self.wgrad_bf16 = bool(wgrad_bf16)
        self.grads = {"dx": torch.empty(x.shape, **f32), "dW_r": torch.empty(W_r.shape, **f32),
                      "dW_up": torch.empty(W_up.shape, **wg),
                      "dW_down": torch.empty(W_down.shape, **wg)}
        if Ws_up is not None:
            self.grads["dWs_up"] = torch.empty(Ws_up.shape, **wg)
            self.grads["dWs_down"] = torch.empty(Ws_down.shape, **wg)
        if W_in is not None:
            self.grads["dW_in"] = torch.empty(W_in.shape, **f32)
            self.grads["dW_out"] = torch.empty(W_out.shape, **f32)
        g = MoeGrads()
        for name, _ in MoeGrads._fields_:
            setattr(g, name, _p(self.grads.get(name)))
        self.g = g
        n = C.c_size_t(0)
        _check(lib().moe_backward_workspace_size(C.byref(self.desc), C.byref(n)),
               "moe_backward_workspace_size")
        self.ws_bytes = n.value
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=x.device)

    def forward_train(self, y=None, stream=None):
        """y of the layer (grouped path), keeping what the backward pass reads in the workspace:
        later calls with ``saved=True`` skip the recompute."""
        x = self._keep[0]
        if y is None:
            y = torch.empty_like(x)
        _need(y, x.shape, "y", x.dtype, x.device)
        rc = lib().moe_layer_forward_train(C.byref(self.desc), C.byref(self.w), _p(y),
                                           _p(self.ws), self.ws_bytes, _stream(stream))
        _check(rc, "moe_layer_forward_train")
        return y

    def __call__(self, dy, stream=None, saved=False):
        x = self._keep[0]
        _need(dy, x.shape, "dy", x.dtype, x.device)
        d = MoeDesc.from_buffer_copy(self.desc)
        if saved:
            d.flags |= SAVED_IN_WORKSPACE
        if self.wgrad_bf16:
            d.flags |= WGRAD_BF16
        rc = lib().moe_layer_backward(C.byref(d), C.byref(self.w), _p(dy), C.byref(self.g),
                                      _p(self.ws), self.ws_bytes, _stream(stream))
        _check(rc, "moe_layer_backward")
        return self.grads


def backward_from(dev: dict, k: int, **kw) -> Backward:
    """A Backward over a ``to_device`` dict (keywords as for Backward)."""
    return Backward(dev["x"], dev["W_r"], dev["b"], dev["W_up"], dev["W_down"], k,
                    Ws_up=dev.get("Ws_up"), Ws_down=dev.get("Ws_down"), W_in=dev.get("W_in"),
                    W_out=dev.get("W_out"), **kw)


def layer_forward(x, W_r, b, W_up, W_down, k, **kw):
    """y = MoE layer (or LatentMoE when W_in / W_out are given) of x; see moe.h."""
    return Layer(x, W_r, b, W_up, W_down, k, **kw)()


def route(b, k, *, logits=None, x=None, W_r=None, stream=None):
    """Router alone. Returns (idx, gates, logits)."""
    src = logits if logits is not None else x
    T = src.shape[0]
    E = b.shape[0]
    dev = src.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    lo = None
    H, dt = 0, MOE_F32
    if logits is None:
        H = x.shape[1]
        dt = _dtype_code(x)
        lo = torch.empty((T, E), dtype=torch.float32, device=dev)
    rc = lib().moe_route(_p(logits), _p(x), _p(W_r), _p(b), T, H, E, k, dt, _p(idx), _p(gates),
                         _p(lo), _stream(stream))
    _check(rc, "moe_route")
    _used_on(stream, idx, gates, lo)
    return idx, gates, (logits if logits is not None else lo)


def dispatch(idx, E, stream=None):
    """(counts, offsets, perm, pos) of idx [T, k]."""
    T, k = idx.shape
    dev = idx.device
    n = C.c_size_t(0)
    _check(lib().moe_dispatch_workspace_size(T, E, k, C.byref(n)), "moe_dispatch_workspace_size")
    ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    rc = lib().moe_dispatch(_p(idx), T, E, k, _p(counts), _p(offsets), _p(perm), _p(pos), _p(ws),
                            n.value, _stream(stream))
    _check(rc, "moe_dispatch")
    # the workspace is dropped here while the kernels may still run on `stream`
    _used_on(stream, ws, counts, offsets, perm, pos)
    return counts, offsets, perm, pos


def bias_update(counts, b, gamma: float, target=None, stream=None) -> None:
    """In place: b[e] += gamma * sign(target[e] - counts[e]) (target None: the mean load)."""
    E = b.numel()
    rc = lib().moe_bias_update(_p(counts), _p(target) if target is not None else None, E,
                               float(gamma), _p(b), _stream(stream))
    _check(rc, "moe_bias_update")


def trace_enable(capacity: int, prefix: str = "") -> None:
    """Record HIP events around every launch whose trace name starts with `prefix`."""
    _check(lib().moe_trace_enable(capacity, prefix.encode()), "moe_trace_enable")


def trace_disable() -> None:
    _check(lib().moe_trace_enable(0, None), "moe_trace_enable")


def trace_reset() -> None:
    lib().moe_trace_reset()


def trace_records() -> list:
    """[(name, ms)] of the recorded launches (synchronise the stream first)."""
    out = []
    for i in range(lib().moe_trace_count()):
        name, ms = C.c_char_p(), C.c_float()
        _check(lib().moe_trace_read(i, C.byref(name), C.byref(ms)), "moe_trace_read")
        out.append((name.value.decode(), ms.value))
    return out


def to_device(inp: dict, device="cuda") -> dict:
    """numpy arrays of a ``moe_inputs.make_layer`` dict -> torch tensors on ``device``
    (uint16 bf16 bit patterns become torch.bfloat16; e4m3, E2M1 and E8M0 codes stay uint8)."""
    import numpy as np
    out = {}
    for name, a in inp.items():
        if isinstance(a, np.ndarray):
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
                else torch.from_numpy(a)
            out[name] = t.to(device)
    return out


def layer_from(dev: dict, k: int, **kw) -> Layer:
    """A Layer over a ``to_device`` dict."""
    return Layer(dev["x"], dev["W_r"], dev["b"], dev["W_up"], dev["W_down"], k,
                 s_up=dev.get("s_up"), s_down=dev.get("s_down"), Ws_up=dev.get("Ws_up"),
                 Ws_down=dev.get("Ws_down"), W_in=dev.get("W_in"), W_out=dev.get("W_out"), **kw)
