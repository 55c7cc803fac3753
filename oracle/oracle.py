"""Python face of the double-precision MoE-layer oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU-baseline leg of the
benchmark, never by the HIP library or its binding. It marshals numpy arrays (in their storage
formats, as produced by ``moe_inputs``) into the C structs and back; all arithmetic is in the C
file, single-threaded, in double precision.

Parity status: every function here is pinned by the CPU tests in ``tests/test_oracle_pins.py``
against brute force, closed forms, library routines or invariants; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "_moe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, E4M3, F64, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE semantics: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcMat(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scale", C.c_void_p), ("dtype", C.c_int32),
                ("pad_", C.c_int32), ("cols", C.c_int64)]


class OrcGrads(C.Structure):
    _fields_ = [("dW_r", C.c_void_p), ("dW_up", C.c_void_p), ("dW_down", C.c_void_p),
                ("dWs_up", C.c_void_p), ("dWs_down", C.c_void_p), ("expert", C.c_int32),
                ("pad_", C.c_int32), ("dW_in", C.c_void_p), ("dW_out", C.c_void_p)]


class OrcLayer(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "E", "k", "I", "I_shared", "latent",
                                         "fp8_emulate")] + \
               [("x", OrcMat), ("W_r", OrcMat), ("b", C.c_void_p), ("W_up", OrcMat),
                ("W_down", OrcMat), ("Ws_up", OrcMat), ("Ws_down", OrcMat), ("W_in", OrcMat),
                ("W_out", OrcMat)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            L = C.CDLL(build())
            i32p, f64p, f32p = (np.ctypeslib.ndpointer(np.int32, flags="C"),
                                np.ctypeslib.ndpointer(np.float64, flags="C"),
                                np.ctypeslib.ndpointer(np.float32, flags="C"))
            L.orc_bf16_to_f64.restype = C.c_double
            L.orc_bf16_to_f64.argtypes = [C.c_uint16]
            L.orc_e4m3_to_f64.restype = C.c_double
            L.orc_e4m3_to_f64.argtypes = [C.c_uint8]
            L.orc_f64_to_e4m3.restype = C.c_uint8
            L.orc_f64_to_e4m3.argtypes = [C.c_double]
            L.orc_e2m1_to_f64.restype = C.c_double
            L.orc_e2m1_to_f64.argtypes = [C.c_uint8]
            L.orc_e8m0_to_f64.restype = C.c_double
            L.orc_e8m0_to_f64.argtypes = [C.c_uint8]
            L.orc_logits.argtypes = [C.POINTER(OrcLayer), C.c_void_p, C.c_int32, f64p]
            L.orc_route.argtypes = [f64p, f32p, C.c_int32, C.c_int32, C.c_int32, i32p, f64p,
                                    f64p]
            L.orc_route_f32.argtypes = [f32p, f32p, C.c_int32, C.c_int32, C.c_int32, i32p, f64p,
                                        f64p]
            L.orc_gates_for.argtypes = [f64p, i32p, C.c_int32, C.c_int32, C.c_int32, f64p]
            L.orc_dispatch.argtypes = [i32p, C.c_int32, C.c_int32, C.c_int32, i32p, i32p, i32p,
                                       i32p]
            L.orc_forward_tokens.argtypes = [C.POINTER(OrcLayer), C.c_void_p, C.c_int32, i32p,
                                             f64p, f64p, f64p]
            L.orc_bias_update.argtypes = [f64p, i32p, f64p, C.c_int32, C.c_double]
            L.orc_backward_tokens.argtypes = [C.POINTER(OrcLayer), C.c_void_p, C.c_int32, i32p,
                                              f64p, C.c_void_p, C.c_void_p, C.POINTER(OrcGrads)]
            _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle call failed with code {rc}")


_DT = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): E4M3,
       np.dtype(np.float64): F64}


_BLOCK_FORMATS = {"mxfp4": MXFP4, "mxfp8": MXFP8}


def _mat(a, scale=None, keep=None, fmt=None):
    """View of one matrix in its storage format. ``fmt`` names a block-scaled format ("mxfp4":
    two E2M1 codes per byte, "mxfp8": e4m3 codes; uint8 E8M0 scales per 32 columns); otherwise
    the format follows the array's dtype (uint8 = e4m3 with fp32 per-row scales)."""
    if a is None:
        return OrcMat()
    a = np.ascontiguousarray(a)
    m = OrcMat()
    m.data = a.ctypes.data
    if fmt in _BLOCK_FORMATS:
        m.dtype = _BLOCK_FORMATS[fmt]
        m.cols = a.shape[-1] * (2 if fmt == "mxfp4" else 1)
        if scale is None or np.asarray(scale).dtype != np.uint8 or \
                np.asarray(scale).shape[-1] * 32 != m.cols:
            raise ValueError(f"{fmt} matrix needs uint8 E8M0 scales, one per 32 columns")
        scale = np.ascontiguousarray(scale)
        m.scale = scale.ctypes.data
        keep.append(scale)
    else:
        m.dtype = _DT[a.dtype]
        m.cols = a.shape[-1]
        if m.dtype == E4M3:
            if scale is None:
                raise ValueError("e4m3 matrix needs its per-row scales")
            scale = np.ascontiguousarray(scale, dtype=np.float32)
            m.scale = scale.ctypes.data
            keep.append(scale)
    keep.append(a)
    return m


def layer(inp: dict, fp8_emulate: bool = False):
    """Build the C layer struct from a ``moe_inputs.make_layer`` dict. Returns (struct, keepalive)."""
    cfg = inp["config"]
    keep = []
    L = OrcLayer()
    L.T, L.H, L.E, L.k, L.I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    L.I_shared, L.latent, L.fp8_emulate = cfg.I_shared, cfg.latent, int(fp8_emulate)
    L.x = _mat(inp.get("x"), keep=keep)
    L.W_r = _mat(inp.get("W_r"), keep=keep)
    b = np.ascontiguousarray(inp["b"], dtype=np.float32) if "b" in inp else None
    if b is not None:
        keep.append(b)
        L.b = b.ctypes.data
    fmt = cfg.expert_dtype
    L.W_up = _mat(inp.get("W_up"), inp.get("s_up"), keep, fmt)
    L.W_down = _mat(inp.get("W_down"), inp.get("s_down"), keep, fmt)
    L.Ws_up = _mat(inp.get("Ws_up"), keep=keep)
    L.Ws_down = _mat(inp.get("Ws_down"), keep=keep)
    L.W_in = _mat(inp.get("W_in"), keep=keep)
    L.W_out = _mat(inp.get("W_out"), keep=keep)
    return L, keep


def _tokens(tokens):
    if tokens is None:
        return None, 0, None
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return t.ctypes.data, t.shape[0], t


def logits(inp: dict, tokens=None) -> np.ndarray:
    """Router logits in double for the listed tokens (all if None): [n, E]."""
    L, keep = layer(inp)
    p, n, tk = _tokens(tokens)
    n = n if tokens is not None else inp["config"].T
    z = np.zeros((n, inp["config"].E), dtype=np.float64)
    _check(lib().orc_logits(C.byref(L), p, n, z))
    return z


def route(z: np.ndarray, b: np.ndarray, k: int):
    """Double-precision routing: (idx [T,k] int32, gates [T,k], margin [T])."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, E = z.shape
    idx = np.zeros((T, k), np.int32)
    g = np.zeros((T, k), np.float64)
    m = np.zeros(T, np.float64)
    _check(lib().orc_route(z, np.ascontiguousarray(b, np.float32), T, E, k, idx, g, m))
    return idx, g, m


def route_f32(z32: np.ndarray, b: np.ndarray, k: int):
    """Routing from fp32 logits, decisions taken on fp32-rounded scores and keys."""
    z32 = np.ascontiguousarray(z32, dtype=np.float32)
    T, E = z32.shape
    idx = np.zeros((T, k), np.int32)
    g = np.zeros((T, k), np.float64)
    m = np.zeros(T, np.float64)
    _check(lib().orc_route_f32(z32, np.ascontiguousarray(b, np.float32), T, E, k, idx, g, m))
    return idx, g, m


def gates_for(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights of a given selection idx [T,k] from double logits z [T,E]."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, E = z.shape
    g = np.zeros(idx.shape, np.float64)
    _check(lib().orc_gates_for(z, idx, T, E, idx.shape[1], g))
    return g


def dispatch(idx: np.ndarray, E: int):
    """(counts [E], offsets [E+1], perm [T*k], pos [T,k]) -- all int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    pos = np.zeros((T, k), np.int32)
    _check(lib().orc_dispatch(idx, T, E, k, counts, offsets, perm, pos))
    return counts, offsets, perm, pos


def forward_tokens(inp: dict, idx: np.ndarray, gates: np.ndarray, tokens=None,
                   fp8_emulate: bool = False) -> np.ndarray:
    """Layer output in double for the listed tokens (all if None) given their routing rows."""
    cfg = inp["config"]
    L, keep = layer(inp, fp8_emulate)
    p, n, tk = _tokens(tokens)
    n = n if tokens is not None else cfg.T
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(n, cfg.k)
    gates = np.ascontiguousarray(gates, dtype=np.float64).reshape(n, cfg.k)
    y = np.zeros((n, cfg.H), np.float64)
    work = np.zeros(2 * cfg.D + max(cfg.I, cfg.I_shared), np.float64)
    _check(lib().orc_forward_tokens(C.byref(L), p, n, idx, gates, y, work))
    return y


def forward(inp: dict, tokens=None, fp8_emulate: bool = False, threads: int = 1) -> dict:
    """Route and run the listed tokens (all if None). Returns logits, idx, gates, margin, y.

    ``threads`` > 1 hands disjoint groups of tokens to that many threads (the C calls release
    the interpreter lock); every token is computed exactly as in a single call."""
    if threads > 1:
        t = np.arange(inp["config"].T) if tokens is None else np.asarray(tokens, dtype=np.int32)
        groups = [g for g in np.array_split(t, min(threads, max(1, len(t)))) if len(g)]
        if len(groups) > 1:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(len(groups)) as ex:
                parts = list(ex.map(lambda g: forward(inp, g, fp8_emulate), groups))
            return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    z = logits(inp, tokens)
    idx, g, m = route(z, inp["b"], inp["config"].k)
    y = forward_tokens(inp, idx, g, tokens, fp8_emulate)
    return dict(logits=z, idx=idx, gates=g, margin=m, y=y)


GRAD_NAMES = ("dx", "dz", "dW_r", "dW_up", "dW_down", "dWs_up", "dWs_down", "dW_in", "dW_out")


def backward(inp: dict, idx: np.ndarray, dy: np.ndarray, tokens=None, want=GRAD_NAMES,
             expert: int = -1, threads: int = 1) -> dict:
    """Gradients in double of the scalar loss sum_t <dy_t, y_t> for the listed tokens (all if
    None), holding the selection idx fixed (one row of k per listed token; dy one row of H).

    Returns the requested names of GRAD_NAMES: dx [n, H] and dz [n, E] per listed token; weight
    gradients summed over the listed tokens, dW_up / dW_down for one expert only when
    ``expert`` >= 0; dW_in / dW_out for a LatentMoE layer. ``threads`` > 1 splits the tokens over threads and adds their weight
    gradients afterwards (float64 sums, so the order of that final addition may differ from a
    single call in the last bits)."""
    cfg = inp["config"]
    t_all = np.arange(cfg.T, dtype=np.int32) if tokens is None else \
        np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(t_all)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(n, cfg.k)
    dy = np.ascontiguousarray(dy, dtype=np.float64).reshape(n, cfg.H)
    if threads > 1 and n > 1:
        groups = [g for g in np.array_split(np.arange(n), min(threads, n)) if len(g)]
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(len(groups)) as ex:
            parts = list(ex.map(lambda g: backward(inp, idx[g], dy[g], t_all[g], want, expert),
                                groups))
        out = {}
        for k in parts[0]:
            out[k] = np.concatenate([p[k] for p in parts]) if k in ("dx", "dz") else \
                sum(p[k] for p in parts)
        return out
    H, E, I, Is, Lw, D = cfg.H, cfg.E, cfg.I, cfg.I_shared, cfg.latent, cfg.D
    shapes = {"dx": (n, H), "dz": (n, E), "dW_r": (E, H),
              "dW_up": (I, D) if expert >= 0 else (E, I, D),
              "dW_down": (D, I) if expert >= 0 else (E, D, I),
              "dWs_up": (Is, H), "dWs_down": (H, Is), "dW_in": (Lw, H), "dW_out": (H, Lw)}
    out = {k: np.zeros(shapes[k], np.float64) for k in want
           if k in shapes and not (k.startswith("dWs") and not Is)
           and not (k in ("dW_in", "dW_out") and not Lw)}
    G = OrcGrads()
    for k in ("dW_r", "dW_up", "dW_down", "dWs_up", "dWs_down", "dW_in", "dW_out"):
        setattr(G, k, out[k].ctypes.data if k in out else None)
    G.expert = expert
    L, keep = layer(inp)
    _check(lib().orc_backward_tokens(C.byref(L), t_all.ctypes.data, n, idx, dy,
                                     out["dx"].ctypes.data if "dx" in out else None,
                                     out["dz"].ctypes.data if "dz" in out else None, C.byref(G)))
    return out


def bias_update(b: np.ndarray, counts: np.ndarray, target: np.ndarray, gamma: float) -> np.ndarray:
    """One aux-loss-free sign step of the routing bias toward per-expert target loads."""
    b = np.array(b, dtype=np.float64, copy=True)
    _check(lib().orc_bias_update(b, np.ascontiguousarray(counts, np.int32),
                                 np.ascontiguousarray(target, np.float64), b.shape[0], gamma))
    return b


def bf16_to_f64(u) -> np.ndarray:
    f = lib().orc_bf16_to_f64
    return np.array([f(int(v)) for v in np.ravel(u)], dtype=np.float64).reshape(np.shape(u))


def e4m3_to_f64(c) -> np.ndarray:
    f = lib().orc_e4m3_to_f64
    return np.array([f(int(v)) for v in np.ravel(c)], dtype=np.float64).reshape(np.shape(c))


def e2m1_to_f64(c) -> np.ndarray:
    f = lib().orc_e2m1_to_f64
    return np.array([f(int(v)) for v in np.ravel(c)], dtype=np.float64).reshape(np.shape(c))


def e8m0_to_f64(c) -> np.ndarray:
    f = lib().orc_e8m0_to_f64
    return np.array([f(int(v)) for v in np.ravel(c)], dtype=np.float64).reshape(np.shape(c))


def f64_to_e4m3(v) -> np.ndarray:
    f = lib().orc_f64_to_e4m3
    return np.array([f(float(x)) for x in np.ravel(v)], dtype=np.uint8).reshape(np.shape(v))
