"""Seeded synthetic inputs for the sparse Mixture-of-Experts layer forward pass.

This module is shared by the HIP path's tests/benchmark and by the oracle's tests. It therefore
holds only random draws, the encoders that put those draws into their storage formats (bf16 bits,
OCP e4m3 weight codes with per-row fp32 scales, OCP microscaling MXFP4 / MXFP8 weight blocks) and
the layer shapes. It holds none of the layer's
own arithmetic: no router, no top-k, no expert MLP, no activation quantisation. The two
router biases that need a calibrated popularity profile are read from text fixtures written by
``tests/golden/make_bias.py``.

Shapes follow the Nemotron 3 pages: a learned router picks k of E routable experts (6 of 128 in
Nano, MarkTechPost article on Nemotron 3, "Hybrid Mamba Transformer MoE architecture"); LatentMoE
runs E' = E*H/l experts with k' = k*H/l in a latent width l (Nemotron 3 white paper summary,
section 2.2 and the speed-read equation).

Random recipe (one ``numpy.random.SeedSequence`` per tensor, per expert for expert weights):
  x ~ N(0, 1)                                    tag 1
  W_r ~ N(0, 1/H)                                tag 2
  b ~ U(-0.1, 0.1) or a stored fixture           tag 3
  W_up[e] ~ N(0, 1/D),  W_down[e] ~ N(0, 1/I)    tags 4, 5 (sequence [seed, tag, e])
  Ws_up ~ N(0, 1/H),    Ws_down ~ N(0, 1/I_s)    tags 6, 7
  W_in ~ N(0, 1/H),     W_out ~ N(0, 1/l)        tags 8, 9
Draws are fp32, then rounded to nearest-even bf16 (bf16 layers), quantised per output row to
e4m3 with scale = row amax / 448 (fp8 expert weights), or quantised in blocks of 32 consecutive
input columns to MXFP4 (E2M1) or MXFP8 (E4M3) codes with one E8M0 scale per block, by the
conversion rule of the OCP Microscaling Formats (MX) v1.0 specification: the block's shared
exponent is floor(log2(amax)) minus the element format's largest exponent (2 for E2M1, 8 for
E4M3), and each value divided by 2^shared is rounded to the nearest element (ties to even),
saturating at the format's largest magnitude.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "TAGS", "make_layer", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "encode_e4m3", "decode_e4m3", "quantize_rows_e4m3", "encode_e2m1", "decode_e2m1",
    "decode_e8m0", "quantize_blocks_mx", "decode_blocks_mx", "BLOCK_FORMATS", "golden_dir",
    "read_bias_fixture",
]

BLOCK_FORMATS = ("mxfp4", "mxfp8")
MX_BLOCK = 32

TAGS = dict(x=1, W_r=2, b=3, W_up=4, W_down=5, Ws_up=6, Ws_down=7, W_in=8, W_out=9, rank=10,
            dy=11)

_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")


def golden_dir() -> str:
    return _GOLDEN


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int = 0
    latent: int = 0              # 0: plain MoE; else the latent width l
    act_dtype: str = "bf16"      # x, W_r, shared expert, W_in / W_out: "f32" | "bf16"
    expert_dtype: str = "bf16"   # W_up / W_down: "f32" | "bf16" | "e4m3" | "mxfp4" | "mxfp8"
    bias: str = "uniform"        # "uniform" or a fixture file name under tests/golden
    description: str = ""

    @property
    def D(self) -> int:
        """Width the routed experts read and write: H, or l for LatentMoE."""
        return self.latent if self.latent else self.H

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_T(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=T)


CONFIGS = {
    "tiny_f32": LayerConfig(
        "tiny_f32", T=64, H=256, E=16, k=2, I=128, act_dtype="f32", expert_dtype="f32",
        description="tiny MoE layer, fp32, T=64 H=256 E=16 k=2 I=128, no shared expert"),
    "nano_decode_bf16": LayerConfig(
        "nano_decode_bf16", T=64, H=2688, E=128, k=6, I=1856, I_shared=3712,
        description="Nano-shaped decode step, bf16, T=64, 6 of 128 experts + shared expert"),
    "nano_prefill_bf16": LayerConfig(
        "nano_prefill_bf16", T=8192, H=2688, E=128, k=6, I=1856, I_shared=3712,
        bias="bias_nano_prefill_zipf.txt",
        description="Nano-shaped prefill, bf16, T=8192, Zipf(1.1) expert popularity"),
    "latent_bf16": LayerConfig(
        "latent_bf16", T=4096, H=4096, E=512, k=24, I=512, latent=1024,
        description="LatentMoE, bf16, T=4096 H=4096 l=1024 E'=512 k'=24 I=512"),
    "latent_decode_bf16": LayerConfig(
        "latent_decode_bf16", T=64, H=4096, E=512, k=24, I=512, latent=1024,
        description="LatentMoE decode step, bf16, T=64 H=4096 l=1024 E'=512 k'=24 I=512"),
    "latent_decode_k22_bf16": LayerConfig(
        "latent_decode_k22_bf16", T=64, H=4096, E=512, k=22, I=512, latent=1024,
        description="LatentMoE decode step with the k'=22 of the published comparison"),
    "nano_fp8_decode": LayerConfig(
        "nano_fp8_decode", T=64, H=2688, E=128, k=6, I=1856, I_shared=3712, expert_dtype="e4m3",
        description="Nano-shaped decode step, e4m3 expert weights, T=64"),
    "nano_mxfp4_decode": LayerConfig(
        "nano_mxfp4_decode", T=64, H=2688, E=128, k=6, I=1856, I_shared=3712,
        expert_dtype="mxfp4",
        description="Nano-shaped decode step, MXFP4 expert weights (E2M1, E8M0 per 32), T=64"),
    "nano_mxfp8_decode": LayerConfig(
        "nano_mxfp8_decode", T=64, H=2688, E=128, k=6, I=1856, I_shared=3712,
        expert_dtype="mxfp8",
        description="Nano-shaped decode step, MXFP8 expert weights (E4M3, E8M0 per 32), T=64"),
    "latent_fp8_decode": LayerConfig(
        "latent_fp8_decode", T=64, H=4096, E=512, k=24, I=512, latent=1024, expert_dtype="e4m3",
        description="LatentMoE decode step, e4m3 expert weights, T=64 H=4096 l=1024 E'=512 k'=24"),
    "latent_mxfp4_decode": LayerConfig(
        "latent_mxfp4_decode", T=64, H=4096, E=512, k=24, I=512, latent=1024,
        expert_dtype="mxfp4",
        description="LatentMoE decode step, MXFP4 expert weights, T=64 H=4096 l=1024 E'=512 k'=24"),
    "nano_fp8": LayerConfig(
        "nano_fp8", T=16384, H=2688, E=128, k=6, I=1856, I_shared=3712, expert_dtype="e4m3",
        bias="bias_nano_fp8_imbalance.txt",
        description="Nano-shaped, e4m3 expert weights, T=16384, heavy expert imbalance"),
}


# ----------------------------------------------------------------------------- format encoders

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 (fn variant): bias 7, no infinities, S.1111.111 is NaN, max 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int32)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest (ties to even), saturating at +-448, OCP E4M3 codes of finite values."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(a)                         # a = f * 2**ex with f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                  # unbiased exponent; subnormals share 2**-6
    q = np.rint(a / np.exp2(e - 3.0))           # 3 mantissa bits: quantum 2**(e-3)
    val = np.minimum(q * np.exp2(e - 3.0), 448.0)
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = val >= 2.0 ** -6
    ef = np.where(normal, e2 + 7, 0)
    mf = np.where(normal, val / np.exp2(e2 - 3.0) - 8.0, val / 2.0 ** -9)
    mf = np.where(val == 0, 0, mf)
    ef = np.where(val == 0, 0, ef)
    code = (ef.astype(np.int32) << 3) | np.rint(mf).astype(np.int32)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows_e4m3(w: np.ndarray):
    """Per-row (output channel) e4m3 codes with fp32 scale = row amax / 448 (1 for a zero row)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = (w / scale[..., None]).astype(np.float32)
    return encode_e4m3(v), scale


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """OCP E2M1 (4-bit): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
    the subnormal 0.5 * m. Codes are the low 4 bits of each entry."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int32) & 0xF
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    v = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(c & 8, -v, v)


# |v| below each bound rounds to the code of that position: the midpoints of the E2M1 grid
# 0, 0.5, 1, 1.5, 2, 3, 4, 6, where a tie goes to the even code (mantissa bit 0)
_E2M1_BOUNDS = ((0.25, True), (0.75, False), (1.25, True), (1.75, False), (2.5, True),
                (3.5, False), (5.0, True))


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to even), saturating at +-6; the sign of v is kept (also on 0)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int32)
    for bound, tie_down in _E2M1_BOUNDS:
        code += (a > bound) if tie_down else (a >= bound)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale: 2^(code - 127); 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int32)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def quantize_blocks_mx(w: np.ndarray, fmt: str):
    """OCP MX conversion of rows of w in blocks of 32 consecutive columns.

    Returns (codes, scales): for "mxfp8" codes [..., cols] e4m3; for "mxfp4" codes
    [..., cols / 2] with element 2i in the low nibble of byte i and 2i + 1 in the high nibble;
    scales [..., cols / 32] E8M0 (an all-zero block gets code 0)."""
    if fmt not in BLOCK_FORMATS:
        raise ValueError(fmt)
    w = np.asarray(w, dtype=np.float64)
    cols = w.shape[-1]
    if cols % MX_BLOCK:
        raise ValueError(f"{cols} columns is not a whole number of {MX_BLOCK}-blocks")
    blk = w.reshape(w.shape[:-1] + (cols // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    emax = 2 if fmt == "mxfp4" else 8
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))   # amax = f * 2**ex, f in [0.5, 1)
    shared = np.clip(ex - 1 - emax, -127, 127)          # floor(log2(amax)) - emax
    scode = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    q = blk / np.exp2(scode.astype(np.float64) - 127.0)[..., None]
    if fmt == "mxfp8":
        codes = encode_e4m3(q).reshape(w.shape)
    else:
        c4 = encode_e2m1(q).reshape(w.shape)
        codes = (c4[..., 0::2] | (c4[..., 1::2] << 4)).astype(np.uint8)
    return codes, scode


def decode_blocks_mx(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """Values of MX blocks as stored by ``quantize_blocks_mx`` (float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "mxfp4":
        el = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), dtype=np.float64)
        el[..., 0::2] = decode_e2m1(codes & 0xF)
        el[..., 1::2] = decode_e2m1(codes >> 4)
    elif fmt == "mxfp8":
        el = decode_e4m3(codes)
    else:
        raise ValueError(fmt)
    return el * np.repeat(decode_e8m0(scales), MX_BLOCK, axis=-1)


# ----------------------------------------------------------------------------- draws

def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def _normal(key, shape, fan_in):
    a = _rng(*key).standard_normal(shape, dtype=np.float32)
    a *= np.float32(1.0 / np.sqrt(fan_in))
    return a


def _store(a: np.ndarray, dtype: str):
    """fp32 draw -> (storage array, per-row scales or None)."""
    if dtype == "f32":
        return a, None
    if dtype == "bf16":
        return f32_to_bf16_bits(a), None
    if dtype == "e4m3":
        return quantize_rows_e4m3(a)
    if dtype in BLOCK_FORMATS:
        return quantize_blocks_mx(a, dtype)
    raise ValueError(dtype)


def read_bias_fixture(fname: str, E: int) -> np.ndarray:
    vals = []
    with open(os.path.join(_GOLDEN, fname)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line))
    b = np.array(vals, dtype=np.float64)
    if b.shape != (E,):
        raise ValueError(f"{fname}: expected {E} values, found {b.shape[0]}")
    out = b.astype(np.float32)
    if not np.array_equal(out.astype(np.float64), b):
        raise ValueError(f"{fname}: values are not exact fp32")
    return out


_THREADS = max(1, min(16, os.cpu_count() or 1))


def _expert_stack(seed, tag, E, rows, cols, fan_in, dtype):
    """[E, rows, cols] weights, one seed sequence per expert, drawn in a thread pool."""
    item = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "mxfp4": np.uint8,
            "mxfp8": np.uint8}[dtype]
    out = np.empty((E, rows, cols // 2 if dtype == "mxfp4" else cols), dtype=item)
    if dtype == "e4m3":
        scales = np.empty((E, rows), dtype=np.float32)
    elif dtype in BLOCK_FORMATS:
        scales = np.empty((E, rows, cols // MX_BLOCK), dtype=np.uint8)
    else:
        scales = None

    def one(e):
        st, sc = _store(_normal((seed, tag, e), (rows, cols), fan_in), dtype)
        out[e] = st
        if scales is not None:
            scales[e] = sc

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, range(E)))
    return out, scales


def make_layer(cfg: LayerConfig, seed: int = 0, tensors=None) -> dict:
    """All inputs of one layer call, in storage formats.

    Returns a dict with numpy arrays: x [T,H], W_r [E,H], b [E] fp32, W_up [E,I,D],
    W_down [E,D,I] (+ s_up [E,I], s_down [E,D] for e4m3; for MXFP4 W_up [E,I,D/2] and W_down
    [E,D,I/2] packed codes, for MXFP4 / MXFP8 s_up [E,I,D/32] and s_down [E,D,I/32] uint8 E8M0
    block scales), Ws_up [I_s,H], Ws_down [H,I_s],
    W_in [l,H], W_out [H,l]. fp32 tensors are float32, bf16 tensors are uint16 bit patterns,
    e4m3 tensors are uint8 codes. ``tensors`` restricts which entries are drawn.
    """
    want = (lambda n: True) if tensors is None else (lambda n: n in tensors)
    T, H, E, I, D, Is, L = cfg.T, cfg.H, cfg.E, cfg.I, cfg.D, cfg.I_shared, cfg.latent
    ad = cfg.act_dtype
    out = {"config": cfg, "seed": seed}
    if want("x"):
        out["x"] = _store(_normal((seed, TAGS["x"]), (T, H), 1.0), ad)[0]
    if want("W_r"):
        out["W_r"] = _store(_normal((seed, TAGS["W_r"]), (E, H), H), ad)[0]
    if want("b"):
        if cfg.bias == "uniform":
            out["b"] = _rng(seed, TAGS["b"]).uniform(-0.1, 0.1, E).astype(np.float32)
        else:
            out["b"] = read_bias_fixture(cfg.bias, E)
    if want("W_up"):
        out["W_up"], out["s_up"] = _expert_stack(seed, TAGS["W_up"], E, I, D, D, cfg.expert_dtype)
    if want("W_down"):
        out["W_down"], out["s_down"] = _expert_stack(seed, TAGS["W_down"], E, D, I, I,
                                                     cfg.expert_dtype)
    if Is and want("Ws_up"):
        out["Ws_up"] = _store(_normal((seed, TAGS["Ws_up"]), (Is, H), H), ad)[0]
    if Is and want("Ws_down"):
        out["Ws_down"] = _store(_normal((seed, TAGS["Ws_down"]), (H, Is), Is), ad)[0]
    if L and want("W_in"):
        out["W_in"] = _store(_normal((seed, TAGS["W_in"]), (L, H), H), ad)[0]
    if L and want("W_out"):
        out["W_out"] = _store(_normal((seed, TAGS["W_out"]), (H, L), L), ad)[0]
    return out


def expert_rank_permutation(seed: int, E: int) -> np.ndarray:
    """Which expert holds popularity rank r (rank 0 = most popular) in the skewed profiles."""
    return _rng(seed, TAGS["rank"]).permutation(E)


def make_grad_output(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """Upstream gradient dy [T, H] for the backward pass: N(0, 1) draws stored in the layer's
    activation format (bf16 bit patterns or fp32)."""
    return _store(_normal((seed, TAGS["dy"]), (cfg.T, cfg.H), 1.0), cfg.act_dtype)[0]
