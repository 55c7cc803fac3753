"""CPU checks of the seeded input generator and of the calibrated bias fixtures."""
import numpy as np
import torch

import moe_inputs as mi
from oracle import oracle as O


def test_generator_is_deterministic_and_seeded():
    c = mi.CONFIGS["tiny_f32"]
    a, b, d = mi.make_layer(c, 0), mi.make_layer(c, 0), mi.make_layer(c, 1)
    for name in ("x", "W_r", "b", "W_up", "W_down"):
        assert np.array_equal(a[name], b[name])
        assert not np.array_equal(a[name], d[name])


def test_generator_shapes_dtypes_and_scales():
    c = mi.LayerConfig("s", T=33, H=64, E=6, k=2, I=48, I_shared=32, latent=0,
                       act_dtype="bf16", expert_dtype="e4m3")
    inp = mi.make_layer(c, 3)
    assert inp["x"].shape == (33, 64) and inp["x"].dtype == np.uint16
    assert inp["W_up"].shape == (6, 48, 64) and inp["W_up"].dtype == np.uint8
    assert inp["s_up"].shape == (6, 48) and inp["s_down"].shape == (6, 64, )
    assert inp["W_down"].shape == (6, 64, 48)
    assert inp["Ws_up"].shape == (32, 64) and inp["Ws_down"].shape == (64, 32)
    # per-row scale makes the largest code of every row +-448
    assert np.all((inp["W_up"] & 0x7F).max(-1) == 0x7E)
    x = mi.bf16_bits_to_f32(inp["x"])
    assert abs(x.mean()) < 0.1 and abs(x.std() - 1) < 0.1


def test_weight_variance_is_one_over_fan_in():
    c = mi.CONFIGS["nano_decode_bf16"]
    inp = mi.make_layer(c.with_T(4), 0, tensors={"W_r", "Ws_down"})
    wr = mi.bf16_bits_to_f32(inp["W_r"]).astype(np.float64)
    assert abs(wr.var() * c.H - 1) < 0.02
    wd = mi.bf16_bits_to_f32(inp["Ws_down"]).astype(np.float64)
    assert abs(wd.var() * c.I_shared - 1) < 0.02


def test_prefix_of_tokens_is_stable_across_T():
    c = mi.CONFIGS["nano_decode_bf16"]
    a = mi.make_layer(c.with_T(5), 0, tensors={"x"})["x"]
    b = mi.make_layer(c.with_T(9), 0, tensors={"x"})["x"]
    assert np.array_equal(a, b[:5])


def test_zipf_bias_fixture_gives_skewed_popularity():
    c = mi.CONFIGS["nano_prefill_bf16"]
    inp = mi.make_layer(c, 0, tensors={"x", "W_r", "b"})
    idx, _, _ = O.route(O.logits(inp), inp["b"], c.k)
    counts = np.sort(np.bincount(idx.ravel(), minlength=c.E))[::-1]
    assert counts.sum() == c.T * c.k
    assert counts[0] == c.T                        # the top expert is capped at one pick per token
    assert counts[1] > 5000 and counts[-1] < 100   # Zipf(1.1) head and tail
    assert np.all(np.diff(counts[:20]) < 0)


def test_imbalance_bias_fixture_subset():
    c = mi.CONFIGS["nano_fp8"]
    sub = c.with_T(4096)
    inp = mi.make_layer(sub, 0, tensors={"x", "W_r", "b"})
    idx, _, _ = O.route(O.logits(inp), inp["b"], c.k)
    counts = np.sort(np.bincount(idx.ravel(), minlength=c.E))[::-1]
    mean = sub.T * sub.k / c.E
    assert np.all(counts[:4] > 8 * mean) and np.all(counts[:4] < 12 * mean)
    assert np.sum(counts == 0) >= 8


def _spec_e2m1():
    vals = []
    with open(f"{mi.golden_dir()}/e2m1_values.txt") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line))
    return np.array(vals)


def test_mx_block_scale_is_floor_log2_amax_minus_emax():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-20, 20, (7, 1)))
    w[3, 32:64] = 0.0                                             # an all-zero block
    for fmt, emax in (("mxfp4", 2), ("mxfp8", 8)):
        _, sc = mi.quantize_blocks_mx(w, fmt)
        amax = np.abs(w.reshape(7, 3, 32)).max(-1)
        want = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - emax + 127, 0)
        assert np.array_equal(sc, want.astype(np.uint8)), fmt


def test_mxfp8_elements_are_torch_e4m3_of_the_scaled_block():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((5, 64)) * np.exp2(rng.integers(-8, 8, (5, 64)))).astype(np.float32)
    codes, sc = mi.quantize_blocks_mx(w, "mxfp8")
    x = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=-1)
    v = np.clip(w / x, -448, 448).astype(np.float32)               # exact: x is a power of two
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_mxfp4_elements_are_nearest_spec_values_ties_even_and_packed_low_first():
    spec = _spec_e2m1()
    rng = np.random.default_rng(7)
    w = rng.standard_normal((4, 128)) * 3.0
    # plant exact midpoints of the E2M1 grid (times the block scale) and out-of-range values
    mags = spec[:8]
    w[0, :7] = (mags[:-1] + mags[1:]) / 2
    w[0, 7] = 6.0                                                  # amax of the block: scale 2^0
    w[1, :3] = [7.9, -7.0, 6.5]                                    # saturate at +-6 times the scale
    codes, sc = mi.quantize_blocks_mx(w, "mxfp4")
    x = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=-1)
    q = w / x
    # brute force: nearest magnitude on the spec grid; on a tie the even code (mantissa bit 0)
    d = np.abs(np.abs(q)[..., None] - mags)
    best = d.min(-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(-1)
    mag_code = np.where(even < 99, even, cand.min(-1))
    want = (mag_code | np.where(np.signbit(q), 8, 0)).astype(np.uint8)
    assert np.array_equal(codes & 0xF, want[:, 0::2]) and np.array_equal(codes >> 4, want[:, 1::2])
    assert sc[0, 0] == 127
    assert mi.decode_blocks_mx(codes, sc, "mxfp4")[0, :8].tolist() == \
        [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    # a zero block: scale code 0 and zero codes
    z, zs = mi.quantize_blocks_mx(np.zeros((1, 32)), "mxfp4")
    assert zs.tolist() == [[0]] and not z.any()
