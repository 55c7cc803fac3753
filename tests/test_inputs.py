"""CPU checks of the seeded input generator and of the calibrated bias fixtures."""
import numpy as np

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
