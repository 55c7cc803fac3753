"""Pins of the double-precision oracle to things other than itself (CPU only).

Each test ties one oracle function to brute force on tiny inputs, a closed form, a special case
that reduces to a library routine (numpy matmul / stable sort, torch's float8 and bfloat16
casts), or an invariant of the layer. Together they are chosen so that a plausible slip anywhere
in the oracle (a dropped term, a wrong sign or index, a transposed operand, biased gates, softmax
for sigmoid, an unstable dispatch) fails at least one of them.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import oracle as O


def cfg(**kw):
    base = dict(name="pin", T=8, H=32, E=4, k=2, I=16, act_dtype="f32", expert_dtype="f32")
    base.update(kw)
    return mi.LayerConfig(**base)


def dense_mlp(x, W_up, W_down):
    """Textbook squared-ReLU MLP through numpy matmul: W_down relu(W_up x)^2, rows of x."""
    a = x @ W_up.T
    return (np.maximum(a, 0.0) ** 2) @ W_down.T


def f64(inp, name):
    a = inp[name]
    fmt = inp["config"].expert_dtype
    if name in ("W_up", "W_down") and fmt in mi.BLOCK_FORMATS:
        # the generator's own decoder (written apart from the oracle's)
        return mi.decode_blocks_mx(a, inp["s_up" if name == "W_up" else "s_down"], fmt)
    if a.dtype == np.uint16:
        return mi.bf16_bits_to_f32(a).astype(np.float64)
    if a.dtype == np.uint8:
        scale = inp["s_up" if name == "W_up" else "s_down"]
        vals = torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
        return vals * scale[..., None].astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------- formats

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2   # S.1111.111 only
    assert np.array_equal(mine[~nan], ref[~nan])
    assert O.e4m3_to_f64(np.array([0x7E]))[0] == 448.0
    assert O.e4m3_to_f64(np.array([0x01]))[0] == 2.0 ** -9


def test_e4m3_encode_roundtrip_and_ties_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.f64_to_e4m3(O.e4m3_to_f64(codes)), codes)
    # midpoints between neighbouring positive codes go to the even mantissa
    vals = O.e4m3_to_f64(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    got = O.f64_to_e4m3(mids)
    want = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(got, want.numpy())
    assert np.all(got % 2 == 0)
    # saturation beyond the largest finite value
    assert O.f64_to_e4m3(np.array([470.0, 1e6, -1e6])).tolist() == [0x7E, 0x7E, 0xFE]


def test_e4m3_encode_random_matches_torch_and_generator():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(4000) * np.exp2(rng.integers(-12, 8, 4000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.f64_to_e4m3(v.astype(np.float64)), ref)
    assert np.array_equal(mi.encode_e4m3(v), ref)


def test_bf16_decode_and_generator_rounding_match_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(5000) * np.exp2(rng.integers(-30, 30, 5000))).astype(np.float32)
    bits = mi.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(O.bf16_to_f64(bits[:500]),
                          torch.from_numpy(ref[:500].view(np.int16)).view(torch.bfloat16)
                          .double().numpy())


def read_e2m1_table():
    vals = []
    with open(f"{mi.golden_dir()}/e2m1_values.txt") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line))
    assert len(vals) == 16
    return np.array(vals)


def test_e2m1_decode_matches_the_spec_table():
    table = read_e2m1_table()
    codes = np.arange(16, dtype=np.uint8)
    for dec in (O.e2m1_to_f64(codes), mi.decode_e2m1(codes)):
        assert np.array_equal(dec, table)
        assert np.array_equal(np.signbit(dec), np.signbit(table))   # 0x8 is -0


def test_e8m0_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    for dec in (O.e8m0_to_f64(codes), mi.decode_e8m0(codes)):
        assert np.isnan(dec[255]) and np.isnan(ref[255])
        assert np.array_equal(dec[:255], ref[:255])
    assert O.e8m0_to_f64(np.array([127]))[0] == 1.0


# ----------------------------------------------------------------------------- routing

def brute_route(key, s, k):
    order = np.lexsort((np.arange(key.shape[0]), -key))   # key descending, index ascending
    sel = order[:k]
    margin = key[order[k - 1]] - key[order[k]] if k < key.shape[0] else np.inf
    return sel, s[sel] / s[sel].sum(), margin


@pytest.mark.parametrize("T,E,k", [(7, 5, 2), (16, 16, 2), (9, 12, 12), (5, 33, 6), (3, 64, 24)])
def test_route_matches_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    z = rng.standard_normal((T, E))
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    z[0, :3] = z[0, 3]            # exact ties in logits
    idx, g, m = O.route(z, b, k)
    for t in range(T):
        s = 1.0 / (1.0 + np.exp(-z[t]))
        sel, gg, mm = brute_route(s + b.astype(np.float64), s, k)
        assert idx[t].tolist() == sel.tolist()
        np.testing.assert_allclose(g[t], gg, rtol=1e-15, atol=0)
        assert m[t] == mm


def test_route_f32_matches_brute_force_in_binary32():
    rng = np.random.default_rng(3)
    T, E, k = 40, 128, 6
    z = rng.standard_normal((T, E)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    z[1, :] = z[1, 0]
    b[:8] = b[0]
    idx, g, m = O.route_f32(z, b, k)
    for t in range(T):
        s32 = (1.0 / (1.0 + np.exp(-z[t].astype(np.float64)))).astype(np.float32)
        key32 = s32 + b                     # numpy binary32 add
        sel, gg, _ = brute_route(key32.astype(np.float64), s32.astype(np.float64), k)
        assert idx[t].tolist() == sel.tolist()
        np.testing.assert_allclose(g[t], gg, rtol=1e-15)


def test_route_exact_ties_take_lowest_index():
    E, k = 10, 4
    z = np.zeros((1, E))
    b = np.zeros(E, np.float32)
    idx, g, m = O.route(z, b, k)
    assert idx[0].tolist() == [0, 1, 2, 3] and m[0] == 0.0
    np.testing.assert_array_equal(g[0], np.full(k, 0.25))


def test_route_forced_by_bias_and_gates_ignore_bias():
    # sigma(log 3) = 3/4 and sigma(0) = 1/2: closed-form gates 0.6 / 0.4 (softmax would be 3/4, 1/4)
    E, k = 6, 2
    z = np.zeros((1, E))
    z[0, 4] = np.log(3.0)
    b = np.zeros(E, np.float32)
    b[[1, 4]] = 4.0                     # scores are in (0, 1): +4 forces experts 1 and 4
    idx, g, _ = O.route(z, b, k)
    assert idx[0].tolist() == [4, 1]
    np.testing.assert_allclose(g[0], [0.6, 0.4], rtol=1e-14)
    b2 = b.copy()
    b2[1] = 5.0                        # expert 1 now first by key; gates still unbiased
    idx2, g2, _ = O.route(z, b2, k)
    assert idx2[0].tolist() == [1, 4]
    np.testing.assert_allclose(g2[0], [0.4, 0.6], rtol=1e-14)


def test_gates_for_a_given_selection():
    # sigma(log 3) = 3/4, sigma(0) = 1/2: selection [4, 0] -> 0.6, 0.4 whatever the bias says
    z = np.zeros((1, 6))
    z[0, 4] = np.log(3.0)
    np.testing.assert_allclose(O.gates_for(z, np.array([[4, 0]])), [[0.6, 0.4]], rtol=1e-14)
    np.testing.assert_allclose(O.gates_for(z, np.array([[0, 4]])), [[0.4, 0.6]], rtol=1e-14)
    np.testing.assert_allclose(O.gates_for(z, np.array([[1, 2, 3]])), [[1 / 3] * 3], rtol=1e-15)


def test_route_invariant_to_common_bias_shift():
    rng = np.random.default_rng(4)
    T, E, k = 50, 32, 4
    z = rng.standard_normal((T, E))
    b = (rng.integers(-100, 100, E) / 1024.0).astype(np.float32)
    i1, g1, _ = O.route(z, b, k)
    i2, g2, _ = O.route(z, (b + np.float32(0.5)).astype(np.float32), k)
    assert np.array_equal(i1, i2)
    np.testing.assert_array_equal(g1, g2)
    np.testing.assert_allclose(g1.sum(1), 1.0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_logits_are_x_times_router_transpose(act):
    # router logits of every token, and of a shuffled token subset with a repeat, against numpy's
    # matmul of the exactly decoded inputs (a dropped or shifted term of the H sum, a transposed
    # W_r or a wrong token row would all show)
    c = cfg(T=29, H=96, E=12, k=3, I=16, act_dtype=act, expert_dtype=act)
    inp = mi.make_layer(c, seed=21)
    want = f64(inp, "x") @ f64(inp, "W_r").T
    np.testing.assert_allclose(O.logits(inp), want, rtol=1e-13, atol=1e-13)
    toks = np.array([17, 3, 28, 0, 3, 11], np.int32)
    np.testing.assert_allclose(O.logits(inp, toks), want[toks], rtol=1e-13, atol=1e-13)


def test_layer_is_gate_weighted_sum_of_selected_expert_mlps():
    # generic routing (k of E, distinct gates per token) plus a shared expert, against numpy's
    # dense squared-ReLU MLPs of the selected experts, on every token and on a token subset
    c = cfg(T=23, H=48, E=9, k=3, I=24, I_shared=16, act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=22)
    r = O.forward(inp)
    x, Wu, Wd = f64(inp, "x"), f64(inp, "W_up"), f64(inp, "W_down")
    want = dense_mlp(x, f64(inp, "Ws_up"), f64(inp, "Ws_down"))
    for t in range(c.T):
        for j in range(c.k):
            e = r["idx"][t, j]
            want[t] += r["gates"][t, j] * dense_mlp(x[t:t + 1], Wu[e], Wd[e])[0]
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)
    toks = np.array([22, 5, 0, 13], np.int32)
    rs = O.forward(inp, toks)
    np.testing.assert_allclose(rs["y"], want[toks], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("latent", [0, 32])
def test_forward_of_a_token_subset_with_threads_equals_the_whole_call(latent):
    # the parity tests at full size run the oracle on token subsets split over threads: every
    # listed token's result must be the whole call's, bit for bit
    c = cfg(T=41, H=64, E=10, k=4, I=24, I_shared=0 if latent else 16, latent=latent,
            act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=23)
    whole = O.forward(inp)
    toks = np.array([40, 2, 7, 7, 19, 0, 33, 25, 11], np.int32)
    for threads in (1, 4):
        part = O.forward(inp, toks, threads=threads)
        for key in ("logits", "idx", "gates", "margin", "y"):
            assert np.array_equal(part[key], whole[key][toks]), (threads, key)


# ----------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (37, 8, 3), (64, 16, 2), (200, 128, 6)])
def test_dispatch_matches_stable_sort(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, pos = O.dispatch(idx, E)
    order = np.argsort(idx.ravel(), kind="stable")          # pairs grouped by expert, in order
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, order // k)
    inv = np.empty(T * k, np.int64)
    inv[order] = np.arange(T * k)
    assert np.array_equal(pos.ravel(), inv)
    for e in range(E):                                       # stable: tokens ascend in an expert
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


# ----------------------------------------------------------------------------- layer math

def test_single_expert_is_dense_squared_relu_mlp():
    c = cfg(E=1, k=1, T=5, H=48, I=24)
    inp = mi.make_layer(c, seed=7)
    r = O.forward(inp)
    assert np.all(r["idx"] == 0) and np.all(r["gates"] == 1.0)
    want = dense_mlp(f64(inp, "x"), f64(inp, "W_up")[0], f64(inp, "W_down")[0])
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_all_experts_with_zero_router_is_uniform_average():
    c = cfg(E=5, k=5, T=6, H=40, I=20)
    inp = mi.make_layer(c, seed=8)
    inp["W_r"] = np.zeros_like(inp["W_r"])
    inp["b"] = np.zeros_like(inp["b"])
    r = O.forward(inp)
    assert np.array_equal(r["idx"], np.tile(np.arange(5), (6, 1)))
    np.testing.assert_allclose(r["gates"], 0.2, rtol=1e-15)
    x, Wu, Wd = f64(inp, "x"), f64(inp, "W_up"), f64(inp, "W_down")
    want = sum(dense_mlp(x, Wu[e], Wd[e]) for e in range(5)) / 5
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_two_expert_gates_weight_each_output():
    # E=2, k=2, logits (0, log 3) via the router: y = 0.4 f0(x) + 0.6 f1(x)  (closed-form gates)
    c = cfg(E=2, k=2, T=1, H=16, I=8)
    inp = mi.make_layer(c, seed=9)
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 1.0
    Wr = np.zeros((2, 16), np.float32)
    Wr[1, 0] = np.float32(np.log(3.0))
    inp["x"], inp["W_r"], inp["b"] = x, Wr, np.zeros(2, np.float32)
    r = O.forward(inp)
    s1 = 1 / (1 + np.exp(-np.float64(np.float32(np.log(3.0)))))
    g = np.array([s1, 0.5]) / (s1 + 0.5)
    assert r["idx"][0].tolist() == [1, 0]
    Wu, Wd = f64(inp, "W_up"), f64(inp, "W_down")
    want = g[0] * dense_mlp(x.astype(np.float64), Wu[1], Wd[1]) + \
        g[1] * dense_mlp(x.astype(np.float64), Wu[0], Wd[0])
    np.testing.assert_allclose(r["y"], want, rtol=1e-13)


def test_shared_expert_alone_is_dense_mlp():
    c = cfg(E=4, k=2, T=5, H=32, I=16, I_shared=24)
    inp = mi.make_layer(c, seed=10)
    inp["W_down"] = np.zeros_like(inp["W_down"])
    r = O.forward(inp)
    want = dense_mlp(f64(inp, "x"), f64(inp, "Ws_up"), f64(inp, "Ws_down"))
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_zero_input_gives_zero_and_doubling_input_quadruples_output():
    c = cfg(E=6, k=3, T=7, H=32, I=16, I_shared=8)
    inp = mi.make_layer(c, seed=11)
    inp["W_r"] = np.zeros_like(inp["W_r"])        # routing then does not depend on x
    r1 = O.forward(inp)
    inp2 = dict(inp, x=(inp["x"] * 2).astype(np.float32))
    r2 = O.forward(inp2)
    assert np.array_equal(r2["y"], 4.0 * r1["y"])     # powers of two: exact
    inp0 = dict(inp, x=np.zeros_like(inp["x"]))
    assert np.all(O.forward(inp0)["y"] == 0.0)


def test_token_permutation_equivariance():
    c = cfg(E=8, k=3, T=12, H=32, I=16, I_shared=8, act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=12)
    perm = np.random.default_rng(0).permutation(12)
    r = O.forward(inp)
    rp = O.forward(dict(inp, x=inp["x"][perm]))
    assert np.array_equal(rp["y"], r["y"][perm])
    assert np.array_equal(rp["idx"], r["idx"][perm])


def test_latent_with_identity_projections_is_plain_moe():
    c = cfg(E=8, k=3, T=6, H=32, I=16, act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=13)
    cl = dataclasses.replace(c, latent=32)
    eye = mi.f32_to_bf16_bits(np.eye(32, dtype=np.float32))
    inpl = dict(inp, config=cl, W_in=eye, W_out=eye)
    assert np.array_equal(O.forward(inpl)["y"], O.forward(inp)["y"])


def test_latent_single_expert_is_projected_dense_mlp():
    c = cfg(E=1, k=1, T=4, H=48, I=8, latent=16)
    inp = mi.make_layer(c, seed=14)
    r = O.forward(inp)
    x, Win, Wout = f64(inp, "x"), f64(inp, "W_in"), f64(inp, "W_out")
    want = dense_mlp(x @ Win.T, f64(inp, "W_up")[0], f64(inp, "W_down")[0]) @ Wout.T
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_latent_scaling_of_expert_count_and_top_k():
    # E' = E*H/l and k' = k*H/l (Nemotron 3 white paper, section 2.2); Table 1 trained k'=22.
    golden = {}
    with open(mi.golden_dir() + "/latent_scaling.txt") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = line.split("=")
                golden[key.strip()] = int(val)
    H, l, E, k = golden["H"], golden["l"], golden["E"], golden["k"]
    assert E * H // l == golden["E_latent"]
    c = mi.CONFIGS["latent_bf16"]
    assert (c.H, c.latent, c.E) == (H, l, golden["E_latent"]) and c.k == k * H // l


def test_fp8_experts_use_dequantised_weights_exactly():
    c = cfg(E=1, k=1, T=4, H=64, I=32, act_dtype="bf16", expert_dtype="e4m3")
    inp = mi.make_layer(c, seed=15)
    r = O.forward(inp)
    want = dense_mlp(f64(inp, "x"), f64(inp, "W_up")[0], f64(inp, "W_down")[0])
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_fp8_emulation_quantises_activation_rows():
    # E=1, k=1: x and h rows quantised per row (scale amax/448, codes = torch's e4m3 cast of
    # the row times fp32(448/amax)), h rounded to bf16 first; the rest is numpy matmul.
    c = cfg(E=1, k=1, T=6, H=64, I=32, act_dtype="bf16", expert_dtype="e4m3")
    inp = mi.make_layer(c, seed=16)
    r = O.forward_tokens(inp, np.zeros((6, 1), np.int32), np.ones((6, 1)), fp8_emulate=True)

    def q(rows):
        rows32 = rows.astype(np.float32)
        amax = np.abs(rows32).max(1)
        sc = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
        inv = np.where(amax > 0, np.float32(448) / amax, np.float32(1)).astype(np.float32)
        v = torch.from_numpy((rows32 * inv[:, None]).astype(np.float32))
        return v.to(torch.float8_e4m3fn).double().numpy() * sc[:, None].astype(np.float64)

    x = q(f64(inp, "x"))
    h = np.maximum(x @ f64(inp, "W_up")[0].T, 0) ** 2
    h = torch.from_numpy(h).float().to(torch.bfloat16).double().numpy()
    want = q(h) @ f64(inp, "W_down")[0].T
    np.testing.assert_allclose(r, want, rtol=1e-12, atol=1e-13)


def test_fp8_emulation_of_a_latent_layer_rounds_the_projection_to_bf16():
    # LatentMoE with e4m3 experts: the projection u = W_in x is rounded to bf16 (where a bf16
    # layer keeps it), then quantised per row like x; E=1, k=1, no shared expert; numpy matmul.
    c = cfg(E=1, k=1, T=5, H=64, I=32, latent=48, act_dtype="bf16", expert_dtype="e4m3")
    inp = mi.make_layer(c, seed=19)
    r = O.forward_tokens(inp, np.zeros((5, 1), np.int32), np.ones((5, 1)), fp8_emulate=True)

    def bf16(a):
        return torch.from_numpy(a).float().to(torch.bfloat16).double().numpy()

    def q(rows):
        rows32 = rows.astype(np.float32)
        amax = np.abs(rows32).max(1)
        sc = (amax / np.float32(448)).astype(np.float32)
        inv = (np.float32(448) / amax).astype(np.float32)
        v = torch.from_numpy((rows32 * inv[:, None]).astype(np.float32))
        return v.to(torch.float8_e4m3fn).double().numpy() * sc[:, None].astype(np.float64)

    u = q(bf16(f64(inp, "x") @ f64(inp, "W_in").T))
    h = q(bf16(np.maximum(u @ f64(inp, "W_up")[0].T, 0) ** 2))
    want = (h @ f64(inp, "W_down")[0].T) @ f64(inp, "W_out").T
    np.testing.assert_allclose(r, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("E,k", [(1, 1), (5, 2)])
def test_block_scaled_experts_use_decoded_weights_exactly(fmt, E, k):
    # Every selected expert is a squared-ReLU MLP over the block-decoded weights: checked with
    # numpy matmul on the generator's decoder, per token and selected expert; several experts
    # check the expert stride of packed codes and of the block scales.
    c = cfg(E=E, k=k, T=5, H=96, I=64, act_dtype="bf16", expert_dtype=fmt)
    inp = mi.make_layer(c, seed=17)
    rng = np.random.default_rng(3)
    for name in ("s_up", "s_down"):   # spread the block scales over 13 binades
        inp[name] = (inp[name] + rng.integers(-6, 7, inp[name].shape)).astype(np.uint8)
    assert len(np.unique(inp["s_up"])) > 8
    r = O.forward(inp)
    x, Wu, Wd = f64(inp, "x"), f64(inp, "W_up"), f64(inp, "W_down")
    want = np.zeros((c.T, c.H))
    for t in range(c.T):
        for j in range(k):
            e = r["idx"][t, j]
            want[t] += r["gates"][t, j] * dense_mlp(x[t:t + 1], Wu[e], Wd[e])[0]
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_block_scaled_emulation_quantises_activation_rows(fmt):
    # Block-scaled expert weights take the activation rows through the same per-row e4m3
    # quantisation as e4m3 weights. With one block scale 2^-5 throughout, the same weights are
    # an e4m3 layer exactly (element codes as e4m3 codes, row scales 2^-5), which must give the
    # same emulated output bit for bit. (Block-scale indexing is pinned by the test above.)
    c = cfg(E=1, k=1, T=6, H=64, I=32, act_dtype="bf16", expert_dtype=fmt)
    inp = mi.make_layer(c, seed=18)
    twin = dict(inp, config=dataclasses.replace(c, expert_dtype="e4m3"))
    for w, sc in (("W_up", "s_up"), ("W_down", "s_down")):
        inp[sc] = np.full_like(inp[sc], 127 - 5)
        elements = mi.decode_blocks_mx(inp[w], np.full_like(inp[sc], 127), fmt)
        twin[w] = mi.encode_e4m3(elements)
        assert np.array_equal(mi.decode_e4m3(twin[w]), elements)
        twin[sc] = np.full(elements.shape[:-1], 2.0 ** -5, np.float32)
    one = (np.zeros((6, 1), np.int32), np.ones((6, 1)))
    a = O.forward_tokens(inp, *one, fp8_emulate=True)
    b = O.forward_tokens(twin, *one, fp8_emulate=True)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, O.forward_tokens(inp, *one))   # emulation did change it


def test_bias_update_sign_rule():
    b = np.array([0.0, 0.5, -0.5, 1.0])
    counts = np.array([10, 3, 7, 7], np.int32)
    target = np.array([5.0, 5.0, 7.0, 9.0])
    nb = O.bias_update(b, counts, target, 0.25)
    np.testing.assert_array_equal(nb, [-0.25, 0.75, -0.5, 1.25])


# ----------------------------------------------------------------------------- backward

_WEIGHTS = ("x", "W_r", "W_up", "W_down", "Ws_up", "Ws_down", "W_in", "W_out")
_GRAD_OF = {"x": "dx", "W_r": "dW_r", "W_up": "dW_up", "W_down": "dW_down", "Ws_up": "dWs_up",
            "Ws_down": "dWs_down", "W_in": "dW_in", "W_out": "dW_out"}


def f64_layer(seed, T=3, H=8, E=5, k=2, I=6, Is=4, latent=0):
    """A tiny layer held in float64 (read exactly by the oracle), with pre-activations kept away
    from the squared-ReLU's kink so that central differences never straddle it."""
    c = cfg(T=T, H=H, E=E, k=k, I=I, I_shared=Is, latent=latent)
    D = latent or H
    rng = np.random.default_rng(seed)
    inp = {"config": c, "x": rng.standard_normal((T, H)),
           "W_r": rng.standard_normal((E, H)) / np.sqrt(H),
           "b": rng.uniform(-0.1, 0.1, E).astype(np.float32),
           "W_up": rng.standard_normal((E, I, D)) / np.sqrt(D),
           "W_down": rng.standard_normal((E, D, I)) / np.sqrt(I)}
    if Is:
        inp["Ws_up"] = rng.standard_normal((Is, H)) / np.sqrt(H)
        inp["Ws_down"] = rng.standard_normal((H, Is)) / np.sqrt(Is)
    u = inp["x"]
    if latent:
        inp["W_in"] = rng.standard_normal((latent, H)) / np.sqrt(H)
        inp["W_out"] = rng.standard_normal((H, latent)) / np.sqrt(latent)
        u = inp["x"] @ inp["W_in"].T
    a = np.einsum("eid,td->tei", inp["W_up"], u)
    gap = np.abs(a).min()
    if Is:
        gap = min(gap, np.abs(inp["x"] @ inp["Ws_up"].T).min())
    return inp, gap


def loss(inp, idx, dy):
    """Sum_t <dy_t, y_t> with the selection idx held fixed and gates recomputed from the logits."""
    g = O.gates_for(O.logits(inp), idx)
    return float(np.sum(O.forward_tokens(inp, idx, g) * dy))


@pytest.mark.parametrize("latent", [0, 4])
def test_backward_matches_central_differences(latent):
    # Pins every gradient of the backward oracle to the forward oracle alone: each entry of
    # every input is nudged by +-eps and the change of the loss compared with the gradient.
    for seed in range(20):
        inp, gap = f64_layer(seed, latent=latent)
        if gap > 1e-2:
            break
    c = inp["config"]
    idx, _, margin = O.route(O.logits(inp), inp["b"], c.k)
    dy = np.random.default_rng(99).standard_normal((c.T, c.H))
    grads = O.backward(inp, idx, dy)
    eps = 1e-6
    for name in [n for n in _WEIGHTS if n in inp]:
        arr = inp[name]
        fd = np.zeros(arr.shape)
        for i in np.ndindex(arr.shape):
            keep = arr[i]
            arr[i] = keep + eps
            up = loss(inp, idx, dy)
            arr[i] = keep - eps
            dn = loss(inp, idx, dy)
            arr[i] = keep
            fd[i] = (up - dn) / (2 * eps)
        got = grads[_GRAD_OF[name]]
        assert np.allclose(got, fd, rtol=1e-6, atol=1e-8), (name, np.abs(got - fd).max())


def torch_layer_loss(t, idx, dy, k):
    """The layer written with torch float64 ops on CPU (selection fixed) for autograd."""
    x, W_r, W_up, W_down = t["x"], t["W_r"], t["W_up"], t["W_down"]
    s = torch.sigmoid(x @ W_r.T)
    u = x @ t["W_in"].T if "W_in" in t else x
    sel = torch.from_numpy(idx.astype(np.int64))
    ss = torch.gather(s, 1, sel)
    g = ss / ss.sum(dim=1, keepdim=True)
    y = torch.zeros_like(u)
    for j in range(k):
        e = sel[:, j]
        a = torch.einsum("tid,td->ti", W_up[e], u)
        h = torch.relu(a) ** 2
        y = y + g[:, j:j + 1] * torch.einsum("tdi,ti->td", W_down[e], h)
    if "W_out" in t:
        y = y @ t["W_out"].T
    if "Ws_up" in t:
        y = y + (torch.relu(x @ t["Ws_up"].T) ** 2) @ t["Ws_down"].T
    return (y * torch.from_numpy(dy)).sum()


@pytest.mark.parametrize("shared,latent", [(0, 0), (24, 0), (24, 16)])
def test_backward_matches_torch_autograd(shared, latent):
    # bf16-valued inputs (the oracle reads the bit patterns exactly; torch gets the same values
    # in float64); gradients from torch's reverse-mode differentiation of the layer.
    c = cfg(T=16, H=32, E=8, k=3, I=16, I_shared=shared, latent=latent, act_dtype="bf16",
            expert_dtype="bf16")
    inp = mi.make_layer(c, seed=4)
    dy64 = mi.bf16_bits_to_f32(mi.make_grad_output(c, seed=4)).astype(np.float64)
    idx, _, _ = O.route(O.logits(inp), inp["b"], c.k)
    grads = O.backward(inp, idx, dy64)
    names = [n for n in _WEIGHTS if n in inp]
    t = {n: torch.tensor(f64(inp, n), dtype=torch.float64, requires_grad=True) for n in names}
    L = torch_layer_loss(t, idx, dy64, c.k)
    auto = torch.autograd.grad(L, [t[n] for n in names])
    for n, gref in zip(names, auto):
        got = grads[_GRAD_OF[n]]
        ref = gref.numpy()
        assert np.allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max()), n
    # dz: only the selected experts carry a logit gradient
    dz = grads["dz"]
    mask = np.zeros_like(dz, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(dz[~mask] == 0.0)


def test_backward_expert_filter_and_threads_agree_with_full_call():
    c = cfg(T=40, H=32, E=6, k=2, I=16, I_shared=8, act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=2)
    dy = mi.bf16_bits_to_f32(mi.make_grad_output(c, seed=2)).astype(np.float64)
    idx, _, _ = O.route(O.logits(inp), inp["b"], c.k)
    full = O.backward(inp, idx, dy)
    split = O.backward(inp, idx, dy, threads=4)
    for n in full:
        assert np.allclose(split[n], full[n], rtol=1e-12, atol=1e-14), n
    e = int(idx[0, 0])
    one = O.backward(inp, idx, dy, want=("dW_up", "dW_down"), expert=e)
    assert np.array_equal(one["dW_up"], full["dW_up"][e])
    assert np.array_equal(one["dW_down"], full["dW_down"][e])
    # tokens that do not route to e contribute nothing to its weight gradients
    sel = np.where((idx == e).any(axis=1))[0]
    sub = O.backward(inp, idx[sel], dy[sel], tokens=sel, want=("dW_up", "dW_down"), expert=e)
    assert np.array_equal(sub["dW_up"], one["dW_up"])


def test_backward_is_linear_in_dy_and_zero_input_gives_zero_weight_gradients():
    c = cfg(T=12, H=32, E=5, k=2, I=16, I_shared=8, act_dtype="bf16", expert_dtype="bf16")
    inp = mi.make_layer(c, seed=6)
    idx, _, _ = O.route(O.logits(inp), inp["b"], c.k)
    dy = mi.bf16_bits_to_f32(mi.make_grad_output(c, seed=6)).astype(np.float64)
    g1 = O.backward(inp, idx, dy)
    g2 = O.backward(inp, idx, 2.0 * dy)
    for n in g1:
        assert np.array_equal(g2[n], 2.0 * g1[n]), n
    z = dict(inp, x=np.zeros_like(inp["x"]))
    g0 = O.backward(z, idx, dy)
    for n in ("dx", "dz", "dW_r", "dW_up", "dW_down", "dWs_up", "dWs_down"):
        assert not np.any(g0[n]), n


def test_latent_backward_with_identity_projections_is_the_plain_backward():
    # l = H with W_in = W_out = I: the LatentMoE layer is the plain layer, and so are all its
    # gradients (dW_in and dW_out themselves are pinned by the difference and autograd tests).
    c = cfg(T=10, H=16, E=6, k=2, I=8, I_shared=8, act_dtype="f32", expert_dtype="f32")
    plain = mi.make_layer(c, seed=8)
    cl = dataclasses.replace(c, latent=16)
    lat = dict(plain, config=cl, W_in=np.eye(16, dtype=np.float32),
               W_out=np.eye(16, dtype=np.float32))
    idx, _, _ = O.route(O.logits(plain), plain["b"], c.k)
    dy = np.random.default_rng(8).standard_normal((c.T, c.H))
    gp = O.backward(plain, idx, dy)
    gl = O.backward(lat, idx, dy)
    for n in ("dx", "dz", "dW_r", "dW_up", "dW_down", "dWs_up", "dWs_down"):
        assert np.allclose(gl[n], gp[n], rtol=1e-12, atol=1e-14), n

