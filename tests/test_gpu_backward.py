"""GPU parity of the backward pass (bf16 plain MoE layer) against the double-precision oracle.

Every gradient the HIP path writes is compared with the oracle's on the same seeded inputs and
the same selection (the GPU's own, checked first against the oracle's routing wherever the
oracle's k-th / (k+1)-th key margin exceeds 1e-4), as a relative Frobenius error.

Tolerance. The path stores five intermediate tensors in bf16 -- relu(a), h, the expert outputs Y,
g * dy and da -- and accumulates in fp32. One bf16 rounding has a relative RMS error of about
2^-9 / sqrt(3) = 1.1e-3. A gradient that passes through two or three of them in sequence (dW_up:
g*dy and relu(a) into da) lands near sqrt(3) * 1.1e-3 = 2e-3; measured: dx up to 2.9e-3, dW_up
3.1e-3, dW_down 2.5e-3, the shared expert's 2.4e-3. LatentMoE adds four bf16 roundings in
sequence with these (u = x W_in^T, z, dy W_out and the per-token sum of the experts' input
gradient): measured 3.3e-3 to 4.2e-3, dW_in and dW_out included. The router gradient is built from the
differences dg_j - sum_m g_m dg_m, which cancel, so its relative error is that of dg (Y rounded)
times the cancellation ratio: measured up to 8.2e-3 on an expert row fed by three tokens. The
bounds are 1e-2 (two to three times the measured expert, shared-expert, projection and dx
errors) and 2e-2 for dW_r.
"""
import os
import sys

import numpy as np
import pytest

import moe_inputs as mi
from oracle import oracle as O

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import torch  # noqa: E402

import sparse_moe_layer_05_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))
TOL = {"dx": 1e-2, "dW_r": 2e-2, "dW_up": 1e-2, "dW_down": 1e-2, "dWs_up": 1e-2,
       "dWs_down": 1e-2, "dW_in": 1e-2, "dW_out": 1e-2}


def say(*a):
    print(*a, flush=True)


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


CASES = {
    # ragged everything: T*k odd, H and I not multiples of the 64-wide K-step or the 192-wide
    # tiles, 24 experts of uneven load
    "bwd_ragged": mi.LayerConfig("bwd_ragged", T=301, H=272, E=24, k=5, I=144, I_shared=208),
    "bwd_no_shared": mi.LayerConfig("bwd_no_shared", T=130, H=256, E=8, k=3, I=96),
    "bwd_one_token": mi.LayerConfig("bwd_one_token", T=1, H=256, E=16, k=4, I=64, I_shared=64),
    # few experts, many tokens each: per-expert K windows of several 64-column steps
    "bwd_few_experts": mi.LayerConfig("bwd_few_experts", T=600, H=256, E=4, k=2, I=128,
                                      I_shared=96),
    # an expert count that is not a multiple of 8, and experts left without tokens
    "bwd_e13_sparse": mi.LayerConfig("bwd_e13_sparse", T=3, H=256, E=13, k=2, I=64),
    # degenerate routings: every expert selected (k = E), and a single expert (a dense MLP)
    "bwd_all_experts": mi.LayerConfig("bwd_all_experts", T=20, H=256, E=8, k=8, I=64,
                                      I_shared=64),
    "bwd_one_expert": mi.LayerConfig("bwd_one_expert", T=50, H=256, E=1, k=1, I=128),
    # the largest routing the ABI takes: 1024 experts, 64 per token
    "bwd_max_routing": mi.LayerConfig("bwd_max_routing", T=150, H=256, E=1024, k=64, I=32,
                                      I_shared=32),
    # LatentMoE: experts in the latent width, without and with a shared expert
    "bwd_latent": mi.LayerConfig("bwd_latent", T=70, H=256, E=64, k=8, I=64, latent=64),
    "bwd_latent_shared": mi.LayerConfig("bwd_latent_shared", T=33, H=256, E=32, k=4, I=48,
                                        latent=96, I_shared=80),
}


def gpu_selection(dev, k):
    """The selection the GPU makes (the backward recomputes it with the same kernels)."""
    T, E = dev["x"].shape[0], dev["W_r"].shape[0]
    routing = moe.alloc_routing(T, E, k, "cuda")
    moe.layer_from(dev, k, path="grouped", routing=routing)()
    torch.cuda.synchronize()
    return routing["idx"].cpu().numpy(), routing["logits"].cpu().numpy()


def check_selection(inp, idx_gpu, tokens=None):
    z = O.logits(inp, tokens)
    idx_o, _, margin = O.route(z, inp["b"], inp["config"].k)
    sure = margin >= 1e-4
    sel = idx_gpu if tokens is None else idx_gpu[tokens]
    assert np.array_equal(sel[sure], idx_o[sure])


def grads_of(dev, k, dy_dev):
    bw = moe.backward_from(dev, k)
    g = bw(dy_dev)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_small_against_oracle(name):
    cfg = CASES[name]
    say(f"[gpu] backward parity {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} "
        f"I_s={cfg.I_shared}")
    inp = mi.make_layer(cfg, seed=3)
    dy = mi.make_grad_output(cfg, seed=3)
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": dy})["dy"]
    idx, _ = gpu_selection(dev, cfg.k)
    check_selection(inp, idx)
    got = grads_of(dev, cfg.k, dy_dev)
    ref = O.backward(inp, idx, mi.bf16_bits_to_f32(dy).astype(np.float64), threads=THREADS)
    for n in got:
        err = rel_frob(got[n], ref[n])
        say(f"[gpu]   {name} {n}: rel Frobenius {err:.3e}")
        assert err <= TOL[n], (n, err)


def test_backward_is_deterministic_and_linear_in_dy():
    cfg = CASES["bwd_ragged"]
    inp = mi.make_layer(cfg, seed=5)
    dy = mi.make_grad_output(cfg, seed=5)
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": dy})["dy"]
    bw = moe.backward_from(dev, cfg.k)
    a = {n: t.clone() for n, t in bw(dy_dev).items()}
    b = {n: t.clone() for n, t in bw(dy_dev).items()}
    c = {n: t.clone() for n, t in bw(2 * dy_dev).items()}   # doubling dy is exact in bf16
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n
        assert torch.equal(c[n], 2 * a[n]), n


def test_backward_zero_input_gives_zero_expert_weight_gradients():
    cfg = CASES["bwd_no_shared"]
    inp = mi.make_layer(cfg, seed=7)
    inp["x"] = np.zeros_like(inp["x"])
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": mi.make_grad_output(cfg, seed=7)})["dy"]
    g = grads_of(dev, cfg.k, dy_dev)
    for n in ("dx", "dW_r", "dW_up", "dW_down"):
        assert not np.any(g[n]), n


@pytest.mark.parametrize("name", ["nano_decode_bf16", "nano_prefill_bf16", "latent_decode_bf16"])
def test_backward_full_size(name):
    # Real Nano shapes. The decode batch (64 tokens) is checked on every token and every
    # gradient but the routed expert stacks, of which three experts are checked whole. The
    # prefill batch (8192 tokens) is checked on sampled tokens' dx and on the least-loaded
    # expert's complete weight and router-row gradients.
    cfg = mi.CONFIGS[name]
    say(f"[gpu] backward full size {name}: T={cfg.T}")
    inp = mi.make_layer(cfg, seed=0)
    dy = mi.make_grad_output(cfg, seed=0)
    dy64 = mi.bf16_bits_to_f32(dy).astype(np.float64)
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": dy})["dy"]
    idx, _ = gpu_selection(dev, cfg.k)
    got = grads_of(dev, cfg.k, dy_dev)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    if cfg.T <= 64:
        check_selection(inp, idx)
        ref = O.backward(inp, idx, dy64, want=("dx", "dW_r", "dWs_up", "dWs_down", "dW_in",
                                                "dW_out"), threads=THREADS)
        for n in ref:
            err = rel_frob(got[n], ref[n])
            say(f"[gpu]   {name} {n}: rel Frobenius {err:.3e}")
            assert err <= TOL[n], (n, err)
        experts = list(np.argsort(-counts)[:2]) + [int(np.flatnonzero(counts)[-1])]
    else:
        rng = np.random.default_rng(11)
        toks = np.sort(rng.choice(cfg.T, 32, replace=False)).astype(np.int32)
        check_selection(inp, idx, toks)
        ref = O.backward(inp, idx[toks], dy64[toks], tokens=toks, want=("dx",), threads=THREADS)
        err = rel_frob(got["dx"][toks], ref["dx"])
        say(f"[gpu]   {name} dx ({len(toks)} sampled tokens): rel Frobenius {err:.3e}")
        assert err <= TOL["dx"]
        experts = [int(np.argmin(np.where(counts > 0, counts, 1 << 30)))]
    for e in experts:
        toks = np.flatnonzero((idx == e).any(axis=1)).astype(np.int32)
        ref = O.backward(inp, idx[toks], dy64[toks], tokens=toks,
                         want=("dW_r", "dW_up", "dW_down"), expert=int(e), threads=THREADS)
        for n, g in (("dW_up", got["dW_up"][e]), ("dW_down", got["dW_down"][e]),
                     ("dW_r", got["dW_r"][e])):
            r = ref[n][e] if n == "dW_r" else ref[n]
            err = rel_frob(g, r)
            say(f"[gpu]   {name} expert {e} ({len(toks)} tokens) {n}: rel Frobenius {err:.3e}")
            assert err <= TOL[n], (n, e, err)


GROUP_BM = 128   # row height of the grouped launches' M-tiles over the pair rows


def tile_cover_tokens(idx, E, T, seed, bm=GROUP_BM):
    """Tokens whose pair rows meet every (expert, bm-row M-tile) of the grouped launches over
    the pair rows (rows in the dispatch order of the selection idx), and every bm-row band of T
    (dense launches over all tokens); a partial tile is met at its last row."""
    rng = np.random.default_rng(seed)
    counts, offsets, perm, pos = (a.astype(np.int64) for a in O.dispatch(idx, E))
    expert_of = np.repeat(np.arange(E), counts)
    tile_of = (np.arange(offsets[-1]) - offsets[expert_of]) // bm
    covered, chosen = set(), set()
    for e in range(E):
        for mt in range(-(-int(counts[e]) // bm)):
            if (e, mt) in covered:
                continue
            lo = offsets[e] + mt * bm
            hi = min(lo + bm, offsets[e + 1])
            t = int(perm[hi - 1 if hi - lo < bm else int(rng.integers(lo, hi))])
            chosen.add(t)
            covered.update((int(expert_of[r]), int(tile_of[r])) for r in pos[t])
    assert len(covered) == int(np.sum(-(-counts // bm)))
    for b0 in range(0, T, bm):
        if not any(b0 <= t < b0 + bm for t in chosen):
            chosen.add(int(rng.integers(b0, min(T, b0 + bm))))
    return np.array(sorted(chosen), np.int32)


def expert_cover_tokens(idx, E, seed):
    """A few tokens that between them select every expert that has any token."""
    rng = np.random.default_rng(seed)
    used = np.zeros(E, bool)
    chosen = []
    for e in range(E):
        if used[e]:
            continue
        holders = np.flatnonzero((idx == e).any(axis=1))
        if holders.size == 0:
            continue
        t = int(rng.choice(holders))
        chosen.append(t)
        used[idx[t]] = True
    return np.array(sorted(chosen), np.int32)


def dy_on(cfg, toks):
    """The seeded upstream gradient, kept on `toks` and zero on every other token."""
    on = np.zeros(cfg.T, bool)
    on[toks] = True
    dy = mi.make_grad_output(cfg, seed=0)
    dy = np.where(on[:, None], dy, np.zeros_like(dy))        # bf16 bit pattern 0 is +0.0
    return on, dy, mi.bf16_bits_to_f32(dy).astype(np.float64)


def expert_stack_errors(inp, idx, dy64, toks, experts, got):
    """Relative Frobenius errors of the GPU's dW_up / dW_down of each listed expert against the
    oracle's over the listed tokens: {expert: (tokens, err_up, err_down)} (one thread per
    expert; each oracle call runs that expert's tokens, and only the errors are kept)."""
    from concurrent.futures import ThreadPoolExecutor

    def one(e):
        mine = toks[(idx[toks] == e).any(axis=1)]
        r = O.backward(inp, idx[mine], dy64[mine], tokens=mine, want=("dW_up", "dW_down"),
                       expert=int(e))
        return (len(mine), rel_frob(got["dW_up"][e], r["dW_up"]),
                rel_frob(got["dW_down"][e], r["dW_down"]))
    with ThreadPoolExecutor(THREADS) as ex:
        return dict(zip(experts, ex.map(one, experts)))


@pytest.mark.parametrize("name", ["nano_prefill_bf16", "latent_bf16"])
def test_backward_full_size_with_dy_on_sampled_tokens(name):
    # Real prefill shapes (the launches the bench times) with dy nonzero only on a token set
    # that meets every tile of the grouped launches over the pair rows (each expert's M-tiles)
    # and every band of the dense launches over all tokens. With the selection held fixed, a
    # token's contribution to every gradient is zero when its dy is, so each gradient is a sum
    # over the sampled tokens that the oracle computes exactly: dx on every token (exactly zero
    # off the sample), dW_r, the shared expert's and the latent projections' gradients whole,
    # and the expert stacks on the three experts the sample uses most.
    cfg = mi.CONFIGS[name]
    inp = mi.make_layer(cfg, seed=0)
    dev = moe.to_device(inp)
    idx, _ = gpu_selection(dev, cfg.k)
    toks = tile_cover_tokens(idx, cfg.E, cfg.T, seed=17)
    say(f"[gpu] backward full size, dy on {len(toks)} tile-covering tokens: {name} T={cfg.T}")
    on, dy, dy64 = dy_on(cfg, toks)
    dy_dev = moe.to_device({"dy": dy})["dy"]
    check_selection(inp, idx, toks)
    got = grads_of(dev, cfg.k, dy_dev)
    assert not np.any(got["dx"][~on])
    ref = O.backward(inp, idx[toks], dy64[toks], tokens=toks,
                     want=("dx", "dW_r", "dWs_up", "dWs_down", "dW_in", "dW_out"), threads=THREADS)
    for n in ref:
        err = rel_frob(got[n][toks] if n == "dx" else got[n], ref[n])
        say(f"[gpu]   {name} {n}: rel Frobenius {err:.3e}")
        assert err <= TOL[n], (n, err)
    used = np.bincount(idx[toks].ravel(), minlength=cfg.E)
    unused = np.flatnonzero(used == 0)
    assert not np.any(got["dW_up"][unused]) and not np.any(got["dW_down"][unused])
    for e in np.argsort(-used, kind="stable")[:3]:
        mine = toks[(idx[toks] == e).any(axis=1)]
        r = O.backward(inp, idx[mine], dy64[mine], tokens=mine, want=("dW_up", "dW_down"),
                       expert=int(e), threads=THREADS)
        for n in ("dW_up", "dW_down"):
            err = rel_frob(got[n][e], r[n])
            say(f"[gpu]   {name} expert {e} ({len(mine)} tokens) {n}: rel Frobenius {err:.3e}")
            assert err <= TOL[n], (n, e, err)


@pytest.mark.parametrize("name", ["nano_prefill_bf16", "latent_bf16"])
def test_backward_full_size_every_expert_stack(name):
    # Real prefill shapes with dy nonzero only on a few tokens that between them select every
    # expert with any token: each expert's weight gradients are then sums over its sampled
    # tokens, and every expert's whole dW_up and dW_down (all of its output tiles) is compared
    # with the oracle; experts no token selects must come out exactly zero.
    cfg = mi.CONFIGS[name]
    inp = mi.make_layer(cfg, seed=0)
    dev = moe.to_device(inp)
    idx, _ = gpu_selection(dev, cfg.k)
    toks = expert_cover_tokens(idx, cfg.E, seed=19)
    say(f"[gpu] backward full size, dy on {len(toks)} expert-covering tokens: {name}")
    on, dy, dy64 = dy_on(cfg, toks)
    check_selection(inp, idx, toks)
    got = grads_of(dev, cfg.k, moe.to_device({"dy": dy})["dy"])
    used = np.bincount(idx[toks].ravel(), minlength=cfg.E)
    assert np.array_equal(used > 0, np.bincount(idx.ravel(), minlength=cfg.E) > 0)
    unused = np.flatnonzero(used == 0)
    assert not np.any(got["dW_up"][unused]) and not np.any(got["dW_down"][unused])
    errs = expert_stack_errors(inp, idx, dy64, toks, [int(e) for e in np.flatnonzero(used)],
                               got)
    up = max(v[1] for v in errs.values())
    down = max(v[2] for v in errs.values())
    say(f"[gpu]   {name}: {len(errs)} experts, worst rel Frobenius dW_up {up:.3e}, "
        f"dW_down {down:.3e}")
    for e, (n_tok, eu, ed) in errs.items():
        assert eu <= TOL["dW_up"] and ed <= TOL["dW_down"], (e, n_tok, eu, ed)


@pytest.mark.parametrize("name", ["bwd_ragged", "bwd_e13_sparse", "bwd_latent_shared"])
def test_training_forward_and_saved_backward_match_the_plain_calls(name):
    # moe_layer_forward_train gives the grouped forward's y bit for bit, and a backward that
    # reads its saved activations gives the recomputing backward's gradients bit for bit, also
    # when called twice after one training forward.
    cfg = CASES[name]
    inp = mi.make_layer(cfg, seed=9)
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": mi.make_grad_output(cfg, seed=9)})["dy"]
    y_ref = moe.layer_from(dev, cfg.k, path="grouped")().clone()
    bw = moe.backward_from(dev, cfg.k)
    plain = {n: t.clone() for n, t in bw(dy_dev).items()}
    y = bw.forward_train()
    first = {n: t.clone() for n, t in bw(dy_dev, saved=True).items()}
    second = {n: t.clone() for n, t in bw(dy_dev, saved=True).items()}
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    for n in plain:
        assert torch.equal(first[n], plain[n]), n
        assert torch.equal(second[n], plain[n]), n



WGRAD = ("dW_up", "dW_down", "dWs_up", "dWs_down")


@pytest.mark.parametrize("name", ["bwd_ragged", "bwd_max_routing", "bwd_latent_shared",
                                  "nano_prefill_bf16"])
def test_bf16_weight_gradients_are_the_fp32_gradients_rounded(name):
    # Under MOE_WGRAD_BF16 the expert weight gradients are the same fp32 sums rounded to nearest
    # even: each equals the fp32 path's rounded by torch, bit for bit, so the parity above holds
    # for them with one more rounding (relative error at most 2^-9 per element). Every other
    # gradient is unchanged, with and without the saved activations.
    cfg = CASES.get(name) or mi.CONFIGS[name]
    say(f"[gpu] bf16 weight gradients {name}: T={cfg.T} E={cfg.E} I={cfg.I} I_s={cfg.I_shared}")
    inp = mi.make_layer(cfg, seed=11)
    dev = moe.to_device(inp)
    dy_dev = moe.to_device({"dy": mi.make_grad_output(cfg, seed=11)})["dy"]
    ref = {n: t.clone() for n, t in moe.backward_from(dev, cfg.k)(dy_dev).items()}
    bw = moe.backward_from(dev, cfg.k, wgrad_bf16=True)
    plain = {n: t.clone() for n, t in bw(dy_dev).items()}
    bw.forward_train()
    saved = bw(dy_dev, saved=True)
    torch.cuda.synchronize()
    assert set(plain) == set(ref)
    for n in ref:
        want = ref[n].to(torch.bfloat16) if n in WGRAD else ref[n]
        assert plain[n].dtype == want.dtype, n
        assert torch.equal(plain[n], want), n
        assert torch.equal(saved[n], want), n
    assert any(n in ref for n in WGRAD)
