"""moe_layer_forward_static (the entry point that allocates nothing: its scratch is the library's
per-GPU device array) against moe_layer_forward / latent_moe_forward with a caller workspace:
identical outputs and routing, bit for bit, on two calls in a row, the second with fewer tokens
(the array keeps the first call's contents)."""
import ctypes as C

import numpy as np
import pytest

import moe_inputs as mi

torch = pytest.importorskip("torch")
import sparse_moe_layer_05_amd as moe  # noqa: E402
from sparse_moe_layer_05_amd import binding as B  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    moe.lib()
    yield


def both(dev, k, path, T):
    """(y, routing) of the workspace call and of the static call on the first T tokens."""
    sub = dict(dev, x=dev["x"][:T].contiguous())
    outs = []
    for no_alloc in (False, True):
        E = sub["W_r"].shape[0]
        rt = moe.alloc_routing(T, E, k, "cuda")
        y = torch.full_like(sub["x"], 3.0)
        moe.layer_from(sub, k, path=path, routing=rt, out=y, no_alloc=no_alloc)()
        torch.cuda.synchronize()
        outs.append((y.cpu(), {n: t.cpu() for n, t in rt.items()}))
    return outs


CASES = [
    ("nano_decode_bf16", "auto"),        # bf16 weight streaming, shared slot in the launches
    ("nano_mxfp4_decode", "auto"),       # narrow decode: side stream, quantised rows
    ("latent_decode_bf16", "auto"),      # LatentMoE decode, split latent projection
    ("bf16_grouped_small", "grouped"),   # grouped GEMMs and the dense shared expert
]


@pytest.mark.parametrize("name,path", CASES)
def test_static_entry_matches_the_workspace_entry_on_two_calls(name, path):
    cfg = mi.LayerConfig("bf16_grouped_small", T=301, H=272, E=24, k=5, I=144, I_shared=208) \
        if name == "bf16_grouped_small" else mi.CONFIGS[name]
    print(f"[gpu] static entry {name} T={cfg.T} then T={cfg.T * 3 // 5} path={path}", flush=True)
    dev = moe.to_device(mi.make_layer(cfg, seed=5))
    for T in (cfg.T, cfg.T * 3 // 5):        # second call smaller: stale contents are ignored
        (y0, r0), (y1, r1) = both(dev, cfg.k, path, T)
        assert torch.equal(y0, y1), (name, T)
        for n in r0:
            assert torch.equal(r0[n], r1[n]), (name, T, n)


def test_static_entry_rejects_calls_beyond_its_scratch():
    cfg = mi.CONFIGS["nano_prefill_bf16"]
    d = B.MoeDesc()
    for f, v in dict(T=cfg.T, H=cfg.H, E=cfg.E, k=cfg.k, I=cfg.I, I_shared=cfg.I_shared,
                     latent=0, act_dtype=B.MOE_BF16, expert_dtype=B.MOE_BF16, flags=0).items():
        setattr(d, f, v)
    n = C.c_size_t(0)
    assert moe.lib().moe_workspace_size(C.byref(d), C.byref(n)) == 0
    assert n.value > (64 << 20)
    w = B.MoeWeights()
    rc = moe.lib().moe_layer_forward_static(C.byref(d), C.byref(w), None, None, None)
    assert rc == B.MOE_ERR_WORKSPACE
