"""CPU checks of the C ABI: the library loads, exports every symbol include/moe.h declares, and
rejects bad arguments before it launches anything (no GPU is touched by these calls)."""
import ctypes as C
import os
import re

import pytest

import sparse_moe_layer_05_amd as moe
from sparse_moe_layer_05_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x10000)    # aligned, never dereferenced: validation fails or returns first


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return set(re.findall(r"^(?:int32_t|const char \*|void)\s*(\w+)\(", text, re.M))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert names == set(B.EXPORTS)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def desc(**kw):
    d = B.MoeDesc()
    base = dict(T=64, H=256, E=16, k=2, I=128, I_shared=0, latent=0, act_dtype=1,
                expert_dtype=1, flags=0)
    base.update(kw)
    for k_, v in base.items():
        setattr(d, k_, v)
    return d


def ws_size(d):
    n = C.c_size_t(0)
    rc = moe.lib().moe_workspace_size(C.byref(d), C.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), B.MOE_ERR_INVALID_ARG), (dict(k=17), B.MOE_ERR_INVALID_ARG),
    (dict(k=65, E=128), B.MOE_ERR_INVALID_ARG), (dict(E=0), B.MOE_ERR_INVALID_ARG),
    (dict(E=1025, k=2), B.MOE_ERR_INVALID_ARG), (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(H=250), B.MOE_ERR_INVALID_ARG), (dict(I=100), B.MOE_ERR_INVALID_ARG),
    (dict(I_shared=8), B.MOE_ERR_INVALID_ARG), (dict(latent=40), B.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=2), B.MOE_ERR_UNSUPPORTED), (dict(act_dtype=0, expert_dtype=2),
                                                  B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=0, expert_dtype=1), B.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=2, flags=B.PATH_STREAM), B.MOE_OK),
    (dict(expert_dtype=2, latent=64, flags=B.PATH_STREAM), B.MOE_OK),
    (dict(act_dtype=0, expert_dtype=0, flags=B.PATH_STREAM), B.MOE_ERR_UNSUPPORTED),
    (dict(flags=3), B.MOE_ERR_INVALID_ARG), (dict(flags=64), B.MOE_ERR_INVALID_ARG),
    # block-scaled experts: bf16 activations, whole 32-blocks, decode path only
    (dict(expert_dtype=B.MOE_MXFP4, flags=B.PATH_STREAM), B.MOE_OK),
    (dict(expert_dtype=B.MOE_MXFP8), B.MOE_OK),
    (dict(expert_dtype=B.MOE_MXFP4, latent=64, flags=B.PATH_STREAM), B.MOE_OK),
    (dict(expert_dtype=B.MOE_MXFP4, flags=B.PATH_GROUPED), B.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=B.MOE_MXFP8, act_dtype=0), B.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=B.MOE_MXFP4, I=144), B.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype=B.MOE_MXFP8, H=272), B.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype=B.MOE_MXFP4, latent=48), B.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype=5), B.MOE_ERR_UNSUPPORTED),
])
def test_descriptor_validation(kw, code):
    assert ws_size(desc(**kw))[0] == code


def test_workspace_grows_with_tokens_and_path():
    a = ws_size(desc(T=64))[1]
    b = ws_size(desc(T=640))[1]
    assert 0 < a < b
    s = ws_size(desc(T=64, flags=B.PATH_STREAM))[1]
    g = ws_size(desc(T=64, flags=B.PATH_GROUPED))[1]
    assert s > 0 and g > 0
    assert ws_size(desc(T=0))[0] == 0
    # block-scaled experts take the stream path whatever the load
    for dt in (B.MOE_MXFP4, B.MOE_MXFP8):
        big = dict(T=6400, expert_dtype=dt)
        assert ws_size(desc(**big)) == ws_size(desc(**big, flags=B.PATH_STREAM))


def forward(d, w=None, y=FAKE, ws=FAKE, ws_bytes=1 << 40, r=None, latent=False):
    if w is None:
        w = B.MoeWeights()
        for n, _ in B.MoeWeights._fields_:
            setattr(w, n, FAKE.value)
    fn = moe.lib().latent_moe_forward if latent else moe.lib().moe_layer_forward
    return fn(C.byref(d), C.byref(w), y, ws, ws_bytes, C.byref(r) if r else None, None)


def test_forward_argument_errors_are_reported_before_launch():
    assert forward(desc(k=0)) == B.MOE_ERR_INVALID_ARG
    assert forward(desc(), y=None) == B.MOE_ERR_INVALID_ARG
    assert forward(desc(), y=C.c_void_p(0x10004)) == B.MOE_ERR_INVALID_ARG   # misaligned
    assert forward(desc(), ws=None) == B.MOE_ERR_WORKSPACE
    assert forward(desc(), ws_bytes=16) == B.MOE_ERR_WORKSPACE
    assert forward(desc(latent=64)) == B.MOE_ERR_INVALID_ARG                # latent via plain call
    assert forward(desc(), latent=True) == B.MOE_ERR_INVALID_ARG            # plain via latent call
    w = B.MoeWeights()
    for n, _ in B.MoeWeights._fields_:
        setattr(w, n, FAKE.value)
    w.W_up = None
    assert forward(desc(), w=w) == B.MOE_ERR_INVALID_ARG
    w.W_up = FAKE.value
    w.Ws_up = None
    assert forward(desc(I_shared=64), w=w) == B.MOE_ERR_INVALID_ARG
    w.Ws_up = FAKE.value
    w.s_up = None
    assert forward(desc(expert_dtype=2), w=w) == B.MOE_ERR_INVALID_ARG
    assert forward(desc(expert_dtype=B.MOE_MXFP4), w=w) == B.MOE_ERR_INVALID_ARG
    assert forward(desc(flags=B.ROUTING_GIVEN)) == B.MOE_ERR_INVALID_ARG   # given but no record
    assert forward(desc(T=0)) == B.MOE_OK                                 # empty: no-op


def test_bias_update_argument_errors():
    L = moe.lib()
    assert L.moe_bias_update(FAKE, None, 0, 1e-3, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(None, None, 8, 1e-3, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(FAKE, None, 8, 1e-3, None, None) == B.MOE_ERR_INVALID_ARG


def test_route_and_dispatch_argument_errors():
    L = moe.lib()
    assert L.moe_route(None, FAKE, FAKE, FAKE, 4, 64, 8, 0, 1, FAKE, FAKE, FAKE, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, FAKE, FAKE, FAKE, 4, 64, 8, 2, 1, FAKE, FAKE, None, None) == \
        B.MOE_ERR_INVALID_ARG                                    # x given but no logits_out
    assert L.moe_route(None, FAKE, FAKE, FAKE, 4, 64, 8, 2, 2, FAKE, FAKE, FAKE, None) == \
        B.MOE_ERR_UNSUPPORTED
    assert L.moe_route(FAKE, None, None, FAKE, 0, 0, 8, 2, 0, FAKE, FAKE, None, None) == B.MOE_OK
    n = C.c_size_t(0)
    assert L.moe_dispatch_workspace_size(300, 16, 2, C.byref(n)) == B.MOE_OK
    assert n.value == 2 * 2 * 16 * 4                             # two [ceil(300/256), E] int tables
    assert L.moe_dispatch_workspace_size(4096, 512, 24, C.byref(n)) == B.MOE_OK
    assert n.value == 2 * 64 * 512 * 4                           # 24 slots: chunks of 64 tokens
    # chunks halve while they hold more than 2048 pairs and the call keeps at most 128 chunks
    for T, k, chunk in ((16384, 6, 256), (8192, 6, 256), (3000, 12, 128), (1000, 64, 64),
                        (32768, 24, 256), (9000, 24, 128)):
        assert L.moe_dispatch_workspace_size(T, 64, k, C.byref(n)) == B.MOE_OK
        assert n.value == 2 * -(-T // chunk) * 64 * 4, (T, k, chunk)
    assert L.moe_dispatch(FAKE, 300, 16, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == \
        B.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(FAKE, 300, 16, 17, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == \
        B.MOE_ERR_INVALID_ARG


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert moe.status_str(code) and moe.status_str(code) != "unknown status"
    assert moe.status_str(7) == "unknown status"


def bwd_ws(d):
    n = C.c_size_t(0)
    rc = moe.lib().moe_backward_workspace_size(C.byref(d), C.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(), B.MOE_OK), (dict(I_shared=64), B.MOE_OK), (dict(T=0), B.MOE_OK),
    (dict(act_dtype=0, expert_dtype=0), B.MOE_ERR_UNSUPPORTED),     # fp32 layer
    (dict(expert_dtype=2), B.MOE_ERR_UNSUPPORTED),                  # e4m3 experts
    (dict(expert_dtype=B.MOE_MXFP4), B.MOE_ERR_UNSUPPORTED),
    (dict(latent=64), B.MOE_OK), (dict(latent=40), B.MOE_ERR_INVALID_ARG),
    (dict(latent=64, expert_dtype=2), B.MOE_ERR_UNSUPPORTED),
    (dict(flags=B.ROUTING_GIVEN), B.MOE_ERR_UNSUPPORTED),
    (dict(flags=64), B.MOE_ERR_INVALID_ARG), (dict(k=0), B.MOE_ERR_INVALID_ARG),
    (dict(H=250), B.MOE_ERR_INVALID_ARG),
])
def test_backward_descriptor_validation(kw, code):
    assert bwd_ws(desc(**kw))[0] == code


NANO = dict(H=2688, E=128, k=6, I=1856, I_shared=3712)


def test_operands_over_2_gib_are_rejected():
    # The matrix-core GEMMs address operands with 32-bit offsets. At Nano width, 100,000 tokens
    # give a bf16 h of 100000 * 6 * 1856 * 2 = 2.23e9 bytes, over 2^31 - 1; e4m3 experts keep h
    # in one byte per element (1.11e9), inside the limit; the fp32 layer's kernels use 64-bit
    # addressing and take any size.
    assert ws_size(desc(T=8192, **NANO))[0] == B.MOE_OK
    assert ws_size(desc(T=100000, **NANO))[0] == B.MOE_ERR_INVALID_ARG
    assert ws_size(desc(T=100000, expert_dtype=2, **NANO))[0] == B.MOE_OK
    assert ws_size(desc(T=100000, act_dtype=0, expert_dtype=0, **NANO))[0] == B.MOE_OK
    # x alone: T * H * 2 over the limit with small experts
    assert ws_size(desc(T=(1 << 30) // 2688 + 1, H=2688, E=8, k=1, I=16))[0] == \
        B.MOE_ERR_INVALID_ARG
    assert ws_size(desc(T=(1 << 30) // 2688, H=2688, E=8, k=1, I=16))[0] == B.MOE_OK
    # one expert's weight matrix over the limit
    assert ws_size(desc(T=64, H=32768, E=8, k=2, I=32768 + 16))[0] == B.MOE_ERR_INVALID_ARG
    # backward: the pair rows [T*k, H] in bf16 (80,000 * 6 * 2688 * 2 = 2.58e9) over the limit
    # while the forward's h (1.78e9) is inside it
    assert ws_size(desc(T=80000, **NANO))[0] == B.MOE_OK
    assert bwd_ws(desc(T=80000, **NANO))[0] == B.MOE_ERR_INVALID_ARG
    assert bwd_ws(desc(T=8192, **NANO))[0] == B.MOE_OK


def test_backward_workspace_holds_no_weight_copies():
    # the weights are read as stored (K-major reads in LDS): the workspace scales with the tokens
    # and holds no copy of the expert stacks
    rc, n = bwd_ws(desc(T=64, H=256, E=16, I=128))
    assert rc == 0 and n < 16 * 256 * 128 * 2
    big = bwd_ws(desc(T=64, H=256, E=16, I=1280))[1]
    assert big < 16 * 256 * 1280 * 2
    assert bwd_ws(desc(T=640))[1] > n
    assert bwd_ws(desc(I_shared=64))[1] > n


def test_backward_argument_errors_are_reported_before_launch():
    L = moe.lib()
    w = B.MoeWeights()
    for n, _ in B.MoeWeights._fields_:
        setattr(w, n, FAKE.value)
    g = B.MoeGrads()
    for n, _ in B.MoeGrads._fields_:
        setattr(g, n, FAKE.value)

    def call(d=None, w=w, dy=FAKE, g=g, ws=FAKE, ws_bytes=1 << 40):
        d = d if d is not None else desc()
        return L.moe_layer_backward(C.byref(d), C.byref(w), dy, C.byref(g) if g else None, ws,
                                    ws_bytes, None)

    assert call(dy=None) == B.MOE_ERR_INVALID_ARG
    assert call(g=None) == B.MOE_ERR_INVALID_ARG
    assert call(dy=C.c_void_p(0x10008)) == B.MOE_ERR_INVALID_ARG      # misaligned
    assert call(ws=None) == B.MOE_ERR_WORKSPACE
    assert call(ws_bytes=16) == B.MOE_ERR_WORKSPACE
    g.dW_in = None
    assert call(desc(latent=64)) == B.MOE_ERR_INVALID_ARG      # dW_in missing
    g.dW_in = FAKE.value
    w.W_out = None
    assert call(desc(latent=64)) == B.MOE_ERR_INVALID_ARG      # W_out missing
    w.W_out = FAKE.value
    g.dW_in = None
    g.dW_up = None
    assert call() == B.MOE_ERR_INVALID_ARG
    g.dW_up = FAKE.value
    g.dWs_up = None
    assert call(desc(I_shared=64)) == B.MOE_ERR_INVALID_ARG
    assert call(desc(T=0)) == B.MOE_OK                                 # empty: no-op


def test_training_forward_and_saved_flag_validation():
    L = moe.lib()
    assert bwd_ws(desc(flags=B.SAVED_IN_WORKSPACE))[0] == B.MOE_OK
    assert ws_size(desc(flags=B.SAVED_IN_WORKSPACE))[0] == B.MOE_ERR_INVALID_ARG  # forward: no
    # bf16 weight gradients: a backward flag (same workspace), refused by the inference calls
    assert bwd_ws(desc(flags=B.WGRAD_BF16)) == bwd_ws(desc())
    assert bwd_ws(desc(flags=B.WGRAD_BF16 | B.SAVED_IN_WORKSPACE))[0] == B.MOE_OK
    assert ws_size(desc(flags=B.WGRAD_BF16))[0] == B.MOE_ERR_INVALID_ARG
    assert bwd_ws(desc(flags=32))[0] == B.MOE_ERR_INVALID_ARG         # unknown bit
    w = B.MoeWeights()
    for n, _ in B.MoeWeights._fields_:
        setattr(w, n, FAKE.value)

    def ft(d=None, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
        d = d if d is not None else desc()
        return L.moe_layer_forward_train(C.byref(d), C.byref(w), y, ws, ws_bytes, None)

    assert ft(y=None) == B.MOE_ERR_INVALID_ARG
    assert ft(desc(flags=B.SAVED_IN_WORKSPACE)) == B.MOE_ERR_INVALID_ARG
    assert ft(ws_bytes=16) == B.MOE_ERR_WORKSPACE
    assert ft(desc(latent=64, expert_dtype=2)) == B.MOE_ERR_UNSUPPORTED
    assert ft(desc(T=0)) == B.MOE_OK


def test_binding_rejects_tensors_that_do_not_match_the_descriptor():
    # the library sees only pointers: the binding checks shapes, dtypes and devices first
    import torch
    bf = torch.bfloat16
    T, H, E, k, I, Is = 8, 64, 4, 2, 32, 16
    x = torch.zeros(T, H, dtype=bf)
    t = dict(W_r=torch.zeros(E, H, dtype=bf), b=torch.zeros(E), W_up=torch.zeros(E, I, H, dtype=bf),
             W_down=torch.zeros(E, H, I, dtype=bf), Ws_up=torch.zeros(Is, H, dtype=bf),
             Ws_down=torch.zeros(H, Is, dtype=bf))
    d = B.make_desc(x, t["W_r"], t["W_up"], k, t["Ws_up"])
    B.check_shapes(d, x, **t)                                   # consistent: no error
    bad = [("W_down", torch.zeros(E, I, H, dtype=bf)),          # transposed expert stack
           ("W_r", torch.zeros(E, H)),                          # fp32 router with bf16 x
           ("b", torch.zeros(E + 1)),
           ("Ws_down", torch.zeros(Is, H, dtype=bf)),
           ("Ws_up", None)]
    for name, v in bad:
        with pytest.raises(ValueError):
            B.check_shapes(d, x, **dict(t, **{name: v}))
    # 4-bit experts: two elements per byte, one scale byte per 32 along K
    u8 = torch.uint8
    mx = dict(W_r=t["W_r"], b=t["b"], W_up=torch.zeros(E, I, H // 2, dtype=u8),
              W_down=torch.zeros(E, H, I // 2, dtype=u8), s_up=torch.zeros(E, I, H // 32, dtype=u8),
              s_down=torch.zeros(E, H, I // 32, dtype=u8))
    dm = B.make_desc(x, mx["W_r"], mx["W_up"], k, s_up=mx["s_up"])
    assert dm.expert_dtype == B.MOE_MXFP4
    B.check_shapes(dm, x, **mx)
    with pytest.raises(ValueError):
        B.check_shapes(dm, x, **dict(mx, s_down=torch.zeros(E, H, I // 16, dtype=u8)))
