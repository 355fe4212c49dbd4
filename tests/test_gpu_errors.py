"""Argument validation of the C ABI on a GPU, with real device buffers.

Each case starts from a valid call (every buffer allocated, padded and in bounds) and changes one
argument to an invalid value; the library must reject it before launching.  Only cases whose
wrong acceptance would still run an in-bounds kernel are used here (bad sizes of the workspace
are passed with a buffer that is physically large enough, misaligned pointers point into padded
buffers); the null-pointer cases are covered without a GPU in tests/test_abi.py, through the same
host code.
"""
import ctypes as ct

import pytest
import torch

lt = pytest.importorskip("long_context_hybrid_amd.lightning")

pytestmark = pytest.mark.gpu

PAD = 4096  # bytes of slack behind every buffer


@pytest.fixture(scope="module")
def bufs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    B, T, H, d = 1, 256, 2, 128
    n = B * T * H * d

    def raw(nbytes):
        return torch.zeros(nbytes + PAD, dtype=torch.uint8, device=dev)

    b = dict(B=B, T=T, H=H, d=d)
    for name in ("q", "k", "v", "g", "y"):
        b[name] = raw(n * 2)
    b["qw"] = torch.ones(H * d + PAD // 4, dtype=torch.float32, device=dev)
    b["kw"] = torch.ones(H * d + PAD // 4, dtype=torch.float32, device=dev)
    b["state"] = raw(B * H * d * d * 4)
    b["ws"] = raw(64 << 20)  # physically large enough for any plan of this shape
    b["positions"] = torch.zeros(64, dtype=torch.int64, device=dev)
    return b


def _ptr(t, off=0):
    return ct.c_void_p(t.data_ptr() + off)


def _prefill(b, **over):
    H = over.pop("H", b["H"])
    lam = over.pop("lam", [0.9] * H)
    a = dict(q=_ptr(b["q"]), k=_ptr(b["k"]), v=_ptr(b["v"]), g=_ptr(b["g"]), qw=_ptr(b["qw"]),
             kw=_ptr(b["kw"]), ow=None, stride=b["d"], lam=(ct.c_double * len(lam))(*lam),
             base=1e6, eps=1e-6, pos0=0, sin=None, sout=_ptr(b["state"]), y=_ptr(b["y"]),
             oraw=None, B=b["B"], T=b["T"], H=H, d=b["d"], dt=lt.LT_BF16, chunk=0, seg=0,
             ws=_ptr(b["ws"]), wsb=64 << 20, ev=None, stream=None)
    a.update(over)
    st = lt.lib.lightning_prefill(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                  a["stride"], a["lam"], a["base"], a["eps"], a["pos0"], a["sin"],
                                  a["sout"], a["y"], a["oraw"], a["B"], a["T"], a["H"], a["d"],
                                  a["dt"], a["chunk"], a["seg"], a["ws"], a["wsb"], a["ev"],
                                  a["stream"])
    torch.cuda.synchronize()
    return st


def test_valid_prefill_call_succeeds(bufs):
    assert _prefill(bufs) == lt.LT_OK
    assert _prefill(bufs, seg=4) == lt.LT_OK


PREFILL_BAD = [
    ("misaligned_k", lambda b: dict(k=_ptr(b["k"], 2)), lt.LT_ERR_INVALID_ARG),
    ("misaligned_y", lambda b: dict(y=_ptr(b["y"], 8)), lt.LT_ERR_INVALID_ARG),
    ("misaligned_state_out", lambda b: dict(sout=_ptr(b["state"], 4)), lt.LT_ERR_INVALID_ARG),
    ("zero_T", lambda b: dict(T=0), lt.LT_ERR_INVALID_ARG),
    ("zero_B", lambda b: dict(B=0), lt.LT_ERR_INVALID_ARG),
    ("bad_dtype", lambda b: dict(dt=7), lt.LT_ERR_INVALID_ARG),
    ("bad_stride", lambda b: dict(stride=5), lt.LT_ERR_INVALID_ARG),
    ("lambda_above_one", lambda b: dict(lam=[0.9, 1.0000001]), lt.LT_ERR_INVALID_ARG),
    ("lambda_nan", lambda b: dict(lam=[float("nan"), 0.5]), lt.LT_ERR_INVALID_ARG),
    ("rope_base_negative", lambda b: dict(base=-1.0), lt.LT_ERR_INVALID_ARG),
    ("eps_negative", lambda b: dict(eps=-1e-6), lt.LT_ERR_INVALID_ARG),
    ("pos0_negative", lambda b: dict(pos0=-5), lt.LT_ERR_INVALID_ARG),
    ("chunk_unsupported", lambda b: dict(chunk=48), lt.LT_ERR_UNSUPPORTED),
    ("workspace_too_small", lambda b: dict(seg=4, wsb=1024), lt.LT_ERR_WORKSPACE),
    ("workspace_misaligned", lambda b: dict(seg=4, ws=_ptr(b["ws"], 8)), lt.LT_ERR_WORKSPACE),
    ("events_null_entries", lambda b: dict(ev=(ct.c_void_p * 2)(None, None)),
     lt.LT_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,over,status", PREFILL_BAD, ids=[c[0] for c in PREFILL_BAD])
def test_prefill_rejects_on_gpu(bufs, name, over, status):
    assert _prefill(bufs, **over(bufs)) == status
    # the rejected call launched nothing that broke the context: a valid call still works
    assert _prefill(bufs) == lt.LT_OK


def _decode(b, **over):
    lam = over.pop("lam", [0.9, 0.99])
    a = dict(q=_ptr(b["q"]), k=_ptr(b["k"]), v=_ptr(b["v"]), g=_ptr(b["g"]), qw=_ptr(b["qw"]),
             kw=_ptr(b["kw"]), ow=None, stride=b["d"], lam=(ct.c_double * 2)(*lam), base=1e6,
             eps=1e-6, pos=_ptr(b["positions"]), sin=_ptr(b["state"]), sout=_ptr(b["state"]),
             y=_ptr(b["y"]), oraw=None, B=1, H=2, d=b["d"], dt=lt.LT_BF16, stream=None)
    a.update(over)
    st = lt.lib.lightning_decode_step(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                      a["stride"], a["lam"], a["base"], a["eps"], a["pos"],
                                      a["sin"], a["sout"], a["y"], a["oraw"], a["B"], a["H"],
                                      a["d"], a["dt"], a["stream"])
    torch.cuda.synchronize()
    return st


DECODE_BAD = [
    ("misaligned_v", lambda b: dict(v=_ptr(b["v"], 2)), lt.LT_ERR_INVALID_ARG),
    ("misaligned_state_in", lambda b: dict(sin=_ptr(b["state"], 4)), lt.LT_ERR_INVALID_ARG),
    ("zero_B", lambda b: dict(B=0), lt.LT_ERR_INVALID_ARG),
    ("lambda_negative", lambda b: dict(lam=[-0.5, 0.5]), lt.LT_ERR_INVALID_ARG),
    ("eps_nan", lambda b: dict(eps=float("nan")), lt.LT_ERR_INVALID_ARG),
    ("rope_base_zero", lambda b: dict(base=0.0), lt.LT_ERR_INVALID_ARG),
]


def test_valid_decode_call_succeeds(bufs):
    assert _decode(bufs) == lt.LT_OK


@pytest.mark.parametrize("name,over,status", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_rejects_on_gpu(bufs, name, over, status):
    assert _decode(bufs, **over(bufs)) == status
    assert _decode(bufs) == lt.LT_OK


def test_state_init_rectangular_copy_and_zero():
    """dk != dv: the fill covers B H dk dv values exactly."""
    dev = torch.device("cuda")
    init = torch.randn(2, 3, 64, 128, device=dev)
    st = torch.full((2 * 3 * 64 * 128 + 64,), 7.0, device=dev)
    view = st[: init.numel()].view(init.shape)
    lt.lightning_state_init(view, init)
    torch.cuda.synchronize()
    assert torch.equal(view, init)
    assert bool((st[init.numel():] == 7.0).all())  # nothing past the end is written
    lt.lightning_state_init(view)
    torch.cuda.synchronize()
    assert int(view.count_nonzero()) == 0 and bool((st[init.numel():] == 7.0).all())


def test_state_init_on_gpu(bufs):
    st = bufs["state"]
    assert lt.lib.lightning_state_init(_ptr(st, 4), 1, 2, 128, 128, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(_ptr(st), 0, 2, 128, 128, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(_ptr(st), 1, 2, 128, 128, None, None) == lt.LT_OK
    torch.cuda.synchronize()
    assert int(st[: 2 * 128 * 128 * 4].count_nonzero()) == 0


def test_prefill_workspace_missing_on_gpu(bufs):
    assert _prefill(bufs, seg=4, ws=None, wsb=0) == lt.LT_ERR_WORKSPACE
    assert _prefill(bufs) == lt.LT_OK


def test_size_queries_on_the_device(bufs):
    """The device-dependent size queries agree with the explicit-CU planner for this device's
    compute-unit count, and the layer's workspace is projections | y | mixer slots."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, T, H, d, dm = 1, 524288, 16, 128, 2048
    pl = lt.lightning_prefill_plan_cus(cus, B, T, H, d)
    assert lt.lightning_prefill_plan(B, T, H, d) == (pl["chunk"], pl["segments"],
                                                     pl["segment_len"])
    mix = lt.lightning_prefill_workspace_size(B, T, H, d)
    assert mix == pl["workspace_bytes"]
    assert lt.lightning_prefill_dd_workspace_size(B, T, H, d) == pl["dd_workspace_bytes"]
    bp = lt.lightning_prefill_plan_cus(cus, 8, 16384, 16, d)
    assert lt.lightning_prefill_backward_workspace_size(8, 16384, 16, d) == \
        bp["backward_workspace_bytes"]
    expect = T * 4 * H * d * 2 + T * H * d * 2 + (mix + 255) // 256 * 256
    assert lt.lightning_layer_prefill_workspace_size(B, T, H, d, dm) == expect


def test_backward_workspace_boundary_on_gpu(bufs):
    """One byte below the reported size is rejected before anything is enqueued (the layout the
    size query reports is the one the call checks, score tiles included)."""
    B, T, H, d = bufs["B"], bufs["T"], bufs["H"], bufs["d"]
    need = lt.lightning_prefill_backward_workspace_size(B, T, H, d)
    assert 0 < need <= 64 << 20
    lam = (ct.c_double * H)(*([0.9] * H))
    p = {n: _ptr(bufs[n]) for n in ("q", "k", "v", "g", "qw", "kw", "y")}

    def call(wsb):
        st = lt.lib.lightning_prefill_backward(
            p["q"], p["k"], p["v"], p["g"], p["qw"], p["kw"], None, d, lam, 1e6, 1e-6, 0, None,
            p["y"], None, p["q"], p["k"], p["v"], p["g"], None, None, None, None, B, T, H, d,
            lt.LT_BF16, 0, _ptr(bufs["ws"]), wsb, None, None)
        torch.cuda.synchronize()
        return st

    # (the gradients are written over the inputs' buffers here: only the status matters)
    assert call(need - 1) == lt.LT_ERR_WORKSPACE
    assert call(0) == lt.LT_ERR_WORKSPACE


def test_layer_workspace_checks_on_gpu():
    dev = torch.device("cuda:0")
    B, T, H, d, dm = 1, 256, 2, 128, 256
    x = torch.zeros((B, T, dm), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((4 * H * d, dm), dtype=torch.bfloat16, device=dev)
    wo = torch.zeros((dm, H * d), dtype=torch.bfloat16, device=dev)
    qw = torch.ones((H, d), dtype=torch.float32, device=dev)
    out = torch.zeros((B, T, dm), dtype=torch.bfloat16, device=dev)
    need = lt.lightning_layer_prefill_workspace_size(B, T, H, d, dm)
    ws = torch.empty(need + 512, dtype=torch.uint8, device=dev)
    lam = (ct.c_double * H)(0.9, 0.99)

    def call(wsp, wsb):
        st = lt.lib.lightning_layer_prefill(_ptr(x), _ptr(w), _ptr(wo), _ptr(qw), _ptr(qw), None,
                                            d, lam, 1e6, 1e-6, 0, None, None, _ptr(out), B, T, H,
                                            d, dm, lt.LT_BF16, 0, 0, wsp, wsb, None, None)
        torch.cuda.synchronize()
        return st

    assert call(None, 0) == lt.LT_ERR_WORKSPACE
    assert call(_ptr(ws), need - 1) == lt.LT_ERR_WORKSPACE
    assert call(_ptr(ws, 16), need) == lt.LT_ERR_WORKSPACE  # not 256-byte aligned
    assert call(_ptr(ws), need) == lt.LT_OK


# ---- the error path of a failing launch (LT_FORCE_FAIL) --------------------------------------------

SENT = 7.0


def _force_fail_cases():
    """name -> (outputs, call): `outputs` are sentinel-filled tensors the call writes, `call()`
    makes one valid call through the binding."""
    import synth

    dev = torch.device("cuda:0")
    pre = synth.make_custom_prefill(1, 300, 2, 128, dtype=torch.bfloat16, seed=11)
    pin = {n: pre[n].to(dev) for n in ("q", "k", "v", "g", "qw", "kw")}
    dec = synth.make_decode(synth.DECODE_B64, device=dev, B=2)
    lay = synth.make_custom_layer(1, 64, 2, 128, 256, dtype=torch.bfloat16, seed=12)
    lin = {n: (lay[n].to(dev) if torch.is_tensor(lay[n]) else lay[n]) for n in lay}
    att = synth.make_custom_attn(1, 64, 4, 2, seed=13)
    ain = {n: (att[n].to(dev) if torch.is_tensor(att[n]) else att[n]) for n in att}

    def full(shape, dtype=torch.float32):
        return torch.full(shape, SENT, dtype=dtype, device=dev)

    cases = {}
    y, s = full(pin["q"].shape, torch.bfloat16), full((1, 2, 128, 128))
    cases["prefill"] = ([y, s], lambda y=y, s=s: lt.lightning_prefill(
        pin["q"], pin["k"], pin["v"], pin["g"], pin["qw"], pin["kw"], pre["lambdas"],
        pre["rope_base"], state_out=s, y=y, segments=2))
    y = full(pin["q"].shape, torch.bfloat16)
    l2 = torch.full((1, 300, 2), -0.01, dtype=torch.float32, device=dev)
    cases["prefill_dd"] = ([y], lambda y=y: lt.lightning_prefill_dd(
        pin["q"], pin["k"], pin["v"], pin["g"], pin["qw"], pin["kw"], l2, pre["rope_base"], y=y,
        segments=2))
    y, s = full(dec["q"].shape, torch.bfloat16), full(dec["state_in"].shape)
    cases["decode_step"] = ([y, s], lambda y=y, s=s: lt.lightning_decode_step(
        dec["q"], dec["k"], dec["v"], dec["g"], dec["qw"], dec["kw"], dec["lambdas"],
        dec["rope_base"], dec["positions"], dec["state_in"], state_out=s, y=y))
    y, s = full(dec["q"].shape, torch.bfloat16), full(dec["state_in"].shape)
    l2d = torch.full((2, dec["H"]), -0.01, dtype=torch.float32, device=dev)
    cases["decode_step_dd"] = ([y, s], lambda y=y, s=s: lt.lightning_decode_step_dd(
        dec["q"], dec["k"], dec["v"], dec["g"], dec["qw"], dec["kw"], l2d, dec["rope_base"],
        dec["positions"], dec["state_in"], state_out=s, y=y))
    s = full((1, 2, 128, 128))
    cases["state_init"] = ([s], lambda s=s: lt.lightning_state_init(s))
    ws = full((lt.lightning_prefill_backward_workspace_size(1, 300, 2, 128),), torch.uint8)
    cases["prefill_backward"] = ([ws], lambda ws=ws: lt.lightning_prefill_backward(
        pin["q"], pin["k"], pin["v"], pin["g"], pin["qw"], pin["kw"], pre["lambdas"],
        pre["rope_base"], pin["v"], workspace=ws))
    out = full(lin["x"].shape, torch.bfloat16)
    cases["layer_prefill"] = ([out], lambda out=out: lt.lightning_layer_prefill(
        lin["x"], lin["w_qkvz"], lin["w_o"], lin["qw"], lin["kw"], lin["lambdas"],
        lin["rope_base"], lin["H"], lin["d"], out=out))
    x1 = lin["x"][:, 0].contiguous()
    out, s = full(x1.shape, torch.bfloat16), full((1, 2, 128, 128))
    pos = torch.zeros(1, dtype=torch.int64, device=dev)
    s_in = torch.zeros((1, 2, 128, 128), device=dev)
    cases["layer_decode_step"] = ([out, s], lambda out=out, s=s: lt.lightning_layer_decode_step(
        x1, lin["w_qkvz"], lin["w_o"], lin["qw"], lin["kw"], lin["lambdas"], lin["rope_base"],
        lin["H"], lin["d"], pos, s_in, state_out=s, out=out))
    y = full(ain["q"].shape, torch.bfloat16)
    cases["attn_prefill"] = ([y], lambda y=y: lt.lightning_attn_prefill(
        ain["q"], ain["k"], ain["v"], ain["g"], ain["a"], q_norm_w=ain["qw"], k_norm_w=ain["kw"],
        y=y))
    q1, g1 = ain["q"][:, 0].contiguous(), ain["g"][:, 0].contiguous()
    k1, v1 = ain["k"][:, 0].contiguous(), ain["v"][:, 0].contiguous()
    kc, vc = full((1, 16, 2, 128), torch.bfloat16), full((1, 16, 2, 128), torch.bfloat16)
    y = full(q1.shape, torch.bfloat16)
    cases["attn_decode_step"] = ([y, kc, vc], lambda y=y, kc=kc, vc=vc: lt.lightning_attn_decode_step(
        q1, k1, v1, g1, kc, vc, [3], ain["a"], q_norm_w=ain["qw"], k_norm_w=ain["kw"], y=y))
    kc, vc = full((1, 16, 2, 128), torch.bfloat16), full((1, 16, 2, 128), torch.bfloat16)
    y = full(q1.shape, torch.bfloat16)
    lens = torch.full((1,), 3, dtype=torch.int64, device=dev)
    cases["attn_decode_step_dev"] = ([y, kc, vc], lambda y=y, kc=kc, vc=vc: lt.lightning_attn_decode_step(
        q1, k1, v1, g1, kc, vc, lens, ain["a"], q_norm_w=ain["qw"], k_norm_w=ain["kw"], y=y))
    return cases


FORCE_FAIL_NAMES = ["state_init", "prefill", "decode_step", "prefill_dd", "decode_step_dd",
                    "prefill_backward", "layer_prefill", "layer_decode_step", "attn_prefill",
                    "attn_decode_step", "attn_decode_step_dev"]


@pytest.mark.parametrize("name", FORCE_FAIL_NAMES)
def test_forced_launch_failure_is_reported(name, monkeypatch):
    """With LT_FORCE_FAIL set every entry point returns LT_ERR_HIP after its argument checks and
    enqueues nothing: every output keeps its sentinel.  With it cleared the same call succeeds
    and writes them."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    outs, call = _force_fail_cases()[name]
    before = [t.clone() for t in outs]
    monkeypatch.setenv("LT_FORCE_FAIL", "1")
    with pytest.raises(lt.LightningError) as e:
        call()
    torch.cuda.synchronize()
    assert e.value.status == lt.LT_ERR_HIP
    for t, b in zip(outs, before):
        assert torch.equal(t, b), "a forced launch failure wrote an output"
    monkeypatch.setenv("LT_FORCE_FAIL", "0")
    call()
    torch.cuda.synchronize()
    assert any(not torch.equal(t, b) for t, b in zip(outs, before)), "the valid call wrote nothing"
