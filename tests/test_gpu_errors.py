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


def test_state_init_on_gpu(bufs):
    st = bufs["state"]
    assert lt.lib.lightning_state_init(_ptr(st, 4), 1, 2, 128, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(_ptr(st), 0, 2, 128, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(_ptr(st), 1, 2, 128, None, None) == lt.LT_OK
    torch.cuda.synchronize()
    assert int(st[: 2 * 128 * 128 * 4].count_nonzero()) == 0
