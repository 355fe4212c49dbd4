"""The C-ABI library on the host: it loads, exports what include/lightning.h declares, and its
host-only logic (the Eq. 19 helper, the plan, argument validation) behaves.  No GPU needed.

The validation cases pass fake (but 16-byte aligned) device addresses together with exactly one
invalid argument, so a call that wrongly passed validation would try to launch.  They therefore
run only where no GPU is visible; the same cases run on the GPU with real buffers in
tests/test_gpu_errors.py.
"""
import ctypes as ct
import math
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "hypenet_gamma_h32.txt")

lt = pytest.importorskip("long_context_hybrid_amd.lightning")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lightning_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(lt.EXPORTS)


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    assert hasattr(lt.lib, name), f"liblightning.so does not export {name}"


def test_status_strings():
    for code in range(5):
        s = lt.lightning_status_string(code)
        assert s.startswith("LT_")
    assert "unknown" in lt.lightning_status_string(99)


def _golden_gamma():
    vals = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            vals.append(float(line))
    return vals


def test_hypenet_gamma_matches_printed_values():
    printed = _golden_gamma()
    assert len(printed) == 32
    got = lt.lightning_hypenet_gamma(32)
    for h, (g, ref) in enumerate(zip(got, printed), start=1):
        assert abs(g - ref) <= 1e-7, f"gamma_{h}: {g} vs printed {ref}"


def test_hypenet_gamma_time_scales():
    # tau_h = 1 / -ln(gamma_h) = 2^(8h/H); the slowest head has tau = 256 tokens, and its
    # decay over 4096 tokens is e^-16 ~ 1.13e-7.
    for H in (16, 32):
        g = lt.lightning_hypenet_gamma(H)
        for h, gh in enumerate(g, start=1):
            assert 0.0 < gh < 1.0
            assert math.isclose(1.0 / -math.log(gh), 2.0 ** (8.0 * h / H), rel_tol=1e-12)
        assert math.isclose(g[-1], math.exp(-1.0 / 256.0), rel_tol=1e-15)
        assert math.isclose(g[-1] ** 4096, 1.13e-7, rel_tol=1e-2)
    with pytest.raises(lt.LightningError):
        lt.lightning_hypenet_gamma(0)


@pytest.mark.parametrize("B,T,H,d,expect_p,expect_sub", [
    (1, 524288, 16, 128, 16, 2),   # 512K-token layer: one segment per CU, state-only pass 2 per CU
    (1, 32768, 16, 128, 16, 2),
    (4, 131072, 32, 128, 2, 4),
    (64, 4096, 16, 128, 1, 1),      # B*H already fills the CUs
    (1, 256, 2, 64, 1, 1),          # too short to split (8 chunks)
    (1, 300, 1, 128, 1, 1),
    (1, 4096, 1, 128, 16, 1),       # 128 chunks, 8 per segment: no further split
    (2, 100000, 2, 64, 64, 2),      # 3125 chunks over 64 segments of 49 (sub-segments 25 + 24)
])
def test_plan_and_workspace(B, T, H, d, expect_p, expect_sub):
    pl = lt.lightning_prefill_plan_cus(256, B, T, H, d)
    p, seg_len = pl["segments"], pl["segment_len"]
    assert pl["chunk"] == 32 and p == expect_p
    # every segment but the last has seg_len tokens (a whole number of chunks); the last is
    # non-empty and no longer; one segment is the whole sequence
    if p > 1:
        assert seg_len % 32 == 0 and 0 < T - (p - 1) * seg_len <= seg_len
        assert pl["state_subsegments"] == expect_sub
    else:
        assert seg_len == T and pl["state_subsegments"] == 0
    # one fp32 d x d state per state-only sub-segment of segments 0 .. P-2, plus the entry state
    # of the last segment
    slots = (p - 1) * expect_sub + 1
    assert pl["workspace_bytes"] == (B * H * slots * d * d * 4 if p > 1 else 0)


@pytest.mark.parametrize("cus,B,T,H,expect_p,expect_sub,expect_len", [
    # 512K tokens, 16 heads on 32 CUs: two segments; the bf16 last segment is made shorter
    # (8533 + 7851 chunks), and each state-only segment is cut in four (4 x 16 = 64 = 2 x 32 slots)
    (32, 1, 524288, 16, 2, 4, 8533 * 32),
    # on 80 CUs: five segments of 3330 chunks (the last 3064), state-only pass in halves
    (80, 1, 524288, 16, 5, 2, 3330 * 32),
    # B*H = 128 already fills 32 or 80 CUs: no segments at all
    (32, 4, 131072, 32, 1, 0, 131072),
    (80, 4, 131072, 32, 1, 0, 131072),
    # 128 chunks of one head: the eight-chunk minimum caps the split at 16 segments on any device
    (32, 1, 4096, 1, 16, 1, 256),
    (80, 1, 4096, 1, 16, 1, 256),
])
def test_plan_on_other_devices(cus, B, T, H, expect_p, expect_sub, expect_len):
    pl = lt.lightning_prefill_plan_cus(cus, B, T, H, 128)
    assert (pl["segments"], pl["state_subsegments"], pl["segment_len"]) == \
        (expect_p, expect_sub, expect_len)
    if expect_p > 1:
        # the main pass gives every CU a workgroup (unless the eight-chunk minimum per segment
        # runs out first); the state-only pass stays within its two slots per CU
        assert B * H * expect_p >= min(cus, B * H * (((T + 31) // 32) // 8))
        assert B * H * (expect_p - 1) * expect_sub <= 2 * cus
    slots = (expect_p - 1) * expect_sub + 1 if expect_p > 1 else 0
    assert pl["workspace_bytes"] == B * H * slots * 128 * 128 * 4


def test_plan_needs_positive_cus():
    for cus in (0, -1):
        with pytest.raises(lt.LightningError) as e:
            lt.lightning_prefill_plan_cus(cus, 1, 1000, 2, 128)
        assert e.value.status == lt.LT_ERR_INVALID_ARG


def test_plan_explicit_segments_and_chunk():
    assert lt.lightning_prefill_plan_cus(256, 1, 1000, 2, 128, segments=3)["segments"] == 3
    # more segments than chunks collapses to one chunk per segment
    pl = lt.lightning_prefill_plan_cus(256, 1, 100, 2, 128, segments=50)
    assert (pl["chunk"], pl["segments"]) == (32, 4)
    for kw in (dict(chunk=48), dict(d=96)):
        a = dict(B=1, T=1000, H=2, d=128)
        a.update(kw)
        with pytest.raises(lt.LightningError) as e:
            lt.lightning_prefill_plan(a["B"], a["T"], a["H"], a["d"], chunk=a.get("chunk", 0))
        assert e.value.status == lt.LT_ERR_UNSUPPORTED
        with pytest.raises(lt.LightningError) as e:
            lt.lightning_prefill_plan_cus(256, a["B"], a["T"], a["H"], a["d"],
                                          chunk=a.get("chunk", 0))
        assert e.value.status == lt.LT_ERR_UNSUPPORTED
    assert lt.lightning_prefill_workspace_size(1, 1000, 2, 96) == 0


def test_plan_chunk64():
    """64-token chunks: segments are whole 64-token chunks (and state-only sub-segments too);
    fp32 with d = 128 (tiles too large for LDS) is unsupported, bf16 and fp32 d = 64 are not."""
    pl = lt.lightning_prefill_plan_cus(256, 1, 524288, 16, 128, chunk=64)
    assert pl["chunk"] == 64 and pl["segments"] > 1
    assert pl["segment_len"] % 64 == 0 and pl["subsegment_len"] % 64 == 0
    assert (pl["segments"] - 1) * pl["segment_len"] < 524288 <= pl["segments"] * pl["segment_len"]
    for dt, d in ((torch.bfloat16, 64), (torch.float32, 64), (torch.bfloat16, 128)):
        assert lt.lightning_prefill_plan_cus(256, 1, 256, 2, d, dtype=dt, chunk=64)["chunk"] == 64
    with pytest.raises(lt.LightningError) as e:
        lt.lightning_prefill_plan_cus(256, 1, 1000, 2, 128, dtype=torch.float32, chunk=64)
    assert e.value.status == lt.LT_ERR_UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the behaviour without a device")
def test_plan_without_a_device_is_a_hip_error():
    """The automatic split depends on the device's compute units: with no device visible the
    device-dependent queries report LT_ERR_HIP (or a size of 0), never a guessed plan."""
    with pytest.raises(lt.LightningError) as e:
        lt.lightning_prefill_plan(1, 524288, 16, 128)
    assert e.value.status == lt.LT_ERR_HIP
    assert lt.lightning_prefill_workspace_size(1, 524288, 16, 128) == 0
    assert lt.lightning_prefill_dd_workspace_size(1, 524288, 16, 128) == 0
    assert lt.lightning_prefill_backward_workspace_size(8, 16384, 16, 128) == 0
    assert lt.lightning_layer_prefill_workspace_size(1, 4096, 16, 128, 2048) == 0


# ---- argument validation with fake device addresses (only where no GPU is visible) ---------

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-address validation cases run only without a GPU")

FAKE = 0x10000  # 16-byte aligned, never dereferenced by a correctly rejected call


def _prefill_args(**over):
    H = over.pop("H", 2)
    lam = over.pop("lam", [0.9] * H)
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128,
             lam=(ct.c_double * len(lam))(*lam), base=1e6, eps=1e-6, pos0=0, sin=None, sout=None,
             y=FAKE, oraw=None, B=1, T=256, H=H, d=128, dt=lt.LT_BF16, chunk=0, seg=0, ws=None,
             wsb=0, ev=None, stream=None)
    a.update(over)
    return a


def _call_prefill(a):
    return lt.lib.lightning_prefill(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                    a["stride"], a["lam"], a["base"], a["eps"], a["pos0"],
                                    a["sin"], a["sout"], a["y"], a["oraw"], a["B"], a["T"],
                                    a["H"], a["d"], a["dt"], a["chunk"], a["seg"], a["ws"],
                                    a["wsb"], a["ev"], a["stream"])


PREFILL_BAD = [
    ("null_q", dict(q=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_k", dict(k=FAKE + 2), lt.LT_ERR_INVALID_ARG),
    ("null_gate", dict(g=None), lt.LT_ERR_INVALID_ARG),
    ("null_y", dict(y=None), lt.LT_ERR_INVALID_ARG),
    ("null_qnorm", dict(qw=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_state_in", dict(sin=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("zero_B", dict(B=0), lt.LT_ERR_INVALID_ARG),
    ("zero_T", dict(T=0), lt.LT_ERR_INVALID_ARG),
    ("neg_H", dict(H=-1, lam=[0.9]), lt.LT_ERR_INVALID_ARG),
    ("d_96", dict(d=96, stride=96), lt.LT_ERR_UNSUPPORTED),
    ("too_many_heads", dict(H=257), lt.LT_ERR_UNSUPPORTED),
    ("bad_dtype", dict(dt=7), lt.LT_ERR_INVALID_ARG),
    ("bad_stride", dict(stride=5), lt.LT_ERR_INVALID_ARG),
    ("lambda_above_one", dict(lam=[0.9, 1.0000001]), lt.LT_ERR_INVALID_ARG),
    ("lambda_negative", dict(lam=[-0.1, 0.5]), lt.LT_ERR_INVALID_ARG),
    ("lambda_nan", dict(lam=[float("nan"), 0.5]), lt.LT_ERR_INVALID_ARG),
    ("rope_base_zero", dict(base=0.0), lt.LT_ERR_INVALID_ARG),
    ("rope_base_inf", dict(base=float("inf")), lt.LT_ERR_INVALID_ARG),
    ("eps_negative", dict(eps=-1e-6), lt.LT_ERR_INVALID_ARG),
    ("pos0_negative", dict(pos0=-1), lt.LT_ERR_INVALID_ARG),
    ("chunk_unsupported", dict(chunk=48), lt.LT_ERR_UNSUPPORTED),
    # Every argument valid: the call then needs the device (its compute units size the plan and
    # the workspace), and without one it reports LT_ERR_HIP before anything else.  The workspace
    # checks themselves run with a device in tests/test_gpu_errors.py.
    ("no_device", dict(T=524288, H=16, lam=[0.9] * 16, ws=FAKE, wsb=1 << 40), lt.LT_ERR_HIP),
    ("no_device_workspace_missing", dict(T=524288, H=16, lam=[0.9] * 16), lt.LT_ERR_HIP),
    ("events_null_entries", dict(ev=(ct.c_void_p * 2)(None, None)), lt.LT_ERR_INVALID_ARG),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", PREFILL_BAD, ids=[c[0] for c in PREFILL_BAD])
def test_prefill_rejects(name, over, status):
    assert _call_prefill(_prefill_args(**over)) == status


DECODE_BAD = [
    ("null_positions", dict(pos=None), lt.LT_ERR_INVALID_ARG),
    ("null_state_in", dict(sin=None), lt.LT_ERR_INVALID_ARG),
    ("null_state_out", dict(sout=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_v", dict(v=FAKE + 2), lt.LT_ERR_INVALID_ARG),
    ("zero_B", dict(B=0), lt.LT_ERR_INVALID_ARG),
    ("d_32", dict(d=32, stride=32), lt.LT_ERR_UNSUPPORTED),
    ("lambda_above_one", dict(lam=[2.0, 0.5]), lt.LT_ERR_INVALID_ARG),
    ("eps_nan", dict(eps=float("nan")), lt.LT_ERR_INVALID_ARG),
    # every argument valid: the launch itself fails without a device
    ("no_device", dict(), lt.LT_ERR_HIP),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_rejects(name, over, status):
    lam = over.pop("lam", [0.9, 0.99])
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128,
             lam=(ct.c_double * 2)(*lam), base=1e6, eps=1e-6, pos=FAKE, sin=FAKE, sout=FAKE,
             y=FAKE, oraw=None, B=4, H=2, d=128, dt=lt.LT_BF16, stream=None)
    a.update(over)
    st = lt.lib.lightning_decode_step(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                      a["stride"], a["lam"], a["base"], a["eps"], a["pos"],
                                      a["sin"], a["sout"], a["y"], a["oraw"], a["B"], a["H"],
                                      a["d"], a["dt"], a["stream"])
    assert st == status


@no_gpu
def test_state_init_rejects():
    assert lt.lib.lightning_state_init(None, 1, 1, 64, 64, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(FAKE + 4, 1, 1, 64, 64, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(FAKE, 0, 1, 64, 64, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(FAKE, 1, 1, 64, 0, None, None) == lt.LT_ERR_INVALID_ARG
    assert lt.lib.lightning_state_init(FAKE, 1, 1, -2, 64, None, None) == lt.LT_ERR_INVALID_ARG


# ---- the whole layer -------------------------------------------------------------------------------

def test_layer_workspace_sizes():
    # decode step: projections and y in bf16, each part 256-byte aligned (no mixer workspace,
    # so no device is needed to size it; the projection GEMMs need no scratch)
    B, H, d, dm = 64, 16, 128, 2048
    assert lt.lightning_layer_decode_workspace_size(B, H, d, dm) == \
        B * 4 * H * d * 2 + B * H * d * 2
    f32 = lt.lightning_layer_decode_workspace_size(3, 2, 64, 64, torch.float32)
    assert f32 == (3 * 512 * 4 + 255) // 256 * 256 + (3 * 128 * 4 + 255) // 256 * 256
    assert lt.lightning_layer_prefill_workspace_size(1, 4096, H, d, 100) == 0  # d_model % 8
    assert lt.lightning_layer_prefill_workspace_size(1, 4096, H, 96, dm) == 0
    assert lt.lightning_layer_decode_workspace_size(0, H, d, dm) == 0


def _layer_args(**over):
    H = over.pop("H", 2)
    lam = over.pop("lam", [0.9] * H)
    a = dict(x=FAKE, w=FAKE, wo=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128,
             lam=(ct.c_double * len(lam))(*lam), base=1e6, eps=1e-6, pos0=0, sin=None, sout=None,
             out=FAKE, B=1, T=256, H=H, d=128, dm=256, dt=lt.LT_BF16, chunk=0, seg=0,
             ws=FAKE * 16, wsb=1 << 40, ev=None, stream=None)
    a.update(over)
    return a


LAYER_BAD = [
    ("null_x", dict(x=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_w_qkvz", dict(w=FAKE + 8), lt.LT_ERR_INVALID_ARG),
    ("null_w_o", dict(wo=None), lt.LT_ERR_INVALID_ARG),
    ("null_out", dict(out=None), lt.LT_ERR_INVALID_ARG),
    ("d_model_not_multiple_of_8", dict(dm=100), lt.LT_ERR_INVALID_ARG),
    ("zero_T", dict(T=0), lt.LT_ERR_INVALID_ARG),
    ("bad_dtype", dict(dt=3), lt.LT_ERR_INVALID_ARG),
    ("d_96", dict(d=96, stride=96), lt.LT_ERR_UNSUPPORTED),
    # valid arguments: sizing the mixer's workspace needs the device, so without one the call
    # reports LT_ERR_HIP (the workspace checks run on the GPU in tests/test_layer_gpu.py)
    ("no_device", dict(), lt.LT_ERR_HIP),
    ("no_device_workspace_missing", dict(ws=None), lt.LT_ERR_HIP),
    # mixer arguments are checked before the first GEMM is enqueued
    ("lambda_nan", dict(lam=[float("nan"), 0.5]), lt.LT_ERR_INVALID_ARG),
    ("null_qnorm", dict(qw=None), lt.LT_ERR_INVALID_ARG),
    ("rope_base_zero", dict(base=0.0), lt.LT_ERR_INVALID_ARG),
    ("misaligned_state_out", dict(sout=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("pos0_negative", dict(pos0=-3), lt.LT_ERR_INVALID_ARG),
    ("events_null_entries", dict(ev=(ct.c_void_p * 4)(FAKE, None, FAKE, FAKE)),
     lt.LT_ERR_INVALID_ARG),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", LAYER_BAD, ids=[c[0] for c in LAYER_BAD])
def test_layer_prefill_rejects(name, over, status):
    a = _layer_args(**over)
    st = lt.lib.lightning_layer_prefill(a["x"], a["w"], a["wo"], a["qw"], a["kw"], a["ow"],
                                        a["stride"], a["lam"], a["base"], a["eps"], a["pos0"],
                                        a["sin"], a["sout"], a["out"], a["B"], a["T"], a["H"],
                                        a["d"], a["dm"], a["dt"], a["chunk"], a["seg"], a["ws"],
                                        a["wsb"], a["ev"], a["stream"])
    assert st == status


LAYER_DECODE_BAD = [
    ("null_x", dict(x=None), lt.LT_ERR_INVALID_ARG),
    ("d_model_not_multiple_of_8", dict(dm=12), lt.LT_ERR_INVALID_ARG),
    ("workspace_small", dict(wsb=4096), lt.LT_ERR_WORKSPACE),
    ("null_positions", dict(pos=None), lt.LT_ERR_INVALID_ARG),
    ("null_state_in", dict(sin=None), lt.LT_ERR_INVALID_ARG),
    ("lambda_above_one", dict(lam=[1.5, 0.5]), lt.LT_ERR_INVALID_ARG),
    ("eps_negative", dict(eps=-1.0), lt.LT_ERR_INVALID_ARG),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", LAYER_DECODE_BAD,
                         ids=[c[0] for c in LAYER_DECODE_BAD])
def test_layer_decode_rejects(name, over, status):
    lam = over.pop("lam", [0.9, 0.99])
    a = dict(x=FAKE, w=FAKE, wo=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128,
             lam=(ct.c_double * 2)(*lam), base=1e6, eps=1e-6, pos=FAKE, sin=FAKE, sout=FAKE,
             out=FAKE, B=4, H=2, d=128, dm=256, dt=lt.LT_BF16, ws=FAKE * 16, wsb=1 << 40,
             stream=None)
    a.update(over)
    st = lt.lib.lightning_layer_decode_step(a["x"], a["w"], a["wo"], a["qw"], a["kw"], a["ow"],
                                            a["stride"], a["lam"], a["base"], a["eps"], a["pos"],
                                            a["sin"], a["sout"], a["out"], a["B"], a["H"], a["d"],
                                            a["dm"], a["dt"], a["ws"], a["wsb"], a["stream"])
    assert st == status


# ---- HyPE attention ---------------------------------------------------------------------------------

def test_attn_workspace_sizes():
    B, T, Hq, Hkv, d = 1, 524288, 16, 8, 128
    q_bytes = B * T * Hq * d * 2
    k_bytes = B * T * Hkv * d * 2
    assert lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, torch.bfloat16, True,
                                                    False) == q_bytes + k_bytes
    assert lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, torch.bfloat16, True,
                                                    True) == q_bytes
    assert lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, torch.bfloat16, False,
                                                    False) == q_bytes
    assert lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, 64) == 0      # d = 128 only
    assert lt.lightning_attn_prefill_workspace_size(B, T, 6, 4, d) == 0          # Hq % Hkv
    assert lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, torch.float32) == 0


ATTN_BAD = [
    ("null_q", dict(q=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_v", dict(v=FAKE + 2), lt.LT_ERR_INVALID_ARG),
    ("null_y", dict(y=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_cache", dict(cache=FAKE + 8), lt.LT_ERR_INVALID_ARG),
    ("zero_T", dict(T=0), lt.LT_ERR_INVALID_ARG),
    ("heads_not_grouped", dict(Hq=6, Hkv=4), lt.LT_ERR_INVALID_ARG),
    ("d_64", dict(d=64, stride=64), lt.LT_ERR_UNSUPPORTED),
    ("fp32", dict(dt=lt.LT_F32), lt.LT_ERR_UNSUPPORTED),
    ("bad_stride", dict(stride=7), lt.LT_ERR_INVALID_ARG),
    ("scale_base_one", dict(a=1.0), lt.LT_ERR_INVALID_ARG),
    ("scale_base_negative", dict(a=-500.0), lt.LT_ERR_INVALID_ARG),
    ("scale_base_inf", dict(a=float("inf")), lt.LT_ERR_INVALID_ARG),
    ("eps_nan", dict(eps=float("nan")), lt.LT_ERR_INVALID_ARG),
    ("pos0_negative", dict(pos0=-1), lt.LT_ERR_INVALID_ARG),
    ("workspace_missing", dict(ws=None), lt.LT_ERR_WORKSPACE),
    ("workspace_small", dict(wsb=1024), lt.LT_ERR_WORKSPACE),
    ("workspace_not_256_aligned", dict(ws=FAKE * 16 + 32), lt.LT_ERR_WORKSPACE),
    ("events_null_entries", dict(ev=(ct.c_void_p * 2)(None, FAKE)), lt.LT_ERR_INVALID_ARG),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", ATTN_BAD, ids=[c[0] for c in ATTN_BAD])
def test_attn_prefill_rejects(name, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=0, a=500.0,
             eps=1e-6, pos0=0, y=FAKE, oraw=None, cache=None, B=1, T=256, Hq=4, Hkv=2, d=128,
             dt=lt.LT_BF16, ws=FAKE * 16, wsb=1 << 40, ev=None, stream=None)
    a.update(over)
    st = lt.lib.lightning_attn_prefill(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                       a["stride"], a["a"], a["eps"], a["pos0"], a["y"],
                                       a["oraw"], a["cache"], a["B"], a["T"], a["Hq"], a["Hkv"],
                                       a["d"], a["dt"], a["ws"], a["wsb"], a["ev"], a["stream"])
    assert st == status


def _attn_decode_call(dev_lengths, **over):
    B = over.get("B", 2)
    lens = (ct.c_int64 * B)(*([3] * B))
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=0, a=500.0,
             eps=1e-6, lengths=FAKE if dev_lengths else lens, maxlen=100, kc=FAKE, vc=FAKE,
             cap=4096, y=FAKE, oraw=None, B=B, Hq=4, Hkv=2, d=128, dt=lt.LT_BF16, ws=FAKE * 16,
             wsb=1 << 40, stream=None)
    a.update(over)
    head = (a["q"], a["kn"], a["vn"], a["g"], a["qw"], a["kw"], a["ow"], a["stride"], a["a"],
            a["eps"], a["lengths"])
    tail = (a["kc"], a["vc"], a["cap"], a["y"], a["oraw"], a["B"], a["Hq"], a["Hkv"], a["d"],
            a["dt"], a["ws"], a["wsb"], a["stream"])
    if dev_lengths:
        return lt.lib.lightning_attn_decode_step_dev(*head, a["maxlen"], *tail)
    return lt.lib.lightning_attn_decode_step(*head, *tail)


ATTN_DECODE_BAD = [
    # (label, device lengths?, overrides, status)
    ("null_lengths", False, dict(lengths=None), lt.LT_ERR_INVALID_ARG),
    ("length_negative", False, dict(lengths=(ct.c_int64 * 2)(3, -1)), lt.LT_ERR_INVALID_ARG),
    ("length_at_capacity", False, dict(lengths=(ct.c_int64 * 2)(4096, 0)), lt.LT_ERR_INVALID_ARG),
    ("host_lengths_b65", False, dict(B=65), lt.LT_ERR_UNSUPPORTED),
    ("group_3", False, dict(Hq=6, Hkv=2), lt.LT_ERR_UNSUPPORTED),
    ("group_16", False, dict(Hq=16, Hkv=1), lt.LT_ERR_UNSUPPORTED),
    ("zero_capacity", False, dict(cap=0), lt.LT_ERR_INVALID_ARG),
    ("null_v_cache", False, dict(vc=None), lt.LT_ERR_INVALID_ARG),
    ("workspace_small", False, dict(wsb=256), lt.LT_ERR_WORKSPACE),
    ("dev_null_lengths", True, dict(lengths=None), lt.LT_ERR_INVALID_ARG),
    ("dev_lengths_misaligned", True, dict(lengths=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("dev_max_length_negative", True, dict(maxlen=-1), lt.LT_ERR_INVALID_ARG),
    ("dev_max_length_at_capacity", True, dict(maxlen=4096), lt.LT_ERR_INVALID_ARG),
    ("dev_group_3", True, dict(Hq=6, Hkv=2), lt.LT_ERR_UNSUPPORTED),
    ("dev_workspace_small", True, dict(wsb=256), lt.LT_ERR_WORKSPACE),
    # valid arguments (B beyond the host path's 64 rows, 8-byte aligned lengths): validation
    # passes and the launch fails for want of a device
    ("dev_b100_passes_validation", True, dict(B=100, lengths=FAKE + 8), lt.LT_ERR_HIP),
]


@no_gpu
@pytest.mark.parametrize("name,dev_lengths,over,status", ATTN_DECODE_BAD,
                         ids=[c[0] for c in ATTN_DECODE_BAD])
def test_attn_decode_rejects(name, dev_lengths, over, status):
    assert _attn_decode_call(dev_lengths, **over) == status


def test_attn_decode_workspace_follows_the_bound():
    one = lt.lightning_attn_decode_workspace_size(3, 8, 2, 128, 2047)
    two = lt.lightning_attn_decode_workspace_size(3, 8, 2, 128, 2048)
    assert one == 3 * 8 * 1 * 130 * 4 // 256 * 256 + 256 and two > one
    assert lt.lightning_attn_decode_workspace_size(3, 8, 2, 128, -1) == 0


# ---- data-dependent decay -------------------------------------------------------------------------

def test_dd_workspace_adds_subsegment_decays():
    B, T, H, d = 1, 524288, 16, 128
    pl = lt.lightning_prefill_plan_cus(256, B, T, H, d)
    base = pl["workspace_bytes"]
    slots = base // (B * H * d * d * 4)  # (P - 1) sub + 1 state slots per (b, h)
    assert slots == (pl["segments"] - 1) * pl["state_subsegments"] + 1
    expect = (base + 255) // 256 * 256 + B * H * (slots - 1) * 4
    assert pl["dd_workspace_bytes"] == expect
    assert lt.lightning_prefill_plan_cus(256, 1, 200, 2, 128)["dd_workspace_bytes"] == 0


@no_gpu
@pytest.mark.parametrize("name,over,status", [
    ("null_decay", dict(dec=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_decay", dict(dec=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("null_q", dict(q=None), lt.LT_ERR_INVALID_ARG),
    ("d_96", dict(d=96, stride=96), lt.LT_ERR_UNSUPPORTED),
    ("no_device_workspace_missing", dict(T=524288, H=16), lt.LT_ERR_HIP),
], ids=lambda x: x if isinstance(x, str) else "")
def test_prefill_dd_rejects(name, over, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128, dec=FAKE,
             base=1e6, eps=1e-6, pos0=0, sin=None, sout=None, y=FAKE, oraw=None, B=1, T=256, H=2,
             d=128, dt=lt.LT_BF16, chunk=0, seg=0, ws=None, wsb=0, ev=None, stream=None)
    a.update(over)
    st = lt.lib.lightning_prefill_dd(a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"],
                                     a["stride"], a["dec"], a["base"], a["eps"], a["pos0"],
                                     a["sin"], a["sout"], a["y"], a["oraw"], a["B"], a["T"], a["H"],
                                     a["d"], a["dt"], a["chunk"], a["seg"], a["ws"], a["wsb"],
                                     a["ev"], a["stream"])
    assert st == status


# ---- prefill backward ----------------------------------------------------------------------------

def test_backward_workspace_layout():
    B, T, H, d = 8, 16384, 16, 128
    pl = lt.lightning_prefill_plan_cus(256, B, T, H, d)
    ws = pl["backward_workspace_bytes"]
    # at least: do (bf16, one activation tensor), the two masked 32 x 32 fp32 score tiles of
    # every chunk, one d x d state gradient per (b, h, segment)
    assert ws >= B * T * H * d * 2 + B * H * (T // 32) * 2 * 32 * 32 * 4 + B * H * d * d * 4
    assert ws % 4 == 0 and pl["backward_segments"] == 2
    # fp32 inputs add five bf16 copies (q, k, v, g, dy) of one activation tensor each
    ws32 = lt.lightning_prefill_plan_cus(256, B, T, H, d, torch.float32)["backward_workspace_bytes"]
    assert ws32 == ws + 5 * B * T * H * d * 2
    # d = 64: smaller by the state and activation parts
    ws64 = lt.lightning_prefill_plan_cus(256, B, T, H, 64)["backward_workspace_bytes"]
    assert B * T * H * 64 * 2 + B * H * 64 * 64 * 4 <= ws64 < ws
    assert lt.lightning_prefill_plan_cus(256, B, T, H, 64, torch.float32)[
        "backward_workspace_bytes"] == ws64 + 5 * B * T * H * 64 * 2
    # one segment (B H fills the CUs): no forward state slots, one gradient per (b, h)
    one = lt.lightning_prefill_plan_cus(256, 16, 256, 16, d)["backward_workspace_bytes"]
    do_bytes = 16 * 256 * 16 * d * 2
    score_bytes = 16 * 16 * (256 // 32) * 2 * 32 * 32 * 4
    assert one >= do_bytes + score_bytes + 16 * 16 * d * d * 4
    assert one < do_bytes + score_bytes + 16 * 16 * d * d * 4 + 3 * 16 * 16 * d * 4 + 1024


def _bwd_args(**over):
    H = over.pop("H", 2)
    lam = over.pop("lam", [0.9] * H)
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, qw=FAKE, kw=FAKE, ow=None, stride=128,
             lam=(ct.c_double * len(lam))(*lam), base=1e6, eps=1e-6, pos0=0, sin=None, dy=FAKE,
             dso=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dsi=None, dqw=None, dkw=None, dow=None,
             B=1, T=256, H=H, d=128, dt=lt.LT_BF16, seg=0, ws=FAKE, wsb=1 << 40, ev=None,
             stream=None)
    a.update(over)
    return a


BWD_BAD = [
    ("null_dy", dict(dy=None), lt.LT_ERR_INVALID_ARG),
    ("null_dq", dict(dq=None), lt.LT_ERR_INVALID_ARG),
    ("null_dgate", dict(dg=None), lt.LT_ERR_INVALID_ARG),
    ("misaligned_dk", dict(dk=FAKE + 2), lt.LT_ERR_INVALID_ARG),
    ("misaligned_d_state_out", dict(dso=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("misaligned_weight_grad", dict(dkw=FAKE + 4), lt.LT_ERR_INVALID_ARG),
    ("null_qnorm", dict(qw=None), lt.LT_ERR_INVALID_ARG),
    ("lambda_above_one", dict(lam=[0.9, 1.5]), lt.LT_ERR_INVALID_ARG),
    ("zero_T", dict(T=0), lt.LT_ERR_INVALID_ARG),
    ("negative_segments", dict(seg=-1), lt.LT_ERR_INVALID_ARG),
    ("pos0_negative", dict(pos0=-3), lt.LT_ERR_INVALID_ARG),
    ("d_96", dict(d=96, stride=96), lt.LT_ERR_UNSUPPORTED),
    ("d_32", dict(d=32, stride=32), lt.LT_ERR_UNSUPPORTED),
    ("events_null_entries", dict(ev=(ct.c_void_p * 4)(None, None, None, None)),
     lt.LT_ERR_INVALID_ARG),
    # valid arguments: the plan needs the device, so without one the call reports LT_ERR_HIP
    # (the workspace checks run on the GPU in tests/test_gpu_errors.py)
    ("no_device", dict(), lt.LT_ERR_HIP),
    ("no_device_fp32", dict(dt=lt.LT_F32), lt.LT_ERR_HIP),
    ("no_device_d64", dict(d=64, stride=64), lt.LT_ERR_HIP),
    ("no_device_workspace_missing", dict(ws=None), lt.LT_ERR_HIP),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", BWD_BAD, ids=[c[0] for c in BWD_BAD])
def test_prefill_backward_rejects(name, over, status):
    a = _bwd_args(**over)
    st = lt.lib.lightning_prefill_backward(
        a["q"], a["k"], a["v"], a["g"], a["qw"], a["kw"], a["ow"], a["stride"], a["lam"],
        a["base"], a["eps"], a["pos0"], a["sin"], a["dy"], a["dso"], a["dq"], a["dk"], a["dv"],
        a["dg"], a["dsi"], a["dqw"], a["dkw"], a["dow"], a["B"], a["T"], a["H"], a["d"], a["dt"],
        a["seg"], a["ws"], a["wsb"], a["ev"], a["stream"])
    assert st == status
