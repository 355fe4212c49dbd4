"""Parity of the HIP path (through the C ABI) with the fp64 oracle on seeded inputs.

Small cases compare every element of every (b, h) slice; they span several chunks with ragged
tails, several segment splits, both storage dtypes and both head widths, and the method's
degenerate cases (lambda = 0, lambda = 1, T = 1, a partial last chunk).  The full-size workloads
run in the launch configuration the benchmark times and are compared on every (b, h) slice
(y, o and the final state), the oracle running them in groups of parallel slices.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import TOL, compare_prefill, gpu_prefill, oracle_prefill
from synth import host_bits, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---- small shapes, every element ----------------------------------------------------------------

SMALL = [
    # (label, B, T, H, d, dtype, lambdas, state, segments list)
    ("tiny_fp32_d64", 1, 256, 2, 64, torch.float32, (0.9, 0.99), "zeros", (0, 1, 2, 4)),
    ("bf16_d128_ragged", 1, 300, 4, 128, torch.bfloat16, None, "randn", (0, 2, 5)),
    ("bf16_d64_ragged", 2, 1000, 3, 64, torch.bfloat16, (0.0, 0.43, 1.0), "zeros", (0, 3, 16)),
    ("fp32_d128_ragged", 1, 777, 2, 128, torch.float32, (0.5, 0.999), "randn", (0, 4)),
    ("bf16_d128_long", 1, 4096 + 17, 2, 128, torch.bfloat16, None, "randn", (0, 7, 65)),
    ("fp32_d64_ragged", 3, 130, 2, 64, torch.float32, (0.0, 1.0), "randn", (0, 3)),
    # segments whose state-only pass is split further (3 and 5 sub-segments per segment)
    ("bf16_d128_subsegments", 1, 8192 + 5, 2, 128, torch.bfloat16, None, "randn", (2, 4)),
    # slow heads: state-only sub-segments close enough to the end to need the low key parts
    # (lambda^(T - end) above 2^-8), a head between, and a fast head whose lazy state scale
    # renormalises every chunk
    ("bf16_d128_slow_heads", 1, 8192 + 33, 3, 128, torch.bfloat16, (0.99999, 0.999, 0.5), "randn", (3, 5)),
    # 3 and 2 sub-segments per segment, fp32 activations
    ("fp32_d64_subsegments", 2, 2048 + 40, 1, 64, torch.float32, (0.9999,), "randn", (2, 3)),
    # the paper's own decay schedule (Appendix A, Eq. 19): gamma_h = exp(-2^(-8h/H)), h = 1..16,
    # from 0.49 (memory of about one token) to 0.996 (about 256 tokens)
    ("bf16_d128_eq19_gamma", 1, 2048 + 9, 16, 128, torch.bfloat16,
     tuple(math.exp(-2.0 ** (-8.0 * h / 16)) for h in range(1, 17)), "randn", (0, 4)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_small(case):
    label, B, T, H, d, dtype, lams, state, seg_list = case
    inp = synth.make_custom_prefill(B, T, H, d, dtype=dtype, seed=zlib.crc32(label.encode()) % 10000,
                                    lambdas=lams, rope_base=1e4 if d == 64 else 1e6, state=state)
    ref = oracle_prefill(inp)
    for seg in seg_list:
        gpu = gpu_prefill(inp, segments=seg)
        compare_prefill(gpu, ref, dtype, label=f"{label} segments={seg}")


# 64-token chunks (the main pass's second instantiation): every small case but fp32 with d = 128,
# whose 64-row tiles do not fit in LDS (the library rejects that combination)
SMALL64 = [c for c in SMALL if not (c[5] == torch.float32 and c[4] == 128)]


@pytest.mark.parametrize("case", SMALL64, ids=[c[0] for c in SMALL64])
def test_prefill_small_chunk64(case):
    label, B, T, H, d, dtype, lams, state, seg_list = case
    inp = synth.make_custom_prefill(B, T, H, d, dtype=dtype, seed=zlib.crc32(label.encode()) % 10000,
                                    lambdas=lams, rope_base=1e4 if d == 64 else 1e6, state=state)
    ref = oracle_prefill(inp)
    for seg in seg_list:
        gpu = gpu_prefill(inp, chunk=64, segments=seg)
        compare_prefill(gpu, ref, dtype, label=f"{label} chunk=64 segments={seg}")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 191])
def test_prefill_chunk64_boundary_lengths(T):
    inp = synth.make_custom_prefill(2, T, 2, 128, dtype=torch.bfloat16, seed=T + 100, state="randn")
    ref = oracle_prefill(inp)
    compare_prefill(gpu_prefill(inp, chunk=64), ref, torch.bfloat16, label=f"T={T} chunk=64")
    compare_prefill(gpu_prefill(inp, chunk=64, segments=2), ref, torch.bfloat16,
                    label=f"T={T} chunk=64 seg=2")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129])
def test_prefill_short_and_boundary_lengths(T):
    inp = synth.make_custom_prefill(2, T, 2, 128, dtype=torch.bfloat16, seed=T, state="randn")
    ref = oracle_prefill(inp)
    compare_prefill(gpu_prefill(inp), ref, torch.bfloat16, label=f"T={T}")
    compare_prefill(gpu_prefill(inp, segments=2), ref, torch.bfloat16, label=f"T={T} seg=2")


def test_tiny_workload_as_specified():
    """The tiny workload as drawn (fp32, d = 64) at its stated chunk length of 64, and at the
    library's default of 32.  The oracle's chunked form at C = 64 equals its recurrence (see the
    oracle pins)."""
    inp = synth.make_prefill(synth.TINY)
    ref = oracle_prefill(inp)
    ref64 = oracle.prefill(*(host_bits(inp[n]) for n in ("q", "k", "v", "g")), inp["qw"].numpy(),
                           inp["kw"].numpy(), inp["lambdas"], inp["rope_base"], chunk=64)
    assert np.max(np.abs(ref64["y"] - ref["y"])) <= 1e-12
    for chunk in (64, 0):
        worst = compare_prefill(gpu_prefill(inp, chunk=chunk), ref, torch.float32,
                                label=f"tiny workload chunk={chunk}")
        assert worst["state"] <= 1e-4


def test_output_norm_weight_shared_norm_weights_and_position_origin():
    B, T, H, d = 1, 200, 3, 128
    inp = synth.make_custom_prefill(B, T, H, d, dtype=torch.bfloat16, seed=77, state="randn")
    inp["qw"] = inp["qw"][0].contiguous()  # one weight vector shared by all heads
    inp["kw"] = inp["kw"][0].contiguous()
    ow = torch.rand((d,), generator=torch.Generator().manual_seed(5)) + 0.5
    for pos0 in (0, 123_457, 524_287):
        ref = oracle_prefill(inp, pos0=pos0, ow=ow)
        gpu = gpu_prefill(inp, pos0=pos0, ow=ow, segments=2)
        compare_prefill(gpu, ref, torch.bfloat16, label=f"shared weights, ow, pos0={pos0}")


def test_deterministic():
    inp = synth.make_custom_prefill(1, 2048, 4, 128, dtype=torch.bfloat16, seed=9, state="randn")
    a = gpu_prefill(inp)
    b = gpu_prefill(inp)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["state"], b["state"])
    assert torch.equal(a["o"], b["o"])


def test_split_prefill_composition():
    """prefill(T1) then prefill(T2, pos0 = T1, state carried) matches the oracle's prefill(T1+T2)."""
    T1, T2 = 1000, 1234
    inp = synth.make_custom_prefill(2, T1 + T2, 3, 128, dtype=torch.bfloat16, seed=11,
                                    state="randn")
    ref = oracle_prefill(inp)
    first = {k: (v[:, :T1].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4
                 and v.shape[1] == T1 + T2 else v) for k, v in inp.items()}
    g1 = gpu_prefill(first, segments=3)
    second = {k: (v[:, T1:].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4
                  and v.shape[1] == T1 + T2 else v) for k, v in inp.items()}
    g2 = gpu_prefill(second, pos0=T1, state_in=g1["state"], segments=2)
    gpu = dict(y=torch.cat([g1["y"], g2["y"]], 1), o=torch.cat([g1["o"], g2["o"]], 1),
               state=g2["state"])
    compare_prefill(gpu, ref, torch.bfloat16, label="split prefill")


def test_state_in_place():
    """state_out may alias state_in."""
    import long_context_hybrid_amd.lightning as lt

    inp = synth.make_custom_prefill(1, 700, 2, 128, dtype=torch.bfloat16, seed=12, state="randn")
    ref = oracle_prefill(inp)
    for seg in (1, 3):
        dev = torch.device("cuda")
        s = inp["state_in"].to(dev).clone()
        y = lt.lightning_prefill(*(inp[n].to(dev) for n in ("q", "k", "v", "g")),
                                 inp["qw"].to(dev), inp["kw"].to(dev), inp["lambdas"],
                                 inp["rope_base"], state_in=s, state_out=s, segments=seg)
        torch.cuda.synchronize()
        compare_prefill(dict(y=y.float().cpu(), state=s.cpu()), ref, torch.bfloat16,
                        what=("y", "state"), label=f"in-place seg={seg}")


# ---- decode ---------------------------------------------------------------------------------------

def gpu_decode(inp, in_place=False):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    s_in = inp["state_in"].to(dev).clone()
    s_out = s_in if in_place else torch.empty_like(s_in)
    o_raw = torch.empty(inp["q"].shape, dtype=torch.float32, device=dev)
    y = lt.lightning_decode_step(*(inp[n].to(dev) for n in ("q", "k", "v", "g")),
                                 inp["qw"].to(dev), inp["kw"].to(dev), inp["lambdas"],
                                 inp["rope_base"], inp["positions"].to(dev), s_in,
                                 state_out=s_out, rms_eps=inp["eps"], o_raw=o_raw)
    torch.cuda.synchronize()
    return y.float().cpu(), o_raw.cpu(), s_out.cpu()


def oracle_decode(inp):
    return oracle.decode_step(host_bits(inp["q"]), host_bits(inp["k"]), host_bits(inp["v"]),
                              host_bits(inp["g"]), inp["qw"].numpy(), inp["kw"].numpy(),
                              inp["lambdas"], inp["rope_base"], inp["positions"].numpy(),
                              inp["state_in"].numpy(), eps=inp["eps"])


def _decode_errors(inp, in_place=False):
    y, o, s = gpu_decode(inp, in_place)
    ref = oracle_decode(inp)
    B, H = inp["B"], inp["H"]
    worst = dict(y=0.0, o=0.0, state=0.0)
    for b in range(B):
        for h in range(H):
            worst["y"] = max(worst["y"], rel_l2(y[b, h].numpy(), ref["y"][b, h]))
            worst["o"] = max(worst["o"], rel_l2(o[b, h].numpy(), ref["o"][b, h]))
            worst["state"] = max(worst["state"], rel_l2(s[b, h].numpy(), ref["state"][b, h]))
    return worst


@pytest.mark.parametrize("in_place", [False, True])
def test_decode_full_workload(in_place):
    """The batched decode workload at full size: B = 64, H = 16, d = 128, every (b, h)."""
    inp = synth.make_decode(synth.DECODE_B64)
    worst = _decode_errors(inp, in_place)
    print(f"[parity] decode B=64 in_place={in_place} " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    tol = TOL[torch.bfloat16]
    for k in worst:
        assert worst[k] <= tol[k], (k, worst[k])


@pytest.mark.parametrize("d,dtype", [(64, torch.float32), (128, torch.float32), (64, torch.bfloat16)])
def test_decode_small(d, dtype):
    spec = synth.DecodeSpec("small", 5, 3, d, dtype, (0.0, 0.9, 1.0), 1e4, 1 << 20, 31)
    inp = synth.make_decode(spec)
    worst = _decode_errors(inp)
    print(f"[parity] decode d={d} {dtype} " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    tol = TOL[dtype]
    for k in worst:
        assert worst[k] <= tol[k], (k, worst[k])


def test_prefill_then_decode():
    """GPU prefill(T) then a GPU decode step at position T equals the oracle's token T of
    prefill(T + 1) and its final state."""
    import long_context_hybrid_amd.lightning as lt

    T, B, H, d = 513, 2, 4, 128
    inp = synth.make_custom_prefill(B, T + 1, H, d, dtype=torch.bfloat16, seed=21, state="randn")
    ref = oracle_prefill(inp)
    head = {k: (v[:, :T].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4
                and v.shape[1] == T + 1 else v) for k, v in inp.items()}
    g = gpu_prefill(head)
    dev = torch.device("cuda")
    s = g["state"].to(dev)
    tok = {n: inp[n][:, T].contiguous().to(dev) for n in ("q", "k", "v", "g")}
    y = lt.lightning_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], inp["qw"].to(dev),
                                 inp["kw"].to(dev), inp["lambdas"], inp["rope_base"],
                                 torch.full((B,), T, dtype=torch.int64, device=dev), s)
    torch.cuda.synchronize()
    y = y.float().cpu()
    s = s.cpu()
    for i, (b, h) in enumerate(ref["slices"]):
        assert rel_l2(y[b, h].numpy(), ref["y"][i][T]) <= 2e-2
        assert rel_l2(s[b, h].numpy(), ref["state"][i]) <= 1e-4


# ---- full-size workloads, every slice --------------------------------------------------------------

def _gather_slices(inp, slices):
    """The inputs of the given (b, h) slices, stacked as the heads of one batch row, so one
    oracle call runs them in parallel (one thread per slice)."""
    def col(name):
        return torch.stack([inp[name][b, :, h].cpu() for b, h in slices], dim=1)[None]

    s_in = None
    if inp["state_in"] is not None:
        s_in = torch.stack([inp["state_in"][b, h].cpu() for b, h in slices])[None]
    return dict(inp, q=col("q"), k=col("k"), v=col("v"), g=col("g"),
                qw=torch.stack([inp["qw"][h].cpu() for _, h in slices]),
                kw=torch.stack([inp["kw"][h].cpu() for _, h in slices]),
                lambdas=[inp["lambdas"][h] for _, h in slices], state_in=s_in)


def _full_size(spec, slices, device_inputs, chunk=0, group=16):
    """One GPU prefill of the full workload in the launch configuration the benchmark times
    (automatic segments; chunk 0 = 32), then y, o and the final state of every listed (b, h)
    slice against the oracle, which runs `group` slices at a time (one thread each) so that
    host memory stays bounded."""
    import long_context_hybrid_amd.lightning as lt

    inp = synth.make_prefill(spec, device="cuda" if device_inputs else "cpu")
    dev = torch.device("cuda")
    B, T, H, d = inp["q"].shape
    s_in = None if inp["state_in"] is None else inp["state_in"].to(dev)
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    o_raw = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    y = lt.lightning_prefill(*(inp[n].to(dev) for n in ("q", "k", "v", "g")), inp["qw"].to(dev),
                             inp["kw"].to(dev), inp["lambdas"], inp["rope_base"],
                             rms_eps=inp["eps"], pos0=inp["pos0"], state_in=s_in,
                             state_out=s_out, o_raw=o_raw, chunk=chunk)
    torch.cuda.synchronize()
    worst = {}
    for i in range(0, len(slices), group):
        part = slices[i:i + group]
        gpu = dict(y=torch.stack([y[b, :, h].float().cpu() for b, h in part], dim=1)[None],
                   o=torch.stack([o_raw[b, :, h].cpu() for b, h in part], dim=1)[None],
                   state=torch.stack([s_out[b, h].cpu() for b, h in part])[None])
        ref = oracle_prefill(_gather_slices(inp, part))
        w = compare_prefill(gpu, ref, torch.bfloat16,
                            label=f"{spec.name} chunk={chunk} slices {part[0]}..{part[-1]}")
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
        del gpu, ref
    print(f"[parity] {spec.name} chunk={chunk}, {len(slices)} slices: " +
          " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    return worst


def test_full_qwen17_32k_all_heads():
    slices = [(0, h) for h in range(16)]
    _full_size(synth.QWEN17_32K, slices, device_inputs=False)


def test_full_qwen17_32k_all_heads_chunk64():
    _full_size(synth.QWEN17_32K, [(0, h) for h in range(16)], device_inputs=False, chunk=64)


@pytest.mark.timeout(600)
def test_full_qwen17_512k_all_heads():
    _full_size(synth.QWEN17_512K, [(0, h) for h in range(16)], device_inputs=True)


@pytest.mark.timeout(900)
def test_full_qwen8_128k_all_slices():
    """Qwen3-8B shape (B = 4, H = 32, T = 128K, nonzero entry states): all 128 (b, h) slices."""
    _full_size(synth.QWEN8_128K, [(b, h) for b in range(4) for h in range(32)], device_inputs=True)
