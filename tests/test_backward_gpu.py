"""Parity of the prefill backward (lightning_prefill_backward) with the fp64 gradient oracle of
oracle/backward.py, on the same seeded inputs, compared per (b, h) slice.

Cases span d = 128 and d = 64, bf16 and fp32 activations (fp32 inputs are rounded once to bf16
copies for the products; the gradients come back in fp32).

Tolerances (relative L2 error per slice): every gradient <= 2e-2.  The backward's products run
on bf16 MFMA operands with fp32 accumulation (q~, k~, v, do and the bf16 copy of the state that
the products contracting over the value dimension read), like the forward's score and output
products, whose bf16 outputs the same bound covers; d_state_in and the norm-weight gradients
are sums of such products, so they carry the same operand rounding (about 2^-9 relative per
operand) and take the same bound rather than the forward state's 1e-4, which the forward reaches
only through its hi/lo split of the decayed keys.

With lambda = 0 the output o_t = (q~_t . k~_t) v_t is parallel to v_t, and the output norm's
gradient do_t is orthogonal to o_t up to a term of relative size eps / mean(o_t^2), so
do_t . v_t ~ 0 and dq, dk nearly vanish.  o_t also crosses zero whenever the score does, and the
output norm's gradient scales with 1/||o_t||, so every gradient is compared on the rows with
||o_t|| >= 5% of the slice's RMS row norm (each gradient of token t only involves token t when
lambda = 0), the others must be finite: dv and dg to the bound above, dq and dk with an absolute
error of at most 2e-2 of the norm of the same rows' gradients for the same inputs with
lambda = 0.5 (where they are of ordinary size).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob
import synth
from synth import host_bits, rel_l2

pytestmark = pytest.mark.gpu

TOL = 2e-2
ILL_ROW_FRAC = 0.05


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_backward(inp, segments=0, ow=None, shared_w=False):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    qw, kw = inp["qw"], inp["kw"]
    if shared_w:
        qw, kw = qw[0], kw[0]
        ow = None if ow is None else ow[0]
    out = lt.lightning_prefill_backward(
        *(inp[n].to(dev) for n in ("q", "k", "v", "g")), qw.to(dev), kw.to(dev), inp["lambdas"],
        inp["rope_base"], inp["dy"].to(dev), rms_eps=inp["eps"], pos0=inp["pos0"],
        state_in=None if inp["state_in"] is None else inp["state_in"].to(dev),
        d_state_out=None if inp["d_state_out"] is None else inp["d_state_out"].to(dev),
        o_norm_w=None if ow is None else ow.to(dev), segments=segments)
    torch.cuda.synchronize()
    return {n: t.float().cpu() for n, t in out.items()}


def oracle_backward(inp, slices=None, ow=None, shared_w=False):
    qw, kw = inp["qw"].numpy(), inp["kw"].numpy()
    owa = None if ow is None else ow.numpy()
    if shared_w:
        qw, kw = qw[0], kw[0]
        owa = None if owa is None else owa[0]
    st = inp["state_in"]
    ds = inp["d_state_out"]
    return ob.prefill_backward(*(host_bits(inp[n]) for n in ("q", "k", "v", "g", "dy")), qw, kw,
                               inp["lambdas"], inp["rope_base"], eps=inp["eps"], pos0=inp["pos0"],
                               state_in=None if st is None else st.numpy(),
                               d_state_out=None if ds is None else ds.numpy(), ow=owa,
                               slices=slices)


def _part(gpu, name, b, h):
    """Slice (b, h) of a GPU result: a full [B, T, H, d] / [B, H, d, d] tensor, or a dict of
    slices keyed by (b, h)."""
    x = gpu[name]
    if isinstance(x, dict):
        return x[(b, h)].numpy()
    return (x[b, :, h] if x.dim() == 4 and name != "d_state_in" else x[b, h]).numpy()


GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dgate"))


def compare(gpu, ref, inp, label, ow=None, ill_rows=False, grads=GRADS):
    B, T, H, d = inp["q"].shape
    worst = {}
    rows_ok = None
    if ill_rows:
        f = oracle.prefill(*(host_bits(inp[n]) for n in ("q", "k", "v", "g")), inp["qw"].numpy(),
                           inp["kw"].numpy(), inp["lambdas"], inp["rope_base"], eps=inp["eps"],
                           pos0=inp["pos0"],
                           state_in=None if inp["state_in"] is None else inp["state_in"].numpy(),
                           slices=ref["slices"])
        norms = np.linalg.norm(f["o"], axis=2)  # [n, T]
        rms = np.sqrt(np.mean(norms ** 2, axis=1, keepdims=True))
        rows_ok = norms >= ILL_ROW_FRAC * rms
    for i, (b, h) in enumerate(ref["slices"]):
        for name, gname in grads:
            x = _part(gpu, gname, b, h)
            r = ref[name][i]
            assert np.all(np.isfinite(x)), f"{label}: {name} not finite"
            if rows_ok is not None:
                x, r = x[rows_ok[i]], r[rows_ok[i]]
            worst[name] = max(worst.get(name, 0.0), rel_l2(x, r))
        if "d_state_in" in gpu:
            worst["dS_in"] = max(worst.get("dS_in", 0.0),
                                 rel_l2(_part(gpu, "d_state_in", b, h), ref["d_state_in"][i]))
    print(f"[parity] backward {label}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= TOL, f"{label}: {k} rel L2 {v:.3e} > {TOL}"
    return dict(worst, rows_ok=rows_ok)


def compare_weights(gpu, ref, inp, label, shared_w=False, want_o=True):
    B, T, H, d = inp["q"].shape
    for name, gname in (("dqw", "d_q_norm_w"), ("dkw", "d_k_norm_w"), ("dow", "d_o_norm_w")):
        if name == "dow" and not want_o:
            continue
        acc = np.zeros((H, d))
        for i, (b, h) in enumerate(ref["slices"]):
            acc[h] += ref[name][i]
        r = acc.sum(axis=0) if shared_w else acc
        e = rel_l2(gpu[gname].numpy(), r)
        print(f"[parity] backward {label}: {name}={e:.2e}")
        assert e <= TOL, f"{label}: {name} rel L2 {e:.3e} > {TOL}"


CASES = [
    # (label, B, T, H, lambdas (None: 1 - 2^-(5 + 8h/H)), state, d_state_out, pos0, segments)
    ("ragged_state_grads", 1, 300, 2, None, "randn", True, 0, (0, 3)),
    ("two_rows_three_heads", 2, 333, 3, None, "zeros", False, 7, (0, 2)),
    ("one_chunk", 1, 32, 2, None, "randn", True, 0, (0,)),
    ("one_chunk_plus_one", 1, 33, 2, None, "randn", True, 0, (0,)),
    ("single_token", 2, 1, 2, None, "randn", True, 5, (0,)),
    ("lambda_one", 1, 200, 1, (1.0,), "randn", True, 0, (0, 2)),
    ("long_position", 1, 257, 2, None, "zeros", True, 500000, (0, 2)),
    ("sub_segments", 1, 4096 + 33, 2, None, "randn", True, 0, (0, 4)),
    # the paper's decay schedule (Appendix A, Eq. 19): gamma_h = exp(-2^(-8h/H)), h = 1..16;
    # the fast heads' lazily scaled state and state gradient renormalise in every chunk
    ("eq19_gamma", 1, 1024 + 5, 16, tuple(math.exp(-2.0 ** (-8.0 * h / 16)) for h in range(1, 17)),
     "randn", True, 0, (0, 3)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_small(case):
    label, B, T, H, lambdas, state, dso, pos0, segs = case
    seed = zlib.crc32(label.encode()) % 9973
    inp = synth.make_custom_prefill(B, T, H, 128, dtype=torch.bfloat16, seed=seed, state=state,
                                    lambdas=lambdas, pos0=pos0)
    gen = torch.Generator().manual_seed(seed + 1)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.bfloat16)
    inp["d_state_out"] = (0.01 * torch.randn((B, H, 128, 128), generator=gen)) if dso else None
    ref = oracle_backward(inp)
    for seg in segs:
        gpu = gpu_backward(inp, segments=seg)
        compare(gpu, ref, inp, f"{label} segments={seg}")
        compare_weights(gpu, ref, inp, f"{label} segments={seg}", want_o=True)


# d = 64 and fp32 activations: the same sweeps at half the head width, and fp32 inputs rounded
# once to bf16 copies (the products take bf16 operands either way) with fp32 gradients written
# out, so the bound stays the bf16 one.
WIDE_CASES = [
    # (label, B, T, H, d, dtype, state, d_state_out, segments)
    ("d64_ragged", 1, 300, 2, 64, torch.bfloat16, "randn", True, (0, 3)),
    ("d64_two_rows", 2, 333, 3, 64, torch.bfloat16, "zeros", False, (0, 2)),
    ("d64_sub_segments", 1, 4096 + 33, 2, 64, torch.bfloat16, "randn", True, (0, 4)),
    ("fp32_d128_ragged", 1, 300, 2, 128, torch.float32, "randn", True, (0, 3)),
    ("fp32_d64_two_rows", 2, 200, 2, 64, torch.float32, "randn", False, (0, 2)),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_backward_d64_and_fp32(case):
    label, B, T, H, d, dtype, state, dso, segs = case
    seed = zlib.crc32(label.encode()) % 9973
    inp = synth.make_custom_prefill(B, T, H, d, dtype=dtype, seed=seed, state=state)
    gen = torch.Generator().manual_seed(seed + 1)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(dtype)
    inp["d_state_out"] = (0.01 * torch.randn((B, H, d, d), generator=gen)) if dso else None
    ref = oracle_backward(inp)
    for seg in segs:
        gpu = gpu_backward(inp, segments=seg)
        compare(gpu, ref, inp, f"{label} segments={seg}")
        compare_weights(gpu, ref, inp, f"{label} segments={seg}")


def test_backward_tiny_workload():
    """The tiny workload as specified (B = 1, H = 2, T = 256, d = 64, fp32, lambda = (0.9, 0.99),
    rope base 1e4, unit norm weights)."""
    inp = synth.make_prefill(synth.TINY)
    gen = torch.Generator().manual_seed(51)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.float32)
    inp["d_state_out"] = None
    ref = oracle_backward(inp)
    gpu = gpu_backward(inp)
    compare(gpu, ref, inp, "tiny workload")
    compare_weights(gpu, ref, inp, "tiny workload")


def test_backward_output_weight_and_shared_norm_weights():
    """An output-norm weight and QK-norm weights shared by all heads (stride 0)."""
    inp = synth.make_custom_prefill(1, 400, 2, 128, dtype=torch.bfloat16, seed=41, state="randn")
    gen = torch.Generator().manual_seed(42)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.bfloat16)
    inp["d_state_out"] = None
    ow = 0.5 + torch.rand((2, 128), generator=gen)
    inp["qw"][1] = inp["qw"][0]
    inp["kw"][1] = inp["kw"][0]
    ow[1] = ow[0]
    ref = oracle_backward(inp, ow=ow, shared_w=True)
    gpu = gpu_backward(inp, ow=ow, shared_w=True)
    compare(gpu, ref, inp, "shared weights")
    compare_weights(gpu, ref, inp, "shared weights", shared_w=True)


def test_backward_lambda_zero():
    inp = synth.make_custom_prefill(1, 160, 2, 128, dtype=torch.bfloat16, seed=43, state="randn",
                                    lambdas=(0.0, 0.0))
    gen = torch.Generator().manual_seed(44)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.bfloat16)
    inp["d_state_out"] = None
    ref = oracle_backward(inp)
    ref_half = oracle_backward(dict(inp, lambdas=[0.5, 0.5]))
    gpu = gpu_backward(inp, segments=2)
    assert float(np.abs(gpu["d_state_in"].numpy()).max()) == 0.0
    rows_ok = compare(gpu, ref, inp, "lambda=0", ill_rows=True, grads=GRADS[2:])["rows_ok"]
    for i, (b, h) in enumerate(ref["slices"]):
        ok = rows_ok[i]
        for name in ("dq", "dk"):
            scale = np.linalg.norm(ref_half[name][i][ok])
            assert np.linalg.norm(ref[name][i][ok]) < 1e-2 * scale  # the near-cancellation
            err = np.linalg.norm(_part(gpu, name, b, h)[ok] - ref[name][i][ok]) / scale
            print(f"[parity] backward lambda=0: {name} error / |{name} at lambda=0.5| = {err:.2e}")
            assert err <= TOL


def test_backward_deterministic():
    inp = synth.make_custom_prefill(1, 1000, 2, 128, dtype=torch.bfloat16, seed=45, state="randn")
    gen = torch.Generator().manual_seed(46)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.bfloat16)
    inp["d_state_out"] = None
    a = gpu_backward(inp, segments=3)
    b = gpu_backward(inp, segments=3)
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.timeout(600)
def test_backward_full_size_sampled_heads():
    """The 16K-token training shape (B = 8, H = 16) in the launch configuration the benchmark
    times; batch rows 0 and 7 of heads 0 and 15 against the oracle."""
    spec = synth.BWD_QWEN17_16K
    inp = synth.make_backward(spec, device="cuda")
    import long_context_hybrid_amd.lightning as lt

    out = lt.lightning_prefill_backward(
        inp["q"], inp["k"], inp["v"], inp["g"], inp["qw"], inp["kw"], inp["lambdas"],
        inp["rope_base"], inp["dy"], rms_eps=inp["eps"], pos0=inp["pos0"])
    torch.cuda.synchronize()
    slices = [(0, 0), (7, 15)]
    host = {n: inp[n].cpu() for n in ("q", "k", "v", "g", "dy", "qw", "kw")}
    sub = dict(inp, **host, state_in=None, d_state_out=None)
    ref = oracle_backward(sub, slices=slices)
    gpu = {n: {(b, h): out[n][b, :, h].float().cpu() for b, h in slices}
           for n in ("dq", "dk", "dv", "dgate")}
    gpu["d_state_in"] = {(b, h): out["d_state_in"][b, h].cpu() for b, h in slices}
    compare(gpu, ref, sub, "16K training shape")


def test_backward_composes_over_split_calls_on_gpu():
    """The backward of two chained prefill calls, the second's d_state_in fed to the first as its
    d_state_out (and the first call's final state as the second's state_in, from the forward
    kernel), equals the backward of the whole call."""
    import long_context_hybrid_amd.lightning as lt

    T, T1 = 1000, 613
    inp = synth.make_custom_prefill(1, T, 2, 128, dtype=torch.bfloat16, seed=47, state="randn")
    gen = torch.Generator().manual_seed(48)
    inp["dy"] = torch.randn(inp["q"].shape, generator=gen).to(torch.bfloat16)
    inp["d_state_out"] = 0.01 * torch.randn((1, 2, 128, 128), generator=gen)
    dev = torch.device("cuda")
    whole = gpu_backward(inp, segments=3)
    first = dict(inp, **{n: inp[n][:, :T1].contiguous() for n in ("q", "k", "v", "g", "dy")})
    second = dict(inp, **{n: inp[n][:, T1:].contiguous() for n in ("q", "k", "v", "g", "dy")},
                  pos0=T1)
    s_mid = torch.empty((1, 2, 128, 128), dtype=torch.float32, device=dev)
    lt.lightning_prefill(*(first[n].to(dev) for n in ("q", "k", "v", "g")), inp["qw"].to(dev),
                         inp["kw"].to(dev), inp["lambdas"], inp["rope_base"],
                         state_in=inp["state_in"].to(dev), state_out=s_mid)
    torch.cuda.synchronize()
    second["state_in"] = s_mid.cpu()
    g2 = gpu_backward(second, segments=2)
    first["d_state_out"] = g2["d_state_in"]
    g1 = gpu_backward(first, segments=2)
    for name in ("dq", "dk", "dv", "dgate"):
        joined = torch.cat([g1[name], g2[name]], 1)
        for h in range(2):
            e = rel_l2(joined[0, :, h].numpy(), whole[name][0, :, h].numpy())
            assert e <= TOL, (name, h, e)
    for h in range(2):
        e = rel_l2(g1["d_state_in"][0, h].numpy(), whole["d_state_in"][0, h].numpy())
        print(f"[parity] backward split calls: d_state_in head {h} {e:.2e}")
        assert e <= TOL
    for name in ("d_q_norm_w", "d_k_norm_w", "d_o_norm_w"):
        e = rel_l2((g1[name] + g2[name]).numpy(), whole[name].numpy())
        assert e <= TOL, (name, e)


def test_backward_state_gradient_only():
    """dy = 0 with a final-state gradient: do vanishes, so dq and dgate are exactly zero, and dk,
    dv and d_state_in come from d_state_out alone (against the oracle)."""
    inp = synth.make_custom_prefill(1, 500, 2, 128, dtype=torch.bfloat16, seed=49, state="randn")
    gen = torch.Generator().manual_seed(50)
    inp["dy"] = torch.zeros(inp["q"].shape, dtype=torch.bfloat16)
    inp["d_state_out"] = torch.randn((1, 2, 128, 128), generator=gen)
    ref = oracle_backward(inp)
    gpu = gpu_backward(inp, segments=3)
    assert float(gpu["dq"].abs().max()) == 0.0 and float(gpu["dgate"].abs().max()) == 0.0
    compare(gpu, ref, inp, "state gradient only", grads=GRADS[1:3])
