"""Parity of the HyPE attention kernels (through the C ABI) with the fp64 oracle.

Small cases compare every element of y and of o (before the output norm) per (b, h) slice,
across the three workgroup shapes (1, 2 or 4 query heads per key/value head), ragged lengths,
T = 1, with and without QK-norm and logits scaling, and a nonzero position origin.  The full
workloads run in the launch configuration the benchmark times and are compared on sampled query
rows of every head (a query row depends on all earlier keys, which the oracle takes in full).

Tolerances are the mixer's (relative L2 <= 2e-2 for bf16 outputs).  The scores are formed from
bf16 queries (already scaled by s_t log2(e)/sqrt(d)) and bf16 keys, and P is rounded to bf16
before P V, which puts o within a few 1e-3 of the exact value.  The key cache written by the
prefill is the normalised key rounded once to bf16 from fp32: each entry must be within one
bf16 ulp (2^-7 relative) plus fp32 rounding of the oracle's fp64 value.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa
import synth
from synth import host_bits, rel_l2

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_attn(inp, with_cache=True):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    q, k, v, g = (inp[n].to(dev) for n in ("q", "k", "v", "g"))
    o_raw = torch.empty(q.shape, dtype=torch.float32, device=dev)
    cache = torch.empty_like(k) if with_cache else None
    qw = None if inp["qw"] is None else inp["qw"].to(dev)
    kw = None if inp["kw"] is None else inp["kw"].to(dev)
    y = lt.lightning_attn_prefill(q, k, v, g, inp["a"], q_norm_w=qw, k_norm_w=kw,
                                  rms_eps=inp["eps"], pos0=inp["pos0"], o_raw=o_raw,
                                  key_cache_out=cache)
    torch.cuda.synchronize()
    return dict(y=y.float().cpu(), o=o_raw.cpu(), cache=None if cache is None else cache.float().cpu())


def oracle_attn(inp, rows=None):
    return oa.attn_prefill(*(host_bits(inp[n].cpu()) for n in ("q", "k", "v", "g")),
                           None if inp["qw"] is None else inp["qw"].cpu().numpy(),
                           None if inp["kw"] is None else inp["kw"].cpu().numpy(),
                           None, a=inp["a"], eps=inp["eps"], pos0=inp["pos0"], rows=rows,
                           want_k_hat=rows is None)


def compare(gpu, ref, inp, rows=None, label=""):
    B, Hq = inp["B"], inp["Hq"]
    rows = slice(None) if rows is None else torch.as_tensor(rows)
    worst = dict(y=0.0, o=0.0)
    for b in range(B):
        for h in range(Hq):
            worst["y"] = max(worst["y"], rel_l2(gpu["y"][b, rows, h].numpy(), ref["y"][b, :, h]))
            worst["o"] = max(worst["o"], rel_l2(gpu["o"][b, rows, h].numpy(), ref["o"][b, :, h]))
    print(f"[parity] attention {label}: " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    assert worst["y"] <= TOL and worst["o"] <= TOL, (label, worst)
    return worst


def check_cache(gpu, ref, label):
    if gpu["cache"] is None:
        return
    got = gpu["cache"].numpy().astype(np.float64)
    exact = ref["k_hat"]
    err = np.abs(got - exact)
    bound = 2.0 ** -7 * np.abs(exact) + 2.0 ** -20 * (np.abs(exact) + 1e-30)
    i = int(np.argmax(err - bound))
    assert err.flat[i] <= bound.flat[i], (label, got.flat[i], exact.flat[i])


SMALL = [
    # (label, B, T, Hq, Hkv, a, qk_norm, pos0)
    ("gqa2_ragged", 1, 300, 4, 2, 500.0, True, 0),
    ("gqa4_two_batches", 2, 1000, 8, 2, 600.0, True, 0),
    ("mha_short_ragged", 1, 65, 2, 2, 900.0, True, 0),
    # one query head per workgroup: three 256-query tiles, so wavefronts run fully masked
    # blocks (up to three per tile) and tiles end mid-block
    ("mha_three_tiles", 1, 700, 2, 2, 500.0, True, 0),
    ("gqa2_no_norm_no_scale", 1, 513, 4, 2, 0.0, False, 0),
    ("gqa8_far_position", 1, 777, 8, 1, 500.0, True, 100000),
    ("single_token", 3, 1, 4, 2, 500.0, True, 5),
    ("gqa2_two_blocks_exact", 1, 128, 2, 1, 300.0, True, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_attn_prefill_small(case):
    label, B, T, Hq, Hkv, a, norm, pos0 = case
    inp = synth.make_custom_attn(B, T, Hq, Hkv, a=a, qk_norm=norm, seed=len(label) * 31 + T,
                                 pos0=pos0)
    ref = oracle_attn(inp)
    gpu = gpu_attn(inp)
    compare(gpu, ref, inp, label=label)
    check_cache(gpu, ref, label)


def test_attn_prefill_deterministic_and_cache_optional():
    inp = synth.make_custom_attn(1, 700, 4, 2, seed=77)
    a = gpu_attn(inp, with_cache=True)
    b = gpu_attn(inp, with_cache=False)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["o"], b["o"])


def _sampled_rows(T, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, n - 4, replace=False).tolist()) | {0, 1, T // 2, T - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("spec_name,n_rows", [("attn_qwen17_32k", 96), ("attn_qwen17_512k", 20)])
@pytest.mark.timeout(600)
def test_attn_prefill_full_sampled_rows(spec_name, n_rows):
    spec = synth.WORKLOADS[spec_name]
    inp = synth.make_attn(spec, device="cuda")
    gpu = gpu_attn(inp, with_cache=False)
    rows = _sampled_rows(inp["T"], n_rows, seed=len(spec_name))
    host = dict(inp, **{n: inp[n].cpu() for n in ("q", "k", "v", "g")},
                qw=inp["qw"].cpu(), kw=inp["kw"].cpu())
    ref = oracle_attn(host, rows=rows)
    compare(gpu, ref, inp, rows=rows, label=f"{spec.name} rows {len(rows)}")


# ---- decode -----------------------------------------------------------------------------------------

def _decode_inputs(B, Hq, Hkv, cap, lengths, seed, qk_norm=True):
    gen = torch.Generator().manual_seed(seed)
    d = 128

    def rnd(*shape):
        return torch.randn(*shape, generator=gen).to(torch.bfloat16)

    inp = dict(q=rnd(B, Hq, d), k_new=rnd(B, Hkv, d), v_new=rnd(B, Hkv, d), g=rnd(B, Hq, d),
               k_cache=rnd(B, cap, Hkv, d), v_cache=rnd(B, cap, Hkv, d), lengths=list(lengths),
               qw=None, kw=None)
    if qk_norm:
        inp["qw"] = 0.5 + torch.rand(d, generator=gen)
        inp["kw"] = 0.5 + torch.rand(d, generator=gen)
    return inp


def _run_decode(inp, a, device_cache=None):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    kc = inp["k_cache"].to(dev) if device_cache is None else device_cache[0]
    vc = inp["v_cache"].to(dev) if device_cache is None else device_cache[1]
    o_raw = torch.empty(inp["q"].shape, dtype=torch.float32, device=dev)
    y = lt.lightning_attn_decode_step(
        inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev), inp["g"].to(dev), kc, vc,
        inp["lengths"], a, q_norm_w=None if inp["qw"] is None else inp["qw"].to(dev),
        k_norm_w=None if inp["kw"] is None else inp["kw"].to(dev), o_raw=o_raw)
    torch.cuda.synchronize()
    return y.float().cpu(), o_raw.cpu(), kc, vc


def _check_decode(inp, a, label, y, o, kc, vc):
    ref = oa.attn_decode_step(*(host_bits(inp[n]) for n in ("q", "k_new", "v_new", "g")),
                              host_bits(inp["k_cache"]), host_bits(inp["v_cache"]),
                              np.array(inp["lengths"]),
                              None if inp["qw"] is None else inp["qw"].numpy(),
                              None if inp["kw"] is None else inp["kw"].numpy(), a=a)
    B, Hq = y.shape[:2]
    worst = dict(y=0.0, o=0.0)
    for b in range(B):
        for h in range(Hq):
            worst["y"] = max(worst["y"], rel_l2(y[b, h].numpy(), ref["y"][b, h]))
            worst["o"] = max(worst["o"], rel_l2(o[b, h].numpy(), ref["o"][b, h]))
    print(f"[parity] attention decode {label}: " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    assert worst["y"] <= TOL and worst["o"] <= TOL, (label, worst)
    # the new token's row: the normalised key (one bf16 rounding) and the value; nothing else
    for b, n in enumerate(inp["lengths"]):
        got_k = kc[b, n].float().cpu().numpy().astype(np.float64)
        exact = ref["k_hat"][b]
        assert np.all(np.abs(got_k - exact) <= 2.0 ** -7 * np.abs(exact) + 1e-30), label
        assert torch.equal(vc[b, n].cpu(), inp["v_new"][b]), label
        keep = torch.ones(kc.shape[1], dtype=torch.bool)
        keep[n] = False
        assert torch.equal(kc[b].cpu()[keep], inp["k_cache"][b][keep]), label
        assert torch.equal(vc[b].cpu()[keep], inp["v_cache"][b][keep]), label


DECODE = [
    # (label, B, Hq, Hkv, capacity, lengths, a, qk_norm)
    ("gqa2_mixed_lengths", 4, 4, 2, 6000, (0, 1, 777, 5000), 500.0, True),
    ("mha", 2, 2, 2, 3000, (2047, 2048), 900.0, True),
    ("gqa4", 3, 8, 2, 4200, (4097, 0, 31), 600.0, True),
    ("gqa8_no_norm_no_scale", 2, 8, 1, 2500, (2499, 100), 0.0, False),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_attn_decode_small(case):
    label, B, Hq, Hkv, cap, lengths, a, norm = case
    inp = _decode_inputs(B, Hq, Hkv, cap, lengths, seed=len(label), qk_norm=norm)
    _check_decode(inp, a, label, *_run_decode(inp, a))


@pytest.mark.timeout(300)
def test_attn_decode_full_context():
    """One token at position 524287 of the Qwen3-1.7B-shaped attention layer (B = 1)."""
    cap = 524288
    inp = _decode_inputs(1, 16, 8, cap, (cap - 1,), seed=99)
    _check_decode(inp, 500.0, "B=1 context 524287", *_run_decode(inp, 500.0))


def test_attn_prefill_then_decode():
    """prefill(T) writing the key cache, then a decode step at position T, equals row T of the
    oracle's prefill of T + 1 tokens."""
    import long_context_hybrid_amd.lightning as lt

    T, Hq, Hkv = 700, 4, 2
    inp = synth.make_custom_attn(1, T + 1, Hq, Hkv, seed=123)
    ref = oracle_attn(inp, rows=np.array([T]))
    dev = torch.device("cuda")
    kc = torch.zeros((1, T + 8, Hkv, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    head = {n: inp[n][:, :T].contiguous().to(dev) for n in ("q", "k", "v", "g")}
    lt.lightning_attn_prefill(head["q"], head["k"], head["v"], head["g"], inp["a"],
                              q_norm_w=inp["qw"].to(dev), k_norm_w=inp["kw"].to(dev),
                              key_cache_out=kc[:, :T])
    vc[:, :T] = head["v"]
    y = lt.lightning_attn_decode_step(inp["q"][:, T].to(dev), inp["k"][:, T].to(dev),
                                      inp["v"][:, T].to(dev), inp["g"][:, T].to(dev), kc, vc, [T],
                                      inp["a"], q_norm_w=inp["qw"].to(dev),
                                      k_norm_w=inp["kw"].to(dev))
    torch.cuda.synchronize()
    for h in range(Hq):
        assert rel_l2(y[0, h].float().cpu().numpy(), ref["y"][0, 0, h]) <= TOL


# ---- decode with the lengths in device memory ------------------------------------------------------

def _run_decode_dev(inp, a, max_length=None, lengths=None):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    o_raw = torch.empty(inp["q"].shape, dtype=torch.float32, device=dev)
    lens = torch.tensor(inp["lengths"] if lengths is None else lengths, dtype=torch.int64,
                        device=dev)
    y = lt.lightning_attn_decode_step(
        inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev), inp["g"].to(dev), kc, vc,
        lens, a, q_norm_w=None if inp["qw"] is None else inp["qw"].to(dev),
        k_norm_w=None if inp["kw"] is None else inp["kw"].to(dev), o_raw=o_raw,
        max_length=max_length)
    torch.cuda.synchronize()
    return y.float().cpu(), o_raw.cpu(), kc, vc


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_attn_decode_device_lengths_match_host(case):
    """The device-lengths entry point runs the same kernels: with the bound at capacity - 1
    (most splits of the short rows exit at once) y, o and both caches equal the host-lengths
    call bit for bit, and the oracle."""
    label, B, Hq, Hkv, cap, lengths, a, norm = case
    inp = _decode_inputs(B, Hq, Hkv, cap, lengths, seed=len(label), qk_norm=norm)
    host = _run_decode(inp, a)
    devr = _run_decode_dev(inp, a)
    for x, y in zip(host, devr):
        assert torch.equal(x, y), label
    _check_decode(inp, a, label + " (device lengths)", *devr)


@pytest.mark.timeout(300)
def test_attn_decode_device_lengths_full_context():
    """One token at position 524287 of the Qwen3-1.7B-shaped attention layer with the length in
    device memory (the bound sizes 256 splits of 2048 keys)."""
    cap = 524288
    inp = _decode_inputs(1, 16, 8, cap, (cap - 1,), seed=98)
    _check_decode(inp, 500.0, "B=1 context 524287 (device lengths)", *_run_decode_dev(inp, 500.0))


def test_attn_decode_device_lengths_large_batch():
    """B = 80, more rows than host lengths allow, lengths from 0 across a split boundary."""
    B, Hq, Hkv, cap = 80, 4, 2, 2100
    lengths = [(i * 523) % 2100 for i in range(B)]
    assert 0 in lengths and max(lengths) >= 2048
    inp = _decode_inputs(B, Hq, Hkv, cap, lengths, seed=80)
    _check_decode(inp, 500.0, "B=80 device lengths",
                  *_run_decode_dev(inp, 500.0, max_length=max(lengths)))


def test_attn_decode_device_lengths_invalid_rows():
    """Rows whose device length is negative or above max_length get NaN outputs and no cache
    write; the other rows are computed as usual."""
    B, Hq, Hkv, cap = 4, 4, 2, 3000
    good = [17, 2500, 0, 900]
    bad = [17, 2999, -5, 900]  # row 1 above the bound 2600, row 2 negative
    inp = _decode_inputs(B, Hq, Hkv, cap, good, seed=5)
    y, o, kc, vc = _run_decode_dev(inp, 500.0, max_length=2600, lengths=bad)
    for b in (1, 2):
        assert torch.isnan(y[b]).all() and torch.isnan(o[b]).all()
        assert torch.equal(kc[b].cpu(), inp["k_cache"][b])
        assert torch.equal(vc[b].cpu(), inp["v_cache"][b])
    ref_y, ref_o, ref_kc, ref_vc = _run_decode(inp, 500.0)
    for b in (0, 3):
        assert torch.equal(y[b], ref_y[b]) and torch.equal(o[b], ref_o[b])
        assert torch.equal(kc[b], ref_kc[b]) and torch.equal(vc[b], ref_vc[b])


def test_attn_decode_device_lengths_graph_loop():
    """A decode loop captured once in a HIP graph: each replay appends one token at the lengths
    held on the GPU, which the loop advances on the device between replays.  Every replay's y and
    the final caches equal eager host-lengths steps with the same inputs."""
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    B, Hq, Hkv, cap, steps = 3, 8, 2, 4200, 4
    start = [2046, 5, 300]  # row 0 crosses the split boundary at 2048
    inp = _decode_inputs(B, Hq, Hkv, cap, start, seed=31)
    gen = torch.Generator().manual_seed(32)
    news = [{n: torch.randn(B, h, 128, generator=gen).to(torch.bfloat16)
             for n, h in (("q", Hq), ("k_new", Hkv), ("v_new", Hkv), ("g", Hq))}
            for _ in range(steps)]
    qw, kw = inp["qw"].to(dev), inp["kw"].to(dev)
    # eager reference: host lengths, one step after another on its own caches
    kc_ref, vc_ref = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    ys_ref = []
    for s in range(steps):
        x = {n: news[s][n].to(dev) for n in news[s]}
        y = lt.lightning_attn_decode_step(x["q"], x["k_new"], x["v_new"], x["g"], kc_ref, vc_ref,
                                          [L + s for L in start], 500.0, q_norm_w=qw, k_norm_w=kw)
        ys_ref.append(y.clone())
    # the graph: static inputs, device lengths, a workspace sized for the bound
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    sq = {n: torch.empty_like(news[0][n], device=dev) for n in news[0]}
    lens = torch.tensor(start, dtype=torch.int64, device=dev)
    y = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    bound = cap - 1
    ws = torch.empty(lt.lightning_attn_decode_workspace_size(B, Hq, Hkv, 128, bound),
                     dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        # capture only (no step runs): the caches are written by the replays alone
        with torch.cuda.graph(graph, stream=side):
            lt.lightning_attn_decode_step(sq["q"], sq["k_new"], sq["v_new"], sq["g"], kc, vc,
                                          lens, 500.0, q_norm_w=qw, k_norm_w=kw, y=y,
                                          workspace=ws, max_length=bound,
                                          stream=torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for s in range(steps):
        for n in sq:
            sq[n].copy_(news[s][n].to(dev))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ys_ref[s]), f"replay {s}"
        lens += 1
        torch.cuda.synchronize()
    assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref)
    assert lens.tolist() == [L + steps for L in start]
