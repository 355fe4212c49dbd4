"""Parity of the whole RNN layer on the GPU (QKVZ GEMM -> mixer -> W_o GEMM) with the oracle.

The library's workspace holds the layer's intermediates after a call (documented in the C
header), so each stage is compared as well as the output:
  * projections: the GEMM accumulates in fp32 and rounds once to the storage dtype, the oracle
    rounds the exact fp64 product.  They can differ only where the fp32 sum s lands on the other
    side of a rounding boundary: with the exact value e, |s - e| <= K 2^-24 sum_i |x_i w_i|
    (the worst-case bound of a K-term fp32 sum), so |got - ref| <= |got - s| + |s - e| +
    |e - ref| <= 2^-8 |got| + K 2^-24 sum_i |x_i w_i| + 2^-8 |ref|.  Ternary inputs (integer
    projections, exact in both) must agree bit for bit.
  * y per (b, h) slice and the layer output per batch row: relative L2 <= 2e-2 (bf16) or 1e-4
    (fp32), the mixer's output tolerances.
  * state per (b, h): 1e-4, the mixer's state tolerance, wherever both sides see the same
    projections (ternary and fp32 cases).  With Gaussian bf16 inputs the projections of the two
    sides differ by one bf16 ulp (relative <= 2^-7) in a fraction f ~ 1e-3 of entries, which
    moves the state by about sqrt(f) 2^-8 ~ 1.2e-4 relative; that case is held to 1e-3.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import layer as ol
import synth
from synth import host_bits, rel_l2

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: dict(y=2e-2, out=2e-2, state=1e-4, state_gauss=1e-3, proj_flips=1e-2),
       torch.float32: dict(y=1e-4, out=1e-4, state=1e-4, state_gauss=1e-4, proj_flips=None)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _round256(n):
    return (n + 255) // 256 * 256


def gpu_layer(inp, segments=0, state_in="inp", pos0=None):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    B, T, H, d, dm, dt = inp["B"], inp["T"], inp["H"], inp["d"], inp["d_model"], inp["dtype"]
    s_in = inp["state_in"] if state_in == "inp" else state_in
    s_in = None if s_in is None else s_in.to(dev)
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    need = lt.lightning_layer_prefill_workspace_size(B, T, H, d, dm, dt, 0, segments)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = lt.lightning_layer_prefill(inp["x"].to(dev), inp["w_qkvz"].to(dev), inp["w_o"].to(dev),
                                     inp["qw"].to(dev), inp["kw"].to(dev), inp["lambdas"],
                                     inp["rope_base"], H, d, rms_eps=inp["eps"],
                                     pos0=inp["pos0"] if pos0 is None else pos0, state_in=s_in,
                                     state_out=s_out, segments=segments, workspace=ws)
    torch.cuda.synchronize()
    es = 2 if dt == torch.bfloat16 else 4
    n_proj = B * T * 4 * H * d * es
    proj = ws[:n_proj].view(dt).reshape(B, T, 4 * H * d)
    y0 = _round256(n_proj)
    y = ws[y0:y0 + B * T * H * d * es].view(dt).reshape(B, T, H * d)
    return dict(out=out.float().cpu(), state=s_out.cpu(), proj=proj.float().cpu(),
                y=y.float().cpu())


def oracle_layer(inp, state_in="inp", pos0=None):
    s_in = inp["state_in"] if state_in == "inp" else state_in
    return ol.layer_prefill(host_bits(inp["x"]), host_bits(inp["w_qkvz"]), host_bits(inp["w_o"]),
                            inp["qw"].numpy(), inp["kw"].numpy(), inp["lambdas"],
                            inp["rope_base"], inp["H"], inp["d"], eps=inp["eps"],
                            pos0=inp["pos0"] if pos0 is None else pos0,
                            state_in=None if s_in is None else s_in.numpy())


def acc_bound(x, w):
    """K 2^-24 sum_i |x_i w_i| for every projection entry: x [rows, K], w [N, K] (torch)."""
    xa = x.double().abs().reshape(-1, x.shape[-1]).numpy()
    wa = w.double().abs().numpy()
    return x.shape[-1] * 2.0 ** -24 * (xa @ wa.T)


def check_proj(got, ref, dtype, exact, label, bound=None):
    got = got.numpy().astype(np.float64).reshape(ref.shape)
    if exact:
        assert np.array_equal(got, ref), f"{label}: projections differ"
        return 0.0
    if dtype == torch.float32:
        err = rel_l2(got, ref)
        assert err <= 1e-6, f"{label}: fp32 projections rel L2 {err:.2e}"
        return err
    diff = got != ref
    frac = float(diff.mean())
    allowed = 2.0 ** -8 * (np.abs(got) + np.abs(ref)) + bound.reshape(ref.shape)
    excess = np.abs(got - ref) - allowed
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (f"{label}: projection {i} is {got.flat[i]!r}, oracle "
                                 f"{ref.flat[i]!r}, allowed difference {allowed.flat[i]:.3e}")
    assert frac <= TOL[dtype]["proj_flips"], f"{label}: {frac:.2e} of projections differ"
    return frac


def compare_layer(gpu, ref, inp, exact_proj=False, label=""):
    dt, B, T, H, d = inp["dtype"], inp["B"], inp["T"], inp["H"], inp["d"]
    tol = TOL[dt]
    bound = None if exact_proj or dt == torch.float32 else acc_bound(inp["x"], inp["w_qkvz"])
    flips = check_proj(gpu["proj"], ref["proj"], dt, exact_proj, label, bound)
    worst = dict(y=0.0, out=0.0, state=0.0)
    y = gpu["y"].numpy().reshape(B, T, H, d)
    ry = ref["y"].reshape(B, T, H, d)
    for b in range(B):
        worst["out"] = max(worst["out"], rel_l2(gpu["out"][b].numpy(), ref["out"][b]))
        for h in range(H):
            worst["y"] = max(worst["y"], rel_l2(y[b, :, h], ry[b, :, h]))
            worst["state"] = max(worst["state"], rel_l2(gpu["state"][b, h].numpy(),
                                                        ref["state"][b, h]))
    print(f"[parity] layer {label}: proj flips {flips:.2e} " +
          " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    stol = tol["state"] if (exact_proj or dt == torch.float32) else tol["state_gauss"]
    assert worst["y"] <= tol["y"], (label, worst)
    assert worst["out"] <= tol["out"], (label, worst)
    assert worst["state"] <= stol, (label, worst)
    return worst


LAYER_CASES = [
    # (label, B, T, H, d, d_model, dtype, values, state, lambdas, segments list)
    ("bf16_gauss_ragged", 1, 300, 2, 128, 256, torch.bfloat16, "gauss", "randn", None, (0, 3)),
    ("bf16_ternary_exact", 2, 1000, 2, 128, 256, torch.bfloat16, "ternary", "randn", None, (0, 4)),
    ("bf16_gauss_wide_model", 1, 777, 4, 64, 640, torch.bfloat16, "gauss", "zeros",
     (0.0, 0.5, 0.99, 1.0), (0, 2)),
    ("fp32_gauss", 2, 257, 2, 64, 96, torch.float32, "gauss", "randn", (0.9, 0.999), (0, 2)),
    ("fp32_d128", 1, 513, 2, 128, 200, torch.float32, "gauss", "zeros", None, (0, 5)),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_prefill_small(case):
    label, B, T, H, d, dm, dt, values, state, lams, segs = case
    inp = synth.make_custom_layer(B, T, H, d, dm, dtype=dt, seed=zlib.crc32(label.encode()) % 9973,
                                  lambdas=lams, rope_base=1e4 if d == 64 else 1e6, state=state,
                                  values=values)
    ref = oracle_layer(inp)
    for seg in segs:
        compare_layer(gpu_layer(inp, segments=seg), ref, inp, exact_proj=values == "ternary",
                      label=f"{label} segments={seg}")


def test_layer_split_composition_and_position_origin():
    """layer(T1) then layer(T2, pos0 = T1, state carried) matches the oracle's layer(T1 + T2)."""
    T1, T2 = 640, 500
    inp = synth.make_custom_layer(1, T1 + T2, 2, 128, 256, seed=41, state="randn",
                                  values="ternary")
    ref = oracle_layer(inp)
    a = dict(inp, x=inp["x"][:, :T1].contiguous(), T=T1)
    g1 = gpu_layer(a, segments=2)
    b = dict(inp, x=inp["x"][:, T1:].contiguous(), T=T2)
    g2 = gpu_layer(b, segments=3, state_in=g1["state"], pos0=T1)
    gpu = dict(out=torch.cat([g1["out"], g2["out"]], 1), state=g2["state"],
               proj=torch.cat([g1["proj"], g2["proj"]], 1), y=torch.cat([g1["y"], g2["y"]], 1))
    compare_layer(gpu, ref, inp, exact_proj=True, label="split layer")


# ---- decode ---------------------------------------------------------------------------------------

def gpu_layer_decode(inp):
    import long_context_hybrid_amd.lightning as lt

    dev = torch.device("cuda")
    B, H, d, dm, dt = inp["B"], inp["H"], inp["d"], inp["d_model"], inp["dtype"]
    s = inp["state_in"].to(dev).clone()
    need = lt.lightning_layer_decode_workspace_size(B, H, d, dm, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = lt.lightning_layer_decode_step(inp["x"].to(dev), inp["w_qkvz"].to(dev),
                                         inp["w_o"].to(dev), inp["qw"].to(dev), inp["kw"].to(dev),
                                         inp["lambdas"], inp["rope_base"], H, d,
                                         inp["positions"].to(dev), s, rms_eps=inp["eps"],
                                         workspace=ws)
    torch.cuda.synchronize()
    es = 2 if dt == torch.bfloat16 else 4
    n_proj = B * 4 * H * d * es
    proj = ws[:n_proj].view(dt).reshape(B, 4 * H * d)
    y0 = _round256(n_proj)
    y = ws[y0:y0 + B * H * d * es].view(dt).reshape(B, H * d)
    return dict(out=out.float().cpu(), state=s.cpu(), proj=proj.float().cpu(), y=y.float().cpu())


@pytest.mark.parametrize("spec_name,values", [("full", "gauss"), ("full_one_row", "gauss"),
                                              ("small_ternary", "ternary"),
                                              ("one_row_ternary", "ternary"),
                                              ("rows_4_ternary", "ternary"),
                                              ("rows_40_ternary", "ternary"),
                                              ("rows_5_wide", "gauss"),
                                              ("rows_33_wide", "gauss"),
                                              ("rows_100_wide", "gauss"),
                                              ("rows_70_ragged_out", "gauss"),
                                              ("small_fp32", "gauss")])
def test_layer_decode(spec_name, values):
    """1, 4, 5, 33, 40, 64, 70 and 100 batch rows (bf16; 64 and 1 with the full-size d_model 2048
    weights) and 3 (fp32): up to four rows take the VALU product, more the MFMA tiles.  5, 33
    and 100 rows (8192 projection columns) take the 64-row ring tiles, one ragged tile and a full
    one plus a ragged one; their output projection (256 and 512 columns, K = 2048) and the 70-row
    case's (200 columns, ragged, K = 512, three 32-row tiles) take the 32-row ring tiles.  The
    ternary inputs' projections are exact integers, so there the projections must match the
    oracle bit for bit."""
    if spec_name == "full":
        inp = synth.make_layer(synth.LAYER_DECODE_B64)
    elif spec_name == "full_one_row":  # the full-size weights with one sequence (batch 1)
        inp = synth.make_layer(synth.LAYER_DECODE_B64, B=1)
    elif spec_name == "small_ternary":
        inp = synth.make_custom_layer(5, 1, 2, 128, 256, seed=8, state="randn", values=values)
    elif spec_name == "one_row_ternary":
        inp = synth.make_custom_layer(1, 1, 2, 128, 256, seed=10, state="randn", values=values)
    elif spec_name == "rows_4_ternary":
        inp = synth.make_custom_layer(4, 1, 2, 128, 256, seed=12, state="randn", values=values)
    elif spec_name == "rows_40_ternary":
        inp = synth.make_custom_layer(40, 1, 2, 128, 256, seed=11, state="randn", values=values)
    elif spec_name == "rows_5_wide":
        inp = synth.make_custom_layer(5, 1, 16, 128, 512, seed=16, state="randn", values=values)
    elif spec_name == "rows_33_wide":
        inp = synth.make_custom_layer(33, 1, 16, 128, 512, seed=13, state="randn", values=values)
    elif spec_name == "rows_100_wide":
        inp = synth.make_custom_layer(100, 1, 16, 128, 256, seed=14, state="randn", values=values)
    elif spec_name == "rows_70_ragged_out":
        inp = synth.make_custom_layer(70, 1, 4, 128, 200, seed=15, state="randn", values=values)
    else:
        inp = synth.make_custom_layer(3, 1, 2, 64, 64, dtype=torch.float32, seed=9,
                                      state="randn", lambdas=(0.0, 0.95))
    ref = ol.layer_decode_step(host_bits(inp["x"]), host_bits(inp["w_qkvz"]),
                               host_bits(inp["w_o"]), inp["qw"].numpy(), inp["kw"].numpy(),
                               inp["lambdas"], inp["rope_base"], inp["H"], inp["d"],
                               inp["positions"].numpy(), inp["state_in"].numpy(), eps=inp["eps"])
    gpu = gpu_layer_decode(inp)
    dt, B, H, d = inp["dtype"], inp["B"], inp["H"], inp["d"]
    bound = acc_bound(inp["x"], inp["w_qkvz"]) if dt == torch.bfloat16 else None
    flips = check_proj(gpu["proj"], ref["proj"], dt, values == "ternary", spec_name, bound)
    tol = TOL[dt]
    worst = dict(out=max(rel_l2(gpu["out"][b].numpy(), ref["out"][b]) for b in range(B)),
                 y=max(rel_l2(gpu["y"][b, h * d:(h + 1) * d].numpy(), ref["y"][b, h * d:(h + 1) * d])
                       for b in range(B) for h in range(H)),
                 state=max(rel_l2(gpu["state"][b, h].numpy(), ref["state"][b, h])
                           for b in range(B) for h in range(H)))
    print(f"[parity] layer decode {spec_name}: proj flips {flips:.2e} " +
          " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    stol = tol["state"] if (values == "ternary" or dt == torch.float32) else tol["state_gauss"]
    assert worst["y"] <= tol["y"] and worst["out"] <= tol["out"] and worst["state"] <= stol, worst


@pytest.mark.timeout(300)
def test_layer_projections_many_tiles_per_workgroup():
    """Every projection of a 10277-token prefill with 8192 projection columns: 41 row blocks (the
    last one 37 rows) by 32 column blocks of the 256 x 256-tile GEMM, about five tiles per
    workgroup of its persistent grid, so each workgroup's later tiles start while its previous
    tile's epilogue stores are in flight.  All of them are compared with the oracle's products,
    and the layer output with the fp64 product of the GPU's own y and W_o."""
    inp = synth.make_custom_layer(1, 10277, 16, 128, 256, seed=21, state="zeros", values="gauss")
    gpu = gpu_layer(inp)
    x = host_bits(inp["x"])
    pq = ol.projections(x, host_bits(inp["w_qkvz"]), inp["H"], inp["d"])
    T, hd = inp["T"], inp["H"] * inp["d"]
    ref = np.concatenate([ol.widen(a).reshape(1, T, hd) for a in pq], -1)
    check_proj(gpu["proj"], ref, torch.bfloat16, False, "10277-token projections",
               acc_bound(inp["x"], inp["w_qkvz"]))
    yw = gpu["y"].double().reshape(T, hd).numpy() @ ol.widen(host_bits(inp["w_o"])).T
    ref_out = ol.widen(ol.store(yw, ol.BF16))
    bound = acc_bound(gpu["y"].reshape(T, hd).to(torch.bfloat16), inp["w_o"])
    check_proj(gpu["out"].reshape(T, -1), ref_out, torch.bfloat16, False,
               "10277-token output projection", bound)


# ---- the benchmarked layer at full size -----------------------------------------------------------

@pytest.mark.timeout(400)  # the oracle's share (two heads over 512K tokens) takes about a minute
def test_full_layer_qwen17_512k_sampled():
    """The 512K-token Qwen3-1.7B-shaped layer in the configuration the benchmark times.

    Checked against the oracle: the projections of 4096 sampled token rows (all heads); y and
    the final state of heads 0 and 15 over the whole sequence (the oracle computes those heads'
    projections for every token and runs its recurrence); and the layer output of the first 2048
    tokens (every head of the oracle over that prefix; a token's output depends on no later
    token).
    """
    import long_context_hybrid_amd.lightning as lt

    spec = synth.LAYER_QWEN17_512K
    dev = torch.device("cuda")
    inp = synth.make_layer(spec, device=dev)
    B, T, H, d, dm = inp["B"], inp["T"], inp["H"], inp["d"], inp["d_model"]
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(lt.lightning_layer_prefill_workspace_size(B, T, H, d, dm), dtype=torch.uint8,
                     device=dev)
    out = lt.lightning_layer_prefill(inp["x"], inp["w_qkvz"], inp["w_o"], inp["qw"], inp["kw"],
                                     inp["lambdas"], inp["rope_base"], H, d, rms_eps=inp["eps"],
                                     state_out=s_out, workspace=ws)
    torch.cuda.synchronize()
    n_proj = B * T * 4 * H * d * 2
    proj = ws[:n_proj].view(torch.bfloat16).reshape(B, T, 4 * H * d)
    y0 = _round256(n_proj)
    y = ws[y0:y0 + B * T * H * d * 2].view(torch.bfloat16).reshape(B, T, H, d)

    x = host_bits(inp["x"].cpu())
    w = host_bits(inp["w_qkvz"].cpu())
    wo = host_bits(inp["w_o"].cpu())
    qw, kw = inp["qw"].cpu().numpy(), inp["kw"].cpu().numpy()
    # 1. projections of sampled rows
    rows = np.sort(np.random.default_rng(0).choice(T, 4096, replace=False))
    pq = ol.projections(x[0, rows], w, H, d)
    ref_p = np.concatenate([ol.widen(a).reshape(len(rows), H * d) for a in pq], -1)
    xs = inp["x"][0, torch.as_tensor(rows, device=dev)].cpu()
    check_proj(proj[0, torch.as_tensor(rows, device=dev)].float().cpu(), ref_p, torch.bfloat16,
               False, "512K sampled projections", acc_bound(xs, inp["w_qkvz"].cpu()))
    # 2. y and state of sampled heads over the whole sequence
    heads = [0, 15]
    from oracle import prefill

    q, k, v, g = ol.projections(x, w, H, d, heads=heads)
    r = prefill(q, k, v, g, qw[heads], kw[heads], [inp["lambdas"][h] for h in heads],
                inp["rope_base"], eps=inp["eps"], want_o=False)
    for i, h in enumerate(heads):
        ey = rel_l2(y[0, :, h].float().cpu().numpy(), r["y"][i])
        es = rel_l2(s_out[0, h].cpu().numpy(), r["state"][i])
        print(f"[parity] layer 512K head {h}: y={ey:.3e} state={es:.3e}")
        assert ey <= 2e-2 and es <= TOL[torch.bfloat16]["state_gauss"], (h, ey, es)
    # 3. the layer output over a prefix
    n = 2048
    pre = ol.layer_prefill(np.ascontiguousarray(x[:, :n]), w, wo, qw, kw, inp["lambdas"],
                           inp["rope_base"], H, d, eps=inp["eps"])
    eo = rel_l2(out[0, :n].float().cpu().numpy(), pre["out"][0])
    print(f"[parity] layer 512K output over the first {n} tokens: out={eo:.3e}")
    assert eo <= 2e-2
