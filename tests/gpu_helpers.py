"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding and the fp64
oracle on the same seeded inputs, and compare them slice by slice.

Tolerances (max over (b, h) slices of the relative L2 error ||x - ref|| / ||ref||):
  * bf16 activations: y and o <= 2e-2; fp32 state <= 1e-4.
  * fp32 activations: y, o and state <= 1e-4.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import host_bits, rel_l2

TOL = {torch.bfloat16: dict(y=2e-2, o=2e-2, state=1e-4),
       torch.float32: dict(y=1e-4, o=1e-4, state=1e-4)}

# y_t = RMSNorm(o_t) * w_o * sigmoid(g_t) is scale invariant in o_t, so a row whose o_t is tiny
# compared with the other rows turns the (absolute) rounding error of the bf16 products into an
# O(1) error of y_t; with lambda = 0, o_t = (q~_t . k~_t) v_t crosses zero whenever the score
# does.  For bf16 activations y is therefore compared on the rows with ||o_t|| >= 5% of the
# slice's RMS row norm; the other rows must still be finite and bounded by sqrt(d) * max|w_o|,
# and may be at most MAX_ILL_ROWS of the slice.  o and the state are compared on every row.
ILL_ROW_FRAC = 0.05
MAX_ILL_ROWS = 0.10


def gpu_prefill(inp, chunk=0, segments=0, want_o=True, want_state=True, pos0=None,
                state_in=None, ow=None, device="cuda"):
    import long_context_hybrid_amd.lightning as lt

    B, T, H, d = inp["q"].shape
    dev = torch.device(device)
    q, k, v, g = (inp[n].to(dev) for n in ("q", "k", "v", "g"))
    s_in = inp["state_in"] if state_in is None else state_in
    s_in = None if s_in is None else s_in.to(dev)
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev) if want_state else None
    o_raw = torch.empty((B, T, H, d), dtype=torch.float32, device=dev) if want_o else None
    ow = inp.get("ow") if ow is None else ow
    y = lt.lightning_prefill(q, k, v, g, inp["qw"].to(dev), inp["kw"].to(dev), inp["lambdas"],
                             inp["rope_base"], rms_eps=inp["eps"],
                             pos0=inp["pos0"] if pos0 is None else pos0, state_in=s_in,
                             state_out=s_out, o_raw=o_raw,
                             o_norm_w=None if ow is None else ow.to(dev), chunk=chunk,
                             segments=segments)
    torch.cuda.synchronize()
    return dict(y=y.float().cpu(), o=None if o_raw is None else o_raw.cpu(),
                state=None if s_out is None else s_out.cpu())


def oracle_prefill(inp, slices=None, pos0=None, state_in=None, ow=None):
    s_in = inp["state_in"] if state_in is None else state_in
    ow = inp.get("ow") if ow is None else ow
    return oracle.prefill(host_bits(inp["q"]), host_bits(inp["k"]), host_bits(inp["v"]),
                          host_bits(inp["g"]), inp["qw"].cpu().numpy(), inp["kw"].cpu().numpy(),
                          inp["lambdas"], inp["rope_base"], eps=inp["eps"],
                          pos0=inp["pos0"] if pos0 is None else pos0,
                          state_in=None if s_in is None else s_in.cpu().numpy(),
                          ow=None if ow is None else ow.cpu().numpy(), slices=slices)


def compare_prefill(gpu, ref, dtype, what=("y", "o", "state"), tol=None, label=""):
    """Max relative L2 error per quantity over the oracle's slices; asserts the tolerance."""
    tol = dict(TOL[dtype], **(tol or {}))
    worst = {}
    ill_rows = 0
    for i, (b, h) in enumerate(ref["slices"]):
        for name in what:
            if gpu.get(name) is None or ref.get(name) is None:
                continue
            got = (gpu[name][b, h] if name == "state" else gpu[name][b, :, h]).numpy()
            want = ref[name][i]
            if name == "y" and dtype == torch.bfloat16 and ref.get("o") is not None:
                norms = np.linalg.norm(ref["o"][i], axis=1)
                keep = norms >= ILL_ROW_FRAC * np.sqrt(np.mean(norms ** 2))
                bad = ~keep
                ill_rows = max(ill_rows, int(bad.sum()))
                assert bad.mean() <= MAX_ILL_ROWS, f"{label}: {bad.mean():.1%} ill-conditioned rows"
                bound = np.sqrt(want.shape[1]) * 1.5 + 1e-6
                assert np.all(np.isfinite(got[bad])) and np.all(
                    np.linalg.norm(got[bad], axis=1) <= bound), f"{label}: bad y on tiny-o rows"
                got, want = got[keep], want[keep]
            err = rel_l2(got, want)
            worst[name] = max(worst.get(name, 0.0), err)
    print(f"[parity] {label} " + " ".join(f"{k}={v:.3e}" for k, v in worst.items())
          + (f" (y skips <= {ill_rows} tiny-o rows per slice)" if ill_rows else ""), flush=True)
    for name, err in worst.items():
        assert np.isfinite(err) and err <= tol[name], f"{label}: {name} rel L2 {err:.3e} > {tol[name]:.1e}"
    return worst
