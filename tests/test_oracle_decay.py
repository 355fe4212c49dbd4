"""Pins of the data-dependent-decay oracle (oracle/decay.py), none of which re-types it.

* A constant per-token decay log2(alpha_t) = log2(lambda_h) reproduces the fixed-decay oracle
  (oracle.prefill, the C recurrence written separately) -- the special case the variant
  generalises.
* Brute force on tiny inputs: o_t = (prod_{s<=t} alpha_s) q~_t S_0 + sum_{j<=t}
  (prod_{j<s<=t} alpha_s)(q~_t . k~_j) v_j, with the products taken directly.
* A decay of 0 at token t (alpha_t = 2^-200) forgets everything before t: the outputs from t on
  equal a fresh prefill starting at t with a zero state (same positions).
* The decode step equals the next token of the prefill, and its state.
"""
import math

import numpy as np
import torch

import oracle
from oracle import decay as od
import synth
from synth import host_bits


def _inputs(B, T, H, d, seed, dtype=torch.float32):
    inp = synth.make_custom_prefill(B, T, H, d, dtype=dtype, seed=seed, state="randn",
                                    rope_base=1e4)
    gen = torch.Generator().manual_seed(seed + 1)
    lg = -torch.rand((B, T, H), generator=gen) * 0.3  # alpha in [0.81, 1]
    return inp, lg.numpy().astype(np.float32)


def _args(inp):
    return [host_bits(inp[n]) for n in ("q", "k", "v", "g")] + [inp["qw"].numpy(), inp["kw"].numpy()]


def test_constant_decay_equals_fixed_decay_oracle():
    inp, _ = _inputs(2, 40, 3, 16, seed=1)
    lams = [0.9, 0.5, 0.999]
    lg = np.broadcast_to(np.log2(np.array(lams, dtype=np.float64)).astype(np.float32),
                         (2, 40, 3)).copy()
    # the fixed oracle takes lambda in fp64; feed it exactly the float32 value used here
    lam32 = [float(2.0 ** float(x)) for x in lg[0, 0]]
    a = od.prefill_dd(*_args(inp), lg, inp["rope_base"], state_in=inp["state_in"].numpy())
    b = oracle.prefill(*_args(inp), lam32, inp["rope_base"], state_in=inp["state_in"].numpy())
    assert np.max(np.abs(a["y"] - b["y"])) <= 1e-12
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-11
    assert np.max(np.abs(a["state"] - b["state"])) <= 1e-12


def test_bruteforce_products():
    B, T, H, d = 1, 9, 1, 8
    inp, lg = _inputs(B, T, H, d, seed=2)
    r = od.prefill_dd(*_args(inp), lg, inp["rope_base"], state_in=inp["state_in"].numpy())
    # the prologue vectors from the (pinned) per-vector routines
    qf = inp["q"][0, :, 0].double().numpy()
    kf = inp["k"][0, :, 0].double().numpy()
    vf = inp["v"][0, :, 0].double().numpy()
    qw, kw = inp["qw"][0].double().numpy(), inp["kw"][0].double().numpy()
    qt = [oracle.rope(oracle.rmsnorm(qf[t], qw), t, inp["rope_base"]) for t in range(T)]
    kt = [oracle.rope(oracle.rmsnorm(kf[t], kw), t, inp["rope_base"]) / math.sqrt(d)
          for t in range(T)]
    a = 2.0 ** lg[0, :, 0].astype(np.float64)
    S0 = inp["state_in"][0, 0].double().numpy()
    for t in range(T):
        o = np.prod(a[:t + 1]) * (qt[t] @ S0)
        for j in range(t + 1):
            o = o + np.prod(a[j + 1:t + 1]) * float(qt[t] @ kt[j]) * vf[j]
        assert np.max(np.abs(o - r["o"][0, t])) <= 1e-12 * max(1.0, np.max(np.abs(o)))


def test_zero_decay_forgets_the_past():
    B, T, H, d, t0 = 1, 30, 2, 16, 11
    inp, lg = _inputs(B, T, H, d, seed=3)
    lg = lg.copy()
    lg[:, t0] = -200.0  # alpha = 2^-200: the state before t0 vanishes at fp64 precision
    full = od.prefill_dd(*_args(inp), lg, inp["rope_base"], state_in=inp["state_in"].numpy())
    tail = {n: inp[n][:, t0:].contiguous() for n in ("q", "k", "v", "g")}
    args = [host_bits(tail[n]) for n in ("q", "k", "v", "g")] + [inp["qw"].numpy(), inp["kw"].numpy()]
    part = od.prefill_dd(*args, np.ascontiguousarray(lg[:, t0:]), inp["rope_base"], pos0=t0)
    assert np.max(np.abs(full["o"][:, t0:] - part["o"])) <= 1e-12
    assert np.max(np.abs(full["state"] - part["state"])) <= 1e-12


def test_decode_matches_next_token():
    B, T, H, d = 2, 25, 2, 16
    inp, lg = _inputs(B, T + 1, H, d, seed=4)
    full = od.prefill_dd(*_args(inp), lg, inp["rope_base"], state_in=inp["state_in"].numpy())
    head = {n: inp[n][:, :T].contiguous() for n in ("q", "k", "v", "g")}
    hargs = [host_bits(head[n]) for n in ("q", "k", "v", "g")] + [inp["qw"].numpy(), inp["kw"].numpy()]
    first = od.prefill_dd(*hargs, np.ascontiguousarray(lg[:, :T]), inp["rope_base"],
                          state_in=inp["state_in"].numpy())
    step = od.decode_step_dd(*(host_bits(inp[n][:, T].contiguous()) for n in ("q", "k", "v", "g")),
                             inp["qw"].numpy(), inp["kw"].numpy(), np.ascontiguousarray(lg[:, T]),
                             inp["rope_base"], np.full(B, T), first["state"].reshape(B, H, d, d))
    y = full["y"].reshape(B, H, T + 1, d)[:, :, T]
    s = full["state"].reshape(B, H, d, d)
    assert np.max(np.abs(step["y"] - y)) <= 1e-12
    assert np.max(np.abs(step["state"] - s)) <= 1e-12
