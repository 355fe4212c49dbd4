"""Pins of the gradient oracle (oracle/backward.py) against things other than itself.

* Finite differences of the forward oracle (the pinned C recurrence of oracle.c): every element
  of q, k, v, g, state_in and the three norm weights, on a tiny case with dyadic inputs so that
  each perturbed input is exact in fp32; Richardson-extrapolated central differences.  A dropped
  term, a wrong sign, index or transposed operand anywhere in the backward fails here.
* Transposition (Euler) identities of the core recurrence at 257 tokens: the outputs are linear
  in q~ and jointly linear in (v, S_0) and in (k~, S_0), so with F = <do, o> + <dS_out, S_T>,
  <dq~, q~> = <do, o> and <dv, v> + <dS_in, S_0> = <dk~, k~> + <dS_in, S_0> = F.
* Composition: the backward of two chained prefill calls (the second's d_state_in fed to the
  first as d_state_out) equals the backward of the whole call.
* lambda = 0 closed form: o_t = (q~_t . k~_t) v_t, so dv_t = (q~_t . k~_t) do_t and dS_in = 0.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob


def _dyadic(rng, shape, lo, hi, bits=8):
    return (np.round(rng.uniform(lo, hi, size=shape) * 2 ** bits) / 2 ** bits).astype(np.float32)


def _case(seed=3, B=1, T=6, H=2, d=8):
    rng = np.random.default_rng(seed)
    c = dict(
        q=_dyadic(rng, (B, T, H, d), -2, 2), k=_dyadic(rng, (B, T, H, d), -2, 2),
        v=_dyadic(rng, (B, T, H, d), -2, 2), g=_dyadic(rng, (B, T, H, d), -2, 2),
        qw=_dyadic(rng, (H, d), 0.5, 1.5), kw=_dyadic(rng, (H, d), 0.5, 1.5),
        ow=_dyadic(rng, (H, d), 0.5, 1.5), state_in=_dyadic(rng, (B, H, d, d), -0.5, 0.5),
        lambdas=np.array([0.9, 0.6][:H]), rope_base=1e4, eps=1e-6, pos0=3)
    c["dy"] = rng.standard_normal((B, T, H, d)).astype(np.float32)
    c["d_state_out"] = rng.standard_normal((B, H, d, d))
    return c


def _loss(c):
    f = oracle.prefill(c["q"], c["k"], c["v"], c["g"], c["qw"], c["kw"], c["lambdas"],
                       c["rope_base"], eps=c["eps"], pos0=c["pos0"], state_in=c["state_in"],
                       ow=c["ow"])
    B, T, H, d = c["q"].shape
    y = f["y"].reshape(B, H, T, d).transpose(0, 2, 1, 3)
    st = f["state"].reshape(B, H, d, d)
    return float(np.sum(c["dy"] * y) + np.sum(c["d_state_out"] * st))


def _fd(c, name, idx, h):
    def at(delta):
        cc = dict(c)
        a = c[name].copy()
        a[idx] += np.float32(delta)
        assert float(a[idx]) - float(c[name][idx]) == delta  # the perturbation is exact
        cc[name] = a
        return _loss(cc)

    d1 = (at(h) - at(-h)) / (2 * h)
    d2 = (at(h / 2) - at(-h / 2)) / h
    return (4 * d2 - d1) / 3


def _analytic(c):
    return ob.prefill_backward(c["q"], c["k"], c["v"], c["g"], c["dy"], c["qw"], c["kw"],
                               c["lambdas"], c["rope_base"], eps=c["eps"], pos0=c["pos0"],
                               state_in=c["state_in"], d_state_out=c["d_state_out"], ow=c["ow"])


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "state_in", "qw", "kw", "ow"])
def test_gradient_matches_finite_differences(name):
    c = _case()
    an = _analytic(c)
    B, T, H, d = c["q"].shape
    slot = {(b, h): i for i, (b, h) in enumerate(an["slices"])}
    h_step = 2.0 ** -10
    worst = 0.0
    for idx in np.ndindex(*c[name].shape):
        fd = _fd(c, name, idx, h_step)
        if name in ("q", "k", "v", "g"):
            b, t, hh, e = idx
            ref = an["d" + name][slot[(b, hh)], t, e]
        elif name == "state_in":
            b, hh, i, j = idx
            ref = an["d_state_in"][slot[(b, hh)], i, j]
        else:  # per-head weights: sum the batch rows' contributions
            hh, e = idx
            ref = sum(an["d" + name][slot[(b, hh)], e] for b in range(B))
        worst = max(worst, abs(fd - ref) / (1.0 + abs(ref)))
    assert worst < 2e-7, f"d{name}: finite differences differ by {worst:.3e}"


def test_core_transposition_identities():
    rng = np.random.default_rng(11)
    T, d, lam = 257, 32, 0.97
    qt, kt, v, do = (rng.standard_normal((T, d)) for _ in range(4))
    S0, dS = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    o, ST = ob.core_forward(qt, kt, v, lam, S0)
    dqt, dkt, dv, dS0 = ob.core_backward(qt, kt, v, lam, do, S0, dS)
    F = np.sum(do * o) + np.sum(dS * ST)
    scale = np.sum(np.abs(do * o)) + np.sum(np.abs(dS * ST))
    assert abs(np.sum(dqt * qt) - np.sum(do * o)) <= 1e-10 * scale
    assert abs(np.sum(dv * v) + np.sum(dS0 * S0) - F) <= 1e-10 * scale
    assert abs(np.sum(dkt * kt) + np.sum(dS0 * S0) - F) <= 1e-10 * scale


def test_lambda_zero_closed_form():
    rng = np.random.default_rng(12)
    T, d = 40, 16
    qt, kt, v, do = (rng.standard_normal((T, d)) for _ in range(4))
    dqt, dkt, dv, dS0 = ob.core_backward(qt, kt, v, 0.0, do, rng.standard_normal((d, d)))
    dots = np.sum(qt * kt, axis=1)
    np.testing.assert_allclose(dv, dots[:, None] * do, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dqt, (do @ v.T).diagonal()[:, None] * kt, rtol=1e-12, atol=1e-12)
    assert np.all(dS0 == 0.0)


def test_backward_composes_over_split_calls():
    c = _case(seed=5, B=2, T=37, H=2, d=16)
    whole = _analytic(c)
    T1 = 23
    first = {n: c[n][:, :T1] for n in ("q", "k", "v", "g", "dy")}
    second = {n: c[n][:, T1:] for n in ("q", "k", "v", "g", "dy")}
    f1 = oracle.prefill(first["q"], first["k"], first["v"], first["g"], c["qw"], c["kw"],
                        c["lambdas"], c["rope_base"], eps=c["eps"], pos0=c["pos0"],
                        state_in=c["state_in"], ow=c["ow"])
    B, H, d = 2, 2, 16
    S_mid = f1["state"].reshape(B, H, d, d)
    kw = dict(eps=c["eps"], ow=c["ow"])
    g2 = ob.prefill_backward(second["q"], second["k"], second["v"], second["g"], second["dy"],
                             c["qw"], c["kw"], c["lambdas"], c["rope_base"], pos0=c["pos0"] + T1,
                             state_in=S_mid, d_state_out=c["d_state_out"], **kw)
    g1 = ob.prefill_backward(first["q"], first["k"], first["v"], first["g"], first["dy"],
                             c["qw"], c["kw"], c["lambdas"], c["rope_base"], pos0=c["pos0"],
                             state_in=c["state_in"],
                             d_state_out=g2["d_state_in"].reshape(B, H, d, d), **kw)
    for name in ("dq", "dk", "dv", "dg"):
        joined = np.concatenate([g1[name], g2[name]], axis=1)
        np.testing.assert_allclose(joined, whole[name], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(g1["d_state_in"], whole["d_state_in"], rtol=1e-9, atol=1e-9)
    for name in ("dqw", "dkw", "dow"):
        np.testing.assert_allclose(g1[name] + g2[name], whole[name], rtol=1e-9, atol=1e-9)


# ---- planted mistakes: each must fail the finite-difference pins -------------------------------

def _fd_all(c, name):
    return {idx: _fd(c, name, idx, 2.0 ** -10) for idx in np.ndindex(*c[name].shape)}


def _worst(c, an, name, fd):
    slot = {(b, h): i for i, (b, h) in enumerate(an["slices"])}
    worst = 0.0
    for idx, f in fd.items():
        if name in ("q", "k", "v", "g"):
            b, t, hh, e = idx
            ref = an["d" + name][slot[(b, hh)], t, e]
        elif name == "state_in":
            b, hh, i, j = idx
            ref = an["d_state_in"][slot[(b, hh)], i, j]
        else:
            hh, e = idx
            ref = sum(an["d" + name][slot[(b, hh)], e] for b in range(c["q"].shape[0]))
        worst = max(worst, abs(f - ref) / (1.0 + abs(ref)))
    return worst


_ROT = ob._rotate_rows  # the unmutated routines the mutants build on
_CORE = ob.core_backward


def _mut_norm_no_mean(dxh, xh, r):
    return r[:, None] * dxh


def _mut_core_late_decay(qt, kt, v, lam, do, S0=None, dS_out=None):
    dqt, dkt, dv, _ = _CORE(qt, kt, v, lam, do, S0, dS_out)
    T, d = qt.shape
    G = np.zeros((d, d)) if dS_out is None else np.array(dS_out, dtype=np.float64)
    for t in range(T - 1, -1, -1):  # decays before adding the token's own term
        G = lam * G + np.outer(qt[t], do[t])
        dkt[t] = G @ v[t]
        dv[t] = kt[t] @ G
    return dqt, dkt, dv, G


def _mut_core_stale_state(qt, kt, v, lam, do, S0=None, dS_out=None):
    _, dkt, dv, dS0 = _CORE(qt, kt, v, lam, do, S0, dS_out)
    T, d = qt.shape
    S = np.zeros((d, d)) if S0 is None else np.array(S0, dtype=np.float64)
    dqt = np.empty((T, d))
    for t in range(T):  # query gradient from the state before the token's update
        dqt[t] = S @ do[t]
        S = lam * S + np.outer(kt[t], v[t])
    return dqt, dkt, dv, dS0


def _mut_rotation_forward(x, pos, base):
    return _ROT(x, np.abs(pos), base)  # adjoint taken as R_p instead of R_-p


@pytest.mark.parametrize("attr,mutant,caught_by", [
    ("_norm_backward", _mut_norm_no_mean, ["q", "g"]),
    ("core_backward", _mut_core_late_decay, ["k", "v", "state_in"]),
    ("core_backward", _mut_core_stale_state, ["q"]),
    ("_rotate_rows", _mut_rotation_forward, ["q", "k"]),
])
def test_planted_mistakes_fail_the_pins(monkeypatch, attr, mutant, caught_by):
    c = _case()
    fds = {name: _fd_all(c, name) for name in caught_by}
    monkeypatch.setattr(ob, attr, mutant)
    an = _analytic(c)
    monkeypatch.undo()
    assert max(_worst(c, an, name, fds[name]) for name in caught_by) > 1e-3
