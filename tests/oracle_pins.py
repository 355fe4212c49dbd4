"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin takes a loaded oracle library (``oracle.load()`` or a mutated build of the same source)
and returns ``(error, tolerance)``; it passes when ``error <= tolerance``.  The kinds of pin:

* library routines: RMSNorm against ``torch.nn.functional.rms_norm`` and the gate against
  ``torch.sigmoid``, both in float64;
* textbook identities of rotary embeddings (RoFormer's complex form, relative-position property,
  norm preservation, identity at position 0);
* brute force on tiny inputs: the unrolled O(T^2) sum of the recurrence (the closed form the
  reading notes derive under Eq. 18/19 of "Hybrid Linear Attention Done Right", with an initial
  state added), written with dense numpy products;
* special cases that reduce to textbook routines: lambda = 1 is plain causal linear attention,
  lambda = 0 is o_t = (q~_t . k~_t) v_t;
* a closed form for RoPE and decay together (a complex geometric series);
* invariants: chunked = recurrent for every chunk length, state carry across split prefills and
  prefill -> decode, invariance of o under a shift of the position origin, joint linearity in
  (v, S_0).

``tests/test_oracle_mutants.py`` builds mutated copies of ``oracle.c`` and checks that every
mutant fails at least one pin.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import host_bits, make_custom_prefill

LAMBDAS = (0.0, 0.43, 0.9, 0.99, 1.0)


def _max_rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = max(float(np.max(np.abs(ref))), 1e-300)
    return float(np.max(np.abs(x - ref))) / den


def _inputs(B, T, H, d, seed, dtype=torch.float32, lambdas=None, state="zeros", norm_w="uniform",
            rope_base=1e4, pos0=0):
    inp = make_custom_prefill(B, T, H, d, dtype=dtype, seed=seed, lambdas=lambdas,
                              rope_base=rope_base, norm_w=norm_w, state=state, pos0=pos0)
    return inp


def _run(lib, inp, **kw):
    s0 = None if inp["state_in"] is None else inp["state_in"].numpy()
    args = dict(eps=inp["eps"], pos0=inp["pos0"], state_in=s0, lib=lib)
    args.update(kw)
    return oracle.prefill(host_bits(inp["q"]), host_bits(inp["k"]), host_bits(inp["v"]),
                          host_bits(inp["g"]), inp["qw"].numpy(), inp["kw"].numpy(),
                          inp["lambdas"], inp["rope_base"], **args)


def _prologue(lib, inp, b, h):
    """q~, k~ for every token of slice (b, h) from the oracle's own per-vector steps (which the
    RMSNorm and RoPE pins check separately)."""
    T, d = inp["T"], inp["d"]
    q = inp["q"].double().numpy()[b, :, h]
    k = inp["k"].double().numpy()[b, :, h]
    qw = inp["qw"].double().numpy()[h]
    kw = inp["kw"].double().numpy()[h]
    Qt = np.empty((T, d))
    Kt = np.empty((T, d))
    for t in range(T):
        p = inp["pos0"] + t
        Qt[t] = oracle.rope(oracle.rmsnorm(q[t], qw, inp["eps"], lib=lib), p, inp["rope_base"],
                            lib=lib)
        Kt[t] = oracle.rope(oracle.rmsnorm(k[t], kw, inp["eps"], lib=lib), p, inp["rope_base"],
                            lib=lib) / np.sqrt(d)
    return Qt, Kt


# ---- per-vector steps --------------------------------------------------------------------------

def pin_rmsnorm_vs_torch(lib):
    rng = np.random.default_rng(1)
    err = 0.0
    for n in (2, 8, 64, 128):
        for scale in (1e-3, 1.0, 40.0):
            x = rng.standard_normal(n) * scale
            w = rng.uniform(0.5, 1.5, n)
            for eps in (0.0, 1e-6, 1e-2):
                ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (n,), torch.from_numpy(w),
                                                   eps).numpy()
                err = max(err, _max_rel(oracle.rmsnorm(x, w, eps, lib=lib), ref))
    return err, 1e-13


def pin_sigmoid_vs_torch(lib):
    xs = np.array([-30.0, -5.0, -1.0, -1e-3, 0.0, 1e-3, 0.5, 1.0, 7.0, 30.0])
    ref = torch.sigmoid(torch.from_numpy(xs)).numpy()
    got = np.array([oracle.sigmoid(x, lib=lib) for x in xs])
    err = float(np.max(np.abs(got - ref)))
    err = max(err, abs(oracle.sigmoid(0.0, lib=lib) - 0.5))
    return err, 1e-15


def pin_rope_complex_form(lib):
    """RoPE of the pair (x_i, x_{i+n/2}) is multiplication of x_i + i x_{i+n/2} by
    exp(i p base^(-2i/n)) (RoFormer's complex form with half-split pairs)."""
    rng = np.random.default_rng(2)
    err = 0.0
    for n in (2, 8, 64, 128):
        half = n // 2
        for base in (500.0, 1e4, 1e6):
            for pos in (0, 1, 17, 4095, 524287, 1_000_003):
                x = rng.standard_normal(n)
                z = (x[:half] + 1j * x[half:]) * np.exp(1j * pos * base ** (-2.0 * np.arange(half) / n))
                ref = np.concatenate([z.real, z.imag])
                err = max(err, _max_rel(oracle.rope(x, pos, base, lib=lib), ref))
    # the angle p * f is ~1e6 rad here, so fp64 argument error bounds the agreement
    return err, 1e-9


def pin_rope_identities(lib):
    """Identity at p = 0, norm preservation, and RoPE_m(q) . RoPE_n(k) = q . RoPE_{n-m}(k)."""
    rng = np.random.default_rng(3)
    err = 0.0
    for n in (8, 64, 128):
        x = rng.standard_normal(n)
        y = rng.standard_normal(n)
        err = max(err, _max_rel(oracle.rope(x, 0, 1e6, lib=lib), x))
        for m, p in ((3, 11), (1000, 250), (524000, 524287)):
            rx = oracle.rope(x, m, 1e6, lib=lib)
            err = max(err, abs(np.linalg.norm(rx) - np.linalg.norm(x)) / np.linalg.norm(x))
            lhs = float(rx @ oracle.rope(y, p, 1e6, lib=lib))
            rhs = float(x @ oracle.rope(y, p - m, 1e6, lib=lib))
            err = max(err, abs(lhs - rhs) / (np.linalg.norm(x) * np.linalg.norm(y)))
    return err, 1e-9


# ---- the recurrence ----------------------------------------------------------------------------

def _bruteforce(Qt, Kt, V, lam, S0):
    """o_t = lam^(t+1) q~_t S_0 + sum_{s<=t} lam^(t-s) (q~_t . k~_s) v_s and
    S_T = lam^T S_0 + sum_s lam^(T-1-s) k~_s^T v_s, with 0^0 = 1."""
    T = Qt.shape[0]
    t = np.arange(T)
    diff = t[:, None] - t[None, :]
    with np.errstate(divide="ignore"):
        D = np.where(diff >= 0, np.power(lam, np.maximum(diff, 0).astype(np.float64)), 0.0)
    D[diff == 0] = 1.0
    carry = np.power(lam, (t + 1).astype(np.float64))
    o = ((Qt @ Kt.T) * D) @ V + carry[:, None] * (Qt @ S0)
    w = np.power(lam, (T - 1 - t).astype(np.float64))
    w[T - 1] = 1.0
    S = lam ** T * S0 + Kt.T @ (w[:, None] * V)
    return o, S


def pin_bruteforce(lib):
    err = 0.0
    seed = 10
    for d in (2, 8, 64):
        for T in (1, 5, 67):
            for state in ("zeros", "randn"):
                lams = LAMBDAS
                inp = _inputs(1, T, len(lams), d, seed, lambdas=lams, state=state,
                              rope_base=1e4, pos0=3)
                seed += 1
                if state == "randn":  # make the initial state comparable to the token terms
                    inp["state_in"] = inp["state_in"] * 50.0
                out = _run(lib, inp)
                for h, lam in enumerate(lams):
                    Qt, Kt = _prologue(lib, inp, 0, h)
                    V = inp["v"].double().numpy()[0, :, h]
                    S0 = (np.zeros((d, d)) if inp["state_in"] is None
                          else inp["state_in"].double().numpy()[0, h])
                    o_ref, S_ref = _bruteforce(Qt, Kt, V, lam, S0)
                    err = max(err, _max_rel(out["o"][h], o_ref), _max_rel(out["state"][h], S_ref))
    return err, 1e-11


def pin_lambda_one_is_causal_linear_attention(lib):
    """lambda = 1: o = tril(Q~ K~^T) V + Q~ S_0 (plain causal linear attention)."""
    inp = _inputs(2, 40, 2, 16, 21, lambdas=(1.0, 1.0), state="randn")
    out = _run(lib, inp)
    err = 0.0
    for i, (b, h) in enumerate(out["slices"]):
        Qt, Kt = _prologue(lib, inp, b, h)
        V = inp["v"].double().numpy()[b, :, h]
        S0 = inp["state_in"].double().numpy()[b, h]
        ref = np.tril(Qt @ Kt.T) @ V + Qt @ S0
        err = max(err, _max_rel(out["o"][i], ref))
        err = max(err, _max_rel(out["state"][i], S0 + Kt.T @ V))
    return err, 1e-11


def pin_lambda_zero_closed_form(lib):
    """lambda = 0: o_t = (q~_t . k~_t) v_t and S_T = k~_{T-1}^T v_{T-1}."""
    inp = _inputs(1, 33, 1, 16, 22, lambdas=(0.0,), state="randn")
    out = _run(lib, inp)
    Qt, Kt = _prologue(lib, inp, 0, 0)
    V = inp["v"].double().numpy()[0, :, 0]
    ref = np.sum(Qt * Kt, axis=1)[:, None] * V
    err = max(_max_rel(out["o"][0], ref), _max_rel(out["state"][0], np.outer(Kt[-1], V[-1])))
    return err, 1e-12


def pin_rope_decay_geometric_series(lib):
    """Constant q, k, v with only rotary pair 0 (entries 0 and d/2) nonzero in q and k.  Pair 0
    rotates by angle p (base^0 = 1), so q~_t . k~_s = Re(A e^{i(t-s)}) with
    A = z_q conj(z_k) / sqrt(d), z = x_0 + i x_{d/2} after RMSNorm.  Hence
    o_t = Re(A (1 - (lam e^i)^(t+1)) / (1 - lam e^i)) v, independent of the position origin, and
    y_t = RMSNorm(o_t) * sigmoid(g_t)."""
    d, T, eps = 8, 50, 1e-6
    lams = (0.43, 0.9, 0.999)
    H = len(lams)
    rng = np.random.default_rng(4)
    qv = np.zeros(d, np.float32)
    kv = np.zeros(d, np.float32)
    qv[0], qv[d // 2] = 0.7, -1.3
    kv[0], kv[d // 2] = 1.1, 0.4
    vv = rng.standard_normal(d).astype(np.float32)
    g = rng.standard_normal((1, T, H, d)).astype(np.float32)
    q = np.broadcast_to(qv, (1, T, H, d)).copy()
    k = np.broadcast_to(kv, (1, T, H, d)).copy()
    v = np.broadcast_to(vv, (1, T, H, d)).copy()
    qw = rng.uniform(0.5, 1.5, (H, d)).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, (H, d)).astype(np.float32)
    err = 0.0
    for pos0 in (0, 100_000):
        out = oracle.prefill(q, k, v, g, qw, kw, lams, 1e6, eps=eps, pos0=pos0, lib=lib)
        for h, lam in enumerate(lams):
            qn = torch.nn.functional.rms_norm(torch.from_numpy(qv).double(), (d,),
                                              torch.from_numpy(qw[h]).double(), eps).numpy()
            kn = torch.nn.functional.rms_norm(torch.from_numpy(kv).double(), (d,),
                                              torch.from_numpy(kw[h]).double(), eps).numpy()
            A = (qn[0] + 1j * qn[d // 2]) * np.conj(kn[0] + 1j * kn[d // 2]) / np.sqrt(d)
            r = lam * np.exp(1j)
            t = np.arange(T)
            coef = np.real(A * (1 - r ** (t + 1)) / (1 - r))
            o_ref = coef[:, None] * vv.astype(np.float64)[None, :]
            y_ref = (torch.nn.functional.rms_norm(torch.from_numpy(o_ref), (d,), None, eps)
                     * torch.sigmoid(torch.from_numpy(g[0, :, h]).double())).numpy()
            err = max(err, _max_rel(out["o"][h], o_ref), _max_rel(out["y"][h], y_ref))
    return err, 1e-11


def pin_output_epilogue(lib):
    """y = RMSNorm(o) (.) w_o (.) sigmoid(g) with a non-trivial output-norm weight, with o taken
    from the oracle itself and the epilogue from torch routines."""
    inp = _inputs(1, 20, 2, 16, 23, lambdas=(0.9, 0.5))
    ow = np.random.default_rng(5).uniform(0.5, 1.5, (2, 16)).astype(np.float32)
    out = _run(lib, inp, ow=ow)
    err = 0.0
    for h in range(2):
        o = torch.from_numpy(out["o"][h])
        ref = (torch.nn.functional.rms_norm(o, (16,), torch.from_numpy(ow[h]).double(), inp["eps"])
               * torch.sigmoid(inp["g"][0, :, h].double())).numpy()
        err = max(err, _max_rel(out["y"][h], ref))
    return err, 1e-13


# ---- invariants --------------------------------------------------------------------------------

def pin_chunked_equals_recurrence(lib):
    err = 0.0
    for T, d in ((64, 8), (131, 16)):
        inp = _inputs(2, T, 3, d, 30 + T, lambdas=(0.43, 0.9, 1.0), state="randn")
        ref = _run(lib, inp)
        for C in (1, 7, 32, 64, T):
            got = _run(lib, inp, chunk=C)
            err = max(err, _max_rel(got["o"], ref["o"]), _max_rel(got["y"], ref["y"]),
                      _max_rel(got["state"], ref["state"]))
    return err, 1e-11


def pin_split_prefill_and_decode(lib):
    """prefill(T1) then prefill(T2, pos0 = T1, S_0 = S_T1) equals prefill(T1 + T2) on the second
    part, and prefill(T) then one decode step at position T equals token T of prefill(T + 1).
    The carried state crosses an fp32 boundary, as it does in the library."""
    T1, T2, d, H = 37, 29, 16, 2
    inp = _inputs(2, T1 + T2, H, d, 40, lambdas=(0.8, 0.97), state="randn")
    full = _run(lib, inp)
    part = {kk: (vv[:, :T1].contiguous() if isinstance(vv, torch.Tensor) and vv.dim() == 4
                 and vv.shape[1] == T1 + T2 else vv) for kk, vv in inp.items()}
    part["T"] = T1
    first = _run(lib, part)
    S1 = first["state"].reshape(2, H, d, d).astype(np.float32)
    rest = {kk: (vv[:, T1:].contiguous() if isinstance(vv, torch.Tensor) and vv.dim() == 4
                 and vv.shape[1] == T1 + T2 else vv) for kk, vv in inp.items()}
    rest["T"] = T2
    rest["pos0"] = T1
    rest["state_in"] = torch.from_numpy(S1)
    second = _run(lib, rest)
    err = max(_max_rel(first["y"], full["y"][:, :T1]), _max_rel(second["y"], full["y"][:, T1:]),
              _max_rel(second["o"], full["o"][:, T1:]), _max_rel(second["state"], full["state"]))
    # decode: feed token T1 of the same inputs at position T1, starting from S_T1
    tok = {kk: host_bits(inp[kk][:, T1]) for kk in ("q", "k", "v", "g")}
    dec = oracle.decode_step(tok["q"], tok["k"], tok["v"], tok["g"], inp["qw"].numpy(),
                             inp["kw"].numpy(), inp["lambdas"], inp["rope_base"],
                             np.full(2, T1, np.int64), S1, eps=inp["eps"], lib=lib)
    ref_pre = _run(lib, {**inp, "q": inp["q"][:, :T1 + 1].contiguous(),
                         "k": inp["k"][:, :T1 + 1].contiguous(),
                         "v": inp["v"][:, :T1 + 1].contiguous(),
                         "g": inp["g"][:, :T1 + 1].contiguous(), "T": T1 + 1})
    last_y = ref_pre["y"][:, T1].reshape(2, H, d)
    last_o = ref_pre["o"][:, T1].reshape(2, H, d)
    err = max(err, _max_rel(dec["y"], last_y), _max_rel(dec["o"], last_o),
              _max_rel(dec["state"], ref_pre["state"].reshape(2, H, d, d)))
    # fp32 rounding of the carried state bounds the agreement
    return err, 1e-6


def pin_position_origin(lib):
    """With S_0 = 0, o and y depend only on relative positions; the final state does not."""
    inp = _inputs(1, 40, 2, 16, 50, lambdas=(0.9, 0.99), rope_base=1e6)
    a = _run(lib, inp)
    b = _run(lib, {**inp, "pos0": 123_457})
    err = max(_max_rel(a["o"], b["o"]), _max_rel(a["y"], b["y"]))
    moved = _max_rel(a["state"], b["state"])
    return (err if moved > 1e-3 else float("inf")), 1e-9


def pin_joint_linearity(lib):
    """o is linear in (v, S_0) jointly; y is invariant to a joint positive rescale (up to eps)."""
    inp = _inputs(1, 30, 2, 16, 60, lambdas=(0.9, 0.6), state="randn")
    inp["eps"] = 0.0  # with eps = 0 the output norm is exactly scale invariant
    a = _run(lib, inp)
    c = 4.0  # a power of two keeps the rescaled fp32 inputs exact
    b = _run(lib, {**inp, "v": inp["v"] * c, "state_in": inp["state_in"] * c})
    err = max(_max_rel(b["o"], c * a["o"]), _max_rel(b["state"], c * a["state"]))
    return max(err, _max_rel(b["y"], a["y"])), 1e-11


def pin_bf16_inputs_widen_exactly(lib):
    """bf16 inputs are widened exactly: feeding the same values as fp32 gives identical output."""
    inp = _inputs(1, 20, 2, 16, 70, dtype=torch.bfloat16, lambdas=(0.9, 0.99))
    a = _run(lib, inp)
    as32 = {**inp, **{kk: inp[kk].float() for kk in ("q", "k", "v", "g")}}
    b = _run(lib, as32)
    return max(_max_rel(a["y"], b["y"]), _max_rel(a["state"], b["state"])), 0.0


ALL_PINS = [
    pin_rmsnorm_vs_torch,
    pin_sigmoid_vs_torch,
    pin_rope_complex_form,
    pin_rope_identities,
    pin_bruteforce,
    pin_lambda_one_is_causal_linear_attention,
    pin_lambda_zero_closed_form,
    pin_rope_decay_geometric_series,
    pin_output_epilogue,
    pin_chunked_equals_recurrence,
    pin_split_prefill_and_decode,
    pin_position_origin,
    pin_joint_linearity,
    pin_bf16_inputs_widen_exactly,
]
