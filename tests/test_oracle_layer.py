"""Pins of the RNN-layer oracle (oracle/layer.py) against facts that do not come from it.

* ``round_bf16`` against torch's float32 -> bfloat16 conversion (round to nearest even) on every
  value torch can take, and on hand-made fp64 ties and near-ties that a double rounding through
  float32 would get wrong.
* The projections' orientation and block order: with permutation matrices as weights, the layer
  must equal the mixer oracle run on permuted copies of x, and its output a permutation of y
  (a transposed weight, swapped q/k/v/z blocks or a transposed W_o give other permutations).
* Invariances of Eq. 18 that hold exactly in fp64 with rms_eps = 0: scaling W_q, W_k or W_v by
  2 leaves the output unchanged (RMSNorm of q and k, and the output RMSNorm of o), scaling W_o
  by 2 doubles it, and scaling W_z changes it (the gate is not normalised).
* The decode step against the prefill path: prefill(T) then a decode step at position T equals
  token T of prefill(T + 1) and its state.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import layer as ol
import synth
from synth import host_bits


# ---- round_bf16 ----------------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_values():
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(200000, generator=g) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    # exact ties of the bf16 grid, both parities, both signs
    ties = (torch.arange(1, 2000, dtype=torch.int32) * 2 ** 15 + (127 << 23)).view(torch.float32)
    x = torch.cat([x, ties, -ties, torch.tensor([0.0, -0.0, 1e-40, -3e-39, 3.3e38])])
    ref = x.to(torch.bfloat16).float().numpy().astype(np.float64)
    got = ol.round_bf16(x.numpy().astype(np.float64))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -8, 1.0),                                  # tie, even below
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),                  # tie, even above
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),         # just above a tie (float32 would
                                                             # round it onto the tie first)
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), -(1.0 + 2.0 ** -7)),
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 1.0),
    (255.5, 256.0),                                          # 8 significant bits
    (257.0, 256.0),                                          # tie at 2^8, even
    (259.0, 260.0),
    (3.0 * 2.0 ** -134, 2.0 ** -132),                        # subnormal tie -> even
    (2.0 ** 128, np.inf),
])
def test_round_bf16_ties_and_near_ties(x, expect):
    assert ol.round_bf16(np.array([x]))[0] == expect


def test_bf16_bits_roundtrip():
    v = ol.round_bf16(np.random.default_rng(1).normal(size=1000))
    assert np.array_equal(ol.widen(ol.bf16_bits(v)), v)
    with pytest.raises(ValueError):
        ol.bf16_bits(np.array([1.0 + 2.0 ** -20]))


# ---- structure of the layer ----------------------------------------------------------------------

def _perm_matrix(perm, dtype=torch.bfloat16):
    """Row n = e_{perm[n]}: (x W^T)[n] = x[perm[n]]."""
    m = torch.zeros((len(perm), len(perm)), dtype=torch.float32)
    m[torch.arange(len(perm)), torch.as_tensor(perm)] = 1.0
    return m.to(dtype)


def test_permutation_weights_select_projection_blocks():
    B, T, H, d = 2, 70, 2, 64
    dm = H * d
    inp = synth.make_custom_layer(B, T, H, d, dm, seed=3, state="randn")
    rng = np.random.default_rng(7)
    perms = [rng.permutation(dm) for _ in range(5)]
    # none of them is an involution, so a transposed matrix would select differently
    for p in perms:
        assert not np.array_equal(p[p], np.arange(dm))
    w_qkvz = torch.cat([_perm_matrix(p) for p in perms[:4]])
    w_o = _perm_matrix(perms[4])
    x = host_bits(inp["x"])
    ref = ol.layer_prefill(x, host_bits(w_qkvz), host_bits(w_o), inp["qw"].numpy(),
                           inp["kw"].numpy(), inp["lambdas"], inp["rope_base"], H, d,
                           state_in=inp["state_in"].numpy())
    sel = [np.ascontiguousarray(x[..., p].reshape(B, T, H, d)) for p in perms[:4]]
    mix = oracle.prefill(*sel, inp["qw"].numpy(), inp["kw"].numpy(), inp["lambdas"],
                         inp["rope_base"], state_in=inp["state_in"].numpy(), want_o=False)
    y = mix["y"].reshape(B, H, T, d).transpose(0, 2, 1, 3).reshape(B, T, dm)
    y = ol.round_bf16(y)
    assert np.array_equal(ref["y"], y)
    assert np.array_equal(ref["out"], y[..., perms[4]])
    assert np.array_equal(ref["state"], mix["state"].reshape(B, H, d, d))
    assert np.array_equal(ref["proj"], np.concatenate([ol.widen(x[..., p]) for p in perms[:4]], -1))


def _run(inp, w_qkvz, w_o, eps):
    return ol.layer_prefill(host_bits(inp["x"]), host_bits(w_qkvz), host_bits(w_o),
                            inp["qw"].numpy(), inp["kw"].numpy(), inp["lambdas"],
                            inp["rope_base"], inp["H"], inp["d"], eps=eps,
                            state_in=None if inp["state_in"] is None else inp["state_in"].numpy())


def test_scale_invariances_of_the_layer():
    inp = synth.make_custom_layer(1, 90, 2, 64, 96, seed=5)
    H, d = 2, 64
    w, wo = inp["w_qkvz"], inp["w_o"]
    base = _run(inp, w, wo, eps=0.0)

    def scaled(block, c=2.0):
        w2 = w.float().clone()
        w2[block * H * d:(block + 1) * H * d] *= c
        return w2.to(w.dtype)

    for block in (0, 1, 2):  # W_q, W_k, W_v
        r = _run(inp, scaled(block), wo, eps=0.0)
        assert np.array_equal(r["out"], base["out"]), block
    r = _run(inp, scaled(3), wo, eps=0.0)  # W_z: the gate changes
    assert not np.allclose(r["out"], base["out"], rtol=1e-3, atol=0)
    r = _run(inp, w, (wo.float() * 2).to(wo.dtype), eps=0.0)
    assert np.array_equal(r["out"], 2 * base["out"])
    # with the default eps the invariance is only approximate, but still close
    r1 = _run(inp, w, wo, eps=1e-6)
    r2 = _run(inp, scaled(2), wo, eps=1e-6)
    assert np.max(np.abs(r1["out"] - r2["out"])) <= 1e-3 * np.max(np.abs(r1["out"]))


def test_layer_decode_matches_prefill_of_one_more_token():
    B, T, H, d, dm = 2, 40, 2, 64, 160
    inp = synth.make_custom_layer(B, T + 1, H, d, dm, seed=9, state="randn")
    args = (host_bits(inp["w_qkvz"]), host_bits(inp["w_o"]), inp["qw"].numpy(),
            inp["kw"].numpy(), inp["lambdas"], inp["rope_base"], H, d)
    x = host_bits(inp["x"])
    full = ol.layer_prefill(x, *args, state_in=inp["state_in"].numpy())
    head = ol.layer_prefill(np.ascontiguousarray(x[:, :T]), *args,
                            state_in=inp["state_in"].numpy())
    step = ol.layer_decode_step(np.ascontiguousarray(x[:, T]), *args,
                                np.full(B, T, dtype=np.int64),
                                head["state"].astype(np.float32))
    # the decode step starts from the fp32-rounded state, so agreement is to fp32 precision
    for b in range(B):
        assert synth.rel_l2(step["out"][b], full["out"][b, T]) <= 1e-6
        assert synth.rel_l2(step["state"][b], full["state"][b]) <= 1e-6
    assert np.array_equal(step["proj"], full["proj"][:, T])


def test_fp32_layer_rounds_to_float32():
    inp = synth.make_custom_layer(1, 20, 1, 64, 64, dtype=torch.float32, seed=2)
    r = ol.layer_prefill(host_bits(inp["x"]), host_bits(inp["w_qkvz"]), host_bits(inp["w_o"]),
                         inp["qw"].numpy(), inp["kw"].numpy(), inp["lambdas"], inp["rope_base"],
                         1, 64)
    assert np.array_equal(r["proj"], r["proj"].astype(np.float32).astype(np.float64))
    assert np.array_equal(r["y"], r["y"].astype(np.float32).astype(np.float64))
    exact = inp["x"].double().numpy() @ inp["w_qkvz"].double().numpy().T
    assert np.max(np.abs(r["proj"][0] - exact[0])) <= 2.0 ** -23 * np.max(np.abs(exact))


def test_ternary_inputs_give_exact_integer_projections():
    inp = synth.make_custom_layer(1, 64, 2, 128, 256, seed=4, values="ternary")
    q, k, v, g = ol.projections(host_bits(inp["x"]), host_bits(inp["w_qkvz"]), 2, 128)
    exact = inp["x"].double() @ inp["w_qkvz"].double().T
    got = np.concatenate([ol.widen(a).reshape(1, 64, 256) for a in (q, k, v, g)], -1)
    assert np.array_equal(got, exact.numpy())
    assert np.all(np.abs(got) <= 256) and np.all(got == np.round(got))
