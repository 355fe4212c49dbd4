"""Pins of the HyPE attention oracle (oracle/attention.py) against facts that do not come from it.

* torch's scaled_dot_product_attention in float64 (causal, default 1/sqrt(d) scale) on
  s_t-scaled queries, with the key/value heads repeated per query group, and torch's rms_norm
  and sigmoid for the normalisations and the gate: the whole prefill, with and without QK-norm.
* The logits scale of Eq. 11: s = 1 at position 0, a^s = pos + a, and (loosely) the worked value
  s ~ 1.87 at position 128K for a = 500 that the summary page gives (the exact value is 1.893).
* Softmax invariances: a common shift of every key leaves o unchanged (without key norm); a
  common shift of every value shifts o by it; with QK-norm and eps = 0 a scaled query changes
  nothing.
* The decode step against the prefill: a decode step at position T over the first T normalised
  keys equals row T of the prefill of T + 1 tokens.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oa


def _draw(B, T, Hq, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, Hq, d, generator=g)
    k = torch.randn(B, T, Hkv, d, generator=g)
    v = torch.randn(B, T, Hkv, d, generator=g)
    gate = torch.randn(B, T, Hq, d, generator=g)
    return q, k, v, gate


def _torch_reference(q, k, v, gate, a, pos0, qw=None, kw=None, ow=None, eps=1e-6):
    q, k, v, gate = (x.double() for x in (q, k, v, gate))
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if qw is not None:
        q = F.rms_norm(q, (d,), qw.double(), eps)
    if kw is not None:
        k = F.rms_norm(k, (d,), kw.double(), eps)
    pos = torch.arange(T, dtype=torch.float64) + pos0
    s = torch.log(pos + a) / math.log(a) if a else torch.ones(T, dtype=torch.float64)
    qs = (q * s[None, :, None, None]).transpose(1, 2)
    kk = k.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    vv = v.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1)
    o = F.scaled_dot_product_attention(qs, kk, vv, is_causal=True).transpose(1, 2)
    y = F.rms_norm(o, (d,), None if ow is None else ow.double(), eps) * torch.sigmoid(gate)
    return o.numpy(), y.numpy()


@pytest.mark.parametrize("Hq,Hkv,a,pos0,norms", [
    (4, 2, 500.0, 0, False),
    (4, 2, 500.0, 123456, True),
    (6, 3, 900.0, 7, True),
    (2, 2, None, 0, False),
    (8, 1, 300.0, 1 << 20, True),
])
def test_prefill_matches_torch_sdpa(Hq, Hkv, a, pos0, norms):
    B, T, d = 2, 37, 16
    q, k, v, gate = _draw(B, T, Hq, Hkv, d, seed=Hq * 7 + Hkv)
    qw = kw = ow = None
    if norms:
        gen = torch.Generator().manual_seed(3)
        qw = 0.5 + torch.rand(Hq, d, generator=gen)
        kw = 0.5 + torch.rand(Hkv, d, generator=gen)
        ow = 0.5 + torch.rand(Hq, d, generator=gen)
    r = oa.attn_prefill(q.numpy(), k.numpy(), v.numpy(), gate.numpy(),
                        None if qw is None else qw.numpy(), None if kw is None else kw.numpy(),
                        None if ow is None else ow.numpy(), a=a, pos0=pos0)
    # torch's rms_norm with a per-head weight: apply per head
    if norms:
        qn = torch.stack([F.rms_norm(q[:, :, h].double(), (d,), qw[h].double(), 1e-6)
                          for h in range(Hq)], 2)
        kn = torch.stack([F.rms_norm(k[:, :, h].double(), (d,), kw[h].double(), 1e-6)
                          for h in range(Hkv)], 2)
        o_ref, _ = _torch_reference(qn, kn, v, gate, a, pos0)
        y_ref = np.stack([(F.rms_norm(torch.from_numpy(o_ref[:, :, h]), (d,), ow[h].double(), 1e-6)
                           * torch.sigmoid(gate[:, :, h].double())).numpy() for h in range(Hq)], 2)
    else:
        o_ref, y_ref = _torch_reference(q, k, v, gate, a, pos0)
    assert np.max(np.abs(r["o"] - o_ref)) <= 1e-12
    assert np.max(np.abs(r["y"] - y_ref)) <= 1e-11


def test_logit_scale_values():
    assert oa.logit_scale(0, 500.0) == 1.0
    assert oa.logit_scale(12345, None) == 1.0
    # the defining relation a^s = pos + a (Eq. 11), checked through exponentiation
    for a, pos in ((500.0, 128000), (900.0, 524287), (300.0, 3)):
        s = float(oa.logit_scale(pos, a))
        assert abs(a ** s - (pos + a)) <= 1e-9 * (pos + a)
    # the summary page's worked value (s ~ 1.87 at 128K, a = 500) is log_500(128500) = 1.893
    # rounded loosely; Eq. 11 itself decides
    assert abs(float(oa.logit_scale(128000, 500.0)) - 1.87) < 0.03
    assert float(oa.logit_scale(128000, 500.0)) > float(oa.logit_scale(64000, 500.0)) > 1.0


def test_softmax_shift_invariances():
    B, T, Hq, Hkv, d = 1, 25, 2, 1, 8
    q, k, v, gate = _draw(B, T, Hq, Hkv, d, seed=5)
    # multiples of 2^-8 of moderate size: the shifted inputs are exact in float32
    k, v = (torch.round(x * 256) / 256 for x in (k, v))
    base = oa.attn_prefill(q.numpy(), k.numpy(), v.numpy(), gate.numpy(), a=500.0)
    c = torch.round(torch.randn(d, generator=torch.Generator().manual_seed(9)) * 256) / 256
    shifted_k = oa.attn_prefill(q.numpy(), (k + c).numpy(), v.numpy(), gate.numpy(), a=500.0)
    # q_t . (k_j + c) adds the same q_t . c to every key of row t: softmax is unchanged
    assert np.max(np.abs(shifted_k["o"] - base["o"])) <= 1e-12
    shifted_v = oa.attn_prefill(q.numpy(), k.numpy(), (v + c).numpy(), gate.numpy(), a=500.0)
    assert np.max(np.abs(shifted_v["o"] - (base["o"] + c.double().numpy()))) <= 1e-12
    qw = np.ones(d, dtype=np.float32)
    r1 = oa.attn_prefill(q.numpy(), k.numpy(), v.numpy(), gate.numpy(), qw=qw, a=500.0, eps=0.0)
    r2 = oa.attn_prefill((2 * q).numpy(), k.numpy(), v.numpy(), gate.numpy(), qw=qw, a=500.0,
                         eps=0.0)
    assert np.array_equal(r1["o"], r2["o"])
    # the first row attends to itself only
    assert np.max(np.abs(base["o"][:, 0, 0] - v[:, 0, 0].double().numpy())) <= 1e-15


def test_decode_matches_prefill_row():
    B, T, Hq, Hkv, d = 2, 30, 4, 2, 16
    q, k, v, gate = _draw(B, T + 1, Hq, Hkv, d, seed=11)
    gen = torch.Generator().manual_seed(4)
    qw, kw = (0.5 + torch.rand(d, generator=gen)).numpy(), (0.5 + torch.rand(d, generator=gen)).numpy()
    full = oa.attn_prefill(q.numpy(), k.numpy(), v.numpy(), gate.numpy(), qw, kw, a=600.0)
    step = oa.attn_decode_step(q[:, T].numpy(), k[:, T].numpy(), v[:, T].numpy(),
                               gate[:, T].numpy(), full["k_hat"][:, :T].astype(np.float32),
                               v[:, :T].numpy(), np.full(B, T), qw, kw, a=600.0)
    # the cache holds the keys rounded to float32: agreement to float32 precision
    assert np.max(np.abs(step["o"] - full["o"][:, T])) <= 1e-5
    assert np.max(np.abs(step["y"] - full["y"][:, T])) <= 1e-5
    assert np.max(np.abs(step["k_hat"] - full["k_hat"][:, T])) <= 1e-12
