"""fp64 CPU oracle of the mixer with a data-dependent scalar decay -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; it imports nothing from the GPU library.

The pages contrast Lightning Attention's fixed per-head decay with RNN mixers whose forget gate
depends on the token ("Hybrid Linear Attention Done Right", Appendix E.1, Fig. 7: the prefill
time of the mixers, Mamba2 among them; Appendix G, Table 11: Mamba2's scalar gate
F_t = alpha_t I).  This oracle is Eq. 18 with the decay gamma of head h replaced by a per-token
alpha_t in (0, 1], given as log2(alpha_t):

    S_t = alpha_t S_{t-1} + k~_t^T v_t,    o_t = q~_t S_t

with the same prologue (RMSNorm, RoPE, 1/sqrt(d) on k) and output gate as the fixed-decay mixer;
the prologue uses the (pinned) RMSNorm and RoPE routines of ``oracle``.  Token by token, in fp64.
"""
from __future__ import annotations

import math

import numpy as np

from . import rmsnorm, rope
from .layer import widen


def _prologue(x, w, pos, base, eps, scale):
    """RMSNorm(x) w, rotated to each token's position, times `scale`: x [T, d] fp64."""
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        out[t] = rope(rmsnorm(x[t], w, eps), int(pos[t]), base)
    return out * scale


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def prefill_dd(q, k, v, g, qw, kw, log2_decay, rope_base, eps=1e-6, pos0=0, state_in=None,
               ow=None, slices=None):
    """q, k, v, g: [B, T, H, d] (bf16 bits or float32); log2_decay: float32 [B, T, H];
    qw, kw (and ow): float32 [H, d] or [d]; state_in: float32 [B, H, d, d] or None.

    Returns y, o [n, T, d] and state [n, d, d] (fp64) for the (b, h) pairs in ``slices``.
    """
    qf, kf, vf, gf = (widen(x) for x in (q, k, v, g))
    B, T, H, d = qf.shape
    lg = np.asarray(log2_decay, dtype=np.float64)
    if lg.shape != (B, T, H):
        raise ValueError("log2_decay must be [B, T, H]")

    def wrow(w, h):
        if w is None:
            return None
        w = np.asarray(w, dtype=np.float64)
        return w if w.ndim == 1 else w[h]

    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    pos = pos0 + np.arange(T)
    n = len(slices)
    y = np.empty((n, T, d))
    o = np.empty((n, T, d))
    st = np.empty((n, d, d))
    for i, (b, h) in enumerate(slices):
        qt = _prologue(qf[b, :, h], wrow(qw, h), pos, rope_base, eps, 1.0)
        kt = _prologue(kf[b, :, h], wrow(kw, h), pos, rope_base, eps, 1.0 / math.sqrt(d))
        S = np.zeros((d, d)) if state_in is None else np.asarray(state_in[b, h], dtype=np.float64)
        alpha = np.exp2(lg[b, :, h])
        wo = wrow(ow, h)
        for t in range(T):
            S = alpha[t] * S + np.outer(kt[t], vf[b, t, h])
            ot = qt[t] @ S
            o[i, t] = ot
            yt = ot / math.sqrt(float(np.mean(ot * ot)) + eps)
            if wo is not None:
                yt = yt * wo
            y[i, t] = yt * _sigmoid(gf[b, t, h])
        st[i] = S
    return {"y": y, "o": o, "state": st, "slices": slices}


def decode_step_dd(q, k, v, g, qw, kw, log2_decay, rope_base, positions, state_in, eps=1e-6,
                   ow=None):
    """One step per (b, h): q, k, v, g [B, H, d]; log2_decay float32 [B, H]; positions int64 [B];
    state_in float32 [B, H, d, d].  Returns y, o [B, H, d] and state [B, H, d, d] (fp64)."""
    qf, kf, vf, gf = (widen(x) for x in (q, k, v, g))
    B, H, d = qf.shape
    lg = np.asarray(log2_decay, dtype=np.float64)
    y = np.empty((B, H, d))
    o = np.empty((B, H, d))
    st = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            wq = None if qw is None else (qw if np.ndim(qw) == 1 else qw[h])
            wk = None if kw is None else (kw if np.ndim(kw) == 1 else kw[h])
            p = np.array([positions[b]])
            qt = _prologue(qf[b, h][None], wq, p, rope_base, eps, 1.0)[0]
            kt = _prologue(kf[b, h][None], wk, p, rope_base, eps, 1.0 / math.sqrt(d))[0]
            S = np.exp2(lg[b, h]) * np.asarray(state_in[b, h], dtype=np.float64) + np.outer(kt, vf[b, h])
            ot = qt @ S
            o[b, h] = ot
            yt = ot / math.sqrt(float(np.mean(ot * ot)) + eps)
            if ow is not None:
                yt = yt * (ow if np.ndim(ow) == 1 else ow[h])
            y[b, h] = yt * _sigmoid(gf[b, h])
            st[b, h] = S
    return {"y": y, "o": o, "state": st}
