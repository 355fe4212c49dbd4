"""fp64 CPU oracle of HypeNet's softmax-attention mixer (HyPE) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; it imports nothing from the GPU library.

It follows "Hybrid Linear Attention Done Right", Appendix A, Eq. 17 (attention layers) with
Section 5.1, Eq. 11 (HyPE: no position encoding in attention layers, and the position-dependent
logits scale s_t = log_a(t + a)), per query head h of a batch row:

    q^ = RMSNorm(q_t) w_q    k^ = RMSNorm(k_j) w_k      (only when QK-norm weights are given; the
                                                         pages leave the attention QK-norm to the
                                                         base model, and Qwen3 has one)
    score(t, j) = s_t (q^_t . k^_j) / sqrt(d)           for keys j <= t (causal), no RoPE
    o_t = sum_j softmax_j(score(t, .)) v_j
    y_t = RMSNorm(o_t) w_o * sigmoid(g_t)               (output gate, Eq. 14 / Eq. 17)

Grouped-query attention: query head h reads key/value head h // (Hq / Hkv), the grouping whose
key/value heads the RNN layers clone (Eq. 13).  Positions are 0-based absolute positions
p_t = pos0 + t, so s = log_a(a) = 1 at the first position; a = None (or 0) means s_t = 1.
A prefill call attends over its own T tokens (keys at positions pos0 .. pos0 + T - 1).

Inputs are bf16 bit patterns (uint16) or float32 arrays, widened exactly; all arithmetic is fp64,
with a max-subtracted softmax (exact in real arithmetic, so no reading is needed for it).
"""
from __future__ import annotations

import math

import numpy as np

from .layer import widen


def logit_scale(pos, a):
    """s = log_a(pos + a), or 1 when a is None or 0 (Eq. 11)."""
    pos = np.asarray(pos, dtype=np.float64)
    if not a:
        return np.ones_like(pos)
    return np.log(pos + a) / math.log(a)


def _rmsnorm(x, w, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _weights(w, H, d):
    if w is None:
        return None
    w = np.asarray(w, dtype=np.float64)
    if w.shape == (d,):
        return np.broadcast_to(w, (H, d))
    if w.shape != (H, d):
        raise ValueError(f"norm weight must be [d] or [{H}, d], got {w.shape}")
    return w


def attn_prefill(q, k, v, g, qw=None, kw=None, ow=None, a=None, eps=1e-6, pos0=0, rows=None,
                 heads=None, batches=None, want_k_hat=True):
    """Causal HyPE attention over one prefill call.

    q, g: [B, T, Hq, d]; k, v: [B, T, Hkv, d] (bf16 bits or float32).  ``rows`` selects query
    tokens (default all), ``heads`` query heads and ``batches`` batch rows.  Returns ``y`` and
    ``o`` of shape [nb, nrows, nheads, d] (fp64) and, with ``want_k_hat``, the normalised keys
    ``k_hat`` [B, T, Hkv, d].  Inputs are widened one (batch row, key/value head) at a time, and
    queries and gates only at the requested rows.
    """
    q, k, v, g = (np.asarray(x) for x in (q, k, v, g))
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows)
    heads = list(range(Hq)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    qwf, kwf, owf = _weights(qw, Hq, d), _weights(kw, Hkv, d), _weights(ow, Hq, d)
    s = logit_scale(pos0 + rows, a)
    y = np.empty((len(batches), len(rows), len(heads), d))
    o = np.empty_like(y)
    k_hat = np.empty((B, T, Hkv, d)) if want_k_hat else None
    for bi, b in enumerate(batches):
        qb = widen(q[b, rows])  # [nrows, Hq, d]
        gb = widen(g[b, rows])
        for kv in sorted({h // grp for h in heads} | (set(range(Hkv)) if want_k_hat else set())):
            K = widen(k[b, :, kv])
            if kwf is not None:
                K = _rmsnorm(K, kwf[kv], eps)
            if want_k_hat:
                k_hat[b, :, kv] = K
            V = widen(v[b, :, kv])
            for hi, h in enumerate(heads):
                if h // grp != kv:
                    continue
                qh = qb[:, h]
                if qwf is not None:
                    qh = _rmsnorm(qh, qwf[h], eps)
                for ri, t in enumerate(rows):
                    sc = s[ri] * (K[:t + 1] @ qh[ri]) / math.sqrt(d)
                    w = np.exp(sc - sc.max())
                    ot = (w @ V[:t + 1]) / w.sum()
                    o[bi, ri, hi] = ot
                    yo = ot / math.sqrt(float(np.mean(ot * ot)) + eps)
                    if owf is not None:
                        yo = yo * owf[h]
                    y[bi, ri, hi] = yo * _sigmoid(gb[ri, h])
    return {"y": y, "o": o, "k_hat": k_hat}


def attn_decode_step(q, k_new, v_new, g, k_cache, v_cache, lengths, qw=None, kw=None, ow=None,
                     a=None, eps=1e-6):
    """One decode step: batch row b's new token sits at position lengths[b] and attends to the
    lengths[b] cached (already normalised) keys and values plus itself.

    q, g: [B, Hq, d]; k_new, v_new: [B, Hkv, d]; k_cache, v_cache: [B, Tmax, Hkv, d].
    Returns y, o [B, Hq, d] and the new token's normalised key k_hat [B, Hkv, d].
    """
    qf, knf, vnf, gf = (widen(x) for x in (q, k_new, v_new, g))
    kc, vc = widen(k_cache), widen(v_cache)
    B, Hq, d = qf.shape
    Hkv = knf.shape[1]
    grp = Hq // Hkv
    qwf, kwf, owf = _weights(qw, Hq, d), _weights(kw, Hkv, d), _weights(ow, Hq, d)
    khat = knf if kwf is None else _rmsnorm(knf, kwf[None], eps)
    y = np.empty((B, Hq, d))
    o = np.empty_like(y)
    for b in range(B):
        n = int(lengths[b])
        s = float(logit_scale(n, a))
        for h in range(Hq):
            kv = h // grp
            qh = qf[b, h] if qwf is None else _rmsnorm(qf[b, h], qwf[h], eps)
            K = np.concatenate([kc[b, :n, kv], khat[b, kv][None]])
            V = np.concatenate([vc[b, :n, kv], vnf[b, kv][None]])
            sc = s * (K @ qh) / math.sqrt(d)
            w = np.exp(sc - sc.max())
            ot = (w @ V) / w.sum()
            o[b, h] = ot
            yo = ot / math.sqrt(float(np.mean(ot * ot)) + eps)
            if owf is not None:
                yo = yo * owf[h]
            y[b, h] = yo * _sigmoid(gf[b, h])
    return {"y": y, "o": o, "k_hat": khat}
