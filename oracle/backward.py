"""fp64 CPU oracle of the mixer's gradients -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; it imports nothing from the GPU library.

The pages train the RNN layers through this mixer (HALO, "Hybrid Linear Attention Done Right",
Section 4.2, Eq. 7: each RNN layer regressed on its attention teacher; Sections 4.4 and 4.5:
end-to-end distillation and long-context finetuning, Appendix B, Table 5) but print no backward
pass.  What the training needs is the derivative of the forward pass of Appendix A, Eq. 18 (with
the QK-norm of Section 5.2, Eq. 12 and the gated output norm of Eq. 14), so this module writes
that derivative out as the adjoint of the token recurrence, per (b, h), in fp64.

Forward, per token t at position p = pos0 + t (as in the forward oracle):

    x^ = q_t r_q, r_q = (mean(q_t^2) + eps)^(-1/2);   q~ = R_p (x^ * w_q)
    k~ = R_p (RMSNorm(k_t) * w_k) / sqrt(d)
    S_t = lambda S_{t-1} + k~^T v_t;   o_t = q~ S_t
    n_t = o_t r_o, r_o = (mean(o_t^2) + eps)^(-1/2);   y_t = n_t * w_o * sigmoid(g_t)

Backward, given dy_t = dL/dy_t and dS_out = dL/dS_{T-1} (zero when absent):

    output gate and norm:  dg = dy n w_o s (1 - s) with s = sigmoid(g);  dn = dy w_o s
                           do = r_o (dn - n mean(dn n));  dw_o += dy n s
    query rule o_t = q~ S_t:           dq~_t = do_t S_t^T
    update rule, in reverse time with G_t = dL/dS_t:
        G_{T-1} = dS_out + q~_{T-1}^T do_{T-1},   G_{t} = lambda G_{t+1} + q~_t^T do_t
        dk~_t = v_t G_t^T,   dv_t = k~_t G_t,   dS_in = lambda G_0
    rotation and norms:    dq^ = R_p^T dq~ = R_{-p} dq~;  dw_q += dq^ x^
                           dq = r_q (dq^ w_q - x^ mean(dq^ w_q x^))
                           (keys alike, with dk^ = R_{-p} dk~ / sqrt(d))

The derivative of RMSNorm, x r with r = (mean(x^2) + eps)^(-1/2), is the usual
d(x r)/dx = r (I - n n^T / d) with n = x r; R_p is orthogonal, so its adjoint is R_{-p}.
The prologue reuses the (pinned) RMSNorm and RoPE routines of ``oracle``.
"""
from __future__ import annotations

import math

import numpy as np

from . import rmsnorm, rope
from .layer import widen


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _wrow(w, h, d):
    if w is None:
        return np.ones(d)
    w = np.asarray(w, dtype=np.float64)
    return w if w.ndim == 1 else w[h]


def _norm_rows(x, eps):
    """x^ = x r per row and r, for x [T, d] (RMSNorm without its weight)."""
    xh = np.empty_like(x)
    for t in range(x.shape[0]):
        xh[t] = rmsnorm(x[t], None, eps)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    return xh, r


def _rotate_rows(x, pos, base):
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        out[t] = rope(x[t], float(pos[t]), base)
    return out


def _norm_backward(dxh, xh, r):
    """Gradient through x^ = x r (rows): r (dx^ - x^ mean(dx^ x^))."""
    m = np.mean(dxh * xh, axis=1, keepdims=True)
    return r[:, None] * (dxh - xh * m)


def core_forward(qt, kt, v, lam, S0=None):
    """The recurrence on already normalised, rotated rows: o [T, d] and the final state."""
    T, d = qt.shape
    S = np.zeros((d, d)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, d))
    for t in range(T):
        S = lam * S + np.outer(kt[t], v[t])
        o[t] = qt[t] @ S
    return o, S


def core_backward(qt, kt, v, lam, do, S0=None, dS_out=None):
    """Adjoint of ``core_forward``: (dq~, dk~, dv, dS_in) for output gradients ``do`` [T, d]
    and the final-state gradient ``dS_out`` (zeros when None)."""
    T, d = qt.shape
    S = np.zeros((d, d)) if S0 is None else np.array(S0, dtype=np.float64)
    dqt = np.empty((T, d))
    for t in range(T):  # query rule: needs S_t, forward in time
        S = lam * S + np.outer(kt[t], v[t])
        dqt[t] = S @ do[t]
    G = np.zeros((d, d)) if dS_out is None else np.array(dS_out, dtype=np.float64)
    dkt = np.empty((T, d))
    dv = np.empty((T, d))
    for t in range(T - 1, -1, -1):  # update rule: reverse time
        G = G + np.outer(qt[t], do[t])
        dkt[t] = G @ v[t]
        dv[t] = kt[t] @ G
        G = lam * G
    return dqt, dkt, dv, G


def prefill_backward(q, k, v, g, dy, qw, kw, lambdas, rope_base, eps=1e-6, pos0=0,
                     state_in=None, d_state_out=None, ow=None, slices=None):
    """Gradients of L = sum(dy * y) + sum(d_state_out * state_out) for the prefill of
    lightning_prefill (fixed per-head decay).

    q, k, v, g, dy: [B, T, H, d] (bf16 bits or float32); qw, kw (and ow): float32 [H, d] or
    [d]; lambdas: [H]; state_in, d_state_out: [B, H, d, d] or None.

    Returns, for the (b, h) pairs in ``slices`` (default all): dq, dk, dv, dg [n, T, d],
    d_state_in [n, d, d], and each pair's contribution to the norm-weight gradients dqw, dkw,
    dow [n, d] (sum them over the pairs that share a weight row).  All fp64.
    """
    q, k, v, g, dy = (np.asarray(x) for x in (q, k, v, g, dy))
    B, T, H, d = q.shape
    lam = np.asarray(lambdas, dtype=np.float64)
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    pos = (pos0 + np.arange(T)).astype(np.float64)
    n = len(slices)
    out = {name: np.empty((n, T, d)) for name in ("dq", "dk", "dv", "dg")}
    out.update({name: np.empty((n, d)) for name in ("dqw", "dkw", "dow")})
    out["d_state_in"] = np.empty((n, d, d))
    out["slices"] = slices
    ks = 1.0 / math.sqrt(d)
    for i, (b, h) in enumerate(slices):
        wq, wk, wo = _wrow(qw, h, d), _wrow(kw, h, d), _wrow(ow, h, d)
        # inputs are widened one (b, h) slice at a time
        xq, rq = _norm_rows(widen(q[b, :, h]), eps)
        xk, rk = _norm_rows(widen(k[b, :, h]), eps)
        qt = _rotate_rows(xq * wq, pos, rope_base)
        kt = _rotate_rows(xk * wk, pos, rope_base) * ks
        vv = widen(v[b, :, h])
        S0 = None if state_in is None else state_in[b, h]
        o, _ = core_forward(qt, kt, vv, lam[h], S0)
        # output gate and norm
        ro = 1.0 / np.sqrt(np.mean(o * o, axis=1) + eps)
        nrm = o * ro[:, None]
        s = _sigmoid(widen(g[b, :, h]))
        dyb = widen(dy[b, :, h])
        out["dg"][i] = dyb * nrm * wo * s * (1.0 - s)
        out["dow"][i] = np.sum(dyb * nrm * s, axis=0)
        do = _norm_backward(dyb * wo * s, nrm, ro)
        dS = None if d_state_out is None else d_state_out[b, h]
        dqt, dkt, dvv, dS0 = core_backward(qt, kt, vv, lam[h], do, S0, dS)
        out["dv"][i] = dvv
        out["d_state_in"][i] = dS0
        # rotation and input norms
        dqh = _rotate_rows(dqt, -pos, rope_base)
        dkh = _rotate_rows(dkt, -pos, rope_base) * ks
        out["dqw"][i] = np.sum(dqh * xq, axis=0)
        out["dkw"][i] = np.sum(dkh * xk, axis=0)
        out["dq"][i] = _norm_backward(dqh * wq, xq, rq)
        out["dk"][i] = _norm_backward(dkh * wk, xk, rk)
    return out
