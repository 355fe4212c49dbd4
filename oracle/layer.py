"""fp64 CPU oracle of the whole HypeNet RNN layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; it imports nothing from the GPU library.

It follows "Hybrid Linear Attention Done Right", Appendix A, Eq. 18 (RNN layers) with the
projections written out: per token, q, k, v and the gate logits are x W_q, x W_k, x W_v and
x W_z for every head, the mixer (the recurrence of ``oracle.prefill`` / ``oracle.decode_step``)
turns them into y, and the layer output is the sum over heads of y^(h) W_o^(h)T (the text after
Eq. 16 says the layer output is the sum of the heads' outputs), i.e. the heads side by side
times W_o^T.

Weights use the library's storage: ``w_qkvz`` is [4 H d, d_model] with row n the weights of
projection output n (blocks q | k | v | z, head-major inside each), and ``w_o`` is
[d_model, H d].  Products are fp64 (numpy's matmul is the only library step).

Precision reading: the layer's tensors between steps (the projections and the mixer output y)
are stored in the activation dtype, as in a bf16 model; this oracle rounds them at the same two
points, to nearest with ties to even from the exact fp64 value (``round_bf16``), and keeps every
other step in fp64.
"""
from __future__ import annotations

import numpy as np

from . import BF16, F32, decode_step, prefill

_BF16_MIN_NORMAL = 2.0 ** -126


def round_bf16(x):
    """Nearest bfloat16 value of each fp64 entry (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits and fp32's exponent range: a normal value m 2^e with
    0.5 <= |m| < 1 rounds m to a multiple of 2^-8; below 2^-126 the spacing is fixed at 2^-133.
    Values beyond the largest finite bfloat16 round to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    with np.errstate(over="ignore", invalid="ignore"):
        normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
        r = np.where(np.abs(x) < _BF16_MIN_NORMAL, sub, normal)
        big = np.abs(r) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, x), r)


def bf16_bits(x):
    """The bfloat16 bit patterns (uint16) of values already on the bfloat16 grid."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16 values")
    return (u >> 16).astype(np.uint16)


def widen(a):
    """fp64 copy of stored activations: bf16 bits (uint16) or float32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError(f"expected bf16 bits (uint16) or float32, got {a.dtype}")


def _dtype_of(a):
    return BF16 if np.asarray(a).dtype == np.uint16 else F32


def store(x, dtype):
    """Round fp64 values to the storage dtype; returns what the oracle's mixer takes (bf16 bits
    or float32)."""
    if dtype == BF16:
        return bf16_bits(round_bf16(x))
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def projections(x, w_qkvz, H, d, heads=None, row_block=65536):
    """The stored projections x W^T for the rows of ``x`` ([..., d_model]).

    Returns q, k, v, g of shape [..., n, d] in the storage dtype of ``x`` for the heads in
    ``heads`` (default: all H), computed ``row_block`` rows at a time to bound memory.
    """
    dt = _dtype_of(x)
    x = np.asarray(x)
    lead, dm = x.shape[:-1], x.shape[-1]
    if w_qkvz.shape != (4 * H * d, dm):
        raise ValueError(f"w_qkvz must be [{4 * H * d}, {dm}], got {w_qkvz.shape}")
    heads = list(range(H)) if heads is None else list(heads)
    cols = np.concatenate([blk * H * d + h * d + np.arange(d)
                           for blk in range(4) for h in heads])
    w = widen(w_qkvz[cols])  # [4 n d, d_model]
    xf = x.reshape(-1, dm)
    rows = xf.shape[0]
    n = len(heads)
    out = np.empty((rows, 4 * n * d), dtype=np.uint16 if dt == BF16 else np.float32)
    for r0 in range(0, rows, row_block):
        p = widen(xf[r0:r0 + row_block]) @ w.T
        out[r0:r0 + row_block] = store(p, dt)
    blocks = out.reshape(*lead, 4, n, d)
    return tuple(np.ascontiguousarray(blocks[..., i, :, :]) for i in range(4))


def layer_prefill(x, w_qkvz, w_o, qw, kw, lambdas, rope_base, H, d, eps=1e-6, pos0=0,
                  state_in=None, ow=None, nthreads=0):
    """The layer over ``x`` [B, T, d_model] (bf16 bits or float32).

    Returns a dict with ``out`` [B, T, d_model] (fp64), ``state`` [B, H, d, d] (fp64), and the
    stored intermediates ``proj`` [B, T, 4 H d] and ``y`` [B, T, H d] as fp64 values.
    """
    dt = _dtype_of(x)
    B, T, dm = x.shape
    if w_o.shape != (dm, H * d):
        raise ValueError(f"w_o must be [{dm}, {H * d}], got {w_o.shape}")
    q, k, v, g = projections(x, w_qkvz, H, d)
    r = prefill(q, k, v, g, qw, kw, lambdas, rope_base, eps=eps, pos0=pos0, state_in=state_in,
                ow=ow, want_o=False, nthreads=nthreads)
    # r["y"] is [(b, h) slices in b-major order, T, d]
    y = r["y"].reshape(B, H, T, d).transpose(0, 2, 1, 3).reshape(B, T, H * d)
    ys = widen(store(y, dt))
    out = ys @ widen(w_o).T
    proj = np.concatenate([widen(a).reshape(B, T, H * d) for a in (q, k, v, g)], axis=-1)
    return {"out": out, "state": r["state"].reshape(B, H, d, d), "proj": proj, "y": ys,
            "threads": r["threads"]}


def layer_decode_step(x, w_qkvz, w_o, qw, kw, lambdas, rope_base, H, d, positions, state_in,
                      eps=1e-6, ow=None):
    """One decode step of the layer on ``x`` [B, d_model]; returns ``out`` [B, d_model],
    ``state`` [B, H, d, d], ``proj`` [B, 4 H d] and ``y`` [B, H d] (fp64)."""
    dt = _dtype_of(x)
    B, dm = x.shape
    q, k, v, g = projections(x, w_qkvz, H, d)
    r = decode_step(q, k, v, g, qw, kw, lambdas, rope_base, positions, state_in, eps=eps, ow=ow)
    ys = widen(store(r["y"].reshape(B, H * d), dt))
    out = ys @ widen(w_o).T
    proj = np.concatenate([widen(a).reshape(B, H * d) for a in (q, k, v, g)], axis=-1)
    return {"out": out, "state": r["state"], "proj": proj, "y": ys}
