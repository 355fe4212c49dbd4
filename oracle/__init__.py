"""fp64 CPU oracle of the HypeNet RNN mixer (Lightning Attention) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU library and its Python binding never import it, and it imports nothing
from them.  It wraps ``liboracle.so`` (built from ``oracle.c`` by ``oracle/build.py``).

The arithmetic lives in ``oracle.c``; see its header for the passages it follows
("Hybrid Linear Attention Done Right", Appendix A, Eq. 18 and Eq. 19; Section 5.2, Eq. 12 and
Eq. 14).  This module only marshals numpy arrays:

* projections q, k, v and gate logits g are ``[B, T, H, d]`` arrays of either ``float32`` or
  ``uint16`` (the raw bits of bf16 values, widened exactly inside the oracle);
* norm weights are float32 ``[H, d]`` (or ``[d]``, shared by all heads);
* ``lambdas`` is one decay per head, float64;
* outputs are float64.
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1

_lib = None


def _bind(lib):
    dp = ct.c_void_p
    i32, i64, f64 = ct.c_int, ct.c_int64, ct.c_double
    lib.oracle_rmsnorm.argtypes = [dp, dp, i32, f64, dp]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_rope.argtypes = [dp, i32, f64, f64, dp]
    lib.oracle_rope.restype = None
    lib.oracle_sigmoid.argtypes = [f64]
    lib.oracle_sigmoid.restype = f64
    common = [dp, dp, dp, dp, i32, dp, dp, dp, i32, dp, f64, f64, i64, dp, i32, i32, i32, i32]
    lib.oracle_prefill_slices.argtypes = common + [dp, dp, i32, dp, dp, dp, i32]
    lib.oracle_prefill_slices.restype = i32
    lib.oracle_chunked_slices.argtypes = common + [i32, dp, dp, i32, dp, dp, dp, i32]
    lib.oracle_chunked_slices.restype = i32
    lib.oracle_decode_step.argtypes = [dp, dp, dp, dp, i32, dp, dp, dp, i32, dp, f64, f64, dp, dp,
                                       i32, i32, i32, dp, dp, dp, i32]
    lib.oracle_decode_step.restype = i32
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library.  ``path`` selects another build of
    the same source, e.g. a deliberately mutated copy used to show that the pins catch it."""
    global _lib
    if path is not None:
        return _bind(ct.CDLL(path))
    if _lib is None:
        alt = os.environ.get("ORACLE_LIBRARY")  # another build of oracle.c (sanitizer runs)
        if alt:
            _lib = _bind(ct.CDLL(alt))
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build as _build

            _build.build()
        _lib = _bind(ct.CDLL(LIB_PATH))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ct.c_void_p)


def _as_input(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    raise TypeError(f"oracle inputs must be float32 or bf16 bits (uint16), got {x.dtype}")


def _weights(w, H, d, name):
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape == (d,):
        return w, 0
    if w.shape == (H, d):
        return w, d
    raise ValueError(f"{name} must be [d] or [H, d], got {w.shape}")


def rmsnorm(x, w=None, eps=1e-6, lib=None):
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    lib.oracle_rmsnorm(_ptr(x), _ptr(wd), x.shape[-1], eps, _ptr(out))
    return out


def rope(x, pos, base, lib=None):
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib.oracle_rope(_ptr(x), x.shape[-1], float(pos), float(base), _ptr(out))
    return out


def sigmoid(x, lib=None):
    lib = lib or load()
    return lib.oracle_sigmoid(float(x))


def prefill(q, k, v, g, qw, kw, lambdas, rope_base, eps=1e-6, pos0=0, state_in=None, ow=None,
            slices=None, chunk=None, want_o=True, want_state=True, nthreads=0, lib=None):
    """Run the oracle over the (b, h) pairs in ``slices`` (default: all).

    ``chunk=None`` runs the token-by-token recurrence; an integer runs the chunkwise form.
    Returns a dict with ``y`` and ``o`` of shape [n, T, d], ``state`` of shape [n, d, d] (all
    float64), ``slices`` and ``threads`` (the number of threads the oracle used).
    """
    lib = lib or load()
    q, dt = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    g, dg = _as_input(g)
    if len({dt, dk, dv, dg}) != 1:
        raise TypeError("q, k, v, g must share one dtype")
    B, T, H, d = q.shape
    for name, a in (("k", k), ("v", v), ("g", g)):
        if a.shape != q.shape:
            raise ValueError(f"{name} shape {a.shape} != q shape {q.shape}")
    qw, ws = _weights(qw, H, d, "qw")
    kw, ws2 = _weights(kw, H, d, "kw")
    if ow is not None:
        ow, ws3 = _weights(ow, H, d, "ow")
        if ws3 != ws:
            raise ValueError("all norm weights must share one layout")
    if ws != ws2:
        raise ValueError("all norm weights must share one layout")
    lam = np.ascontiguousarray(lambdas, dtype=np.float64)
    if lam.shape != (H,):
        raise ValueError("one lambda per head")
    s0 = None if state_in is None else np.ascontiguousarray(state_in, dtype=np.float32)
    if s0 is not None and s0.shape != (B, H, d, d):
        raise ValueError("state_in must be [B, H, d, d]")
    if slices is None:
        slices = [(b, h) for b in range(B) for h in range(H)]
    bi = np.array([s[0] for s in slices], dtype=np.int32)
    hi = np.array([s[1] for s in slices], dtype=np.int32)
    n = len(slices)
    y = np.empty((n, T, d), dtype=np.float64)
    o = np.empty((n, T, d), dtype=np.float64) if want_o else None
    st = np.empty((n, d, d), dtype=np.float64) if want_state else None
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), dt, _ptr(qw), _ptr(kw), _ptr(ow), ws, _ptr(lam),
            float(rope_base), float(eps), int(pos0), _ptr(s0), B, T, H, d)
    if chunk is None:
        rc = lib.oracle_prefill_slices(*head, _ptr(bi), _ptr(hi), n, _ptr(y), _ptr(o), _ptr(st),
                                       int(nthreads))
    else:
        rc = lib.oracle_chunked_slices(*head, int(chunk), _ptr(bi), _ptr(hi), n, _ptr(y), _ptr(o),
                                       _ptr(st), int(nthreads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    return {"y": y, "o": o, "state": st, "slices": slices, "threads": rc}


def decode_step(q, k, v, g, qw, kw, lambdas, rope_base, positions, state_in, eps=1e-6, ow=None,
                nthreads=0, lib=None):
    """One recurrence step per (b, h).  q, k, v, g: [B, H, d]; positions: int64 [B];
    state_in: float32 [B, H, d, d].  Returns y, o [B, H, d] and state [B, H, d, d] (float64)."""
    lib = lib or load()
    q, dt = _as_input(q)
    k, _ = _as_input(k)
    v, _ = _as_input(v)
    g, _ = _as_input(g)
    B, H, d = q.shape
    qw, ws = _weights(qw, H, d, "qw")
    kw, _ = _weights(kw, H, d, "kw")
    if ow is not None:
        ow, _ = _weights(ow, H, d, "ow")
    lam = np.ascontiguousarray(lambdas, dtype=np.float64)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    s0 = np.ascontiguousarray(state_in, dtype=np.float32)
    if s0.shape != (B, H, d, d) or pos.shape != (B,) or lam.shape != (H,):
        raise ValueError("bad decode shapes")
    y = np.empty((B, H, d), dtype=np.float64)
    o = np.empty((B, H, d), dtype=np.float64)
    st = np.empty((B, H, d, d), dtype=np.float64)
    rc = lib.oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), dt, _ptr(qw), _ptr(kw),
                                _ptr(ow), ws, _ptr(lam), float(rope_base), float(eps), _ptr(pos),
                                _ptr(s0), B, H, d, _ptr(y), _ptr(o), _ptr(st), int(nthreads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    return {"y": y, "o": o, "state": st, "threads": rc}
