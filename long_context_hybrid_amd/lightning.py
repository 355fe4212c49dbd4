"""Python binding of ``liblightning.so``, the gfx950 Lightning Attention mixer library.

Argument marshalling only: every step of the mixer runs in the library's HIP kernels.  PyTorch
provides device memory (outputs and the workspace are allocated here with ``torch.empty`` when
the caller does not pass them) and the stream (the current stream unless one is given).  The
functions carry the names of the C entry points declared in ``include/lightning.h``; see that
header for the mathematics, layouts and error behaviour.  A missing library raises at import.
"""
from __future__ import annotations

import ctypes as ct
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LIGHTNING_LIBRARY selects another build of the same sources (e.g. the host-sanitizer build).
LIB_PATH = os.environ.get("LIGHTNING_LIBRARY") or os.path.join(HERE, "liblightning.so")

LT_OK, LT_ERR_INVALID_ARG, LT_ERR_UNSUPPORTED, LT_ERR_WORKSPACE, LT_ERR_HIP = range(5)
LT_F32, LT_BF16 = 0, 1
LT_MAX_HEADS = 256

EXPORTS = (
    "lightning_status_string",
    "lightning_hypenet_gamma",
    "lightning_state_init",
    "lightning_prefill_plan",
    "lightning_prefill_plan_cus",
    "lightning_prefill_workspace_size",
    "lightning_prefill",
    "lightning_prefill_noalloc",
    "lightning_decode_step",
    "lightning_prefill_dd_workspace_size",
    "lightning_prefill_dd",
    "lightning_decode_step_dd",
    "lightning_prefill_backward_workspace_size",
    "lightning_prefill_backward",
    "lightning_layer_prefill_workspace_size",
    "lightning_layer_prefill",
    "lightning_layer_decode_workspace_size",
    "lightning_layer_decode_step",
    "lightning_attn_prefill_workspace_size",
    "lightning_attn_prefill",
    "lightning_attn_decode_workspace_size",
    "lightning_attn_decode_step",
    "lightning_attn_decode_step_dev",
)


class PrefillPlan(ct.Structure):
    """lt_prefill_plan of include/lightning.h."""
    _fields_ = [("chunk", ct.c_int), ("segments", ct.c_int), ("segment_len", ct.c_int),
                ("state_subsegments", ct.c_int), ("subsegment_len", ct.c_int),
                ("backward_segments", ct.c_int), ("backward_segment_len", ct.c_int),
                ("reserved", ct.c_int), ("workspace_bytes", ct.c_size_t),
                ("dd_workspace_bytes", ct.c_size_t), ("backward_workspace_bytes", ct.c_size_t)]


class LightningError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.lightning_status_string(status).decode()}")


def _load() -> ct.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m long_context_hybrid_amd.build` first")
    h = ct.CDLL(LIB_PATH)
    vp, i32, i64, f64, sz = ct.c_void_p, ct.c_int, ct.c_int64, ct.c_double, ct.c_size_t
    h.lightning_status_string.argtypes = [i32]
    h.lightning_status_string.restype = ct.c_char_p
    h.lightning_hypenet_gamma.argtypes = [i32, vp]
    h.lightning_hypenet_gamma.restype = i32
    h.lightning_state_init.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    h.lightning_state_init.restype = i32
    h.lightning_prefill_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    h.lightning_prefill_plan.restype = i32
    h.lightning_prefill_plan_cus.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                             ct.POINTER(PrefillPlan)]
    h.lightning_prefill_plan_cus.restype = i32
    h.lightning_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    h.lightning_prefill_workspace_size.restype = sz
    h.lightning_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, i64, vp, vp,
                                    vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp, vp]
    h.lightning_prefill.restype = i32
    h.lightning_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, i64,
                                            vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    h.lightning_prefill_noalloc.restype = i32
    h.lightning_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, vp, vp,
                                        vp, vp, vp, i32, i32, i32, i32, vp]
    h.lightning_decode_step.restype = i32
    h.lightning_prefill_dd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    h.lightning_prefill_dd_workspace_size.restype = sz
    h.lightning_prefill_dd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, i64, vp, vp,
                                       vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp, vp]
    h.lightning_prefill_dd.restype = i32
    h.lightning_prefill_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    h.lightning_prefill_backward_workspace_size.restype = sz
    # q k v gate qw kw ow stride lambda base eps pos0 state_in dy d_state_out dq dk dv dgate
    # d_state_in dqw dkw dow B T H d dtype segments workspace bytes events stream
    h.lightning_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, i64,
                                             vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                             i32, i32, i32, i32, vp, sz, vp, vp]
    h.lightning_prefill_backward.restype = i32
    h.lightning_decode_step_dd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, vp, vp,
                                           vp, vp, vp, i32, i32, i32, i32, vp]
    h.lightning_decode_step_dd.restype = i32
    h.lightning_layer_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    h.lightning_layer_prefill_workspace_size.restype = sz
    h.lightning_layer_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, i64, vp, vp,
                                          vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp,
                                          vp]
    h.lightning_layer_prefill.restype = i32
    h.lightning_layer_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    h.lightning_layer_decode_workspace_size.restype = sz
    h.lightning_layer_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, f64, f64, vp, vp,
                                              vp, vp, i32, i32, i32, i32, i32, vp, sz, vp]
    h.lightning_layer_decode_step.restype = i32
    h.lightning_attn_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    h.lightning_attn_prefill_workspace_size.restype = sz
    h.lightning_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, f64, f64, i64, vp, vp,
                                         vp, i32, i32, i32, i32, i32, i32, vp, sz, vp, vp]
    h.lightning_attn_prefill.restype = i32
    h.lightning_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i64]
    h.lightning_attn_decode_workspace_size.restype = sz
    h.lightning_attn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, f64, f64, vp, vp,
                                             vp, i64, vp, vp, i32, i32, i32, i32, i32, vp, sz, vp]
    h.lightning_attn_decode_step.restype = i32
    h.lightning_attn_decode_step_dev.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, f64, f64, vp,
                                                 i64, vp, vp, i64, vp, vp, i32, i32, i32, i32,
                                                 i32, vp, sz, vp]
    h.lightning_attn_decode_step_dev.restype = i32
    return h


lib = _load()


def _check(status: int, where: str):
    if status != LT_OK:
        raise LightningError(status, where)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LT_BF16
    if dt == torch.float32:
        return LT_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {dt}")


def _dev(t, name, dtype=None, shape=None, device=None):
    """Device pointer of a tensor, after checking it is a contiguous GPU tensor of the expected
    dtype/shape (a host pointer handed to a kernel would fault the GPU)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return ct.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ct.c_void_p(stream.cuda_stream)


def _norm_weights(qw, kw, ow, H, d, device):
    shape = tuple(qw.shape)
    if shape == (d,):
        stride = 0
    elif shape == (H, d):
        stride = d
    else:
        raise ValueError(f"norm weights must be [d] or [H, d], got {shape}")
    ptrs = [_dev(qw, "q_norm_w", torch.float32, shape, device),
            _dev(kw, "k_norm_w", torch.float32, shape, device),
            _dev(ow, "o_norm_w", torch.float32, shape, device)]
    return ptrs, stride


def _lambda_array(lambdas, H):
    lam = [float(x) for x in lambdas]
    if len(lam) != H:
        raise ValueError(f"need one lambda per head ({H}), got {len(lam)}")
    return (ct.c_double * H)(*lam)


def lightning_status_string(status: int) -> str:
    return lib.lightning_status_string(int(status)).decode()


def lightning_hypenet_gamma(H: int) -> list:
    out = (ct.c_double * max(int(H), 1))()
    _check(lib.lightning_hypenet_gamma(int(H), out), "lightning_hypenet_gamma")
    return list(out)[:H]


def lightning_state_init(state: torch.Tensor, init: torch.Tensor | None = None, stream=None):
    """Zero `state` [B, H, dk, dv] (fp32), or copy `init` (same shape) into it."""
    B, H, dk, dv = state.shape
    dev = state.device
    sp = _dev(state, "state", torch.float32, None, dev)
    ip = _dev(init, "init", torch.float32, state.shape, dev)
    _check(lib.lightning_state_init(sp, B, H, dk, dv, ip, _stream(stream, dev)),
           "lightning_state_init")
    return state


def lightning_prefill_plan(B, T, H, d, dtype=torch.bfloat16, chunk=0, segments=0):
    """(chunk, segments, tokens per segment but the last) that lightning_prefill will use."""
    c, p, n = ct.c_int(0), ct.c_int(0), ct.c_int(0)
    _check(lib.lightning_prefill_plan(B, T, H, d, _dtype_code(dtype), chunk, segments,
                                      ct.byref(c), ct.byref(p), ct.byref(n)),
           "lightning_prefill_plan")
    return c.value, p.value, n.value


def lightning_prefill_plan_cus(num_cus, B, T, H, d, dtype=torch.bfloat16, chunk=0,
                               segments=0) -> dict:
    """The plan (and workspace sizes) of a prefill request on a device with num_cus compute
    units, as a dict of the lt_prefill_plan fields.  Host-only."""
    out = PrefillPlan()
    _check(lib.lightning_prefill_plan_cus(num_cus, B, T, H, d, _dtype_code(dtype), chunk,
                                          segments, ct.byref(out)),
           "lightning_prefill_plan_cus")
    return {name: getattr(out, name) for name, _ in PrefillPlan._fields_ if name != "reserved"}


def lightning_prefill_workspace_size(B, T, H, d, dtype=torch.bfloat16, chunk=0, segments=0) -> int:
    return int(lib.lightning_prefill_workspace_size(B, T, H, d, _dtype_code(dtype), chunk,
                                                    segments))


def lightning_prefill(q, k, v, gate, q_norm_w, k_norm_w, lambdas, rope_base, rms_eps=1e-6,
                      pos0=0, state_in=None, state_out=None, y=None, o_raw=None, o_norm_w=None,
                      chunk=0, segments=0, workspace=None, main_kernel_events=None, stream=None):
    """Prefill ``[B, T, H, d]`` activations; returns ``y`` (allocated if not given).  Pass a
    ``state_out`` tensor ([B, H, d, d] fp32) to receive the final state and an ``o_raw`` tensor
    ([B, T, H, d] fp32) to receive o before the output norm.  ``main_kernel_events`` is None or
    a pair of raw hipEvent_t handles (integers) recorded around the main chunk kernel."""
    B, T, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if y is None:
        y = torch.empty_like(q)
    yp = _dev(y, "y", **act)
    sshape = (B, H, d, d)
    sip = _dev(state_in, "state_in", torch.float32, sshape, dev)
    sop = _dev(state_out, "state_out", torch.float32, sshape, dev)
    orp = _dev(o_raw, "o_raw", torch.float32, q.shape, dev)
    need = lightning_prefill_workspace_size(B, T, H, d, q.dtype, chunk, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsp = _dev(workspace, "workspace", None, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    evp = None
    if main_kernel_events is not None:
        evp = (ct.c_void_p * 2)(*(ct.c_void_p(int(e)) for e in main_kernel_events))
    st = lib.lightning_prefill(*ptrs, qwp, kwp, owp, stride, _lambda_array(lambdas, H),
                               float(rope_base), float(rms_eps), int(pos0), sip, sop, yp, orp,
                               B, T, H, d, dt, int(chunk), int(segments), wsp, wbytes, evp,
                               _stream(stream, dev))
    _check(st, "lightning_prefill")
    return y


def lightning_prefill_noalloc(q, k, v, gate, q_norm_w, k_norm_w, lambdas, rope_base,
                              rms_eps=1e-6, pos0=0, state_in=None, state_out=None, y=None,
                              o_raw=None, o_norm_w=None, chunk=0, segments=0, stream=None):
    """lightning_prefill through the entry point that allocates nothing (its segment states live
    in the library's static device scratch).  ``y`` must be given or is allocated here, before
    the call."""
    B, T, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if y is None:
        y = torch.empty_like(q)
    sshape = (B, H, d, d)
    st = lib.lightning_prefill_noalloc(
        *ptrs, qwp, kwp, owp, stride, _lambda_array(lambdas, H), float(rope_base),
        float(rms_eps), int(pos0), _dev(state_in, "state_in", torch.float32, sshape, dev),
        _dev(state_out, "state_out", torch.float32, sshape, dev), _dev(y, "y", **act),
        _dev(o_raw, "o_raw", torch.float32, q.shape, dev), B, T, H, d, dt, int(chunk),
        int(segments), _stream(stream, dev))
    _check(st, "lightning_prefill_noalloc")
    return y


def lightning_decode_step(q, k, v, gate, q_norm_w, k_norm_w, lambdas, rope_base, positions,
                          state_in, state_out=None, rms_eps=1e-6, y=None, o_raw=None,
                          o_norm_w=None, stream=None):
    """One decode step on ``[B, H, d]`` activations.  ``state_out`` defaults to ``state_in``
    (in-place update).  Returns ``y``."""
    B, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if y is None:
        y = torch.empty_like(q)
    if state_out is None:
        state_out = state_in
    sshape = (B, H, d, d)
    st = lib.lightning_decode_step(*ptrs, qwp, kwp, owp, stride, _lambda_array(lambdas, H),
                                   float(rope_base), float(rms_eps),
                                   _dev(positions, "positions", torch.int64, (B,), dev),
                                   _dev(state_in, "state_in", torch.float32, sshape, dev),
                                   _dev(state_out, "state_out", torch.float32, sshape, dev),
                                   _dev(y, "y", **act), _dev(o_raw, "o_raw", torch.float32, q.shape, dev),
                                   B, H, d, dt, _stream(stream, dev))
    _check(st, "lightning_decode_step")
    return y


# ---- the whole RNN layer ---------------------------------------------------------------------------

def lightning_layer_prefill_workspace_size(B, T, H, d, d_model, dtype=torch.bfloat16, chunk=0,
                                           segments=0) -> int:
    return int(lib.lightning_layer_prefill_workspace_size(B, T, H, d, d_model, _dtype_code(dtype),
                                                          chunk, segments))


def lightning_layer_decode_workspace_size(B, H, d, d_model, dtype=torch.bfloat16) -> int:
    return int(lib.lightning_layer_decode_workspace_size(B, H, d, d_model, _dtype_code(dtype)))


def _layer_weights(w_qkvz, w_o, H, d, d_model, dtype, dev):
    return (_dev(w_qkvz, "w_qkvz", dtype, (4 * H * d, d_model), dev),
            _dev(w_o, "w_o", dtype, (d_model, H * d), dev))


def _workspace(workspace, need, dev):
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, _dev(workspace, "workspace", None, None, dev), \
        workspace.numel() * workspace.element_size()


def lightning_layer_prefill(x, w_qkvz, w_o, q_norm_w, k_norm_w, lambdas, rope_base, H, d,
                            rms_eps=1e-6, pos0=0, state_in=None, state_out=None, out=None,
                            o_norm_w=None, chunk=0, segments=0, workspace=None,
                            stage_events=None, stream=None):
    """The RNN layer on ``x`` [B, T, d_model]: x W_qkvz^T -> mixer -> W_o; returns ``out``
    [B, T, d_model] (allocated if not given).  ``workspace`` (uint8, at least the size query's
    bytes) receives the projections and the mixer output at the offsets the C header gives.
    ``stage_events``: None or four raw hipEvent_t handles (integers)."""
    B, T, d_model = x.shape
    dev = x.device
    dt = _dtype_code(x.dtype)
    xp = _dev(x, "x", x.dtype, x.shape, dev)
    wqp, wop = _layer_weights(w_qkvz, w_o, H, d, d_model, x.dtype, dev)
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if out is None:
        out = torch.empty_like(x)
    outp = _dev(out, "out", x.dtype, x.shape, dev)
    sshape = (B, H, d, d)
    sip = _dev(state_in, "state_in", torch.float32, sshape, dev)
    sop = _dev(state_out, "state_out", torch.float32, sshape, dev)
    need = lightning_layer_prefill_workspace_size(B, T, H, d, d_model, x.dtype, chunk, segments)
    workspace, wsp, wbytes = _workspace(workspace, need, dev)
    evp = None
    if stage_events is not None:
        evp = (ct.c_void_p * 4)(*(ct.c_void_p(int(e)) for e in stage_events))
    st = lib.lightning_layer_prefill(xp, wqp, wop, qwp, kwp, owp, stride,
                                     _lambda_array(lambdas, H), float(rope_base), float(rms_eps),
                                     int(pos0), sip, sop, outp, B, T, H, d, d_model, dt,
                                     int(chunk), int(segments), wsp, wbytes, evp,
                                     _stream(stream, dev))
    _check(st, "lightning_layer_prefill")
    return out


def lightning_layer_decode_step(x, w_qkvz, w_o, q_norm_w, k_norm_w, lambdas, rope_base, H, d,
                                positions, state_in, state_out=None, rms_eps=1e-6, out=None,
                                o_norm_w=None, workspace=None, stream=None):
    """One decode step of the RNN layer on ``x`` [B, d_model]; ``state_out`` defaults to
    ``state_in`` (in place).  Returns ``out`` [B, d_model]."""
    B, d_model = x.shape
    dev = x.device
    dt = _dtype_code(x.dtype)
    xp = _dev(x, "x", x.dtype, x.shape, dev)
    wqp, wop = _layer_weights(w_qkvz, w_o, H, d, d_model, x.dtype, dev)
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if out is None:
        out = torch.empty_like(x)
    if state_out is None:
        state_out = state_in
    sshape = (B, H, d, d)
    need = lightning_layer_decode_workspace_size(B, H, d, d_model, x.dtype)
    workspace, wsp, wbytes = _workspace(workspace, need, dev)
    st = lib.lightning_layer_decode_step(xp, wqp, wop, qwp, kwp, owp, stride,
                                         _lambda_array(lambdas, H), float(rope_base),
                                         float(rms_eps),
                                         _dev(positions, "positions", torch.int64, (B,), dev),
                                         _dev(state_in, "state_in", torch.float32, sshape, dev),
                                         _dev(state_out, "state_out", torch.float32, sshape, dev),
                                         _dev(out, "out", x.dtype, x.shape, dev), B, H, d, d_model,
                                         dt, wsp, wbytes, _stream(stream, dev))
    _check(st, "lightning_layer_decode_step")
    return out


# ---- HyPE softmax attention ------------------------------------------------------------------------

def lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, dtype=torch.bfloat16,
                                          has_key_norm=True, has_key_cache=False) -> int:
    return int(lib.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, _dtype_code(dtype),
                                                         int(bool(has_key_norm)),
                                                         int(bool(has_key_cache))))


def _opt_weight(w, H, d, name, dev, stride):
    if w is None:
        return None
    shape = (d,) if stride == 0 else (H, d)
    return _dev(w, name, torch.float32, shape, dev)


def lightning_attn_prefill(q, k, v, gate, logit_scale_base, q_norm_w=None, k_norm_w=None,
                           o_norm_w=None, rms_eps=1e-6, pos0=0, y=None, o_raw=None,
                           key_cache_out=None, workspace=None, main_kernel_events=None,
                           stream=None):
    """Causal HyPE attention: q, gate [B, T, Hq, d], k, v [B, T, Hkv, d] (bf16).  Norm weights
    are None or fp32 [d] / [heads, d] (all given ones share one layout).  Returns ``y``."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    dev = q.device
    dt = _dtype_code(q.dtype)
    given = [w for w in (q_norm_w, k_norm_w, o_norm_w) if w is not None]
    stride = 0 if all(w.dim() == 1 for w in given) else d
    ptrs = [_dev(q, "q", q.dtype, (B, T, Hq, d), dev), _dev(k, "k", q.dtype, (B, T, Hkv, d), dev),
            _dev(v, "v", q.dtype, (B, T, Hkv, d), dev),
            _dev(gate, "gate", q.dtype, (B, T, Hq, d), dev)]
    wq = _opt_weight(q_norm_w, Hq, d, "q_norm_w", dev, stride)
    wk = _opt_weight(k_norm_w, Hkv, d, "k_norm_w", dev, stride)
    wo = _opt_weight(o_norm_w, Hq, d, "o_norm_w", dev, stride)
    if y is None:
        y = torch.empty_like(q)
    yp = _dev(y, "y", q.dtype, q.shape, dev)
    orp = _dev(o_raw, "o_raw", torch.float32, q.shape, dev)
    kcp = _dev(key_cache_out, "key_cache_out", q.dtype, k.shape, dev)
    need = lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, q.dtype, k_norm_w is not None,
                                                 key_cache_out is not None)
    workspace, wsp, wbytes = _workspace(workspace, need, dev)
    evp = None
    if main_kernel_events is not None:
        evp = (ct.c_void_p * 2)(*(ct.c_void_p(int(e)) for e in main_kernel_events))
    st = lib.lightning_attn_prefill(*ptrs, wq, wk, wo, stride, float(logit_scale_base or 0.0),
                                    float(rms_eps), int(pos0), yp, orp, kcp, B, T, Hq, Hkv, d, dt,
                                    wsp, wbytes, evp, _stream(stream, dev))
    _check(st, "lightning_attn_prefill")
    return y


def lightning_attn_decode_workspace_size(B, Hq, Hkv, d, max_length, dtype=torch.bfloat16) -> int:
    return int(lib.lightning_attn_decode_workspace_size(B, Hq, Hkv, d, _dtype_code(dtype),
                                                        int(max_length)))


def lightning_attn_decode_step(q, k_new, v_new, gate, k_cache, v_cache, lengths,
                               logit_scale_base, q_norm_w=None, k_norm_w=None, o_norm_w=None,
                               rms_eps=1e-6, y=None, o_raw=None, workspace=None, stream=None,
                               max_length=None):
    """One decode step: q, gate [B, Hq, d], k_new, v_new [B, Hkv, d], caches
    [B, capacity, Hkv, d] (bf16).  ``lengths``: a sequence of B ints (host;
    lightning_attn_decode_step), or an int64 CUDA tensor [B] read by the kernels
    (lightning_attn_decode_step_dev), whose values must not exceed ``max_length`` (default
    capacity - 1).  The new token's key and value are written into row lengths[b] of the
    caches.  Returns ``y``."""
    B, Hq, d = q.shape
    Hkv = k_new.shape[1]
    cap = k_cache.shape[1]
    dev = q.device
    dt = _dtype_code(q.dtype)
    given = [w for w in (q_norm_w, k_norm_w, o_norm_w) if w is not None]
    stride = 0 if all(w.dim() == 1 for w in given) else d
    on_device = isinstance(lengths, torch.Tensor) and lengths.is_cuda
    if on_device:
        lp = _dev(lengths, "lengths", torch.int64, (B,), dev)
        bound = cap - 1 if max_length is None else int(max_length)
    else:
        lens = [int(x) for x in lengths]
        if len(lens) != B:
            raise ValueError(f"need one length per batch row ({B})")
        bound = max(lens) if lens else 0
    ptrs = [_dev(q, "q", q.dtype, (B, Hq, d), dev), _dev(k_new, "k_new", q.dtype, (B, Hkv, d), dev),
            _dev(v_new, "v_new", q.dtype, (B, Hkv, d), dev),
            _dev(gate, "gate", q.dtype, (B, Hq, d), dev)]
    wq = _opt_weight(q_norm_w, Hq, d, "q_norm_w", dev, stride)
    wk = _opt_weight(k_norm_w, Hkv, d, "k_norm_w", dev, stride)
    wo = _opt_weight(o_norm_w, Hq, d, "o_norm_w", dev, stride)
    kcp = _dev(k_cache, "k_cache", q.dtype, (B, cap, Hkv, d), dev)
    vcp = _dev(v_cache, "v_cache", q.dtype, (B, cap, Hkv, d), dev)
    if y is None:
        y = torch.empty_like(q)
    yp = _dev(y, "y", q.dtype, q.shape, dev)
    orp = _dev(o_raw, "o_raw", torch.float32, q.shape, dev)
    need = lightning_attn_decode_workspace_size(B, Hq, Hkv, d, max(bound, 0), q.dtype)
    workspace, wsp, wbytes = _workspace(workspace, need, dev)
    if on_device:
        st = lib.lightning_attn_decode_step_dev(
            *ptrs, wq, wk, wo, stride, float(logit_scale_base or 0.0), float(rms_eps), lp, bound,
            kcp, vcp, cap, yp, orp, B, Hq, Hkv, d, dt, wsp, wbytes, _stream(stream, dev))
        _check(st, "lightning_attn_decode_step_dev")
        return y
    st = lib.lightning_attn_decode_step(*ptrs, wq, wk, wo, stride, float(logit_scale_base or 0.0),
                                        float(rms_eps), (ct.c_int64 * B)(*lens), kcp, vcp, cap,
                                        yp, orp, B, Hq, Hkv, d, dt, wsp, wbytes,
                                        _stream(stream, dev))
    _check(st, "lightning_attn_decode_step")
    return y


# ---- data-dependent scalar decay ------------------------------------------------------------------

def lightning_prefill_dd_workspace_size(B, T, H, d, dtype=torch.bfloat16, chunk=0,
                                        segments=0) -> int:
    return int(lib.lightning_prefill_dd_workspace_size(B, T, H, d, _dtype_code(dtype), chunk,
                                                       segments))


def lightning_prefill_dd(q, k, v, gate, q_norm_w, k_norm_w, log2_decay, rope_base, rms_eps=1e-6,
                         pos0=0, state_in=None, state_out=None, y=None, o_raw=None,
                         o_norm_w=None, chunk=0, segments=0, workspace=None,
                         main_kernel_events=None, stream=None):
    """lightning_prefill with a per-token decay: ``log2_decay`` fp32 [B, T, H] (log2 alpha_t)."""
    B, T, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    lgp = _dev(log2_decay, "log2_decay", torch.float32, (B, T, H), dev)
    if y is None:
        y = torch.empty_like(q)
    sshape = (B, H, d, d)
    need = lightning_prefill_dd_workspace_size(B, T, H, d, q.dtype, chunk, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsp = _dev(workspace, "workspace", None, None, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    evp = None
    if main_kernel_events is not None:
        evp = (ct.c_void_p * 2)(*(ct.c_void_p(int(e)) for e in main_kernel_events))
    st = lib.lightning_prefill_dd(*ptrs, qwp, kwp, owp, stride, lgp, float(rope_base),
                                  float(rms_eps), int(pos0),
                                  _dev(state_in, "state_in", torch.float32, sshape, dev),
                                  _dev(state_out, "state_out", torch.float32, sshape, dev),
                                  _dev(y, "y", **act), _dev(o_raw, "o_raw", torch.float32, q.shape, dev),
                                  B, T, H, d, dt, int(chunk), int(segments), wsp, wbytes, evp,
                                  _stream(stream, dev))
    _check(st, "lightning_prefill_dd")
    return y


def lightning_decode_step_dd(q, k, v, gate, q_norm_w, k_norm_w, log2_decay, rope_base, positions,
                             state_in, state_out=None, rms_eps=1e-6, y=None, o_raw=None,
                             o_norm_w=None, stream=None):
    """lightning_decode_step with a per-token decay: ``log2_decay`` fp32 [B, H]."""
    B, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    if y is None:
        y = torch.empty_like(q)
    if state_out is None:
        state_out = state_in
    sshape = (B, H, d, d)
    st = lib.lightning_decode_step_dd(*ptrs, qwp, kwp, owp, stride,
                                      _dev(log2_decay, "log2_decay", torch.float32, (B, H), dev),
                                      float(rope_base), float(rms_eps),
                                      _dev(positions, "positions", torch.int64, (B,), dev),
                                      _dev(state_in, "state_in", torch.float32, sshape, dev),
                                      _dev(state_out, "state_out", torch.float32, sshape, dev),
                                      _dev(y, "y", **act),
                                      _dev(o_raw, "o_raw", torch.float32, q.shape, dev), B, H, d, dt,
                                      _stream(stream, dev))
    _check(st, "lightning_decode_step_dd")
    return y


def lightning_prefill_backward_workspace_size(B, T, H, d, dtype=torch.bfloat16, segments=0) -> int:
    return int(lib.lightning_prefill_backward_workspace_size(B, T, H, d, _dtype_code(dtype),
                                                             segments))


def lightning_prefill_backward(q, k, v, gate, q_norm_w, k_norm_w, lambdas, rope_base, dy,
                               rms_eps=1e-6, pos0=0, state_in=None, d_state_out=None,
                               o_norm_w=None, want_state_grad=True, want_weight_grads=True,
                               segments=0, workspace=None, kernel_events=None, stream=None):
    """Gradients of sum(dy * y) + sum(d_state_out * state_out) for lightning_prefill on the same
    inputs.  Returns a dict: dq, dk, dv, dgate (like q), d_state_in [B, H, d, d] fp32 (with
    ``want_state_grad``) and d_q_norm_w, d_k_norm_w, d_o_norm_w (with ``want_weight_grads``;
    shaped like the weights, d_o_norm_w also when o_norm_w is None)."""
    B, T, H, d = q.shape
    dev = q.device
    dt = _dtype_code(q.dtype)
    act = dict(dtype=q.dtype, shape=q.shape, device=dev)
    ptrs = [_dev(t, n, **act) for t, n in ((q, "q"), (k, "k"), (v, "v"), (gate, "gate"))]
    (qwp, kwp, owp), stride = _norm_weights(q_norm_w, k_norm_w, o_norm_w, H, d, dev)
    out = {n: torch.empty_like(q) for n in ("dq", "dk", "dv", "dgate")}
    sshape = (B, H, d, d)
    if want_state_grad:
        out["d_state_in"] = torch.empty(sshape, dtype=torch.float32, device=dev)
    wshape = (H, d) if stride else (d,)
    if want_weight_grads:
        for n in ("d_q_norm_w", "d_k_norm_w", "d_o_norm_w"):
            out[n] = torch.empty(wshape, dtype=torch.float32, device=dev)
    need = lightning_prefill_backward_workspace_size(B, T, H, d, q.dtype, segments)
    workspace, wsp, wbytes = _workspace(workspace, need, dev)
    evp = None
    if kernel_events is not None:
        evp = (ct.c_void_p * 4)(*(ct.c_void_p(int(e)) for e in kernel_events))
    st = lib.lightning_prefill_backward(
        *ptrs, qwp, kwp, owp, stride, _lambda_array(lambdas, H), float(rope_base),
        float(rms_eps), int(pos0), _dev(state_in, "state_in", torch.float32, sshape, dev),
        _dev(dy, "dy", **act), _dev(d_state_out, "d_state_out", torch.float32, sshape, dev),
        *(_dev(out[n], n, **act) for n in ("dq", "dk", "dv", "dgate")),
        _dev(out.get("d_state_in"), "d_state_in", torch.float32, sshape, dev),
        *(_dev(out.get(n), n, torch.float32, wshape, dev)
          for n in ("d_q_norm_w", "d_k_norm_w", "d_o_norm_w")),
        B, T, H, d, dt, int(segments), wsp, wbytes, evp, _stream(stream, dev))
    _check(st, "lightning_prefill_backward")
    return out
