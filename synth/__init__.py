"""Seeded synthetic workloads for the Lightning Attention mixer.

This module only draws inputs: it holds none of the mixer's arithmetic, and both the GPU path
(through the tests and the benchmark) and the fp64 oracle receive the identical tensors it
returns.  Values are drawn in float32 from a seeded ``torch.Generator`` and rounded once to the
storage dtype, so the bits that reach the GPU are the bits the oracle widens.

The named workloads mirror the shapes of the layers the pages benchmark (Qwen3-shaped RNN
layers with 128-wide heads, batch 1, long context; "Hybrid Linear Attention Done Right",
Table 6 and Section 6.6).  Real activations need trained weights and datasets that are not
available here; after the prologue's RMSNorm and RoPE the q/k statistics have the realistic
scale, and only v and the gate logits are idealised as N(0, 1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


def qwen_lambdas(H: int) -> list[float]:
    """Per-head decays 1 - 2^-(5 + 8h/H), h = 0..H-1, used by the Qwen3-shaped workloads."""
    return [1.0 - 2.0 ** (-(5.0 + 8.0 * h / H)) for h in range(H)]


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    T: int
    H: int
    d: int
    dtype: torch.dtype
    lambdas: tuple
    rope_base: float
    norm_w: str  # "ones" or "uniform" (U(0.5, 1.5) per head and channel)
    state: str  # "zeros" or "randn" (0.01 * N(0, 1))
    chunk: int  # 0 = library default
    seed: int
    eps: float = 1e-6
    pos0: int = 0


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    B: int
    H: int
    d: int
    dtype: torch.dtype
    lambdas: tuple
    rope_base: float
    max_pos: int
    seed: int
    eps: float = 1e-6


TINY = PrefillSpec("tiny prefill B=1 H=2 T=256 d=64 fp32", 1, 256, 2, 64, torch.float32,
                   (0.9, 0.99), 1e4, "ones", "zeros", 64, 1000)
QWEN17_32K = PrefillSpec("Qwen3-1.7B-shaped RNN layer prefill B=1 H=16 T=32768 d=128 bf16", 1,
                         32768, 16, 128, torch.bfloat16, tuple(qwen_lambdas(16)), 1e6, "uniform",
                         "zeros", 0, 1001)
QWEN17_512K = dataclasses.replace(
    QWEN17_32K, name="Qwen3-1.7B-shaped RNN layer prefill B=1 H=16 T=524288 d=128 bf16",
    T=524288, seed=1002)
DECODE_B64 = DecodeSpec("batched decode step B=64 H=16 d=128 bf16, fp32 state", 64, 16, 128,
                        torch.bfloat16, tuple(qwen_lambdas(16)), 1e6, 524288, 1003)
QWEN8_128K = PrefillSpec("Qwen3-8B-shaped RNN layer prefill B=4 H=32 T=131072 d=128 bf16", 4,
                         131072, 32, 128, torch.bfloat16, tuple(qwen_lambdas(32)), 1e6, "uniform",
                         "randn", 0, 1004)

@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Inputs of the whole RNN layer: x [B, T, d_model] and the projection weights.

    values = "gauss": x ~ N(0, 1) (the layer input is an RMS-normalised residual stream) and
    weights ~ N(0, 1/fan_in), so the projections have unit scale like the mixer workloads.
    values = "ternary": x and the weights drawn from {-1, 0, 1} (weights mostly 0), so that with
    d_model <= 256 every projection is an integer of magnitude <= 256, exactly representable in
    bf16 and summed exactly in fp32 (a case where the projections carry no rounding at all).
    """
    name: str
    B: int
    T: int  # 1 for a decode step
    H: int
    d: int
    d_model: int
    dtype: torch.dtype
    lambdas: tuple
    rope_base: float
    norm_w: str
    state: str
    seed: int
    values: str = "gauss"
    eps: float = 1e-6
    pos0: int = 0
    max_pos: int = 524288  # decode positions ~ U[0, max_pos)


LAYER_QWEN17_512K = LayerSpec(
    "Qwen3-1.7B-shaped RNN layer (projections + mixer) B=1 T=524288 H=16 d=128 d_model=2048 bf16",
    1, 524288, 16, 128, 2048, torch.bfloat16, tuple(qwen_lambdas(16)), 1e6, "uniform", "zeros",
    1005)
LAYER_DECODE_B64 = LayerSpec(
    "Qwen3-1.7B-shaped RNN layer decode step B=64 H=16 d=128 d_model=2048 bf16, fp32 state",
    64, 1, 16, 128, 2048, torch.bfloat16, tuple(qwen_lambdas(16)), 1e6, "uniform", "randn", 1006)

@dataclasses.dataclass(frozen=True)
class AttnSpec:
    """Inputs of one HyPE attention layer (Eq. 17): q, gate [B, T, Hq, d], k, v [B, T, Hkv, d]
    ~ N(0, 1) in bf16; QK-norm weights shared over heads ([d], U(0.5, 1.5)) as in Qwen3's
    attention layers, or none; the logits scale base a of Eq. 11."""
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    a: float
    qk_norm: bool
    seed: int
    eps: float = 1e-6
    pos0: int = 0


ATTN_QWEN17_32K = AttnSpec(
    "HyPE attention layer (Qwen3-1.7B shape) B=1 T=32768 Hq=16 Hkv=8 d=128 bf16, a=500",
    1, 32768, 16, 8, 128, 500.0, True, 1007)
ATTN_QWEN17_512K = dataclasses.replace(
    ATTN_QWEN17_32K,
    name="HyPE attention layer (Qwen3-1.7B shape) B=1 T=524288 Hq=16 Hkv=8 d=128 bf16, a=500",
    T=524288, seed=1008)

# Training shape of the mixer's backward: HALO's long-context stage trains at 16K tokens
# (Section 4.5, Appendix B); the per-device micro-batch is not given, 8 sequences are taken here.
BWD_QWEN17_16K = PrefillSpec(
    "Qwen3-1.7B-shaped RNN layer backward B=8 H=16 T=16384 d=128 bf16 (16K training context)",
    8, 16384, 16, 128, torch.bfloat16, tuple(qwen_lambdas(16)), 1e6, "uniform", "zeros", 0, 1009)

WORKLOADS = {
    "tiny": TINY,
    "qwen17_32k": QWEN17_32K,
    "qwen17_512k": QWEN17_512K,
    "decode_b64": DECODE_B64,
    "qwen8_128k": QWEN8_128K,
    "layer_qwen17_512k": LAYER_QWEN17_512K,
    "layer_decode_b64": LAYER_DECODE_B64,
    "attn_qwen17_32k": ATTN_QWEN17_32K,
    "attn_qwen17_512k": ATTN_QWEN17_512K,
    "bwd_qwen17_16k": BWD_QWEN17_16K,
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, device, dtype, scale=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def make_prefill(spec: PrefillSpec, device="cpu", T: int | None = None) -> dict:
    """Draw one prefill batch.  ``T`` overrides the sequence length (same distributions)."""
    T = spec.T if T is None else T
    B, H, d = spec.B, spec.H, spec.d
    gen = _gen(spec.seed, device)
    shape = (B, T, H, d)
    q = _randn(shape, gen, device, spec.dtype)
    k = _randn(shape, gen, device, spec.dtype)
    v = _randn(shape, gen, device, spec.dtype)
    g = _randn(shape, gen, device, spec.dtype)
    if spec.norm_w == "ones":
        qw = torch.ones((H, d), device=device, dtype=torch.float32)
        kw = torch.ones((H, d), device=device, dtype=torch.float32)
    else:
        qw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
        kw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
    state = None
    if spec.state == "randn":
        state = _randn((B, H, d, d), gen, device, torch.float32, 0.01)
    return dict(q=q, k=k, v=v, g=g, qw=qw, kw=kw, ow=None, lambdas=list(spec.lambdas),
                rope_base=spec.rope_base, eps=spec.eps, pos0=spec.pos0, state_in=state,
                B=B, T=T, H=H, d=d, dtype=spec.dtype, chunk=spec.chunk)


def make_backward(spec: PrefillSpec, device="cpu", T: int | None = None, B: int | None = None,
                  d_state_out: bool = False) -> dict:
    """A prefill batch (as make_prefill) plus the upstream gradients of the backward: dy ~ N(0, 1)
    in the activations' dtype and, with ``d_state_out``, a 0.01 N(0, 1) fp32 gradient of the final
    state (else None).  ``B`` keeps the first B rows of the spec's batch."""
    out = make_prefill(spec, device, T)
    if B is not None and B != out["B"]:
        for n in ("q", "k", "v", "g"):
            out[n] = out[n][:B].contiguous()
        if out["state_in"] is not None:
            out["state_in"] = out["state_in"][:B].contiguous()
        out["B"] = B
    gen = _gen(spec.seed + 500, device)
    out["dy"] = _randn(out["q"].shape, gen, device, spec.dtype)
    out["d_state_out"] = None
    if d_state_out:
        out["d_state_out"] = _randn((out["B"], out["H"], out["d"], out["d"]), gen, device,
                                    torch.float32, 0.01)
    return out


def make_decode(spec: DecodeSpec, device="cpu", B: int | None = None) -> dict:
    B = spec.B if B is None else B
    H, d = spec.H, spec.d
    gen = _gen(spec.seed, device)
    q = _randn((B, H, d), gen, device, spec.dtype)
    k = _randn((B, H, d), gen, device, spec.dtype)
    v = _randn((B, H, d), gen, device, spec.dtype)
    g = _randn((B, H, d), gen, device, spec.dtype)
    qw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
    kw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
    state = _randn((B, H, d, d), gen, device, torch.float32, 0.01)
    positions = torch.randint(0, spec.max_pos, (B,), generator=gen, device=device,
                              dtype=torch.int64)
    return dict(q=q, k=k, v=v, g=g, qw=qw, kw=kw, ow=None, lambdas=list(spec.lambdas),
                rope_base=spec.rope_base, eps=spec.eps, positions=positions, state_in=state,
                B=B, H=H, d=d, dtype=spec.dtype)


def make_custom_prefill(B, T, H, d, dtype=torch.bfloat16, seed=0, lambdas=None, rope_base=1e6,
                        norm_w="uniform", state="zeros", pos0=0, eps=1e-6, device="cpu",
                        v_scale=1.0) -> dict:
    """Arbitrary-shape prefill batch with the same distributions as the named workloads."""
    if lambdas is None:
        lambdas = qwen_lambdas(H)
    spec = PrefillSpec("custom", B, T, H, d, dtype, tuple(lambdas), rope_base, norm_w, state, 0,
                       seed, eps, pos0)
    out = make_prefill(spec, device)
    if v_scale != 1.0:
        out["v"] = (out["v"].float() * v_scale).to(dtype)
    return out


def _ternary(shape, gen, device, p_nonzero):
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    s = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    return torch.where(u < p_nonzero, torch.where(s < 0.5, -1.0, 1.0), 0.0)


def make_layer(spec: LayerSpec, device="cpu", T: int | None = None, B: int | None = None) -> dict:
    """Draw one layer batch: x [B, T, d_model] (prefill) or [B, d_model] (a decode step, T = 1
    in the spec), w_qkvz [4 H d, d_model], w_o [d_model, H d] and the mixer's parameters."""
    T = spec.T if T is None else T
    B = spec.B if B is None else B
    H, d, dm = spec.H, spec.d, spec.d_model
    gen = _gen(spec.seed, device)
    decode = spec.T == 1
    xshape = (B, dm) if decode else (B, T, dm)
    if spec.values == "ternary":
        if dm > 256 or H * d > 256:
            raise ValueError("ternary layer inputs need d_model <= 256 and H d <= 256")
        x = _ternary(xshape, gen, device, 0.5).to(spec.dtype)
        w_qkvz = _ternary((4 * H * d, dm), gen, device, 0.125).to(spec.dtype)
        w_o = _ternary((dm, H * d), gen, device, 0.125).to(spec.dtype)
    else:
        x = _randn(xshape, gen, device, spec.dtype)
        w_qkvz = _randn((4 * H * d, dm), gen, device, spec.dtype, dm ** -0.5)
        w_o = _randn((dm, H * d), gen, device, spec.dtype, (H * d) ** -0.5)
    if spec.norm_w == "ones":
        qw = torch.ones((H, d), device=device, dtype=torch.float32)
        kw = torch.ones((H, d), device=device, dtype=torch.float32)
    else:
        qw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
        kw = 0.5 + torch.rand((H, d), generator=gen, device=device, dtype=torch.float32)
    state = None
    if spec.state == "randn":
        state = _randn((B, H, d, d), gen, device, torch.float32, 0.01)
    out = dict(x=x, w_qkvz=w_qkvz, w_o=w_o, qw=qw, kw=kw, ow=None, lambdas=list(spec.lambdas),
               rope_base=spec.rope_base, eps=spec.eps, pos0=spec.pos0, state_in=state, B=B, T=T,
               H=H, d=d, d_model=dm, dtype=spec.dtype)
    if decode:
        out["positions"] = torch.randint(0, spec.max_pos, (B,), generator=gen, device=device,
                                         dtype=torch.int64)
    return out


def make_custom_layer(B, T, H, d, d_model, dtype=torch.bfloat16, seed=0, lambdas=None,
                      rope_base=1e6, norm_w="uniform", state="zeros", values="gauss", pos0=0,
                      eps=1e-6, device="cpu") -> dict:
    """Arbitrary-shape layer batch (T = 1 draws a decode step with random positions)."""
    if lambdas is None:
        lambdas = qwen_lambdas(H)
    spec = LayerSpec("custom", B, T, H, d, d_model, dtype, tuple(lambdas), rope_base, norm_w,
                     state, seed, values, eps, pos0)
    return make_layer(spec, device)


def make_attn(spec: AttnSpec, device="cpu", T: int | None = None) -> dict:
    T = spec.T if T is None else T
    B, Hq, Hkv, d = spec.B, spec.Hq, spec.Hkv, spec.d
    gen = _gen(spec.seed, device)
    q = _randn((B, T, Hq, d), gen, device, torch.bfloat16)
    k = _randn((B, T, Hkv, d), gen, device, torch.bfloat16)
    v = _randn((B, T, Hkv, d), gen, device, torch.bfloat16)
    g = _randn((B, T, Hq, d), gen, device, torch.bfloat16)
    qw = kw = None
    if spec.qk_norm:
        qw = 0.5 + torch.rand((d,), generator=gen, device=device, dtype=torch.float32)
        kw = 0.5 + torch.rand((d,), generator=gen, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, qw=qw, kw=kw, ow=None, a=spec.a, eps=spec.eps,
                pos0=spec.pos0, B=B, T=T, Hq=Hq, Hkv=Hkv, d=d)


def make_custom_attn(B, T, Hq, Hkv, d=128, a=500.0, qk_norm=True, seed=0, pos0=0, eps=1e-6,
                     device="cpu") -> dict:
    spec = AttnSpec("custom", B, T, Hq, Hkv, d, a, qk_norm, seed, eps, pos0)
    return make_attn(spec, device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """The raw storage of a CPU tensor as numpy: bf16 -> uint16 bits, fp32 -> float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole array (float64)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = math.sqrt(float(np.sum(ref * ref)))
    num = math.sqrt(float(np.sum((x - ref) ** 2)))
    return num / den if den > 0 else num
