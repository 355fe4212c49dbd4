"""lightning_prefill_noalloc (the prefill whose segment states live in the library's static device
scratch) against lightning_prefill (caller-owned workspace) on the same inputs.

Both entry points run the same kernels with the same plan, so their outputs must be
bit-identical; the comparison also holds them to the parity bars (relative L2 per (b, h) slice:
2e-2 on y, 1e-4 on the state for bf16 activations).  Calls in a row, each smaller than the one
before, show that what a call leaves in the shared scratch does not leak into the next.  A request
whose workspace exceeds the scratch is refused before anything is launched.
"""
import pytest
import torch

lt = pytest.importorskip("long_context_hybrid_amd.lightning")
import synth  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rel(a, b):
    return float((a.double() - b.double()).norm() / b.double().norm().clamp_min(1e-300))


def _compare(inp, segments):
    dev = torch.device("cuda:0")
    q, k, v, g = (inp[n].to(dev) for n in ("q", "k", "v", "g"))
    qw, kw = inp["qw"].to(dev), inp["kw"].to(dev)
    B, T, H, d = q.shape
    s_in = None if inp.get("state_in") is None else inp["state_in"].to(dev)
    ws_need = lt.lightning_prefill_workspace_size(B, T, H, d, q.dtype, 0, segments)
    assert 0 < ws_need <= 64 << 20, "the case must use the scratch and fit in it"
    ref_s = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ref_y = lt.lightning_prefill(q, k, v, g, qw, kw, inp["lambdas"], inp["rope_base"],
                                 state_in=s_in, state_out=ref_s, segments=segments)
    y = torch.full_like(q, float("nan"))
    s = torch.full((B, H, d, d), float("nan"), dtype=torch.float32, device=dev)
    out = lt.lightning_prefill_noalloc(q, k, v, g, qw, kw, inp["lambdas"], inp["rope_base"],
                                       state_in=s_in, state_out=s, y=y, segments=segments)
    torch.cuda.synchronize()
    assert out is y
    for b in range(B):
        for h in range(H):
            assert _rel(y[b, :, h], ref_y[b, :, h]) <= 2e-2
            assert _rel(s[b, h], ref_s[b, h]) <= 1e-4
    assert torch.equal(y, ref_y), "same kernels, same plan: y must be bit-identical"
    assert torch.equal(s, ref_s), "same kernels, same plan: the state must be bit-identical"


def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row():
    _need_gpu()
    dev = torch.device("cuda:0")
    # first call: the Qwen3-8B-shaped workload, the largest (B = 4, H = 32, 128K tokens: 40 MiB
    # of segment states, nonzero initial state)
    big = synth.make_prefill(synth.QWEN8_128K, device=dev)
    _compare(big, 0)
    del big
    # second call, smaller: the 512K-token Qwen3-1.7B-shaped layer (31 MiB of states)
    big = synth.make_prefill(synth.QWEN17_512K, device=dev)
    _compare(big, 0)
    del big
    # third call, smaller again: fewer heads and tokens, a ragged tail, a nonzero initial state,
    # an explicit segment count; the scratch still holds the earlier calls' states
    small = synth.make_custom_prefill(1, 1000, 4, 128, dtype=torch.bfloat16, seed=21,
                                      state="randn")
    _compare(small, 3)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    _need_gpu()
    dev = torch.device("cuda:0")
    B, T, H, d = 1, 8192, 64, 128  # 32 segments: 64 heads x 32 slots x 64 KiB = 128 MiB
    assert lt.lightning_prefill_workspace_size(B, T, H, d, torch.bfloat16, 0, 32) > 64 << 20
    x = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device=dev)
    w = torch.ones((H, d), dtype=torch.float32, device=dev)
    y = torch.full_like(x, 3.0)
    with pytest.raises(lt.LightningError) as e:
        lt.lightning_prefill_noalloc(x, x, x, x, w, w, [0.9] * H, 1e6, y=y, segments=32)
    assert e.value.status == lt.LT_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a refused call wrote its output"
