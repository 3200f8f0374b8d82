"""The forward and the allocation-free backward captured into a HIP graph
(torch.cuda.graph) and replayed.  Neither entry point allocates or records a
memset, so the captured launches replay on whatever the static buffers hold:
each replay runs on new inputs copied in eagerly, with eager work and
synchronisations between the replays, and is compared bitwise with eager
calls (fa_fwd, fa_bwd with a workspace) on the same inputs.  Debug mode
under capture prints its plan but skips its scan (which would wait for the
stream)."""
import math

import pytest

import exact_attention_21_amd as fa
import fa_inputs
from tests.helpers import say, to_device

pytestmark = pytest.mark.gpu


def test_forward_and_noalloc_backward_replay(gpu, monkeypatch):
    import torch
    monkeypatch.delenv("FA_DEBUG", raising=False)
    monkeypatch.delenv("FLASH_ATTENTION_DEBUG", raising=False)
    B, H, N, d, dtype, causal = 2, 4, 700, 128, "bf16", True
    scale = 1 / math.sqrt(d)

    def draw(seed):
        bits = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=seed, with_dout=True)
        return [to_device(x, dtype, gpu) for x in bits]

    q, k, v, do = draw(5200)
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=gpu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale, causal)
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale, causal)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        new = draw(5300 + rep)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el = fa.fwd(*new[:3], causal=causal, scale=scale)
        eg = fa.bwd(*new[:3], eo, new[3], el, causal=causal, scale=scale)
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}: comparing O, LSE, dQ, dK, dV with eager calls")
        assert torch.equal(o, eo) and torch.equal(lse, el)
        for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), eg):
            assert torch.equal(a, b), name


def test_debug_mode_skips_its_scan_under_capture(gpu, monkeypatch, capfd):
    # the scan waits for the stream, which a capture forbids: it is skipped,
    # the plan is still printed, and the captured forward replays correctly
    import torch
    monkeypatch.setenv("FA_DEBUG", "1")
    B, H, N, d, dtype = 1, 2, 300, 64, "f16"
    q, k, v = (to_device(x, dtype, gpu) for x in fa_inputs.qkv_bits(B, H, N, d, dtype, seed=5400))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=gpu)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_fwd(q, k, v, o, lse, 0.125, True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    capfd.readouterr()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_fwd(q, k, v, o, lse, 0.125, True)
    err = capfd.readouterr().err
    assert "[FA_DEBUG] fa_fwd: B=1 H=2 Nq=300" in err
    assert "[FA_DEBUG] fa_fwd: stream is being captured; no scan" in err
    monkeypatch.delenv("FA_DEBUG")
    o.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    eo, el = fa.fwd(q, k, v, causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, eo) and torch.equal(lse, el)
