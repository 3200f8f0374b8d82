"""fa_bwd_noalloc (the backward for callers that cannot allocate: its row
statistics live in the library's static per-GPU scratch) against fa_bwd, the
entry point it is a variant of: called through the C ABI twice in a row, the
second call on a smaller problem of another shape, dtype and mask, each time
bitwise equal to fa_bwd on the same inputs (the same kernels run)."""
import ctypes
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
from tests.helpers import say, to_device

pytestmark = pytest.mark.gpu


def _run_both(gpu, B, H, N, d, dtype, causal, seed):
    import torch
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=seed, with_dout=True)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    ref = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fa.lib().fa_bwd_noalloc(P(q), P(k), P(v), P(o), P(do), P(lse), P(got[0]), P(got[1]), P(got[2]),
                                 B, H, N, d, ctypes.c_float(scale), int(causal),
                                 fa.FA_BF16 if dtype == "bf16" else fa.FA_F16, stream)
    assert rc == 0, fa.fa_status_str(rc)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        diff = float((a.float() - b.float()).abs().max())
        say(f"    {name}: max |noalloc - fa_bwd| = {diff:.3e}")
        assert torch.equal(a, b), name


def test_noalloc_matches_fa_bwd_twice_then_smaller(gpu):
    say("[noalloc] call 1: B=2 H=4 N=1000 d=128 bf16 causal")
    _run_both(gpu, 2, 4, 1000, 128, "bf16", True, seed=5100)
    say("[noalloc] call 2 (smaller): B=1 H=2 N=300 d=64 f16 non-causal")
    _run_both(gpu, 1, 2, 300, 64, "f16", False, seed=5101)


def test_noalloc_rejects_problems_beyond_the_scratch(gpu):
    import torch
    lib = fa.lib()
    p = ctypes.c_void_p(256)
    # B*H*N = 4194305 > FA_BWD_NOALLOC_MAX_ROWS: rejected before any launch
    rc = lib.fa_bwd_noalloc(*([p] * 9), 1, 1, fa.FA_BWD_NOALLOC_MAX_ROWS + 1, 64, ctypes.c_float(0.1), 0,
                            fa.FA_BF16, None)
    assert rc == 10, fa.fa_status_str(rc)
    torch.cuda.synchronize()
