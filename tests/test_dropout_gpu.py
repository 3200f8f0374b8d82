"""Dropout on the attention weights on the GPU (fa_fwd_dropout, fa_bwd_dropout)
against the fp64 oracle with the same Philox4x32-10 mask, on the same seeded
inputs: O, LSE and gradients to the forward / backward bars; the forward's
and backward's masks are regenerated in three different lane layouts (the
forward's and dQ pass's query-major one, the dK/dV pass's key-major one), so
agreement of all of O, dQ, dK and dV with the oracle checks each of them."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_ABS, TOL_GRAD_RELF, TOL_LSE, TOL_O, max_abs, rel_frob, say,
                           to_device, to_host_f64)
from tests.test_padded_gpu import inputs, lens_tensor

pytestmark = pytest.mark.gpu

SEED = 0x0DDBA11C0FFEE123
# (Nq, Nk, Lq, Lk, p)
CASES = {
    "n130_p25": (130, 130, None, None, 0.25),
    "n257_p50": (257, 257, None, None, 0.5),
    "cross_q100_k200_padded_p10": (100, 200, [100, 61], [200, 97], 0.1),
}


def run(q, k, v, do, lq, lk, dtype, causal, p, offset, device):
    import torch
    tq, tk, tv, tdo = (to_device(x, dtype, device) for x in (q, k, v, do))
    Lq, Lk = lens_tensor(lq, device), lens_tensor(lk, device)
    o, lse = fa.fwd_dropout(tq, tk, tv, p, SEED, offset, Lq, Lk, causal=causal)
    dq, dk, dv = fa.bwd_dropout(tq, tk, tv, o, tdo, lse, p, SEED, offset, Lq, Lk, causal=causal)
    torch.cuda.synchronize()
    return tuple(to_host_f64(x) for x in (o, lse, dq, dk, dv))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(CASES))
def test_dropout_against_oracle(gpu, case, d, causal, dtype):
    Nq, Nk, lq, lk, p = CASES[case]
    offset = 17
    say(f"[dropout] {case} d={d} causal={causal} {dtype}")
    q, k, v, do = inputs(Nq, Nk, d, dtype, 4500 + d, B=2, H=2)
    o, lse, dq, dk, dv = run(q, k, v, do, lq, lk, dtype, causal, p, offset, gpu)
    scale = float(np.float32(1 / math.sqrt(d)))
    w = [fa_inputs.widen(x, dtype) for x in (q, k, v, do)]
    drop = (fa.dropout_threshold(p), SEED, offset)
    ro, rl = oracle.fwd_padded(w[0], w[1], w[2], scale, causal, lq, lk, dropout=drop)
    rq, rk, rv = oracle.bwd_padded(*w, scale, causal, lq, lk, dropout=drop)
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead)
    live = ~dead
    eo, el = max_abs(o[live], ro[live]), max_abs(lse[live], rl[live])
    say(f"    O max-abs {eo:.3e}  LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        ea, er = max_abs(got, ref), rel_frob(got, ref)
        say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
        assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF, (name, ea, er)


def test_zero_probability_equals_no_dropout(gpu):
    import torch
    q, k, v, do = inputs(200, 200, 128, "bf16", 4600, B=2, H=2)
    tq, tk, tv, tdo = (to_device(x, "bf16", gpu) for x in (q, k, v, do))
    o1, l1 = fa.fwd_padded(tq, tk, tv, causal=True)
    o2, l2 = fa.fwd_dropout(tq, tk, tv, 0.0, SEED, 3, causal=True)
    g1 = fa.bwd_padded(tq, tk, tv, o1, tdo, l1, causal=True)
    g2 = fa.bwd_dropout(tq, tk, tv, o2, tdo, l2, 0.0, SEED, 3, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dropout_repeatable_and_offset_dependent(gpu):
    q, k, v, do = inputs(160, 160, 64, "f16", 4700, B=1, H=2)
    a = run(q, k, v, do, None, None, "f16", False, 0.3, 5, gpu)
    b = run(q, k, v, do, None, None, "f16", False, 0.3, 5, gpu)
    c = run(q, k, v, do, None, None, "f16", False, 0.3, 6, gpu)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert np.array_equal(a[1], c[1])  # LSE is taken before dropout


def test_bad_dropout_probability_is_rejected(gpu):
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16, device=gpu)
    for p in (-0.1, 1.0, float("nan")):
        with pytest.raises(fa.FaError) as e:
            fa.fwd_dropout(q, q, q, p, 1)
        assert e.value.status == 9  # FA_ERR_ARG
