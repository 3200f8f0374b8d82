"""Parity at the full sizes of the benchmark's padded, cross-attention and dropout
workloads (the entry points and launch configurations bench.py times), on
sampled heads against the fp64 oracle: a variable-length causal batch (B=8 H=16
N=4096, lengths drawn in [512, 4096]), cross-attention (B=2 H=16 Nq=4096
Nk=16384) and dropout p = 0.1 (B=8 H=16 N=4096 causal).  The whole batch runs on
the GPU; the oracle takes the sampled heads (for dropout, heads of the first
batch entry, whose head index b*H + h, a Philox counter word, a slice keeps;
the oracle's forward runs on one thread, so few heads are sampled).
Bars: O max-abs <= 2e-2 (bf16), LSE <= 1e-3 on live rows, dead rows O = 0 and
LSE = -inf exactly, padding keys dK = dV = 0 exactly; gradients max-abs <= 5e-2
and relative Frobenius <= 1e-2."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_ABS, TOL_GRAD_RELF, TOL_LSE, TOL_O, max_abs, rel_frob, say,
                           to_device, to_host_f64)

pytestmark = pytest.mark.gpu


def _inputs(c):
    B, H, N, d, dt = c["B"], c["H"], c["N"], c["d"], c["dtype"]
    Nk = c.get("Nk", N)
    q = fa_inputs.normal_bits(B * H * N * d, dt, c["seed"], fa_inputs.STREAM_Q).reshape(B, H, N, d)
    k = fa_inputs.normal_bits(B * H * Nk * d, dt, c["seed"], fa_inputs.STREAM_K).reshape(B, H, Nk, d)
    v = fa_inputs.normal_bits(B * H * Nk * d, dt, c["seed"], fa_inputs.STREAM_V).reshape(B, H, Nk, d)
    do = fa_inputs.normal_bits(B * H * N * d, dt, c["seed"], fa_inputs.STREAM_DO).reshape(B, H, N, d)
    return q, k, v, do


def _check_fwd(o, lse, ro, rl, dtype):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), "rows with LSE = -inf differ"
    assert np.all(o[dead] == 0)
    live = ~dead
    eo, el = max_abs(o[live], ro[live]), max_abs(lse[live], rl[live])
    say(f"    O max-abs {eo:.3e}  LSE max-abs {el:.3e}  dead rows {int(dead.sum())}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE


def _check_grads(got, ref):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        ea, er = max_abs(g, r), rel_frob(g, r)
        say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
        assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF, (name, ea, er)


def _heads(t, b, hs):
    """Device tensor [B, H, ...] -> float64 host array [1, len(hs), ...] of batch b, heads hs."""
    return to_host_f64(t[b:b + 1, hs[0]:hs[-1] + 1])


@pytest.mark.parametrize("name", ["p1_varlen_causal_b8_n4096_d128_bf16", "p2_cross_q4096_k16384_d128_bf16"])
def test_padded_and_cross_full_size_sampled_heads(gpu, name):
    import torch
    c = fa_inputs.CONFIGS[name]
    B, H, d, dt, causal = c["B"], c["H"], c["d"], c["dtype"], c["causal"]
    lens = fa_inputs.seq_lengths(B, c["len_lo"], c["len_hi"], c["seed"]) if "len_lo" in c else None
    say(f"[bench workload] {name} lengths {None if lens is None else lens.tolist()}")
    q, k, v, do = _inputs(c)
    tq, tk, tv, tdo = (to_device(x, dt, gpu) for x in (q, k, v, do))
    L = None if lens is None else torch.from_numpy(lens).to(gpu)
    o, lse = fa.fwd_padded(tq, tk, tv, L, L, causal=causal)
    dq, dk, dv = fa.bwd_padded(tq, tk, tv, o, tdo, lse, L, L, causal=causal)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / math.sqrt(d)))
    # the first and the last head of the batch; at Nk = 16384 the last only (the
    # oracle's forward and backward of one such head take ~20 s each)
    for b, h in ((0, 0), (B - 1, H - 1)) if lens is not None else ((B - 1, H - 1),):
        say(f"  head b={b} h={h}")
        lb = None if lens is None else [int(lens[b])]
        w = [fa_inputs.widen(x[b:b + 1, h:h + 1], dt) for x in (q, k, v, do)]
        ro, rl = oracle.fwd_padded(w[0], w[1], w[2], scale, causal, lb, lb)
        _check_fwd(_heads(o, b, [h]), _heads(lse, b, [h]), ro, rl, dt)
        ref = oracle.bwd_padded(*w, scale, causal, lb, lb)
        got = [_heads(x, b, [h]) for x in (dq, dk, dv)]
        if lb is not None:  # padding rows and keys: exact zeros
            assert np.all(got[0][:, :, lb[0]:] == 0)
            assert np.all(got[1][:, :, lb[0]:] == 0) and np.all(got[2][:, :, lb[0]:] == 0)
        _check_grads(got, ref)


def test_dropout_full_size_sampled_heads(gpu):
    import torch
    c = fa_inputs.CONFIGS["p3_dropout10_causal_n4096_d128_bf16"]
    B, H, d, dt, causal, p = c["B"], c["H"], c["d"], c["dtype"], c["causal"], c["dropout"]
    seed, offset = c["seed"], 5
    say(f"[bench workload] dropout p={p}")
    q, k, v, do = _inputs(c)
    tq, tk, tv, tdo = (to_device(x, dt, gpu) for x in (q, k, v, do))
    o, lse = fa.fwd_dropout(tq, tk, tv, p, seed, offset, causal=causal)
    dq, dk, dv = fa.bwd_dropout(tq, tk, tv, o, tdo, lse, p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / math.sqrt(d)))
    drop = (fa.dropout_threshold(p), seed, offset)
    # forward over heads 0 .. 3 of batch entry 0 (their head indices as in the
    # full batch), backward over heads 0 and 1
    w = [fa_inputs.widen(x[0:1, 0:4], dt) for x in (q, k, v, do)]
    ro, rl = oracle.fwd_padded(w[0], w[1], w[2], scale, causal, dropout=drop)
    _check_fwd(_heads(o, 0, [0, 1, 2, 3]), _heads(lse, 0, [0, 1, 2, 3]), ro, rl, dt)
    w2 = [x[:, 0:2] for x in w]
    ref = oracle.bwd_padded(*w2, scale, causal, dropout=drop)
    _check_grads([_heads(x, 0, [0, 1]) for x in (dq, dk, dv)], ref)
