"""Scale and NaN semantics on the GPU.

Scale: any finite float is a valid scale (the formula softmax(Q K^T * scale) V
takes it as a free parameter; the pages use 1/sqrt(d_k)).  The masks are
applied to the scaled scores, so they hold at scale = 0 (uniform weights over
the visible keys: O = mean of the visible V rows, LSE = ln n, dQ = dK = 0) and
at negative scales (the smallest raw scores get the largest weights), where
the outputs are compared element by element with the fp64 oracle through every
entry point (square, padded / cross-attention, dropout, split over keys).

NaN: inputs are IEEE values and NaN propagates.  A NaN anywhere in query row i
makes O row i and LSE row i NaN and leaves every other row of O and LSE
bit-identical; a NaN in key row j does the same to exactly the rows that see
key j; a NaN in V[j][c] makes column c of O NaN in every row that sees key j
and leaves the other columns bit-identical (rows that do not see key j but
share a wave's 32-row query block with one that does may get a NaN in column
c too: the tile products multiply their zero weights by the NaN; a wave whose
rows all end before key j skips that key's tile)."""
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


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_zero_scale_closed_form(gpu, d, causal, dtype):
    B, H, N = 2, 2, 300
    say(f"[scale 0] d={d} causal={causal} {dtype}")
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4100 + d, with_dout=True)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.0)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=0.0)
    _sync()
    vw, dow = fa_inputs.widen(vb, dtype), fa_inputs.widen(dob, dtype)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    ref_o = (np.cumsum(vw, axis=2) / n[:, None]) if causal else np.broadcast_to(vw.mean(axis=2, keepdims=True), vw.shape)
    eo = max_abs(to_host_f64(o), ref_o)
    el = max_abs(to_host_f64(lse), np.broadcast_to(np.log(n), (B, H, N)))
    say(f"    O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE
    # dQ and dK carry the factor scale: exactly zero
    assert not to_host_f64(dq).any() and not to_host_f64(dk).any()
    # dV_j = sum over the rows i that see key j of dO_i / n_i
    w = dow / n[:, None]
    ref_dv = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2) if causal else \
        np.broadcast_to(w.sum(axis=2, keepdims=True), w.shape)
    g = to_host_f64(dv)
    ea, er = max_abs(g, ref_dv), rel_frob(g, ref_dv)
    say(f"    dV max-abs {ea:.3e} rel-F {er:.3e}")
    assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF
    # and the oracle at scale 0 agrees with the closed form on the same bits
    ro, rl = oracle.fwd(*(fa_inputs.widen(x, dtype) for x in (qb, kb, vb)), 0.0, causal)
    assert max_abs(to_host_f64(o), ro) <= TOL_O[dtype] and max_abs(to_host_f64(lse), rl) <= TOL_LSE


def _check_fwd(o, lse, ro, rl, dtype, what):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert np.all(o[dead] == 0), what
    live = ~dead
    eo = max_abs(o[live], ro[live]) if live.any() else 0.0
    el = max_abs(lse[live], rl[live]) if live.any() else 0.0
    say(f"    {what}: O max-abs {eo:.3e}  LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, what


def _check_grads(grads, ref):
    for name, got, want in zip(("dQ", "dK", "dV"), grads, ref):
        g = to_host_f64(got)
        ea, er = max_abs(g, want), rel_frob(g, want)
        say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
        assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF, (name, ea, er)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("factor", [-1.0, -0.5])
def test_negative_scale_square(gpu, factor, d, causal, dtype):
    # scores of the workloads' magnitude (|scale| = 1/sqrt(d) and half of it),
    # for which the gradient tolerances are set
    B, H, N = 1, 3, 333
    scale = factor / math.sqrt(d)
    say(f"[scale {scale}] square N={N} d={d} causal={causal} {dtype}")
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4200 + d, with_dout=True)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    _sync()
    w = [fa_inputs.widen(x, dtype) for x in (qb, kb, vb, dob)]
    s32 = float(np.float32(scale))
    ro, rl = oracle.fwd(*w[:3], s32, causal)
    _check_fwd(to_host_f64(o), to_host_f64(lse), ro, rl, dtype, "forward")
    _check_grads(grads, oracle.bwd(*w, s32, causal))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_negative_scale_padded_dropout_and_split(gpu, d, causal, dtype):
    # cross-attention with ragged lengths (an empty key range included), then
    # the same with dropout, then the split-over-keys forward and one decode row
    Nq, Nk, lq, lk = 200, 450, [200, 90, 17], [450, 0, 300]
    scale = -1.0 / math.sqrt(d)
    s32 = float(np.float32(scale))
    say(f"[scale {scale}] padded Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype}")
    qb, kb, vb, dob = inputs(Nq, Nk, d, dtype, 4300 + d)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    Lq, Lk = lens_tensor(lq, gpu), lens_tensor(lk, gpu)
    w = [fa_inputs.widen(x, dtype) for x in (qb, kb, vb, dob)]

    o, lse = fa.fwd_padded(q, k, v, Lq, Lk, causal=causal, scale=scale)
    grads = fa.bwd_padded(q, k, v, o, do, lse, Lq, Lk, causal=causal, scale=scale)
    so, sl = fa.fwd_splitkv(q, k, v, Lq, Lk, causal=causal, scale=scale)
    _sync()
    ro, rl = oracle.fwd_padded(*w[:3], s32, causal, lq, lk)
    _check_fwd(to_host_f64(o), to_host_f64(lse), ro, rl, dtype, "padded forward")
    _check_fwd(to_host_f64(so), to_host_f64(sl), ro, rl, dtype, "split forward")
    _check_grads(grads, oracle.bwd_padded(*w, s32, causal, lq, lk))

    p, seed, offset = 0.2, 0x5CA1E0000001, 3
    o, lse = fa.fwd_dropout(q, k, v, p, seed, offset, Lq, Lk, causal=causal, scale=scale)
    grads = fa.bwd_dropout(q, k, v, o, do, lse, p, seed, offset, Lq, Lk, causal=causal, scale=scale)
    _sync()
    drop = (fa.dropout_threshold(p), seed, offset)
    ro, rl = oracle.fwd_padded(*w[:3], s32, causal, lq, lk, dropout=drop)
    _check_fwd(to_host_f64(o), to_host_f64(lse), ro, rl, dtype, "dropout forward")
    _check_grads(grads, oracle.bwd_padded(*w, s32, causal, lq, lk, dropout=drop))

    # decode: one query row per head over the keys
    q1 = q[:, :, :1].contiguous()
    so, sl = fa.fwd_splitkv(q1, k, v, None, Lk, causal=causal, scale=scale)
    _sync()
    ro, rl = oracle.fwd_padded(w[0][:, :, :1].copy(), w[1], w[2], s32, causal, None, lk)
    _check_fwd(to_host_f64(so), to_host_f64(sl), ro, rl, dtype, "decode forward")


# --------------------------------------------------------------------------
# NaN propagation (forward)
# --------------------------------------------------------------------------

def _nan_bits(dtype):
    return np.uint16(0x7FC0 if dtype == "bf16" else 0x7E00)


def _fwd_pair(qb, kb, vb, dtype, causal, gpu, poisoned):
    """Forward on clean inputs and on inputs with one NaN planted (by `poisoned`)."""
    clean = fa.fwd(*(to_device(x, dtype, gpu) for x in (qb, kb, vb)), causal=causal)
    bad = fa.fwd(*(to_device(x, dtype, gpu) for x in poisoned(qb.copy(), kb.copy(), vb.copy())), causal=causal)
    _sync()
    return [to_host_f64(x) for x in clean], [to_host_f64(x) for x in bad]


def _same_bits(a, b):
    return np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_in_query_row(gpu, causal, dtype):
    B, H, N, d, i, c = 1, 2, 300, 128, 77, 5
    say(f"[nan q] causal={causal} {dtype}")
    qb, kb, vb = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4400)

    def poison(q, k, v):
        q[0, 1, i, c] = _nan_bits(dtype)
        return q, k, v

    (o0, l0), (o1, l1) = _fwd_pair(qb, kb, vb, dtype, causal, gpu, poison)
    assert np.isnan(o1[0, 1, i]).all() and np.isnan(l1[0, 1, i])
    keep = np.ones((B, H, N), bool)
    keep[0, 1, i] = False
    assert _same_bits(o1[keep], o0[keep]) and _same_bits(l1[keep], l0[keep])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_in_key_row(gpu, causal, dtype):
    B, H, N, d, j = 1, 2, 300, 64, 150
    say(f"[nan k] causal={causal} {dtype}")
    qb, kb, vb = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4401)

    def poison(q, k, v):
        k[0, 0, j, 3] = _nan_bits(dtype)
        return q, k, v

    (o0, l0), (o1, l1) = _fwd_pair(qb, kb, vb, dtype, causal, gpu, poison)
    sees = np.zeros((B, H, N), bool)
    sees[0, 0, j if causal else 0:] = True  # the rows that see key j
    assert np.isnan(o1[sees]).all() and np.isnan(l1[sees]).all()
    assert _same_bits(o1[~sees], o0[~sees]) and _same_bits(l1[~sees], l0[~sees])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_in_value_element(gpu, causal, dtype):
    B, H, N, d, j, c = 1, 2, 600, 128, 450, 9
    say(f"[nan v] causal={causal} {dtype}")
    qb, kb, vb = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4402)

    def poison(q, k, v):
        v[0, 1, j, c] = _nan_bits(dtype)
        return q, k, v

    (o0, l0), (o1, l1) = _fwd_pair(qb, kb, vb, dtype, causal, gpu, poison)
    assert _same_bits(l1, l0)  # the LSE does not involve V
    first = j if causal else 0  # the rows that see key j
    assert np.isnan(o1[0, 1, first:, c]).all()
    others = np.ones(d, bool)
    others[c] = False
    assert _same_bits(o1[..., others], o0[..., others])
    assert _same_bits(o1[0, 0], o0[0, 0])  # another head
    if causal:  # a wave's 32 query rows that end before key j never use its tile
        clean_rows = (j // 32) * 32
        assert _same_bits(o1[0, 1, :clean_rows, c], o0[0, 1, :clean_rows, c])
