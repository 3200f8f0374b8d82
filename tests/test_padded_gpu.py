"""Padded batches and cross-attention on the GPU (fa_fwd_padded, fa_bwd_padded)
against the fp64 oracle's padded definition on the same seeded inputs.

Per batch entry b, Lq[b] valid queries out of Nq and Lk[b] valid keys out of
Nk; causal is aligned to the last query and key.  Valid rows follow the
forward / backward bars (O max-abs <= 2e-2 bf16 / 4e-3 fp16, LSE <= 1e-3,
gradients max-abs <= 5e-2 and rel-Frobenius <= 1e-2); rows that see no key and
padding rows must be exactly O = 0, LSE = -inf, dQ = 0, and padding keys
exactly dK = dV = 0."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_ABS, TOL_GRAD_RELF, TOL_LSE, TOL_O, max_abs, rel_frob, say,
                           to_device, to_host_f64)

pytestmark = pytest.mark.gpu

# B = 3; (Nq, Nk, Lq per batch, Lk per batch); None = all valid
CASES = {
    "cross_q130_k300": (130, 300, [130, 77, 0], [300, 33, 160]),
    "cross_q300_k130": (300, 130, [300, 250, 45], [130, 0, 97]),
    "same_n257_padded": (257, 257, [257, 100, 200], [257, 257, 31]),
    "one_query_k513": (1, 513, [1, 1, 1], [513, 200, 1]),
    "cross_full_q100_k700": (100, 700, None, None),
}


def inputs(Nq, Nk, d, dtype, seed, B=3, H=2):
    q = fa_inputs.normal_bits(B * H * Nq * d, dtype, seed, fa_inputs.STREAM_Q).reshape(B, H, Nq, d)
    k = fa_inputs.normal_bits(B * H * Nk * d, dtype, seed, fa_inputs.STREAM_K).reshape(B, H, Nk, d)
    v = fa_inputs.normal_bits(B * H * Nk * d, dtype, seed, fa_inputs.STREAM_V).reshape(B, H, Nk, d)
    do = fa_inputs.normal_bits(B * H * Nq * d, dtype, seed, fa_inputs.STREAM_DO).reshape(B, H, Nq, d)
    return q, k, v, do


def lens_tensor(lens, device):
    import torch
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device=device)


def run(q, k, v, do, lq, lk, dtype, causal, device):
    import torch
    tq, tk, tv, tdo = (to_device(x, dtype, device) for x in (q, k, v, do))
    Lq, Lk = lens_tensor(lq, device), lens_tensor(lk, device)
    o, lse = fa.fwd_padded(tq, tk, tv, Lq, Lk, causal=causal)
    dq, dk, dv = fa.bwd_padded(tq, tk, tv, o, tdo, lse, Lq, Lk, causal=causal)
    torch.cuda.synchronize()
    return tuple(to_host_f64(x) for x in (o, lse, dq, dk, dv))


def check_against_oracle(case, d, dtype, causal, gpu, seed):
    Nq, Nk, lq, lk = CASES[case]
    say(f"[padded] {case} d={d} causal={causal} {dtype}")
    q, k, v, do = inputs(Nq, Nk, d, dtype, seed)
    o, lse, dq, dk, dv = run(q, k, v, do, lq, lk, dtype, causal, gpu)
    scale = float(np.float32(1 / math.sqrt(d)))
    w = [fa_inputs.widen(x, dtype) for x in (q, k, v, do)]
    ro, rl = oracle.fwd_padded(w[0], w[1], w[2], scale, causal, lq, lk)
    rq, rk, rv = oracle.bwd_padded(*w, scale, causal, lq, lk)
    dead = np.isneginf(rl)  # padding rows and rows that see no key
    assert np.array_equal(np.isneginf(lse), dead), "rows with LSE = -inf differ"
    assert np.all(o[dead] == 0) and np.all(dq[dead] == 0)
    live = ~dead
    eo = max_abs(o[live], ro[live])
    el = max_abs(lse[live], rl[live])
    say(f"    O max-abs {eo:.3e}  LSE max-abs {el:.3e}  dead rows {int(dead.sum())}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE
    B = q.shape[0]
    for b in range(B):
        Lk = Nk if lk is None else lk[b]
        assert np.all(dk[b, :, Lk:] == 0) and np.all(dv[b, :, Lk:] == 0)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        ea, er = max_abs(got, ref), rel_frob(got, ref)
        say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
        assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF, (name, ea, er)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(CASES))
def test_padded_against_oracle(gpu, case, d, causal, dtype):
    check_against_oracle(case, d, causal=causal, dtype=dtype, gpu=gpu, seed=4100 + d + len(case))


@pytest.mark.parametrize("causal", [False, True])
def test_full_lengths_equal_square_entry_points(gpu, causal):
    """With Nq = Nk and every length full, the padded entry points give the
    square ones' results bit for bit."""
    import torch
    B, H, N, d, dtype = 2, 2, 300, 128, "bf16"
    q, k, v, do = inputs(N, N, d, dtype, 4200, B=B, H=H)
    tq, tk, tv, tdo = (to_device(x, dtype, gpu) for x in (q, k, v, do))
    full = torch.full((B,), N, dtype=torch.int32, device=gpu)
    o1, l1 = fa.fwd(tq, tk, tv, causal=causal)
    o2, l2 = fa.fwd_padded(tq, tk, tv, full, full, causal=causal)
    g1 = fa.bwd(tq, tk, tv, o1, tdo, l1, causal=causal)
    g2 = fa.bwd_padded(tq, tk, tv, o2, tdo, l2, full, full, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_padding_contents_are_not_read(gpu):
    """Garbage (huge values, NaN) in padding rows and keys changes nothing."""
    import torch
    Nq, Nk, lq, lk = 70, 90, [70, 33], [90, 40]
    d, dtype = 64, "f16"
    q, k, v, do = inputs(Nq, Nk, d, dtype, 4300, B=2, H=2)
    a = run(q, k, v, do, lq, lk, dtype, True, gpu)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    nan16 = np.uint16(0x7E00)
    for b in range(2):
        q2[b, :, lq[b]:] = nan16
        do2[b, :, lq[b]:] = nan16
        k2[b, :, lk[b]:] = nan16
        v2[b, :, lk[b]:] = nan16
    b_ = run(q2, k2, v2, do2, lq, lk, dtype, True, gpu)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y, equal_nan=False)


def test_padded_gradients_repeatable(gpu):
    case = "cross_q300_k130"
    Nq, Nk, lq, lk = CASES[case]
    q, k, v, do = inputs(Nq, Nk, 128, "bf16", 4400)
    a = run(q, k, v, do, lq, lk, "bf16", True, gpu)
    b = run(q, k, v, do, lq, lk, "bf16", True, gpu)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_misaligned_lengths_are_rejected(gpu):
    import torch
    q = torch.zeros((2, 1, 8, 64), dtype=torch.float16, device=gpu)
    o = torch.empty_like(q)
    lse = torch.empty((2, 1, 8), dtype=torch.float32, device=gpu)
    buf = torch.zeros(8, dtype=torch.int32, device=gpu)
    bad = buf.view(torch.uint8)[2:10]  # 2-byte offset, 8 bytes = two int32 lengths
    import ctypes
    rc = fa.lib().fa_fwd_padded(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                                ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(bad.data_ptr()),
                                ctypes.c_void_p(None), 2, 1, 8, 8, 64, 0.125, 0, fa.FA_F16, None)
    assert rc == 5  # FA_ERR_ALIGN
