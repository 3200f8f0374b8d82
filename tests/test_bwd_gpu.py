"""Backward parity on the GPU: dQ, dK, dV from the HIP kernels against the fp64
oracle's gradients on the same seeded inputs (the GPU backward consumes the GPU
forward's O and LSE).  Bar for each tensor: max-abs <= 5e-2 and relative
Frobenius error <= 1e-2."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_ABS, TOL_GRAD_RELF, max_abs, rel_frob, say, to_device,
                           to_host_f64)

pytestmark = pytest.mark.gpu


def run_fwd_bwd(qb, kb, vb, dob, dtype, causal, device):
    import torch
    q, k, v, do = (to_device(x, dtype, device) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(name, got, ref):
    ea, er = max_abs(got, ref), rel_frob(got, ref)
    say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
    assert ea <= TOL_GRAD_ABS, (name, ea)
    assert er <= TOL_GRAD_RELF, (name, er)


SMALL = [(1, 2, 1, 64), (1, 2, 17, 128), (1, 3, 100, 64), (2, 4, 130, 128), (1, 2, 257, 64),
         (1, 1, 384, 128), (1, 2, 700, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_all_elements(gpu, shape, causal, dtype):
    B, H, N, d = shape
    say(f"[bwd small] B={B} H={H} N={N} d={d} causal={causal} {dtype}")
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=2000 + N + d, with_dout=True)
    dq, dk, dv = run_fwd_bwd(qb, kb, vb, dob, dtype, causal, gpu)
    scale = float(np.float32(1 / math.sqrt(d)))
    rq, rk, rv = oracle.bwd(*(fa_inputs.widen(x, dtype) for x in (qb, kb, vb, dob)), scale, causal)
    compare("dQ", to_host_f64(dq), rq)
    compare("dK", to_host_f64(dk), rk)
    compare("dV", to_host_f64(dv), rv)


@pytest.mark.parametrize("name", ["c5_bwd_causal_n4096_d128_bf16", "c3_bwd_causal_n8192_d128_bf16"])
def test_full_size_sampled_heads(gpu, name):
    c = fa_inputs.CONFIGS[name]
    B, H, N, d, dtype, causal = c["B"], c["H"], c["N"], c["d"], c["dtype"], c["causal"]
    say(f"[bwd full] {name}")
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, c["seed"], with_dout=True)
    dq, dk, dv = run_fwd_bwd(qb, kb, vb, dob, dtype, causal, gpu)
    dq_h, dk_h, dv_h = (to_host_f64(x) for x in (dq, dk, dv))
    for x in (dq_h, dk_h, dv_h):
        assert np.isfinite(x).all()
    # first and last heads; at N = 8192 also an interior one (XCD 2, its third
    # pair of heads) so that heads away from the grid's ends are covered
    heads = [0, B * H - 1] if N <= 4096 else [0, 42, B * H - 1]
    scale = float(np.float32(1 / math.sqrt(d)))
    for bh in heads:
        b, h = divmod(bh, H)
        sub = [fa_inputs.widen(x[b:b + 1, h:h + 1], dtype) for x in (qb, kb, vb, dob)]
        rq, rk, rv = oracle.bwd_heads(*sub, scale, causal, [0])
        say(f"  head {bh}")
        compare("dQ", dq_h[b, h], rq[0])
        compare("dK", dk_h[b, h], rk[0])
        compare("dV", dv_h[b, h], rv[0])


def test_gradients_bitwise_repeatable(gpu):
    # no atomics anywhere: two runs give identical bits (the determinism check of
    # the FA1-vs-FA2 page's troubleshooting section, tightened to bitwise)
    import torch
    qb, kb, vb, dob = fa_inputs.qkv_bits(2, 8, 1024, 128, "bf16", seed=90, with_dout=True)
    r1 = run_fwd_bwd(qb, kb, vb, dob, "bf16", True, gpu)
    r2 = run_fwd_bwd(qb, kb, vb, dob, "bf16", True, gpu)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,dt", [(128, "f16"), (64, "bf16")])
def test_staged_entry_points_match_fa_bwd(gpu, d, dt):
    import torch
    B, H, N = 1, 4, 300
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dt, seed=92, with_dout=True)
    q, k, v, do = (to_device(x, dt, gpu) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True)
    ref = fa.bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    scale = 1 / math.sqrt(d)
    fa.fa_bwd_preprocess(o, do, lse, ws)
    fa.fa_bwd_dq(q, k, v, do, dq, scale, True, ws)
    fa.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, True, ws)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)

    # the workspace holds -D and LSE*log2(e), fp32 [B][H][N] each, the second
    # at the first 256-byte boundary after the first
    rows = B * H * N
    second = (rows * 4 + 255) // 256 * 256

    def stats(w):
        return w[: rows * 4].clone(), w[second: second + rows * 4].clone()

    pre = stats(ws)
    # the dQ pass that computes the statistics itself writes the same values
    ws.fill_(0xFF)
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd_dq_preprocess(q, k, v, o, do, lse, dq2, scale, True, ws)
    fa.fa_bwd_dkdv(q, k, v, do, dk2, dv2, scale, True, ws)
    torch.cuda.synchronize()
    for a, b in zip(stats(ws), pre):
        assert torch.equal(a, b)
    for a, b in zip((dq2, dk2, dv2), ref):
        assert torch.equal(a, b)


def test_single_query_gradients(gpu):
    # N = 1: softmax of one score is constant, so dQ = dK = 0 and dV = dO.  On the
    # GPU, P = exp(s - LSE) is 1 up to fp32 rounding of LSE and dP - D cancels up to
    # fp32 summation order, so dQ and dK are ~1e-7 rather than exactly 0.
    qb, kb, vb, dob = fa_inputs.qkv_bits(2, 4, 1, 128, "bf16", seed=91, with_dout=True)
    dq, dk, dv = run_fwd_bwd(qb, kb, vb, dob, "bf16", False, gpu)
    assert np.abs(to_host_f64(dq)).max() <= 1e-5 and np.abs(to_host_f64(dk)).max() <= 1e-5
    assert np.array_equal(to_host_f64(dv), fa_inputs.widen(dob, "bf16"))


def test_workspace_too_small_is_rejected(gpu):
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16, device=gpu)
    lse = torch.zeros(1, 1, 64, device=gpu)
    ws = torch.empty(fa.fa_bwd_workspace_size(1, 1, 64, 64) - 16, dtype=torch.uint8, device=gpu)
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd(q, q, q, q, q, lse, q.clone(), q.clone(), q.clone(), 0.125, False, ws)
    assert e.value.status == 6


@pytest.mark.parametrize("B,H", [(32, 8), (21, 13)], ids=["xcd_grouped", "not_grouped"])
def test_large_grid_covers_every_block(gpu, B, H):
    # Many heads of short sequences: 2048+ key blocks of the dK/dV pass and as
    # many query blocks of the dQ pass, heads grouped per XCD (B*H a multiple
    # of 8) or not.  Outputs are pre-filled with NaN, so a block that no
    # workgroup wrote would show; two calls in a row give the same bits.
    import torch
    N, d, dtype = 1024, 128, "bf16"
    say(f"[bwd large grid] B={B} H={H} N={N}")
    qb, kb, vb, dob = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=2300 + H, with_dout=True)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu)
    runs = []
    for _ in range(2):
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, 1 / math.sqrt(d), True, ws)
        torch.cuda.synchronize()
        runs.append((dq, dk, dv))
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    dq_h, dk_h, dv_h = (to_host_f64(x) for x in runs[0])
    for x in (dq_h, dk_h, dv_h):
        assert np.isfinite(x).all()
    # every head: sum_j dV_j = sum_i dO_i (probability rows sum to 1) and sum_j dK_j = 0
    dow = fa_inputs.widen(dob, dtype)
    assert max_abs(dv_h.sum(axis=2), dow.sum(axis=2)) <= 0.5
    assert np.abs(dk_h.sum(axis=2)).max() <= 0.5
    scale = float(np.float32(1 / math.sqrt(d)))
    for bh in (0, (B * H) // 2, B * H - 1):
        b, h = divmod(bh, H)
        sub = [fa_inputs.widen(x[b:b + 1, h:h + 1], dtype) for x in (qb, kb, vb, dob)]
        rq, rk, rv = oracle.bwd_heads(*sub, scale, True, [0])
        say(f"  head {bh}")
        compare("dQ", dq_h[b, h], rq[0])
        compare("dK", dk_h[b, h], rk[0])
        compare("dV", dv_h[b, h], rv[0])

