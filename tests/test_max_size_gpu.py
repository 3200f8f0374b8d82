"""The largest heads the library accepts, on the GPU.

One head is addressed through a 32-bit buffer resource, so a head's K (or Q)
may hold up to 2^32 - 1 bytes: at d = 128 that is N = 16 777 215 rows (the
next size is rejected with FA_ERR_SHAPE, checked on the CPU in test_abi).
Both ends are exercised with cross-attention shapes whose compute stays
small: 130 queries over the maximum number of keys, and the maximum number
of queries over 100 keys.  Inputs are seeded draws made on the device (host
generation of 2^31 values would take minutes); the fp64 oracle gets the
same bits, widened.

Rows are independent in the forward and in dQ (row i's output and gradient
depend only on q_i, dO_i, K and V), so the oracle checks sampled rows through
a subproblem made of those rows; with the causal mask aligned to the last
query and key, the last r rows of a problem are the r rows of the subproblem
with the same keys, so the sample is the last rows.  dK and dV sum over every
row: they are checked against the oracle where only a few rows see any key,
and otherwise through identities that hold at any size: the rows of P sum to
one, so sum_j dV_j = sum_i dO_i over the rows that see a key, and sum_j dS_ij
= 0, so sum_j dK_j = 0."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_ABS, TOL_GRAD_RELF, TOL_LSE, TOL_O, max_abs, rel_frob, say,
                           to_host_f64)

pytestmark = pytest.mark.gpu

NMAX_D128 = (1 << 32) // (2 * 128) - 1  # 16 777 215


def _draw(shape, dtype, seed, device, chunk=1 << 22):
    """Seeded N(0,1) rows drawn on the device in chunks, rounded to dtype."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1, shape[-1])
    for s in range(0, flat.shape[0], chunk):
        e = min(flat.shape[0], s + chunk)
        flat[s:e] = torch.randn((e - s, shape[-1]), generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def _host64(t):
    return to_host_f64(t)


def _check_rows(o, lse, ro, rl, dtype, what):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert np.all(o[dead] == 0), what
    live = ~dead
    eo = max_abs(o[live], ro[live]) if live.any() else 0.0
    el = max_abs(lse[live], rl[live]) if live.any() else 0.0
    say(f"    {what}: O max-abs {eo:.3e}  LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, what


def _grad_close(name, got, want):
    ea, er = max_abs(got, want), rel_frob(got, want)
    say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e}")
    assert ea <= TOL_GRAD_ABS and er <= TOL_GRAD_RELF, (name, ea, er)


def test_maximum_keys(gpu):
    # 130 queries (two query tiles, the second ragged) over 2^24 - 1 keys, causal
    import torch
    Nq, Nk, d, dtype = 130, NMAX_D128, 128, "bf16"
    tdt = torch.bfloat16
    say(f"[max keys] Nq={Nq} Nk={Nk} d={d} {dtype} causal")
    q = _draw((1, 1, Nq, d), tdt, 61, gpu)
    k = _draw((1, 1, Nk, d), tdt, 62, gpu)
    v = _draw((1, 1, Nk, d), tdt, 63, gpu)
    do = _draw((1, 1, Nq, d), tdt, 64, gpu)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd_padded(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.bwd_padded(q, k, v, o, do, lse, causal=True, scale=scale)
    so, sl = fa.fwd_splitkv(q[:, :, -1:].contiguous(), k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    # every gradient finite; identities over all keys (every row sees keys)
    for name, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(x.float()).all(), name
    sv = dv.double().sum(dim=2)
    sdo = do.double().sum(dim=2)
    assert float((sv - sdo).abs().max()) <= 1e-2 * max(1.0, float(sdo.abs().max()))
    sk = dk.double().sum(dim=2)
    assert float(sk.abs().max()) <= 1e-2 * max(1e-6, float(dk.double().abs().sum(dim=2).max()))
    # the last three rows through the oracle (same bottom-right alignment)
    r = 3
    w = [_host64(x) for x in (q[:, :, -r:].contiguous(), k, v, do[:, :, -r:].contiguous())]
    s32 = float(np.float32(scale))
    ro, rl = oracle.fwd_padded(w[0], w[1], w[2], s32, True)
    _check_rows(_host64(o)[:, :, -r:], _host64(lse)[:, :, -r:], ro, rl, dtype, "forward, last 3 rows")
    _check_rows(_host64(so), _host64(sl), ro[:, :, -1:], rl[:, :, -1:], dtype, "decode of the last row")
    rq, _, _ = oracle.bwd_padded(*w, s32, True)
    _grad_close("dQ (last 3 rows)", _host64(dq)[:, :, -r:], rq)


@pytest.mark.parametrize("causal", [False, True])
def test_maximum_queries(gpu, causal):
    # 2^24 - 1 queries over 100 keys; causal aligned to the last query and key,
    # so every row but the last 100 sees no key (O = 0, LSE = -inf, dQ = 0)
    import torch
    Nq, Nk, d, dtype = NMAX_D128, 100, 128, "f16"
    tdt = torch.float16
    say(f"[max queries] Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}")
    q = _draw((1, 1, Nq, d), tdt, 71, gpu)
    k = _draw((1, 1, Nk, d), tdt, 72, gpu)
    v = _draw((1, 1, Nk, d), tdt, 73, gpu)
    do = _draw((1, 1, Nq, d), tdt, 74, gpu)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd_padded(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_padded(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    s32 = float(np.float32(scale))
    if causal:
        first_live = Nq - Nk
        assert bool(torch.isneginf(lse[:, :, :first_live]).all())
        assert not bool(o[:, :, :first_live].any()) and not bool(dq[:, :, :first_live].any())
        # the live rows are the last Nk: their subproblem is exact for dK and dV too
        w = [_host64(x) for x in (q[:, :, first_live:].contiguous(), k, v, do[:, :, first_live:].contiguous())]
        ro, rl = oracle.fwd_padded(w[0], w[1], w[2], s32, True)
        _check_rows(_host64(o)[:, :, first_live:], _host64(lse)[:, :, first_live:], ro, rl, dtype, "forward, live rows")
        rq, rk, rv = oracle.bwd_padded(*w, s32, True)
        _grad_close("dQ (live rows)", _host64(dq)[:, :, first_live:], rq)
        _grad_close("dK", _host64(dk), rk)
        _grad_close("dV", _host64(dv), rv)
    else:
        rows = np.array([0, 1, 127, 128, Nq // 2, Nq - 130, Nq - 2, Nq - 1])
        idx = torch.from_numpy(rows).to(gpu)
        w = [_host64(x.index_select(2, idx).contiguous()) for x in (q, do)]
        kk, vv = _host64(k), _host64(v)
        ro, rl = oracle.fwd_padded(w[0], kk, vv, s32, False)
        _check_rows(_host64(o.index_select(2, idx)), _host64(lse.index_select(2, idx)), ro, rl, dtype,
                    "forward, sampled rows")
        rq, _, _ = oracle.bwd_padded(w[0], kk, vv, w[1], s32, False)
        _grad_close("dQ (sampled rows)", _host64(dq.index_select(2, idx)), rq)
        for name, x in (("dK", dk), ("dV", dv)):
            assert torch.isfinite(x.float()).all(), name
        sv, sdo = dv.double().sum(dim=2), do.double().sum(dim=2)
        assert float((sv - sdo).abs().max()) <= 1e-3 * float(sdo.abs().max() + 1)
        sk = dk.double().sum(dim=2)
        assert float(sk.abs().max()) <= 1e-2 * max(1e-6, float(dk.double().abs().sum(dim=2).max()))
