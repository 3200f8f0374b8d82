"""Seeded random shapes through every forward and backward entry point, against
the fp64 oracle on the same inputs: batch, heads, Nq and Nk (equal or not),
head size, dtype, causal or not, per-batch valid lengths (including empty
ones), dropout or not.  Each case runs the padded (or dropout) forward and
backward and, without dropout, the split-over-keys forward too.  Bars as in
the other parity tests: O max-abs <= 2e-2 (bf16) / 4e-3 (fp16), LSE <= 1e-3,
gradients max-abs <= 5e-2 and rel-Frobenius <= 1e-2; rows that see no key are
exactly O = 0, LSE = -inf.  A gradient entry large enough that one unit in the
last place of its 16-bit storage exceeds 5e-2 (|x| >= 8 in bf16, as when
one valid key collects the gradients of hundreds of rows) is held to that
unit instead: the rounding of the stored value alone can reach it.

The rel-Frobenius bar of dQ and dK is widened by a bound computed per case:
the backward forms D = rowsum(dO * O) from the 16-bit O it is given, and with
few live rows one row can carry the whole norm of a gradient; a row whose
weight sits on one key (P = 0.92, 0.05, 0.02 over 3 keys, say) has
dS = P (dP - D) made of near-cancelling terms, so the rounding of O alone
moves its fp64 reference gradient by ~1e-2 relative.  The gradients are affine
in D (dS changes by -P dD, with no dropout factor), so that change is exact:
with dD = rowsum(dO * (round(O) - O)) from the oracle's own O,
  delta dQ = -scale dD (P K)   and   delta dK = -scale P^T (dD * Q),
where P K is the oracle's forward with V = K and P^T X the oracle's dV for the
upstream gradient X.  dQ and dK must be within 1e-2 + 2 |delta| / |ref|
(twice: the O the GPU hands its backward is within about one unit in the last
place of the exact O, the rounding within half of one); dV does not involve D
and always has the plain 1e-2 bar.  The bar is checked multiplied out,
|err| <= 1e-2 |ref| + 2 |delta|, so that it also holds where the reference is
exactly zero: over a single visible key P = 1 and D = dP, so dS = P (dP - D)
vanishes identically and dQ = dK = 0, while the D formed from the rounded O
leaves a gradient of the size of delta; where delta is zero too (O = V
exactly), the fp32 difference dP - D leaves round-off, which an rms floor of
1e-4 per element (500x below the max-abs bar) admits.  Max-abs is checked in
every case, with the same change as slack element by element (2 |delta_ij|):
where dS cancels for every row (one visible key), the rounded O's effect on D
sums over all of the rows into that key's dK.  It also takes the first-order
bound of the 16-bit rounding of P and dS, the operands of the gradient
products: u * sum |terms| per element (u = 2^-9 bf16, 2^-11 fp16; plus
n * 2^-24 for the fp32 accumulation).  That is ~1e-3 where the weights are
spread, but a few valid keys collecting hundreds of rows give entries of
magnitude 10-30 and sums of |terms| up to ~180 (found in a 4000 + 200 case
run: 0.07 off at such an entry, against a bound of 0.37).
"""
import math
import os

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import (TOL_GRAD_RELF, TOL_LSE, TOL_O, grad_abs_excess, max_abs, rel_frob, say, to_device,
                           to_host_f64)
from tests.test_padded_gpu import inputs, lens_tensor

pytestmark = pytest.mark.gpu

# 64 cases by default; FA_RANDOM_SHAPE_CASES=n runs the first n of the same
# seeded sequence (a longer sweep for kernel changes)
NCASES = int(os.environ.get("FA_RANDOM_SHAPE_CASES", "64"))
RMS_FLOOR = 1e-4  # 500x below the max-abs bar
DROP_SEED = 0x5EEDFACE12345678


def draw_case(i: int):
    rng = np.random.default_rng(0xCA5E0000 + i)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    Nq = 1 if rng.random() < 0.15 else int(rng.integers(1, 401))  # one row: the decode kernel
    Nk = Nq if rng.random() < 0.4 else int(rng.integers(1, 401))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.random() < 0.5)
    lq = lk = None
    if rng.random() < 0.6:
        lq = [int(x) for x in rng.integers(0, Nq + 1, size=B)]
        lk = [int(x) for x in rng.integers(0, Nk + 1, size=B)]
    p = float(rng.choice([0.1, 0.3])) if rng.random() < 0.3 else 0.0
    return B, H, Nq, Nk, d, dtype, causal, lq, lk, p


# Larger shapes: several tiles per head, up to 32 heads (B*H a multiple of 8
# selects the XCD-grouped dispatch), Nq and Nk up to 1500
NCASES_LARGE = int(os.environ.get("FA_RANDOM_LARGE_CASES", "12"))


def draw_large_case(i: int):
    rng = np.random.default_rng(0xB16C0000 + i)
    B, H = int(rng.integers(1, 5)), int(rng.choice([1, 2, 4, 8]))
    Nq = 1 if rng.random() < 0.1 else int(rng.integers(1, 1501))
    Nk = Nq if rng.random() < 0.4 else int(rng.integers(1, 1501))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.random() < 0.5)
    lq = lk = None
    if rng.random() < 0.5:
        lq = [int(x) for x in rng.integers(0, Nq + 1, size=B)]
        lk = [int(x) for x in rng.integers(0, Nk + 1, size=B)]
    p = float(rng.choice([0.1, 0.3])) if rng.random() < 0.25 else 0.0
    return B, H, Nq, Nk, d, dtype, causal, lq, lk, p


def check_fwd(o, lse, ro, rl, dtype, what):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert np.all(o[dead] == 0), what
    live = ~dead
    eo = max_abs(o[live], ro[live]) if live.any() else 0.0
    el = max_abs(lse[live], rl[live]) if live.any() else 0.0
    say(f"    {what}: O max-abs {eo:.3e}  LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, what


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape(gpu, i):
    say(f"[random {i}]")
    run_case(gpu, draw_case(i), 7000 + i, i)


@pytest.mark.parametrize("i", range(NCASES_LARGE))
def test_random_large_shape(gpu, i):
    say(f"[random large {i}]")
    run_case(gpu, draw_large_case(i), 9000 + i, 1000 + i)


def run_case(gpu, case, seed, i):
    """One case through the padded (or dropout) forward and backward and the
    split forward, against the oracle; i is the dropout offset."""
    import torch
    B, H, Nq, Nk, d, dtype, causal, lq, lk, p = case
    say(f"    B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} lq={lq} lk={lk} p={p}")
    q, k, v, do = inputs(Nq, Nk, d, dtype, seed, B=B, H=H)
    tq, tk, tv, tdo = (to_device(x, dtype, gpu) for x in (q, k, v, do))
    Lq, Lk = lens_tensor(lq, gpu), lens_tensor(lk, gpu)
    if p > 0:
        o, lse = fa.fwd_dropout(tq, tk, tv, p, DROP_SEED, i, Lq, Lk, causal=causal)
        grads = fa.bwd_dropout(tq, tk, tv, o, tdo, lse, p, DROP_SEED, i, Lq, Lk, causal=causal)
        drop = (fa.dropout_threshold(p), DROP_SEED, i)
    else:
        o, lse = fa.fwd_padded(tq, tk, tv, Lq, Lk, causal=causal)
        grads = fa.bwd_padded(tq, tk, tv, o, tdo, lse, Lq, Lk, causal=causal)
        drop = None
    split = fa.fwd_splitkv(tq, tk, tv, Lq, Lk, causal=causal) if p == 0 else None
    torch.cuda.synchronize()

    scale = float(np.float32(1 / math.sqrt(d)))
    w = [fa_inputs.widen(x, dtype) for x in (q, k, v, do)]
    ro, rl = oracle.fwd_padded(w[0], w[1], w[2], scale, causal, lq, lk, dropout=drop)
    check_fwd(to_host_f64(o), to_host_f64(lse), ro, rl, dtype, "forward")
    if split is not None:
        check_fwd(to_host_f64(split[0]), to_host_f64(split[1]), ro, rl, dtype, "split forward")
    ref = oracle.bwd_padded(*w, scale, causal, lq, lk, dropout=drop)
    live_rows = int(np.isfinite(rl).sum())
    delta = d_rounding_delta(w, ro, scale, causal, lq, lk, dtype)
    sums = abs_sums(w, ro, rl, scale, causal, lq, lk, drop)
    for name, got, want in zip(("dQ", "dK", "dV"), grads, ref):
        g = to_host_f64(got)
        ea, er = max_abs(g, want), rel_frob(g, want)
        # rel-F <= 1e-2 + 2 |delta| / |ref|, multiplied out so that it also
        # holds where the reference is exactly zero, plus an rms floor of
        # RMS_FLOOR per element for the fp32 round-off left where it is
        dl = delta.get(name)
        err, den = float(np.linalg.norm(g - want)), float(np.linalg.norm(want))
        allowed = TOL_GRAD_RELF * den + (2.0 * float(np.linalg.norm(dl)) if dl is not None else 0.0) \
            + RMS_FLOOR * math.sqrt(g.size)
        say(f"    {name}: max-abs {ea:.3e} rel-F {er:.3e} (|err| {err:.3e}, allowed {allowed:.3e}; "
            f"{live_rows} live rows)")
        # max-abs: the same exact change, element by element, and the
        # rounding of the 16-bit operands of the product (first-order bound)
        slack = 2.0 * np.abs(dl) if dl is not None else 0.0
        sm, n = sums[name]
        slack = slack + (UNIT_ROUNDOFF[dtype] + n * 2.0 ** -24) * sm
        assert grad_abs_excess(g, want, dtype, slack) <= 0.0, (name, ea)
        assert err <= allowed, (name, err, allowed)


# unit roundoff (half the relative spacing) of the 16-bit operands
UNIT_ROUNDOFF = {"bf16": 2.0 ** -9, "f16": 2.0 ** -11}


def abs_sums(w, ro, rl, scale, causal, lq, lk, drop):
    """Sums of |terms| of the gradient products, per element: dV_j = sum_i
    Z_ij P_ij dO_i, dK_j = scale sum_i dS_ij Q_i, dQ_i = scale sum_j dS_ij K_j
    with dS = P (Z dP - D) (Z the dropout factor, 1 without dropout).  The
    kernels round P and dS to 16 bits before these products, which moves
    each by at most u * (its sum of |terms|) (first order, u the operand's
    unit roundoff); the fp32 accumulation adds at most n * 2^-24 * the same
    sum.  P is formed from the oracle's LSE over the visible pairs (valid
    query i < Lq and key j < Lk; causal: j <= i + Lk - Lq), D from its O."""
    q, k, v, do = w
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    z_all = None
    if drop is not None:
        p8, seed, offset = drop
        keep = oracle.dropout_mask(B, H, Nq, Nk, p8, seed, offset).reshape(B, H, Nq, Nk)
        z_all = keep.astype(np.float64) * (256.0 / (256.0 - p8))
    s_dq, s_dk, s_dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(k)
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    for b in range(B):
        Lq = lq[b] if lq is not None else Nq
        Lk = lk[b] if lk is not None else Nk
        vis = (i < Lq) & (j < Lk)
        if causal:
            vis &= j <= i + (Lk - Lq)
        for h in range(H):
            with np.errstate(over="ignore", invalid="ignore"):
                pm = np.where(vis, np.exp(q[b, h] @ k[b, h].T * scale - rl[b, h][:, None]), 0.0)
            z = 1.0 if z_all is None else z_all[b, h]
            dpm = do[b, h] @ v[b, h].T
            dd = np.sum(do[b, h] * ro[b, h], axis=-1)[:, None]
            ads = np.abs(pm * (z * dpm - dd))
            s_dv[b, h] = (z * pm).T @ np.abs(do[b, h])
            s_dk[b, h] = scale * ads.T @ np.abs(q[b, h])
            s_dq[b, h] = scale * ads @ np.abs(k[b, h])
    return {"dQ": (s_dq, Nk), "dK": (s_dk, Nq), "dV": (s_dv, Nq)}


def d_rounding_delta(w, ro, scale, causal, lq, lk, dtype):
    """Change of the oracle's dQ and dK when D is formed from its own O rounded
    to the storage dtype (exact: the gradients are affine in D)."""
    q, k, v, do = w
    o16 = fa_inputs.widen(fa_inputs.narrow(ro, dtype), dtype)
    dD = np.sum(do * (o16 - ro), axis=-1)                      # [B, H, Nq]
    pk, _ = oracle.fwd_padded(q, k, k, scale, causal, lq, lk)  # P K
    delta_dq = -scale * dD[..., None] * pk
    delta_dk = -scale * oracle.bwd_padded(q, k, v, dD[..., None] * q, scale, causal, lq, lk)[2]  # P^T (dD Q)
    return {"dQ": delta_dq, "dK": delta_dk}
