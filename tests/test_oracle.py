"""Pins for the fp64 oracle: closed forms, a hand-derived worked example,
invariants, brute force in extended precision, an independent tiled (online
softmax) evaluation, library autograd and finite differences.

Each check is chosen so that a plausible mistake in the oracle (a dropped scale,
a wrong mask boundary, a transposed operand, a sign error in the softmax
gradient, a missing max subtraction) fails at least one of them; the mutation
tests at the end plant such mistakes in a copy of the oracle and assert that.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------------
# worked example derived by hand (tests/golden/tiny_n2_d2.json)
# --------------------------------------------------------------------------

def load_golden():
    with open(os.path.join(GOLDEN, "tiny_n2_d2.json")) as f:
        g = json.load(f)
    as4 = lambda a: np.array(a, np.float64)[None, None]
    return g, as4(g["q"]), as4(g["k"]), as4(g["v"]), as4(g["dout"])


def test_golden_forward_noncausal():
    g, q, k, v, _ = load_golden()
    o, lse = oracle.fwd(q, k, v, g["scale"], False)
    np.testing.assert_allclose(o[0, 0], g["noncausal"]["o"], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], g["noncausal"]["lse"], atol=1e-12)


def test_golden_forward_causal():
    g, q, k, v, _ = load_golden()
    o, lse = oracle.fwd(q, k, v, g["scale"], True)
    np.testing.assert_allclose(o[0, 0], g["causal"]["o"], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], g["causal"]["lse"], atol=1e-12)


def test_golden_backward_noncausal():
    g, q, k, v, do = load_golden()
    dq, dk, dv = oracle.bwd(q, k, v, do, g["scale"], False)
    np.testing.assert_allclose(dq[0, 0], g["noncausal"]["dq"], atol=1e-12)
    np.testing.assert_allclose(dk[0, 0], g["noncausal"]["dk"], atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], g["noncausal"]["dv"], atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    B, H, N, d = 1, 2, 13, 8
    q = rnd((B, H, N, d), 1)
    v = rnd((B, H, N, d), 2)
    k = np.broadcast_to(rnd((B, H, 1, d), 3), (B, H, N, d)).copy()
    scale = 0.37
    o, lse = oracle.fwd(q, k, v, scale, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n_vis].mean(axis=2), atol=1e-12)
        s = scale * np.einsum("bhc,bhc->bh", q[:, :, i], k[:, :, 0])
        np.testing.assert_allclose(lse[:, :, i], s + math.log(n_vis), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_of_visible_values(causal):
    # scale = 0: every visible score is 0, so the weights are uniform over the
    # visible keys: O_i = mean of V over them (prefix means when causal),
    # LSE_i = ln n_i; dQ = dK = 0 (both carry the factor scale) and
    # dV_j = sum over the rows i that see key j of dO_i / n_i
    B, H, N, d = 2, 2, 11, 8
    q, k, v, do = (rnd((B, H, N, d), 300 + i, 3.0) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.0, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.0, causal)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    for i in range(N):
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n[i]].mean(axis=2), atol=1e-12)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(n), lse.shape), atol=1e-14)
    assert not dq.any() and not dk.any()
    for j in range(N):
        rows = [i for i in range(N) if (i >= j or not causal)]
        want = sum(do[:, :, i] / n[i] for i in rows)
        np.testing.assert_allclose(dv[:, :, j], want, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_equals_negated_keys(causal):
    # softmax(-s q.k) = softmax(s q.(-k)): the forward at -s on K equals the
    # forward at s on -K; by the chain rule dQ and dV agree and dK changes sign
    q, k, v, do = (rnd((1, 2, 9, 6), 310 + i) for i in range(4))
    o1, l1 = oracle.fwd(q, k, v, -0.45, causal)
    o2, l2 = oracle.fwd(q, -k, v, 0.45, causal)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    g1 = oracle.bwd(q, k, v, do, -0.45, causal)
    g2 = oracle.bwd(q, -k, v, do, 0.45, causal)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], -g2[1], atol=1e-13)
    np.testing.assert_allclose(g1[2], g2[2], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key_returns_v_exactly(causal):
    q, k, v = rnd((2, 3, 1, 16), 4), rnd((2, 3, 1, 16), 5), rnd((2, 3, 1, 16), 6)
    o, lse = oracle.fwd(q, k, v, 0.25, causal)
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse[..., 0], 0.25 * (q[..., 0, :] * k[..., 0, :]).sum(-1), atol=1e-13)


def test_causal_row0_is_v0():
    q, k, v = rnd((1, 2, 9, 8), 7), rnd((1, 2, 9, 8), 8), rnd((1, 2, 9, 8), 9)
    o, lse = oracle.fwd(q, k, v, 0.5, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.5 * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    # with V = identity (N = d) the output rows are the softmax rows themselves
    N = 12
    q, k = rnd((1, 1, N, N), 10), rnd((1, 1, N, N), 11)
    v = np.eye(N)[None, None]
    p, _ = oracle.fwd(q, k, v, 0.3, causal)
    p = p[0, 0]
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    if causal:
        assert np.count_nonzero(np.triu(p, 1)) == 0
        assert (np.diag(p) > 0).all()


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mag", [1.0, 12.0])
@pytest.mark.parametrize("scale", [0.5, -0.8, 0.0])
def test_lse_and_output_match_50_digit_brute_force(N, causal, mag, scale):
    # the scale is a free argument of the formula: the usual 1/sqrt(d) (d = 4),
    # a negative one (the smallest raw scores get the largest weights) and 0
    d = 4
    q, k, v = rnd((1, 1, N, d), 20 + N, mag), rnd((1, 1, N, d), 30 + N, mag), rnd((1, 1, N, d), 40 + N)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    mpmath.mp.dps = 50
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        # no max subtraction: plain log of the plain sum, at 50 digits
        e = {j: mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, 0, i, c]) * mpmath.mpf(k[0, 0, j, c])
                                                          for c in range(d))) for j in js}
        tot = mpmath.fsum(e.values())
        assert abs(float(mpmath.log(tot)) - lse[0, 0, i]) <= 1e-12 * max(1.0, abs(lse[0, 0, i]))
        for c in range(d):
            ref = mpmath.fsum(e[j] * mpmath.mpf(v[0, 0, j, c]) for j in js) / tot
            assert abs(float(ref) - o[0, 0, i, c]) <= 1e-12


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v = rnd((1, 2, 10, 6), 50), rnd((1, 2, 10, 6), 51), rnd((1, 2, 10, 6), 52)
    u = rnd((1, 2, 1, 6), 53)
    o1, l1 = oracle.fwd(q, k, v, 0.4, causal)
    o2, l2 = oracle.fwd(q, k + u, v, 0.4, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.4 * np.einsum("bhnc,bhkc->bhn", q, u), atol=1e-12)


def test_permutation_equivariance_noncausal():
    q, k, v = rnd((1, 1, 11, 5), 60), rnd((1, 1, 11, 5), 61), rnd((1, 1, 11, 5), 62)
    perm = np.random.default_rng(63).permutation(11)
    o, lse = oracle.fwd(q, k, v, 0.7, False)
    o2, lse2 = oracle.fwd(q, k[:, :, perm], v[:, :, perm], 0.7, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    o3, lse3 = oracle.fwd(q[:, :, perm], k, v, 0.7, False)
    np.testing.assert_allclose(o3, o[:, :, perm], atol=1e-12)
    np.testing.assert_allclose(lse3, lse[:, :, perm], atol=1e-12)


def test_huge_scores_stay_finite():
    q, k, v = rnd((1, 1, 16, 8), 70, 40.0), rnd((1, 1, 16, 8), 71, 40.0), rnd((1, 1, 16, 8), 72)
    o, lse = oracle.fwd(q, k, v, 1.0, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert (np.abs(o) <= np.abs(v).max(axis=2, keepdims=True) + 1e-12).all()


# --------------------------------------------------------------------------
# an independent evaluation: block-wise online softmax (running max, running
# sum, rescaling of the partial output), as the tuning handbook's
# "engineering implementation" section describes, written here in numpy
# --------------------------------------------------------------------------

def tiled_online(q, k, v, scale, causal, block):
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    lse = np.full((B, H, N), -np.inf)
    for i0 in range(0, N, block):
        i1 = min(N, i0 + block)
        m = np.full((B, H, i1 - i0, 1), -np.inf)
        l = np.zeros((B, H, i1 - i0, 1))
        acc = np.zeros((B, H, i1 - i0, d))
        for j0 in range(0, N, block):
            j1 = min(N, j0 + block)
            s = scale * q[:, :, i0:i1] @ np.swapaxes(k[:, :, j0:j1], -1, -2)
            if causal:
                ii = np.arange(i0, i1)[:, None]
                jj = np.arange(j0, j1)[None, :]
                s = np.where(jj <= ii, s, -np.inf)
            bm = s.max(-1, keepdims=True)
            m_new = np.maximum(m, bm)
            safe = np.where(np.isfinite(m_new), m_new, 0.0)
            p = np.exp(s - safe)
            alpha = np.exp(m - safe)
            l = alpha * l + p.sum(-1, keepdims=True)
            acc = alpha * acc + p @ v[:, :, j0:j1]
            m = m_new
        o[:, :, i0:i1] = acc / l
        lse[:, :, i0:i1] = (m + np.log(l))[..., 0]
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,block", [(64, 16), (77, 16), (33, 64)])
def test_online_tiled_equals_plain(causal, N, block):
    q, k, v = rnd((2, 2, N, 16), 80), rnd((2, 2, N, 16), 81), rnd((2, 2, N, 16), 82)
    o, lse = oracle.fwd(q, k, v, 0.25, causal)
    o2, lse2 = tiled_online(q, k, v, 0.25, causal, block)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


# --------------------------------------------------------------------------
# library routine: torch fp64 CPU, forward and autograd backward
# --------------------------------------------------------------------------

def torch_reference(q, k, v, dout, scale, causal):
    import torch
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Q, K, V = t(q), t(k), t(v)
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
    if causal:
        N = q.shape[2]
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.matmul(torch.softmax(s, dim=-1), V)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return o.detach().numpy(), lse.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.25, -0.7, 0.0])
def test_matches_torch_fp64_autograd(causal, scale):
    shape = (2, 3, 40, 16)
    q, k, v, do = (rnd(shape, 90 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, scale, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    to, tl, tdq, tdk, tdv = torch_reference(q, k, v, do, scale, causal)
    np.testing.assert_allclose(o, to, atol=1e-12)
    np.testing.assert_allclose(lse, tl, atol=1e-12)
    np.testing.assert_allclose(dq, tdq, atol=1e-12)
    np.testing.assert_allclose(dk, tdk, atol=1e-12)
    np.testing.assert_allclose(dv, tdv, atol=1e-12)


# --------------------------------------------------------------------------
# backward: finite differences of L = sum(dO * O), and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (5, 4), (8, 2)])
def test_backward_central_differences(causal, N, d):
    q, k, v, do = (rnd((1, 1, N, d), 100 + i + 10 * N) for i in range(4))
    scale = 0.6
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    loss = lambda q_, k_, v_: float((oracle.fwd(q_, k_, v_, scale, causal)[0] * do).sum())
    h = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        fd = np.zeros_like(grad)
        for idx in np.ndindex(q.shape[2:]):
            args = {"q": q, "k": k, "v": v}
            plus = {a: b.copy() for a, b in args.items()}
            minus = {a: b.copy() for a, b in args.items()}
            plus[which][(0, 0) + idx] += h
            minus[which][(0, 0) + idx] -= h
            fd[(0, 0) + idx] = (loss(plus["q"], plus["k"], plus["v"]) -
                                loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
        np.testing.assert_allclose(grad, fd, atol=2e-8, rtol=1e-6, err_msg=which)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v, do = (rnd((1, 2, 24, 8), 120 + i) for i in range(4))
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.35, causal)
    # dS rows sum to zero, so the key gradients sum to zero over keys
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # P rows sum to one, so dV summed over keys equals dO summed over queries
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    if causal:
        # query 0 sees only key 0: its softmax is constant, so its gradient vanishes
        np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)
        # the last key is seen only by the last query: dV_last = P_last,last * dO_last
        _, lse = oracle.fwd(q, k, v, 0.35, causal)
        p_ll = np.exp(0.35 * (q[:, :, -1] * k[:, :, -1]).sum(-1) - lse[:, :, -1])
        np.testing.assert_allclose(dv[:, :, -1], p_ll[..., None] * do[:, :, -1], atol=1e-12)


# --------------------------------------------------------------------------
# entry points agree with each other
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_and_heads_subsets_match_full(causal):
    B, H, N, d = 2, 3, 21, 8
    q, k, v, do = (rnd((B, H, N, d), 130 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.3, causal, threads=1)
    rows = np.array([0, 5, N - 1, N, 2 * H * N - 1, 3 * N + 7])
    o_r, l_r = oracle.fwd_rows(q, k, v, 0.3, causal, rows, threads=3)
    assert np.array_equal(o_r, o.reshape(-1, d)[rows])
    assert np.array_equal(l_r, lse.reshape(-1)[rows])
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.3, causal, threads=4)
    heads = np.array([4, 0])
    hq, hk, hv = oracle.bwd_heads(q, k, v, do, 0.3, causal, heads, threads=1)
    for x, hh in enumerate(heads):
        assert np.array_equal(hq[x], dq.reshape(B * H, N, d)[hh])
        assert np.array_equal(hk[x], dk.reshape(B * H, N, d)[hh])
        assert np.array_equal(hv[x], dv.reshape(B * H, N, d)[hh])


def test_bad_arguments_are_rejected():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(RuntimeError):
        oracle.fwd_rows(q, q, q, 1.0, False, [4])
    with pytest.raises(RuntimeError):
        oracle.bwd_heads(q, q, q, q, 1.0, False, [1])


# --------------------------------------------------------------------------
# padded batches and cross-attention: per-batch valid lengths Lq <= Nq,
# Lk <= Nk, causal aligned to the last query and key (oracle.fwd_padded /
# oracle.bwd_padded)
# --------------------------------------------------------------------------

def visible_mask(Nq, Nk, Lq, Lk, causal):
    """[Nq, Nk] bool: query i sees key j (the definition, written as a mask)."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    m = (i < Lq) & (j < Lk)
    if causal:
        m &= j <= i + (Lk - Lq)
    return m


def torch_padded_reference(q, k, v, dout, scale, causal, lq, lk):
    """torch fp64 (library softmax, logsumexp, matmul, autograd) with an explicit
    mask; rows that see no key get O = 0 and LSE = -inf and no gradient."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Q, K, V = t(q), t(k), t(v)
    mask = torch.stack([torch.from_numpy(visible_mask(Nq, Nk, lq[b], lk[b], causal)) for b in range(B)])
    mask = mask[:, None]                                   # [B, 1, Nq, Nk]
    rowvalid = mask.any(-1, keepdim=True)                  # [B, 1, Nq, 1]
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    s_safe = torch.where(rowvalid, s, torch.zeros_like(s))
    p = torch.softmax(s_safe, dim=-1) * rowvalid
    o = torch.matmul(p, V)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return o.detach().numpy(), lse.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


PADDED_CASES = [
    # Nq, Nk, lq, lk
    (29, 41, [29, 17, 0], [41, 5, 30]),
    (40, 13, [40, 33, 12], [13, 13, 0]),
    (16, 16, [16, 9, 3], [16, 12, 16]),
]


@pytest.mark.parametrize("case", range(len(PADDED_CASES)))
@pytest.mark.parametrize("causal", [False, True])
def test_padded_matches_torch_masked_reference(case, causal):
    Nq, Nk, lq, lk = PADDED_CASES[case]
    B, H, d = 3, 2, 8
    q, do = rnd((B, H, Nq, d), 200 + case), rnd((B, H, Nq, d), 210 + case)
    k, v = rnd((B, H, Nk, d), 220 + case), rnd((B, H, Nk, d), 230 + case)
    scale = 0.4
    o, lse = oracle.fwd_padded(q, k, v, scale, causal, lq, lk)
    dq, dk, dv = oracle.bwd_padded(q, k, v, do, scale, causal, lq, lk)
    to, tl, tdq, tdk, tdv = torch_padded_reference(q, k, v, do, scale, causal, lq, lk)
    np.testing.assert_allclose(o, to, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(tl))
    fin = np.isfinite(tl)
    np.testing.assert_allclose(lse[fin], tl[fin], atol=1e-12)
    np.testing.assert_allclose(dq, tdq, atol=1e-12)
    np.testing.assert_allclose(dk, tdk, atol=1e-12)
    np.testing.assert_allclose(dv, tdv, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_full_lengths_equal_square_oracle(causal):
    q, k, v, do = (rnd((2, 2, 37, 8), 240 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.3, causal)
    for lens in (None, [37, 37]):
        po, pl = oracle.fwd_padded(q, k, v, 0.3, causal, lens, lens)
        pq, pk, pv = oracle.bwd_padded(q, k, v, do, 0.3, causal, lens, lens)
        assert np.array_equal(po, o) and np.array_equal(pl, lse)
        assert np.array_equal(pq, dq) and np.array_equal(pk, dk) and np.array_equal(pv, dv)


@pytest.mark.parametrize("causal", [False, True])
def test_padding_contents_do_not_matter(causal):
    B, H, Nq, Nk, d = 2, 2, 19, 23, 4
    lq, lk = [11, 19], [23, 7]
    q, do = rnd((B, H, Nq, d), 250), rnd((B, H, Nq, d), 251)
    k, v = rnd((B, H, Nk, d), 252), rnd((B, H, Nk, d), 253)
    o, lse = oracle.fwd_padded(q, k, v, 0.5, causal, lq, lk)
    dq, dk, dv = oracle.bwd_padded(q, k, v, do, 0.5, causal, lq, lk)
    q2, do2, k2, v2 = q.copy(), do.copy(), k.copy(), v.copy()
    for b in range(B):
        q2[b, :, lq[b]:] = 1e3
        do2[b, :, lq[b]:] = -7.0
        k2[b, :, lk[b]:] = 1e3
        v2[b, :, lk[b]:] = 5.0
    o2, lse2 = oracle.fwd_padded(q2, k2, v2, 0.5, causal, lq, lk)
    dq2, dk2, dv2 = oracle.bwd_padded(q2, k2, v2, do2, 0.5, causal, lq, lk)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    for b in range(B):
        assert np.all(o[b, :, lq[b]:] == 0) and np.all(np.isneginf(lse[b, :, lq[b]:]))
        assert np.all(dq[b, :, lq[b]:] == 0)
        assert np.all(dk[b, :, lk[b]:] == 0) and np.all(dv[b, :, lk[b]:] == 0)


def test_bottom_right_causal_closed_forms():
    # identical keys: query i of a causal cross-attention with Lk > Lq averages
    # the first i + Lk - Lq + 1 values; with Lk < Lq the first Lq - Lk rows see nothing
    d = 3
    for Lq, Lk in ((4, 9), (9, 4), (1, 6)):
        q = rnd((1, 1, Lq, d), 260)
        k = np.tile(rnd((1, 1, 1, d), 261), (1, 1, Lk, 1))
        v = rnd((1, 1, Lk, d), 262)
        o, lse = oracle.fwd_padded(q, k, v, 0.7, True)
        for i in range(Lq):
            n = i + Lk - Lq + 1
            if n <= 0:
                assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
            else:
                s = 0.7 * float(q[0, 0, i] @ k[0, 0, 0])
                np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-13)
                np.testing.assert_allclose(lse[0, 0, i], s + math.log(n), atol=1e-13)
    # a single query sees every key (it is the last query), causal or not
    q, k, v = rnd((1, 2, 1, 5), 263), rnd((1, 2, 7, 5), 264), rnd((1, 2, 7, 5), 265)
    a = oracle.fwd_padded(q, k, v, 0.4, True)
    b = oracle.fwd_padded(q, k, v, 0.4, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [False, True])
def test_padded_backward_central_differences(causal):
    Nq, Nk, d = 4, 6, 3
    lq, lk = [3], [5]
    q, do = rnd((1, 1, Nq, d), 270), rnd((1, 1, Nq, d), 271)
    k, v = rnd((1, 1, Nk, d), 272), rnd((1, 1, Nk, d), 273)
    scale = 0.6
    dq, dk, dv = oracle.bwd_padded(q, k, v, do, scale, causal, lq, lk)
    loss = lambda q_, k_, v_: float((oracle.fwd_padded(q_, k_, v_, scale, causal, lq, lk)[0] * do).sum())
    h = 1e-6
    for which, grad, shp in (("q", dq, q.shape), ("k", dk, k.shape), ("v", dv, v.shape)):
        fd = np.zeros_like(grad)
        for idx in np.ndindex(shp[2:]):
            args = {"q": q, "k": k, "v": v}
            plus = {a: b.copy() for a, b in args.items()}
            minus = {a: b.copy() for a, b in args.items()}
            plus[which][(0, 0) + idx] += h
            minus[which][(0, 0) + idx] -= h
            fd[(0, 0) + idx] = (loss(plus["q"], plus["k"], plus["v"]) -
                                loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
        np.testing.assert_allclose(grad, fd, atol=2e-8, rtol=1e-6, err_msg=which)


def test_padded_bad_lengths_are_rejected():
    q = np.zeros((2, 1, 4, 2))
    k = np.zeros((2, 1, 3, 2))
    with pytest.raises(RuntimeError):
        oracle.fwd_padded(q, k, k, 1.0, False, [4, 5], None)
    with pytest.raises(RuntimeError):
        oracle.bwd_padded(q, k, k, q, 1.0, False, None, [-1, 3])


# --------------------------------------------------------------------------
# dropout: Philox4x32-10 (published known answers), the mask rule, keep rate,
# unbiasedness, a masked torch fp64 reference and finite differences
# --------------------------------------------------------------------------

def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        out = oracle.philox4x32_10([int(x, 16) for x in vec["counter"]], [int(x, 16) for x in vec["key"]])
        assert out == [int(x, 16) for x in vec["out"]]


def test_dropout_mask_follows_the_documented_rule():
    # pair (i, j) of head bh kept iff byte j%4 of word i%4 of
    # Philox(counter = (j/4, i/4, bh, offset), key = (seed lo, seed hi)) >= p8
    B, H, Nq, Nk, p8, seed, offset = 2, 3, 9, 13, 77, 0x0123456789ABCDEF, 5
    keep = oracle.dropout_mask(B, H, Nq, Nk, p8, seed, offset)
    rng = np.random.default_rng(7)
    for _ in range(60):
        b, h, i, j = (int(rng.integers(0, n)) for n in (B, H, Nq, Nk))
        out = oracle.philox4x32_10([j // 4, i // 4, b * H + h, offset], [seed & 0xFFFFFFFF, seed >> 32])
        byte = (out[i % 4] >> (8 * (j % 4))) & 0xFF
        assert keep[b, h, i, j] == (byte >= p8)


@pytest.mark.parametrize("p8", [0, 26, 128, 255])
def test_dropout_keep_rate(p8):
    keep = oracle.dropout_mask(2, 4, 64, 96, p8, 42, 0)
    n, p = keep.size, 1 - p8 / 256
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - n * p) <= 5 * sigma + (0 if 0 < p < 1 else 0.5)
    # different offsets and seeds give different masks
    if 0 < p8 < 255:
        assert not np.array_equal(keep, oracle.dropout_mask(2, 4, 64, 96, p8, 42, 1))
        assert not np.array_equal(keep, oracle.dropout_mask(2, 4, 64, 96, p8, 43, 0))


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_zero_equals_no_dropout(causal):
    q, k, v, do = (rnd((2, 2, 21, 8), 300 + i) for i in range(4))
    a = oracle.fwd_padded(q, k, v, 0.3, causal)
    b = oracle.fwd_padded(q, k, v, 0.3, causal, dropout=(0, 99, 3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ga = oracle.bwd_padded(q, k, v, do, 0.3, causal)
    gb = oracle.bwd_padded(q, k, v, do, 0.3, causal, dropout=(0, 99, 3))
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def torch_dropout_reference(q, k, v, dout, scale, causal, keep, p8):
    """torch fp64: O = (softmax(S) * Z) V with Z = keep * 256 / (256 - p8); autograd."""
    import torch
    Nq, Nk = q.shape[2], k.shape[2]
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Q, K, V = t(q), t(k), t(v)
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
    if causal:
        mask = torch.from_numpy(~visible_mask(Nq, Nk, Nq, Nk, True))
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    z = torch.from_numpy(keep.astype(np.float64)) * (256.0 / (256.0 - p8))
    o = torch.matmul(torch.softmax(s, dim=-1) * z, V)
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return o.detach().numpy(), lse.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_matches_torch_masked_reference(causal):
    B, H, Nq, Nk, d, p8, seed, offset = 2, 2, 27, 35 if not causal else 27, 8, 51, 1234, 9
    q, do = rnd((B, H, Nq, d), 310), rnd((B, H, Nq, d), 311)
    k, v = rnd((B, H, Nk, d), 312), rnd((B, H, Nk, d), 313)
    drop = (p8, seed, offset)
    o, lse = oracle.fwd_padded(q, k, v, 0.45, causal, dropout=drop)
    dq, dk, dv = oracle.bwd_padded(q, k, v, do, 0.45, causal, dropout=drop)
    keep = oracle.dropout_mask(B, H, Nq, Nk, *drop)
    to, tl, tdq, tdk, tdv = torch_dropout_reference(q, k, v, do, 0.45, causal, keep, p8)
    for got, ref in ((o, to), (lse, tl), (dq, tdq), (dk, tdk), (dv, tdv)):
        np.testing.assert_allclose(got, ref, atol=1e-12)


def test_dropout_is_unbiased():
    # E[O] over dropout masks is the output without dropout: average over offsets
    q, k, v = rnd((1, 1, 6, 4), 320), rnd((1, 1, 6, 4), 321), rnd((1, 1, 6, 4), 322)
    ref, _ = oracle.fwd_padded(q, k, v, 0.5, False)
    n = 3000
    acc = np.zeros_like(ref)
    for off in range(n):
        acc += oracle.fwd_padded(q, k, v, 0.5, False, dropout=(96, 2024, off))[0]
    # per-element std of one sample is below max|V|; 5 standard errors
    tol = 5 * np.abs(v).max() * math.sqrt((96 / 256) / (1 - 96 / 256)) / math.sqrt(n)
    np.testing.assert_allclose(acc / n, ref, atol=tol)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_central_differences(causal):
    Nq = Nk = 5
    d = 3
    q, k, v, do = (rnd((1, 1, Nq, d), 330 + i) for i in range(4))
    drop = (100, 77, 1)
    dq, dk, dv = oracle.bwd_padded(q, k, v, do, 0.6, causal, dropout=drop)
    loss = lambda q_, k_, v_: float((oracle.fwd_padded(q_, k_, v_, 0.6, causal, dropout=drop)[0] * do).sum())
    h = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        fd = np.zeros_like(grad)
        for idx in np.ndindex(grad.shape[2:]):
            args = {"q": q, "k": k, "v": v}
            plus = {a: b.copy() for a, b in args.items()}
            minus = {a: b.copy() for a, b in args.items()}
            plus[which][(0, 0) + idx] += h
            minus[which][(0, 0) + idx] -= h
            fd[(0, 0) + idx] = (loss(plus["q"], plus["k"], plus["v"]) -
                                loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
        np.testing.assert_allclose(grad, fd, atol=2e-8, rtol=1e-6, err_msg=which)
