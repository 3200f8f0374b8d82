"""Debug mode on the GPU: with FA_DEBUG set, every computing entry point, after
its launches, waits for the stream and prints the NaN / +inf / -inf counts of
its inputs and outputs; results are bit-identical to those without it.  The
counts are checked against what the inputs fix: none on clean inputs; a NaN
planted in one element of query row i shows as one NaN in q, a NaN in every
element of O row i and in LSE row i; rows that see no key show as -inf in the
LSE (one per such row), never as NaN.  Calls with per-batch lengths print
them, flagging values outside [0, N] (the kernels clamp them)."""
import re

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
from tests.helpers import say, to_device, to_host_f64
from tests.test_padded_gpu import inputs, lens_tensor

pytestmark = pytest.mark.gpu

LINE = re.compile(r"^\[FA_DEBUG\] (\w+): (.+?): (\d+) NaN, (\d+) \+inf, (\d+) -inf of (\d+) values")


def _scan(err):
    """{(entry point, tensor): (nan, +inf, -inf, n)} from the debug lines."""
    out = {}
    for line in err.splitlines():
        m = LINE.match(line)
        if m:
            out[(m.group(1), m.group(2))] = tuple(int(m.group(i)) for i in range(3, 7))
    return out


def _bits(t):
    import torch
    t = t.detach().cpu()
    return t.view(torch.int32).numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy()


def _run_twice(monkeypatch, capfd, fn):
    """fn() without and with debug mode; returns both results and the scan of the second."""
    import torch
    monkeypatch.delenv("FA_DEBUG", raising=False)
    monkeypatch.delenv("FLASH_ATTENTION_DEBUG", raising=False)
    plain = fn()
    torch.cuda.synchronize()
    capfd.readouterr()
    monkeypatch.setenv("FA_DEBUG", "1")
    dbg = fn()
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    monkeypatch.delenv("FA_DEBUG", raising=False)
    for a, b in zip(plain, dbg):
        assert np.array_equal(_bits(a), _bits(b))
    return _scan(err), err


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_clean_inputs_square(gpu, monkeypatch, capfd, dtype):
    B, H, N, d = 1, 2, 300, 128
    say(f"[debug] square N={N} d={d} {dtype}")
    qb, kb, vb = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4700)
    dob = fa_inputs.normal_bits(B * H * N * d, dtype, 4700, fa_inputs.STREAM_DO).reshape(B, H, N, d)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))

    def run():
        o, lse = fa.fwd(q, k, v, causal=True)
        return (o, lse, *fa.bwd(q, k, v, o, do, lse, causal=True))

    scan, err = _run_twice(monkeypatch, capfd, run)
    assert "[FA_DEBUG] fa_fwd: B=1 H=2 Nq=300 Nk=300 d=128" in err
    n = B * H * N
    for name in ("q", "k", "v", "o"):
        assert scan[("fa_fwd", name)] == (0, 0, 0, n * d), name
    assert scan[("fa_fwd", "lse")] == (0, 0, 0, n)
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        assert scan[("fa_bwd", name)] == (0, 0, 0, n * d), name
    assert scan[("fa_bwd", "lse")] == (0, 0, 0, n)


def test_dead_rows_are_reported_as_minus_inf(gpu, monkeypatch, capfd):
    # padded cross-attention: batch entries with 77 and 0 valid queries of 130
    dtype, d = "bf16", 64
    Lq, Lk = [130, 77, 0], [300, 33, 160]
    qb, kb, vb, dob = inputs(130, 300, d, dtype, 4701)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    lq, lk = lens_tensor(Lq, gpu), lens_tensor(Lk, gpu)

    def run():
        o, lse = fa.fwd_padded(q, k, v, lq, lk, causal=False)
        so, sl = fa.fwd_splitkv(q, k, v, lq, lk, causal=False)
        return (o, lse, so, sl, *fa.bwd_padded(q, k, v, o, do, lse, lq, lk, causal=False))

    scan, err = _run_twice(monkeypatch, capfd, run)
    for fn in ("fa_fwd_padded", "fa_fwd_splitkv", "fa_bwd_padded"):
        assert f"[FA_DEBUG] {fn}: seqlens_q (B=3, N=130): [130, 77, 0]\n" in err, fn
        assert f"[FA_DEBUG] {fn}: seqlens_k (B=3, N=300): [300, 33, 160]\n" in err, fn
    H = 2
    dead = H * sum(130 - x for x in Lq)
    assert dead == 366
    o, lse = fa.fwd_padded(q, k, v, lq, lk, causal=False)
    assert int(np.isneginf(to_host_f64(lse)).sum()) == dead
    for fn in ("fa_fwd_padded", "fa_fwd_splitkv"):
        assert scan[(fn, "lse")] == (0, 0, dead, 3 * H * 130), fn
        assert scan[(fn, "o")][:3] == (0, 0, 0), fn
    assert scan[("fa_bwd_padded", "lse")] == (0, 0, dead, 3 * H * 130)
    for name in ("dq", "dk", "dv"):
        assert scan[("fa_bwd_padded", name)][:3] == (0, 0, 0), name


def test_planted_nan_is_reported(gpu, monkeypatch, capfd):
    B, H, N, d, dtype = 1, 2, 300, 128, "bf16"
    i, c = 77, 5
    qb, kb, vb = fa_inputs.qkv_bits(B, H, N, d, dtype, seed=4702)
    dob = fa_inputs.normal_bits(B * H * N * d, dtype, 4702, fa_inputs.STREAM_DO).reshape(B, H, N, d)
    qb = qb.copy()
    qb[0, 1, i, c] = np.uint16(0x7FC0)
    q, k, v, do = (to_device(x, dtype, gpu) for x in (qb, kb, vb, dob))
    say("[debug] NaN planted in q[0, 1, 77, 5]")

    def run():
        o, lse = fa.fwd(q, k, v, causal=False)
        ws = torch_empty_ws(q)
        fa.fa_bwd_preprocess(o, do, lse, ws)
        dq = q.new_empty(q.shape)
        fa.fa_bwd_dq(q, k, v, do, dq, fa.default_scale(d), False, ws)
        return o, lse, dq

    scan, _ = _run_twice(monkeypatch, capfd, run)
    n = B * H * N
    assert scan[("fa_fwd", "q")] == (1, 0, 0, n * d)
    assert scan[("fa_fwd", "k")] == (0, 0, 0, n * d)
    # O row i and LSE row i are NaN, nothing else
    assert scan[("fa_fwd", "o")] == (d, 0, 0, n * d)
    assert scan[("fa_fwd", "lse")] == (1, 0, 0, n)
    assert scan[("fa_bwd_preprocess", "o")] == (d, 0, 0, n * d)
    assert scan[("fa_bwd_preprocess", "workspace LSE*log2(e)")] == (1, 0, 0, n)
    assert scan[("fa_bwd_preprocess", "workspace -D")] == (1, 0, 0, n)
    assert scan[("fa_bwd_dq", "dq")] == (d, 0, 0, n * d)


def torch_empty_ws(q):
    import torch
    B, H, N, d = q.shape
    return torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)


def test_out_of_range_lengths_are_flagged(gpu, monkeypatch, capfd):
    # lengths past N are clamped on the device; debug mode says so
    dtype, d = "f16", 64
    qb, kb, vb, _ = inputs(40, 50, d, dtype, 4703, B=2, H=1)
    q, k, v = (to_device(x, dtype, gpu) for x in (qb, kb, vb))
    lq, lk = lens_tensor([40, 99], gpu), lens_tensor([-3, 50], gpu)
    scan, err = _run_twice(monkeypatch, capfd, lambda: fa.fwd_padded(q, k, v, lq, lk, causal=True))
    assert "seqlens_q (B=2, N=40): [40, 99]; outside [0, N], clamped on the device" in err
    assert "seqlens_k (B=2, N=50): [-3, 50]; outside [0, N], clamped on the device" in err
    # batch entry 0 sees no key (Lk clamped to 0): its 40 rows are dead
    assert scan[("fa_fwd_padded", "lse")] == (0, 0, 40, 80)

