"""Forward split over key blocks (fa_fwd_splitkv) on decode-shaped inputs --
few queries over a long K/V, with per-batch cache lengths -- against the fp64
oracle's padded definition (the same function) on the same seeded inputs.
Bars: O max-abs <= 2e-2 (bf16) / 4e-3 (fp16), LSE <= 1e-3; rows that see no
key exactly O = 0, LSE = -inf."""
import math

import numpy as np
import pytest

import exact_attention_21_amd as fa
import fa_inputs
import oracle
from tests.helpers import TOL_LSE, TOL_O, max_abs, say, to_device, to_host_f64
from tests.test_padded_gpu import inputs, lens_tensor

pytestmark = pytest.mark.gpu

# B, H, Nq, Nk, Lq per batch, Lk per batch
CASES = {
    "decode_q1_k5000": (4, 8, 1, 5000, None, [5000, 1, 0, 3333]),
    "spec_q7_k2048": (2, 4, 7, 2048, None, [2048, 900]),
    "prefill_q300_k9000": (1, 2, 300, 9000, [300], [9000]),
    "decode_q1_k40000": (1, 4, 1, 40000, None, None),
    "decode_q1_padding_row": (2, 4, 1, 3000, [1, 0], [3000, 2999]),
    "decode_q1_k5": (1, 2, 1, 5, None, None),
}


def run(q, k, v, lq, lk, dtype, causal, device):
    import torch
    tq, tk, tv = (to_device(x, dtype, device) for x in (q, k, v))
    o, lse = fa.fwd_splitkv(tq, tk, tv, lens_tensor(lq, device), lens_tensor(lk, device), causal=causal)
    torch.cuda.synchronize()
    return to_host_f64(o), to_host_f64(lse)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(CASES))
def test_splitkv_against_oracle(gpu, case, d, causal, dtype):
    B, H, Nq, Nk, lq, lk = CASES[case]
    say(f"[splitkv] {case} d={d} causal={causal} {dtype}")
    q, k, v, _ = inputs(Nq, Nk, d, dtype, 4800 + d, B=B, H=H)
    o, lse = run(q, k, v, lq, lk, dtype, causal, gpu)
    scale = float(np.float32(1 / math.sqrt(d)))
    ro, rl = oracle.fwd_padded(*(fa_inputs.widen(x, dtype) for x in (q, k, v)), scale, causal, lq, lk)
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead)
    assert np.all(o[dead] == 0)
    live = ~dead
    eo, el = max_abs(o[live], ro[live]), max_abs(lse[live], rl[live])
    say(f"    O max-abs {eo:.3e}  LSE max-abs {el:.3e}")
    assert eo <= TOL_O[dtype] and el <= TOL_LSE


def test_splitkv_close_to_unsplit_and_repeatable(gpu):
    import torch
    B, H, Nq, Nk, d = 2, 4, 3, 7000, 128
    q, k, v, _ = inputs(Nq, Nk, d, "bf16", 4900, B=B, H=H)
    tq, tk, tv = (to_device(x, "bf16", gpu) for x in (q, k, v))
    o1, l1 = fa.fwd_splitkv(tq, tk, tv, causal=True)
    o2, l2 = fa.fwd_splitkv(tq, tk, tv, causal=True)
    o3, l3 = fa.fwd_padded(tq, tk, tv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert float((o1.float() - o3.float()).abs().max()) <= 2e-2
    assert float((l1 - l3).abs().max()) <= 1e-3


def test_splitkv_workspace_checked(gpu):
    import torch
    q = torch.zeros((1, 1, 1, 64), dtype=torch.float16, device=gpu)
    k = torch.zeros((1, 1, 4096, 64), dtype=torch.float16, device=gpu)
    need = fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 4096, 64)
    assert need > 0
    ws = torch.empty(need - 256, dtype=torch.uint8, device=gpu)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 1), dtype=torch.float32, device=gpu)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv(q, k, k, o, lse, None, None, 0.125, False, ws)
    assert e.value.status == 6  # FA_ERR_WORKSPACE


def test_decode_full_size_sampled_heads(gpu):
    # the benchmark's decode call: B=32 H=32, one query per (batch, head) over
    # 16384 keys, bf16, causal (one workgroup of four partials per head); inputs
    # N(0,1) drawn on the device from a fixed seed, sampled heads checked
    import torch
    B, H, Nk, d = 32, 32, 16384, 128
    say(f"[splitkv full] decode B={B} H={H} Nk={Nk}")
    gen = torch.Generator(device=gpu).manual_seed(4950)
    draw = lambda n: torch.randn((B, H, n, d), generator=gen, device=gpu, dtype=torch.float32).to(torch.bfloat16)
    q, k, v = draw(1), draw(Nk), draw(Nk)
    o, lse = fa.fwd_splitkv(q, k, v, causal=True)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / math.sqrt(d)))
    worst_o = worst_l = 0.0
    for b, h in [(0, 0), (0, 31), (13, 7), (31, 0), (31, 31)]:
        sub = [to_host_f64(x[b:b + 1, h:h + 1]) for x in (q, k, v)]
        ro, rl = oracle.fwd_padded(*sub, scale, True, None, None)
        worst_o = max(worst_o, max_abs(to_host_f64(o[b:b + 1, h:h + 1]), ro))
        worst_l = max(worst_l, max_abs(to_host_f64(lse[b:b + 1, h:h + 1]), rl))
    say(f"    5 heads: O max-abs {worst_o:.3e}  LSE max-abs {worst_l:.3e}")
    assert worst_o <= TOL_O["bf16"] and worst_l <= TOL_LSE
