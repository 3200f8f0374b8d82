"""Shared helpers for the GPU parity tests (marshalling and error metrics only)."""
import sys

import numpy as np

import fa_inputs

TOL_O = {"bf16": 2e-2, "f16": 4e-3}
TOL_LSE = 1e-3
TOL_GRAD_ABS = 5e-2
TOL_GRAD_RELF = 1e-2


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def to_device(bits: np.ndarray, dtype: str, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).to(device)


def to_host_f64(t) -> np.ndarray:
    """Exact widening of a 16-bit or fp32 device tensor to float64."""
    import torch
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy().astype(np.float64)
    bits = t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return fa_inputs.widen(bits, "bf16" if t.dtype == torch.bfloat16 else "f16")


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def ulp16(x, dtype: str) -> np.ndarray:
    """Unit in the last place of |x| in the 16-bit storage type (elementwise)."""
    mant, emin = (7, -126) if dtype == "bf16" else (10, -14)
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def grad_abs_excess(got, want, dtype: str, slack=0.0) -> float:
    """Largest |got - want| beyond max(TOL_GRAD_ABS, one 16-bit ulp of the
    larger magnitude) + slack over all elements (<= 0 passes; slack may be an
    array of the same shape).  The gradients are stored in 16 bits, so an
    entry whose magnitude makes one unit in the last place exceed the absolute
    bar (|x| >= 8 in bf16, >= 64 in fp16) is held to that unit: rounding the
    exact value alone can be that far off when the fp32 result sits on the
    other side of a rounding midpoint."""
    g, w = np.asarray(got, np.float64), np.asarray(want, np.float64)
    if g.size == 0:
        return 0.0
    bar = np.maximum(TOL_GRAD_ABS, ulp16(np.maximum(np.abs(g), np.abs(w)), dtype)) + slack
    return float(np.max(np.abs(g - w) - bar))


def rel_frob(a, b) -> float:
    ref = np.asarray(b, np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(np.asarray(a, np.float64) - ref))
    return num / den if den > 0 else num


def sample_rows(N: int, BM: int, count: int, seed: int) -> np.ndarray:
    """Query rows for sampled checks: both ends, tile edges and random rows."""
    rng = np.random.default_rng(seed)
    edges = {0, 1, N - 1, N - 2, min(N - 1, BM - 1), min(N - 1, BM), N // 2}
    for t in range(1, 4):
        edges.add(min(N - 1, t * BM - 1))
        edges.add(min(N - 1, t * BM))
    rest = rng.integers(0, N, size=max(0, count - len(edges)))
    return np.unique(np.concatenate([np.array(sorted(edges)), rest]).clip(0, N - 1))
