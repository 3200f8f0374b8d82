"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic: it only draws i.i.d. standard normal
samples from a fixed seed, rounds them to the 16-bit storage type, and widens
16-bit patterns back to float64 exactly.  Both the HIP path and the oracle take
their inputs from here, so the two see the very same bits.

Generator: numpy's PCG64 stream seeded by SeedSequence([seed, stream]);
standard_normal in float32, then round-to-nearest-even to fp16 or bf16.
Streams: Q=0, K=1, V=2, dO=3.
"""
from __future__ import annotations

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 0, 1, 2, 3
BASE_SEED = 0x5EED0000

_CHUNK = 1 << 24  # elements per conversion chunk (bounds temporary memory)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); finite inputs."""
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_bits(n: int, dtype: str, seed: int, stream: int) -> np.ndarray:
    """n i.i.d. N(0,1) samples rounded to `dtype` ("bf16" | "f16"), as uint16 bits."""
    if dtype not in ("bf16", "f16"):
        raise ValueError(f"dtype must be bf16 or f16, got {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if dtype == "f16":
            out[s:e] = x.astype(np.float16).view(np.uint16)  # IEEE RNE
        else:
            out[s:e] = _f32_to_bf16_bits(x)
    return out


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns to float64 (same shape)."""
    bits = np.ascontiguousarray(bits).view(np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to `dtype` bits (RNE), for hand-built inputs."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(x32.ravel()).reshape(x32.shape)
    raise ValueError(dtype)


def qkv_bits(B: int, H: int, N: int, d: int, dtype: str, seed: int, with_dout: bool = False):
    """Q, K, V (and dO) as uint16 arrays of shape [B, H, N, d]."""
    n = B * H * N * d
    streams = [STREAM_Q, STREAM_K, STREAM_V] + ([STREAM_DO] if with_dout else [])
    return tuple(normal_bits(n, dtype, seed, s).reshape(B, H, N, d) for s in streams)


def seq_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """B valid sequence lengths drawn uniformly from [lo, hi] (int32), for padded batches."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


# The workloads: shapes, dtypes, mask mode and seeds (no arithmetic).
# Padded / cross-attention workloads add Nk (keys per head; default N) and
# len_lo / len_hi (per-batch valid lengths, the same for queries and keys).
CONFIGS = {
    "c1_fwd_n256_d64_f16": dict(B=1, H=2, N=256, d=64, dtype="f16", causal=False, seed=BASE_SEED + 1, bwd=False),
    "c2_fwd_n4096_d128_bf16": dict(B=1, H=32, N=4096, d=128, dtype="bf16", causal=False, seed=BASE_SEED + 2, bwd=False),
    "c3_fwd_causal_n8192_d128_bf16": dict(B=4, H=32, N=8192, d=128, dtype="bf16", causal=True, seed=BASE_SEED + 3, bwd=False),
    "c4_causal_n1024_d128_f16": dict(B=32, H=16, N=1024, d=128, dtype="f16", causal=True, seed=BASE_SEED + 41, bwd=False),
    "c4_causal_n4096_d128_f16": dict(B=8, H=16, N=4096, d=128, dtype="f16", causal=True, seed=BASE_SEED + 42, bwd=False),
    "c4_causal_n16384_d128_f16": dict(B=2, H=16, N=16384, d=128, dtype="f16", causal=True, seed=BASE_SEED + 43, bwd=False),
    "c4_causal_n32768_d128_f16": dict(B=1, H=16, N=32768, d=128, dtype="f16", causal=True, seed=BASE_SEED + 44, bwd=False),
    "c4_causal_n16384_d64_f16": dict(B=2, H=32, N=16384, d=64, dtype="f16", causal=True, seed=BASE_SEED + 45, bwd=False),
    "c5_bwd_causal_n4096_d128_bf16": dict(B=2, H=16, N=4096, d=128, dtype="bf16", causal=True, seed=BASE_SEED + 5, bwd=True),
    "c3_bwd_causal_n8192_d128_bf16": dict(B=4, H=32, N=8192, d=128, dtype="bf16", causal=True, seed=BASE_SEED + 6, bwd=True),
    "p1_varlen_causal_b8_n4096_d128_bf16": dict(B=8, H=16, N=4096, d=128, dtype="bf16", causal=True,
                                                seed=BASE_SEED + 61, bwd=True, len_lo=512, len_hi=4096),
    "p2_cross_q4096_k16384_d128_bf16": dict(B=2, H=16, N=4096, Nk=16384, d=128, dtype="bf16",
                                            causal=False, seed=BASE_SEED + 62, bwd=True),
    "p3_dropout10_causal_n4096_d128_bf16": dict(B=8, H=16, N=4096, d=128, dtype="bf16", causal=True,
                                                seed=BASE_SEED + 63, bwd=True, dropout=0.1),
    # decoding one token per sequence against a 16k key/value cache
    "p4_decode_b32_h32_q1_k16384_d128_bf16": dict(B=32, H=32, N=1, Nk=16384, d=128, dtype="bf16",
                                                  causal=True, seed=BASE_SEED + 64, bwd=False,
                                                  splitkv=True),
}
