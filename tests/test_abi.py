"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and its planner / argument validation behave (no GPU needed)."""
import ctypes
import os
import re

import pytest

import exact_attention_21_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_status_str"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"libfa.so does not export {n}"


def test_status_strings():
    for s in range(11):
        assert fa.fa_status_str(s) and fa.fa_status_str(s) != "unknown status"
    assert fa.fa_status_str(99) == "unknown status"


@pytest.mark.parametrize("N,d,causal", [(256, 64, 0), (4096, 128, 0), (8192, 128, 1), (1, 128, 1), (1000, 64, 1)])
def test_forward_plan(N, d, causal):
    p = fa.fa_fwd_plan(4, 32, N, d, causal, fa.FA_BF16)
    assert p.threads == 256 and p.block_m in (128, 256) and p.block_n in (32, 64, 128)
    assert p.grid == -(-N // p.block_m) * 4 * 32
    assert p.lds_bytes <= 160 * 1024
    assert p.xcd_grouped == 1
    assert fa.fa_fwd_plan(1, 2, N, d, causal, fa.FA_F16).xcd_grouped == 0


def test_backward_plan_and_workspace():
    p = fa.fa_bwd_plan(2, 16, 4096, 128, 1, fa.FA_BF16)
    assert p.grid == (4096 // p.block_n) * 32
    assert p.lds_bytes <= 160 * 1024
    ws = fa.fa_bwd_workspace_size(2, 16, 4096, 128)
    assert ws >= 2 * (2 * 16 * 4096 * 4)
    assert fa.fa_bwd_workspace_size(0, 16, 4096, 128) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 96) == 0


@pytest.mark.parametrize("args,status", [
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(d=96), 3), (dict(d=32), 3),
    (dict(dtype=2), 4), (dict(causal=2), 9),
])
def test_plan_rejects_bad_arguments(args, status):
    kw = dict(B=1, H=1, N=16, d=64, causal=0, dtype=0)
    kw.update(args)
    plan = fa.fa_plan_t()
    rc = fa.lib().fa_fwd_plan(kw["B"], kw["H"], kw["N"], kw["d"], kw["causal"], kw["dtype"], ctypes.byref(plan))
    assert rc == status
    rc = fa.lib().fa_bwd_plan(kw["B"], kw["H"], kw["N"], kw["d"], kw["causal"], kw["dtype"], ctypes.byref(plan))
    assert rc == status


def _fwd_raw(ptr=16, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dtype=0):
    p = ctypes.c_void_p(ptr) if ptr else None
    return fa.lib().fa_fwd(p, p, p, p, p, B, H, N, d, scale, causal, dtype, None)


def test_forward_validation_order_without_gpu():
    assert _fwd_raw(ptr=0) == 1                     # null
    assert _fwd_raw(N=0) == 2                       # shape
    assert _fwd_raw(d=80) == 3                      # head dim
    assert _fwd_raw(dtype=7) == 4                   # dtype
    assert _fwd_raw(scale=float("nan")) == 9       # scale must be finite
    assert _fwd_raw(scale=float("inf")) == 9
    assert _fwd_raw(scale=float("-inf")) == 9
    assert _fwd_raw(ptr=24) == 5                    # misaligned
    # zero and negative scales are valid arguments: they pass to the later checks
    assert _fwd_raw(ptr=24, scale=0.0) == 5
    assert _fwd_raw(ptr=24, scale=-1.0) == 5
    # valid arguments: the device gate is the only thing left
    import torch
    if not torch.cuda.is_available():
        assert _fwd_raw(ptr=64) == 7


def test_backward_validation_without_gpu():
    lib = fa.lib()
    p = ctypes.c_void_p(64)
    args = [p] * 9 + [1, 1, 16, 64, 0.125, 0, 0]
    need = fa.fa_bwd_workspace_size(1, 1, 16, 64)
    assert lib.fa_bwd(*args, None, need, None) == 1
    assert lib.fa_bwd(*args, p, need - 1, None) == 6
    assert lib.fa_bwd(*([p] * 9 + [1, 1, 16, 128, float("nan"), 0, 0]), p, 10 ** 9, None) == 9
    # a negative scale is valid: the call gets as far as the workspace check
    assert lib.fa_bwd(*([p] * 9 + [1, 1, 16, 128, -0.5, 0, 0]), p, 1, None) == 6
    assert lib.fa_bwd(*([ctypes.c_void_p(72)] + [p] * 8 + [1, 1, 16, 64, 0.125, 0, 0]), p, need, None) == 5


def test_product_path_does_not_import_the_oracle():
    src_dir = os.path.join(ROOT, "exact_attention_21_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "liboracle" not in text and "oracle.c" not in text, f


def _align256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("B,H,Nk,d,partials", [
    (32, 32, 16384, 128, 4),   # 1024 heads: one workgroup (4 waves, 4 partials) per head
    (1, 4, 40000, 128, 160),   # 4 heads: 40 workgroups per head, chunks of >= 256 keys
    (1, 2, 5, 64, 4),          # fewer keys than one tile: a single workgroup per head
])
def test_decode_split_workspace(B, H, Nk, d, partials):
    # one query row: fp32 partial output rows and LSEs, one per wave of the decode kernel
    rows = B * H * partials
    assert fa.fa_fwd_splitkv_workspace_size(B, H, 1, Nk, d) == _align256(rows * d * 4) + _align256(rows * 4)


def test_split_workspace_covers_every_chunk():
    for B, H, Nq, Nk, d in [(2, 4, 7, 2048, 128), (1, 2, 300, 9000, 64), (8, 16, 128, 65536, 128)]:
        ws = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d)
        assert ws >= B * H * Nq * d * 4 + B * H * Nq * 4  # at least one chunk
        assert ws % 256 == 0
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 16, 96) == 0  # unsupported head size


def test_noalloc_limits_without_gpu():
    lib = fa.lib()
    p = ctypes.c_void_p(64)
    rows = fa.FA_BWD_NOALLOC_MAX_ROWS
    assert re.search(r"#define FA_BWD_NOALLOC_MAX_ROWS %d\b" % rows, open(HEADER).read())
    args = lambda B, H, N, d=64: [p] * 9 + [B, H, N, d, ctypes.c_float(0.125), 0, 0, None]
    assert lib.fa_bwd_noalloc(*([None] + [p] * 8 + args(1, 1, 16)[9:])) == 1   # null
    assert lib.fa_bwd_noalloc(*args(1, 1, 16, 80)) == 3                          # head dim
    assert lib.fa_bwd_noalloc(*args(1, 1, rows + 1)) == 10                       # beyond the scratch
    assert lib.fa_bwd_noalloc(*args(4, 32, 32768 + 1)) == 10
    # at the limit the argument checks pass: the device gate is what remains
    import torch
    if not torch.cuda.is_available():
        assert lib.fa_bwd_noalloc(*args(4, 32, rows // 128)) == 7
        assert lib.fa_bwd_noalloc(*args(1, 1, rows)) == 7


def test_head_size_limit_without_gpu():
    # one head is addressed through a 32-bit buffer resource: N * d * 2 < 2^32
    for d, nmax in ((128, (1 << 32) // 256 - 1), (64, (1 << 32) // 128 - 1)):
        assert fa.fa_fwd_plan(1, 1, nmax, d, 0, fa.FA_BF16).grid > 0
        with pytest.raises(fa.FaError) as e:
            fa.fa_fwd_plan(1, 1, nmax + 1, d, 0, fa.FA_BF16)
        assert e.value.status == 2
        assert fa.fa_bwd_workspace_size(1, 1, nmax, d) > 0
        assert fa.fa_bwd_workspace_size(1, 1, nmax + 1, d) == 0



def test_dropout_probability_range_without_gpu():
    # p is checked before it is rounded to 8 bits: a value past the range of
    # the rounding (1e30, inf) is rejected, not wrapped to a small threshold
    lib = fa.lib()
    p = ctypes.c_void_p(64)

    def call(prob):
        return lib.fa_fwd_dropout(p, p, p, p, p, None, None, 1, 1, 16, 16, 64, ctypes.c_float(0.125), 0,
                                  ctypes.c_float(prob), ctypes.c_uint64(1), ctypes.c_uint32(0), 0, None)

    for bad in (1e30, float("inf"), float("nan"), -1e-3, 1.0, 255.5 / 256, 3e38):
        assert call(bad) == 9, bad
    import torch
    if not torch.cuda.is_available():
        for ok in (0.0, -0.0, 0.1, 255.4 / 256):
            assert call(ok) == 7, ok
