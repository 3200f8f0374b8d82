"""CPU tests of the Python binding's argument checks: every wrapper must reject
a host tensor (or a tensor on another device) in any position before a pointer
reaches the library, because a host pointer handed to a kernel faults the GPU
instead of raising.  The library is replaced by a recorder, and the "GPU"
tensors are host tensors that report a GPU device, so no GPU is needed."""
import ctypes

import pytest
import torch

import exact_attention_21_amd as fa


class FakeGpu:
    """A host tensor that reports being on `device` (default cuda:0)."""

    def __init__(self, t, device="cuda:0"):
        self._t = t
        self.device = torch.device(device)
        self.is_cuda = True

    @property
    def __class__(self):  # passes the binding's isinstance(x, torch.Tensor) checks
        return torch.Tensor

    def __getattr__(self, name):
        return getattr(self._t, name)


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            if name.endswith("_workspace_size"):
                return 1 << 20
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(fa, "lib", lambda: r)
    return r


B, H, N, Nk, D = 2, 2, 64, 96, 64


def t16(n=N):
    return FakeGpu(torch.zeros((B, H, n, D), dtype=torch.bfloat16))


def f32(n=N):
    return FakeGpu(torch.zeros((B, H, n), dtype=torch.float32))


def ws():
    return FakeGpu(torch.zeros(1 << 20, dtype=torch.uint8))


def lens():
    return FakeGpu(torch.full((B,), 7, dtype=torch.int32))


# wrapper name -> (argument names, builder of valid arguments, keyword args)
CASES = {
    "fa_fwd": ("q k v o lse".split(), lambda: [t16(), t16(), t16(), t16(), f32()], dict(scale=0.1, causal=True)),
    "fa_bwd": ("q k v o dout lse dq dk dv".split(),
               lambda: [t16(), t16(), t16(), t16(), t16(), f32(), t16(), t16(), t16()],
               dict(scale=0.1, causal=True, workspace=ws())),
    "fa_bwd_preprocess": ("o dout lse".split(), lambda: [t16(), t16(), f32()], dict(workspace=ws())),
    "fa_bwd_dkdv": ("q k v dout dk dv".split(),
                    lambda: [t16(), t16(), t16(), t16(), t16(), t16()],
                    dict(scale=0.1, causal=True, workspace=ws())),
    "fa_bwd_dq": ("q k v dout dq".split(),
                  lambda: [t16(), t16(), t16(), t16(), t16()], dict(scale=0.1, causal=True, workspace=ws())),
    "fa_bwd_dq_preprocess": ("q k v o dout lse dq".split(),
                             lambda: [t16(), t16(), t16(), t16(), t16(), f32(), t16()],
                             dict(scale=0.1, causal=True, workspace=ws())),
    "fa_fwd_padded": ("q k v o lse seqlens_q seqlens_k".split(),
                      lambda: [t16(), t16(Nk), t16(Nk), t16(), f32(), lens(), lens()],
                      dict(scale=0.1, causal=True)),
    "fa_bwd_padded": ("q k v o dout lse dq dk dv seqlens_q seqlens_k".split(),
                      lambda: [t16(), t16(Nk), t16(Nk), t16(), t16(), f32(), t16(), t16(Nk), t16(Nk),
                               lens(), lens()], dict(scale=0.1, causal=True, workspace=ws())),
    "fa_fwd_dropout": ("q k v o lse seqlens_q seqlens_k".split(),
                       lambda: [t16(), t16(Nk), t16(Nk), t16(), f32(), lens(), lens()],
                       dict(scale=0.1, causal=True, dropout_p=0.1, seed=1, offset=0)),
    "fa_bwd_dropout": ("q k v o dout lse dq dk dv seqlens_q seqlens_k".split(),
                       lambda: [t16(), t16(Nk), t16(Nk), t16(), t16(), f32(), t16(), t16(Nk), t16(Nk),
                                lens(), lens()],
                       dict(scale=0.1, causal=True, dropout_p=0.1, seed=1, offset=0, workspace=ws())),
    "fa_fwd_splitkv": ("q k v o lse seqlens_q seqlens_k".split(),
                       lambda: [t16(), t16(Nk), t16(Nk), t16(), f32(), lens(), lens()],
                       dict(scale=0.1, causal=True, workspace=ws())),
}


def _host(x):
    return x._t if isinstance(x, FakeGpu) else x


def _other_gpu(x):
    return FakeGpu(x._t, "cuda:1")


@pytest.mark.parametrize("name", sorted(CASES))
def test_valid_arguments_reach_the_library(rec, name):
    _, build, kw = CASES[name]
    getattr(fa, name)(*build(), stream=0, **kw)
    assert rec.calls == [name]


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("how", ["host", "other_gpu"])
def test_misplaced_tensor_is_rejected_before_the_library(rec, name, how):
    names, build, kw = CASES[name]
    positions = list(range(len(names))) + (["workspace"] if "workspace" in kw else [])
    for pos in positions:
        args, kws = build(), dict(kw)
        if pos == "workspace":
            kws["workspace"] = _host(kws["workspace"]) if how == "host" else _other_gpu(kws["workspace"])
            what = "workspace"
        else:
            args[pos] = _host(args[pos]) if how == "host" else _other_gpu(args[pos])
            what = names[pos]
        with pytest.raises(ValueError):
            getattr(fa, name)(*args, stream=0, **kws)
        assert rec.calls == [], (name, what)
