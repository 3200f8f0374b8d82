"""Debug mode of the C ABI on the host: with FA_DEBUG (or FLASH_ATTENTION_DEBUG,
the name the FA1-vs-FA2 page's troubleshooting section uses) set to anything but "0",
each computing entry point prints its launch plan to stderr once its
arguments have passed the host checks, before the device check, so the plan
shows on a host without a usable GPU too; unset or "0" prints nothing.  (The
scan of non-finite values after the launches needs a GPU: see
test_debug_mode_gpu.)"""
import ctypes

import pytest

import exact_attention_21_amd as fa


@pytest.fixture
def no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("the fake device pointers of this test must not reach a GPU")


def _p(x=64):
    return ctypes.c_void_p(x)


def _calls(lib):
    p = _p()
    need = fa.fa_bwd_workspace_size(1, 2, 300, 128)
    split = fa.fa_fwd_splitkv_workspace_size(2, 4, 1, 5000, 128)
    return {
        "fa_fwd": lambda: lib.fa_fwd(p, p, p, p, p, 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, None),
        "fa_fwd_padded": lambda: lib.fa_fwd_padded(p, p, p, p, p, p, p, 3, 2, 130, 300, 64, 0.125, 0,
                                                   fa.FA_F16, None),
        "fa_fwd_splitkv": lambda: lib.fa_fwd_splitkv(p, p, p, p, p, None, None, 2, 4, 1, 5000, 128, 0.088,
                                                     0, fa.FA_BF16, p, split, None),
        "fa_bwd": lambda: lib.fa_bwd(*([p] * 9), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, p, need, None),
        "fa_bwd_dq": lambda: lib.fa_bwd_dq(*([p] * 5), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, p, need, None),
        "fa_bwd_dkdv": lambda: lib.fa_bwd_dkdv(*([p] * 6), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, p, need,
                                               None),
        "fa_bwd_preprocess": lambda: lib.fa_bwd_preprocess(p, p, p, 1, 2, 300, 128, fa.FA_BF16, p, need,
                                                           None),
    }


def test_plan_lines(no_gpu, monkeypatch, capfd):
    lib = fa.lib()
    monkeypatch.setenv("FA_DEBUG", "1")
    for name, call in _calls(lib).items():
        assert call() == 7, name  # FA_ERR_DEVICE: no GPU here
        err = capfd.readouterr().err
        lines = [l for l in err.splitlines() if l.startswith("[FA_DEBUG] ")]
        assert len(lines) == 1 and lines[0].startswith(f"[FA_DEBUG] {name}: "), (name, err)
    # the planner's figures appear in the line
    lib.fa_fwd(_p(), _p(), _p(), _p(), _p(), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, None)
    err = capfd.readouterr().err
    plan = fa.fa_fwd_plan(1, 2, 300, 128, 1, fa.FA_BF16)
    assert "Nq=300 Nk=300 d=128 dtype=bf16 causal=1" in err
    assert f"grid {plan.grid} x {plan.threads} threads" in err
    assert f"{plan.lds_bytes} bytes of LDS" in err
    lib.fa_bwd(*([_p()] * 9), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, _p(),
               fa.fa_bwd_workspace_size(1, 2, 300, 128), None)
    err = capfd.readouterr().err
    assert "dQ grid 6 (128 query rows per workgroup)" in err and "dK/dV grid 6 (128 keys" in err
    lib.fa_fwd_splitkv(*([_p()] * 5), None, None, 2, 4, 1, 5000, 128, 0.088, 0, fa.FA_BF16, _p(),
                       fa.fa_fwd_splitkv_workspace_size(2, 4, 1, 5000, 128), None)
    assert "decode (one partial per wave)" in capfd.readouterr().err
    lib.fa_fwd_splitkv(*([_p()] * 5), None, None, 2, 4, 300, 5000, 128, 0.088, 0, fa.FA_BF16, _p(),
                       fa.fa_fwd_splitkv_workspace_size(2, 4, 300, 5000, 128), None)
    assert "split forward" in capfd.readouterr().err


def test_the_pages_variable_name_also_turns_it_on(no_gpu, monkeypatch, capfd):
    monkeypatch.delenv("FA_DEBUG", raising=False)
    monkeypatch.setenv("FLASH_ATTENTION_DEBUG", "1")
    assert _calls(fa.lib())["fa_fwd"]() == 7
    assert "[FA_DEBUG] fa_fwd: " in capfd.readouterr().err


@pytest.mark.parametrize("value", [None, "0", ""])
def test_off_prints_nothing(no_gpu, monkeypatch, capfd, value):
    monkeypatch.delenv("FLASH_ATTENTION_DEBUG", raising=False)
    if value is None:
        monkeypatch.delenv("FA_DEBUG", raising=False)
    else:
        monkeypatch.setenv("FA_DEBUG", value)
    for name, call in _calls(fa.lib()).items():
        assert call() == 7, name
    assert "[FA_DEBUG]" not in capfd.readouterr().err


def test_rejected_arguments_print_no_plan(monkeypatch, capfd):
    # a call the host checks reject returns its status before any plan line
    monkeypatch.setenv("FA_DEBUG", "1")
    lib = fa.lib()
    p = _p()
    assert lib.fa_fwd(p, p, p, p, p, 1, 2, 0, 128, 0.088, 1, fa.FA_BF16, None) == 2
    assert lib.fa_fwd(_p(24), p, p, p, p, 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, None) == 5
    assert lib.fa_bwd(*([p] * 9), 1, 2, 300, 128, 0.088, 1, fa.FA_BF16, p, 1, None) == 6
    assert "[FA_DEBUG]" not in capfd.readouterr().err
