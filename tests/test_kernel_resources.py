"""Register budget of the gfx950 kernels, from the compiler's own report (no GPU
needed): the kernels are compiled to assembly with the library's flags and the
per-kernel metadata and loop bodies are checked.

- No kernel keeps spilled registers inside a loop: scratch reloads count in
  vmcnt like the K/V (or Q/dO) tile loads, so a reload would wait for the
  next tile and undo the prefetch.  The only spills allowed at all are the
  forward's with dropout at d = 128 (two registers, outside the loop).
- The occupancy each kernel is built for is met: forward d = 128 <= 168 VGPRs
  (3 waves per SIMD), forward d = 64 and the d = 64 dQ pass <= 128 (4), the
  d = 128 backward passes <= 256 (2)."""
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_21_amd", "csrc")


def _build_module():
    spec = importlib.util.spec_from_file_location("fa_build", os.path.join(ROOT, "exact_attention_21_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    b = _build_module()
    out = {}
    for src in ("fa_fwd.hip", "fa_bwd.hip", "fa_bwd_dkdv.hip", "fa_bwd_dkdv_ilp.hip"):
        dst = tmp_path_factory.mktemp("asm") / (src + ".s")
        cmd = [b.hipcc(), *b.source_flags(src), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = dst.read_text()
    return out


def kernels(text):
    """name -> (metadata dict, body lines) for every kernel in the assembly."""
    meta = {}
    for blk in text[text.index("amdhsa.kernels:"):].split("\n  - ")[1:]:
        fields = dict(re.findall(r"^\s+\.([a-z_]+):\s+(\S+)$", blk, re.M))
        if "name" in fields:  # (the list that follows, amdhsa.version, has no names)
            meta[fields["name"]] = fields
    res = {}
    for name, fields in meta.items():
        start = re.search(r"^" + re.escape(name) + r":", text, re.M).start()
        end = text.index("s_endpgm", start)
        res[name] = (fields, text[start:end].splitlines())
    return res


def in_loop_scratch(body):
    """Scratch instructions between a loop header and its last back-branch."""
    hits = []
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\w+):.*Loop Header", line)
        if not m:
            continue
        back = [j for j in range(i + 1, len(body)) if re.search(r"s_c?branch\w*\s+" + re.escape(m.group(1)) + r"\b", body[j])]
        if back:
            hits += [body[j].strip() for j in range(i, back[-1] + 1) if "scratch_" in body[j]]
    return hits


def test_no_spills_in_loops(assembly):
    for src, text in assembly.items():
        for name, (fields, body) in kernels(text).items():
            assert not in_loop_scratch(body), f"{src}: {name} reloads spilled registers inside a loop"
            spills = int(fields.get("vgpr_spill_count", 0))
            forward_dropout_d128 = "fwd_kernel" in name and re.search(r"ELi128ELi1ELb[01]ELb1ELb0E", name)
            assert spills == 0 or (forward_dropout_d128 and spills <= 4), f"{src}: {name} spills {spills} VGPRs"


def test_occupancy_budgets(assembly):
    def vgprs(fields):
        return int(fields["vgpr_count"]) + int(fields.get("agpr_count", 0))
    seen = set()
    for src, text in assembly.items():
        for name, (fields, _) in kernels(text).items():
            fwd = re.search(r"fwd_kernel\w*?ELi(64|128)ELi(1|2)E", name)
            dq64 = re.search(r"bwd_dq_kernel\w*?ELi64ELb[01]ELb0E", name)  # d = 64, no dropout
            bwd = re.search(r"bwd_(dq|dkdv)_kernel\w*?ELi(64|128)E", name)
            if fwd and fwd.group(2) == "1":
                limit = 168 if fwd.group(1) == "128" else 128
                assert vgprs(fields) <= limit, (name, vgprs(fields))
                seen.add("fwd" + fwd.group(1))
            if dq64:
                assert vgprs(fields) <= 128, (name, vgprs(fields))
                seen.add("dq64")
            if bwd:
                assert vgprs(fields) <= 256, (name, vgprs(fields))
                seen.add("bwd")
    assert {"fwd128", "fwd64", "dq64", "bwd"} <= seen
