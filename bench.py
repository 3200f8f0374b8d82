#!/usr/bin/env python3
"""Attention throughput on one MI355X: fused forward + recompute backward.

One step = one pass of the whole hot path over one batch: fa_fwd (O, LSE) then
the backward's two passes as fa_bwd runs them (the dQ pass, which also forms
D = rowsum(dO*O), then the dK/dV pass) on the causal workload B=4, H=32, N=8192,
d=128, bf16, with Q, K, V, dO i.i.d. N(0,1) from a fixed seed, all resident in
HBM before timing starts.

FLOP convention: 4*B*H*N^2*d for the forward, halved when causal; the backward
counts 2.5x the forward.  `value` is (forward + backward FLOP) / step time.

Per-kernel figures are measured live with HIP events recorded on the stream the
kernels run on (mean, median and minimum over the timed steps; FLOP rates as
executed work and as the method's share of the work).  The CPU baseline times
the fp64 oracle on bounded samples on the host's cores: one head of this
workload (the forward over 2048 rows spread over it and the backward of the
whole head), and per configuration of the family a forward row sample (and the
4096 backward configuration's backward of one head).

After the headline step the other configurations of the workload family (the
sequence-length sweep N = 1k..32k at 32768 tokens per batch, the d=64 variant,
the non-causal 4096 forward, the 4096 backward, a variable-length causal batch
and a cross-attention shape through the padded entry points) are timed too and
reported under "sweep" (skip with --no-sweep; --sweep-only runs just those).

Extra modes: --copy-ref MiB runs a plain device copy of known size (the
reference for scaling hardware byte counters); --gemm-ref times the vendor
library's bf16 matrix product (torch.matmul) on large square shapes, the
dense-bf16 rate this GPU sustains under its power limit; --fwd-only times the
forward alone.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
SWEEP_WARMUP_S = 0.5  # seconds of untimed work per sweep configuration before its timed steps
WORKLOAD = dict(name="c3_fwd_bwd_causal_n8192_d128_bf16", B=4, H=32, N=8192, d=128, dtype="bf16",
                causal=True)


# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# workload (FETCH_SIZE scaled x2.0, WRITE_SIZE x1.0 by a plain 1 GiB copy; see
# profiles/fwd_bwd_causal_n8192_d128_bf16_hbm_traffic.md).  Valid only for the
# kernel code they were taken on: the hash of the kernel sources (comments and
# blank lines removed, so that a comment edit keeps the figures) must match.
MEASURED_TRAFFIC = {
    "source_sha256_16": "8cf321c434fc002b",
    "bytes": {"fwd_kernel": 3.559e9, "bwd_dq_kernel": 2.392e9,
              "bwd_dkdv_kernel": 1.910e9},
}
KERNEL_SOURCES = ["exact_attention_21_amd/csrc/fa_bwd.hip", "exact_attention_21_amd/csrc/fa_bwd_common.h",
                  "exact_attention_21_amd/csrc/fa_bwd_dkdv.h", "exact_attention_21_amd/csrc/fa_bwd_dkdv.hip",
                  "exact_attention_21_amd/csrc/fa_bwd_dkdv_ilp.hip", "exact_attention_21_amd/csrc/fa_fwd.hip",
                  "exact_attention_21_amd/csrc/fa_device.h", "exact_attention_21_amd/csrc/fa_kernels.h",
                  "exact_attention_21_amd/build.py"]


def _code_only(text: str) -> str:
    """C/C++ source without comments, trailing blanks and empty lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        h.update((_code_only(text) if f.endswith((".hip", ".h")) else text).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    if kernel_source_hash() != MEASURED_TRAFFIC["source_sha256_16"]:
        return None  # kernels changed since the counters were taken
    return MEASURED_TRAFFIC["bytes"].get(kernel)


def nominal_flop(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
    return f, 2.5 * f


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_inputs(w, device):
    import numpy as np
    import torch
    import fa_inputs
    seed = fa_inputs.CONFIGS["c3_bwd_causal_n8192_d128_bf16"]["seed"]
    bits = fa_inputs.qkv_bits(w["B"], w["H"], w["N"], w["d"], w["dtype"], seed, with_dout=True)
    tdt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float16
    tens = [torch.from_numpy(b.view(np.int16)).view(tdt).to(device) for b in bits]
    return bits, tens


def cpu_info():
    """CPU model, logical CPUs and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def _timed(fn, reps):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return ts


def _stats(ts, flop):
    med = statistics.median(ts)
    return {"median_s": med, "min_s": min(ts), "mean_s": sum(ts) / len(ts), "runs": len(ts),
            "flop": flop, "tflops_median": flop / med / 1e12, "tflops_best": flop / min(ts) / 1e12}


def cpu_baseline(bits, w, max_bwd_n, fwd_rows=2048, reps=3):
    """The fp64 oracle, as it is, on bounded samples of the workloads, on the
    host's cores (its default thread count).

    Headline (the bench workload, one head of it): the forward over `fwd_rows`
    rows spread evenly over head (0,0) plus the backward of that whole head;
    value = their nominal FLOP / time (4 d FLOP per visible (query, key) pair
    forward, 2.5x that backward).  Per configuration of the family: the
    forward over the same kind of row sample of head (0,0) (median, minimum and
    mean of `reps` runs), and for the backward configuration also the
    backward of head (0,0).  Inputs are the seeded draws of each workload."""
    import numpy as np
    import fa_inputs
    import oracle
    threads = oracle.default_threads()
    info = cpu_info()

    def fwd_sample(q, k, v, N, d, causal):
        rows = np.unique(np.linspace(0, N - 1, min(N, fwd_rows)).round().astype(np.int64))
        vis = (rows + 1) if causal else np.full(len(rows), N)
        return rows, 4.0 * d * float(vis.sum())

    # headline: the bench workload's head (0,0)
    N, d, causal = w["N"], w["d"], w["causal"]
    scale = float(np.float32(1 / math.sqrt(d)))
    sub = [fa_inputs.widen(x[0:1, 0:1], w["dtype"]) for x in bits]
    rows, f_rows = fwd_sample(*sub[:3], N, d, causal)
    t_fwd = _timed(lambda: oracle.fwd_rows(*sub[:3], scale, causal, rows, threads=threads), reps)
    flop, secs = f_rows, statistics.median(t_fwd)
    sample = f"head (0,0) of {w['name']}: forward over {len(rows)} rows spread over the head ({secs:.2f} s median of {reps})"
    head = {"fwd": _stats(t_fwd, f_rows)}
    if N <= max_bwd_n:
        _, f_bwd = nominal_flop(1, 1, N, d, causal)
        t_bwd = _timed(lambda: oracle.bwd_heads(*sub, scale, causal, [0], threads=threads), 1)
        head["bwd"] = _stats(t_bwd, f_bwd)
        flop += f_bwd
        secs += t_bwd[0]
        sample += f" + backward of the whole head ({t_bwd[0]:.1f} s)"
    per = {w["name"]: head}
    # the other configurations of the family (forward samples; the backward
    # configuration also with its backward)
    for name, c in fa_inputs.CONFIGS.items():
        if name.startswith("c3_") or not name.startswith(("c1_", "c2_", "c4_", "c5_")):
            continue
        B, H, Nc, dc, cc = c["B"], c["H"], c["N"], c["d"], c["causal"]
        xb = fa_inputs.qkv_bits(1, 1, Nc, dc, c["dtype"], c["seed"], with_dout=c.get("bwd", False))
        xs = [fa_inputs.widen(x, c["dtype"]) for x in xb]
        sc = float(np.float32(1 / math.sqrt(dc)))
        r, f = fwd_sample(*xs[:3], Nc, dc, cc)
        entry = {"fwd": _stats(_timed(lambda: oracle.fwd_rows(*xs[:3], sc, cc, r, threads=threads), reps), f),
                 "rows": int(len(r)), "N": Nc, "d": dc, "causal": cc}
        if c.get("bwd"):
            _, fb = nominal_flop(1, 1, Nc, dc, cc)
            entry["bwd"] = _stats(_timed(lambda: oracle.bwd_heads(*xs, sc, cc, [0], threads=threads), 1), fb)
        per[name] = entry
        log(f"[bench] cpu baseline {name}: fwd {entry['fwd']['tflops_median'] * 1e3:.2f} GFLOP/s"
            + (f", bwd {entry['bwd']['tflops_median'] * 1e3:.2f} GFLOP/s" if "bwd" in entry else ""))
    return {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample + f"; nominal FLOP {flop:.3e} in {secs:.1f} s",
            "threads": threads, **info, "per_config": per}


def visible_pairs(Lq: int, Lk: int, causal: bool) -> int:
    """(query, key) pairs of one head with valid lengths Lq, Lk (causal aligned to the
    last query and key): the work unit of the padded FLOP count."""
    if not causal:
        return Lq * Lk
    # row i sees min(Lk, max(0, i + Lk - Lq + 1)) keys
    total = 0
    for i in range(Lq):
        total += min(Lk, max(0, i + Lk - Lq + 1))
    return total


def decode_timing(fa, c, q, k, v, steps, warmup):
    """Decode-shaped forward (few queries, long K/V): fa_fwd_splitkv against the
    unsplit fa_fwd_padded on the same inputs.  The bound is HBM: bytes = Q, K, V
    read and O, LSE written."""
    import torch
    stream = torch.cuda.current_stream()
    B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
    Nk = c["Nk"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, Nk, d), dtype=torch.uint8, device=q.device)
    scale = 1 / math.sqrt(d)

    def timed(fn):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(warmup + steps):
            e = ev[i - warmup] if i >= warmup else None
            if e:
                e[0].record(stream)
            fn()
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        return sum(e[0].elapsed_time(e[1]) for e in ev) / steps

    split_ms = timed(lambda: fa.fa_fwd_splitkv(q, k, v, o, lse, None, None, scale, causal, ws, stream))
    plain_ms = timed(lambda: fa.fa_fwd_padded(q, k, v, o, lse, None, None, scale, causal, stream))
    nbytes = 2.0 * B * H * d * (2 * N + 2 * Nk) + 4.0 * B * H * N
    flop = 4.0 * d * B * H * visible_pairs(N, Nk, causal)
    r = {"B": B, "H": H, "N": N, "Nk": Nk, "d": d, "dtype": c["dtype"], "causal": causal,
         "fwd_ms": split_ms, "fwd_tflops": flop / (split_ms * 1e-3) / 1e12,
         "hbm_bytes": nbytes, "hbm_gbps": nbytes / (split_ms * 1e-3) / 1e9,
         "hbm_frac_of_8tbps": nbytes / (split_ms * 1e-3) / 8e12, "unsplit_fwd_ms": plain_ms}
    log(f"[bench] sweep {c.get('name', '')}decode B={B} H={H} Nq={N} Nk={Nk}: split-KV {split_ms:.3f} ms "
        f"({r['hbm_gbps']:.0f} GB/s, {100 * r['hbm_frac_of_8tbps']:.0f} % of 8 TB/s); unsplit {plain_ms:.3f} ms")
    return r


def sweep(fa, device, steps, warmup, only=None):
    """Forward and backward timings over the other configurations of the workload
    family (sequence-length sweep at 32768 tokens per batch, the d=64 variant, the
    non-causal 4096 forward, the 4096 backward, a variable-length causal batch, a
    cross-attention shape, a dropout workload and a decode shape timed through the
    split-over-keys forward).  Inputs are seeded N(0,1) draws made on the device
    (timing only; parity is the tests' job).  Padded workloads count FLOP over the
    visible pairs only: 4 d per pair forward, 2.5x that backward."""
    import torch
    import fa_inputs
    stream = torch.cuda.current_stream()
    res = {}
    for name, c in fa_inputs.CONFIGS.items():
        if name.startswith("c1_") or name.startswith("c3_"):
            continue  # c1 is the oracle-sized case; c3 is the headline above
        if only and only not in name:
            continue
        B, H, N, d, causal = c["B"], c["H"], c["N"], c["d"], c["causal"]
        Nk = c.get("Nk", N)
        drop = c.get("dropout", 0.0)
        padded = "len_lo" in c or Nk != N or drop > 0
        tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float16
        gen = torch.Generator(device=device).manual_seed(c["seed"])
        draw = lambda n: torch.randn((B, H, n, d), generator=gen, device=device,
                                     dtype=torch.float32).to(tdt)
        q, do = draw(N), draw(N)
        k, v = draw(Nk), draw(Nk)
        if c.get("splitkv"):
            res[name] = decode_timing(fa, c, q, k, v, steps, warmup)
            del q, k, v, do
            continue
        lens = None
        if "len_lo" in c:
            lens = fa_inputs.seq_lengths(B, c["len_lo"], c["len_hi"], c["seed"])
        lq = lk = None if lens is None else torch.from_numpy(lens).to(device)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=device)
        scale = 1 / math.sqrt(d)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        # untimed warm-up of at least `warmup` steps and SWEEP_WARMUP_S seconds:
        # the power-limited clock takes milliseconds to settle after the
        # previous configuration's load
        t_warm, i = time.perf_counter(), 0
        while i < warmup or time.perf_counter() - t_warm < SWEEP_WARMUP_S:
            if drop > 0:
                fa.fa_fwd_dropout(q, k, v, o, lse, lq, lk, scale, causal, drop, c["seed"], i, stream)
                fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, lq, lk, scale, causal, drop, c["seed"], i,
                                  ws, stream)
            elif padded:
                fa.fa_fwd_padded(q, k, v, o, lse, lq, lk, scale, causal, stream)
                fa.fa_bwd_padded(q, k, v, o, do, lse, dq, dk, dv, lq, lk, scale, causal, ws, stream)
            else:
                fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
                fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, ws, stream)
            i += 1
            if i % max(1, warmup) == 0:
                torch.cuda.synchronize()
        for i in range(warmup, warmup + steps):
            e = ev[i - warmup]
            e[0].record(stream)
            if drop > 0:
                fa.fa_fwd_dropout(q, k, v, o, lse, lq, lk, scale, causal, drop, c["seed"], i, stream)
            elif padded:
                fa.fa_fwd_padded(q, k, v, o, lse, lq, lk, scale, causal, stream)
            else:
                fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
            e[1].record(stream)
            if drop > 0:
                fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, lq, lk, scale, causal, drop, c["seed"], i,
                                  ws, stream)
            elif padded:
                fa.fa_bwd_padded(q, k, v, o, do, lse, dq, dk, dv, lq, lk, scale, causal, ws, stream)
            else:
                fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, ws, stream)
            e[2].record(stream)
        torch.cuda.synchronize()
        if padded:
            pairs = sum(visible_pairs(int(lens[b]) if lens is not None else N,
                                      int(lens[b]) if lens is not None else Nk, causal)
                        for b in range(B)) * H
            f_fwd = 4.0 * d * pairs
            f_bwd = 2.5 * f_fwd
        else:
            f_fwd, f_bwd = nominal_flop(B, H, N, d, causal)
        fts = [e[0].elapsed_time(e[1]) for e in ev]
        bts = [e[1].elapsed_time(e[2]) for e in ev]
        fms, bms = sum(fts) / steps, sum(bts) / steps
        res[name] = {"B": B, "H": H, "N": N, "Nk": Nk, "d": d, "dtype": c["dtype"], "causal": causal,
                     "dropout": drop,
                     "lengths": None if lens is None else [int(x) for x in lens],
                     "fwd_ms": fms, "fwd_tflops": f_fwd / (fms * 1e-3) / 1e12,
                     "fwd_ms_median": statistics.median(fts), "fwd_ms_min": min(fts),
                     "bwd_ms": bms, "bwd_tflops": f_bwd / (bms * 1e-3) / 1e12,
                     "bwd_ms_median": statistics.median(bts), "bwd_ms_min": min(bts)}
        log(f"[bench] sweep {name}: fwd {fms:.3f} ms ({res[name]['fwd_tflops']:.0f} TFLOP/s)  "
            f"bwd {bms:.3f} ms ({res[name]['bwd_tflops']:.0f} TFLOP/s nominal)")
        if not padded:
            # the forward alone, back to back: in the loop above each forward
            # follows a backward, which leaves other data in the caches
            evr = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for i in range(warmup + steps):
                e = evr[i - warmup] if i >= warmup else None
                if e:
                    e[0].record(stream)
                fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
                if e:
                    e[1].record(stream)
            torch.cuda.synchronize()
            rms = sum(e[0].elapsed_time(e[1]) for e in evr) / steps
            res[name]["fwd_repeat_ms"] = rms
            res[name]["fwd_repeat_tflops"] = f_fwd / (rms * 1e-3) / 1e12
            log(f"[bench] sweep {name}: forward back to back {rms:.3f} ms "
                f"({res[name]['fwd_repeat_tflops']:.0f} TFLOP/s)")
        if not padded and not causal:
            # a grid of equal workgroups that fills the resident slots 1.33
            # times (C2): the split-over-keys entry point, whose plan fills
            # whole rounds, on the same inputs (back to back, like the
            # fwd_repeat figure it compares with)
            wss = torch.empty(fa.fa_fwd_splitkv_workspace_size(B, H, N, N, d), dtype=torch.uint8, device=device)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for i in range(warmup + steps):
                e = evs[i - warmup] if i >= warmup else None
                if e:
                    e[0].record(stream)
                fa.fa_fwd_splitkv(q, k, v, o, lse, None, None, scale, causal, wss, stream)
                if e:
                    e[1].record(stream)
            torch.cuda.synchronize()
            sms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
            res[name]["splitkv_fwd_ms"] = sms
            res[name]["splitkv_fwd_tflops"] = f_fwd / (sms * 1e-3) / 1e12
            log(f"[bench] sweep {name} through fa_fwd_splitkv: fwd {sms:.3f} ms "
                f"({res[name]['splitkv_fwd_tflops']:.0f} TFLOP/s)")
            del wss
        del q, k, v, do, o, lse, dq, dk, dv, ws
    return res


def copy_ref(mib, device):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_ref_bytes_per_launch": n, "launches": 5}), flush=True)


def gemm_ref(device):
    """bf16 C = A B through torch.matmul (2-D contiguous operands: the vendor
    GEMM library) at n = 4096, 8192, 16384, ~20 TFLOP per shape after warm-up."""
    import torch
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device=device, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=device, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=device, dtype=torch.bfloat16)
        for _ in range(5):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        reps = max(5, int(2e13 / (2.0 * n ** 3)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        print(json.dumps({"gemm_ref": f"{n}x{n}x{n} bf16", "ms_per_call": ms, "calls": reps,
                          "tflops": 2.0 * n ** 3 / (ms * 1e-3) / 1e12,
                          "frac_of_peak": 2.0 * n ** 3 / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}), flush=True)
        del a, b, c


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-bwd-max-n", type=int, default=8192,
                    help="largest N for which the CPU baseline includes the backward")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB")
    ap.add_argument("--gemm-ref", action="store_true", help="time the vendor bf16 GEMM (power-limited dense rate)")
    ap.add_argument("--fwd-only", action="store_true", help="time only the forward (diagnostics)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the other configurations' timings")
    ap.add_argument("--sweep-only", action="store_true", help="time only the other configurations")
    ap.add_argument("--only", default=None, help="with --sweep-only: configurations whose name contains this")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the kernels would shard by head or batch with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_21_amd as fa

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.copy_ref:
        copy_ref(args.copy_ref, device)
        return
    if args.gemm_ref:
        gemm_ref(device)
        return

    if args.sweep_only:
        print(json.dumps({"sweep": sweep(fa, device, args.steps, args.warmup, args.only)}), flush=True)
        return

    w = WORKLOAD
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    log(f"[bench] generating inputs {w['name']}")
    bits, (q, k, v, do) = make_inputs(w, device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=device)
    scale = 1 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    # one step: forward, then the backward's two passes as fa_bwd runs them
    # (the dQ pass also computes the row statistics the dK/dV pass reads);
    # events bracket each kernel on the stream it runs on
    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
        rec(1)
        if not args.fwd_only:
            fa.fa_bwd_dq_preprocess(q, k, v, o, do, lse, dq, scale, causal, ws, stream)
            rec(2)
            fa.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, causal, ws, stream)
            rec(3)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def times_ms(i, j):
        return [e[i].elapsed_time(e[j]) for e in evs]

    def avg_ms(i, j):
        t = times_ms(i, j)
        return sum(t) / len(t)

    f_fwd, f_bwd = nominal_flop(B, H, N, d, causal)
    ms_step = wall * 1e3 / args.steps
    # per kernel: event times and two FLOP counts.  Every tile product is
    # 2 B H N^2 d (halved when causal), half the nominal forward.  "executed":
    # the products the kernel runs; "method": its share of the method's work
    # (forward 2 products, backward 5: S and dP recomputed, dV, dK, dQ).  The
    # dK/dV pass runs four (S, dP, dV, dK), all method work; the dQ pass runs
    # three (S, dP, dQ) of which only dQ is not also done by the dK/dV pass.
    half = 0.5 * f_fwd
    kern = {"fwd_kernel": ((0, 1), 2 * half, 2 * half)}
    if not args.fwd_only:
        kern["bwd_dq_kernel"] = ((1, 2), 3 * half, 1 * half)
        kern["bwd_dkdv_kernel"] = ((2, 3), 4 * half, 4 * half)
    fwd_avg = avg_ms(0, 1)
    bwd_avg = avg_ms(1, 3) if not args.fwd_only else 0.0
    total_flop = f_fwd + (0 if args.fwd_only else f_bwd)
    fwd_tf = f_fwd / (fwd_avg * 1e-3) / 1e12
    bwd_tf = f_bwd / (bwd_avg * 1e-3) / 1e12 if not args.fwd_only else None
    kernels = {}
    for name, ((i, j), f_exec, f_meth) in kern.items():
        t = times_ms(i, j)
        ms = sum(t) / len(t)
        kernels[name] = {"avg_ms": ms, "median_ms": statistics.median(t), "min_ms": min(t),
                         "executed_flop": f_exec, "method_flop": f_meth,
                         "executed_tflops": f_exec / (ms * 1e-3) / 1e12,
                         "method_tflops": f_meth / (ms * 1e-3) / 1e12,
                         "method_frac_of_peak": f_meth / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        log(f"[bench] {name}: {ms:.3f} ms (median {statistics.median(t):.3f}, min {min(t):.3f}); "
            f"executed {kernels[name]['executed_tflops']:.0f} TFLOP/s, method {kernels[name]['method_tflops']:.0f}")
    log(f"[bench] fwd {fwd_avg:.3f} ms ({fwd_tf:.0f} TFLOP/s)"
        + ("" if args.fwd_only else f"  bwd {bwd_avg:.3f} ms ({bwd_tf:.0f} TFLOP/s nominal)"))

    # the roofline entry is for the longest kernel (method work = executed work there)
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"])
    dom_ms, dom_flop = kernels[dom]["avg_ms"], kernels[dom]["method_flop"]
    dom_tf = dom_flop / (dom_ms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": dom_tf, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dom_tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom),
                "avg_launch_ms": dom_ms, "algorithmic_flop_per_launch": dom_flop}

    swp = None
    if not args.no_sweep and not args.fwd_only:
        del q, k, v, do, o, lse, dq, dk, dv, ws
        swp = sweep(fa, device, max(3, args.steps // 2), 2)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(bits, w, args.cpu_bwd_max_n)

    out = {
        "metric": "attention TFLOPS and % of MI355X bf16 MFMA peak, fwd/bwd, N=1k-32k, d=128",
        "value": total_flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) Q, K, V, dO from a fixed seed (no datasets or weights)",
        "config": {"workload": w["name"] if not args.fwd_only else w["name"] + " (forward only)",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "pass": "fwd+bwd" if not args.fwd_only else "fwd",
                   "flop_per_step": total_flop},
        "fwd_ms": fwd_avg, "bwd_ms": bwd_avg if not args.fwd_only else None,
        "fwd_ms_median": statistics.median(times_ms(0, 1)), "fwd_ms_min": min(times_ms(0, 1)),
        "bwd_ms_median": statistics.median(times_ms(1, 3)) if not args.fwd_only else None,
        "bwd_ms_min": min(times_ms(1, 3)) if not args.fwd_only else None,
        "fwd_tflops": fwd_tf, "bwd_tflops": bwd_tf,
        "fwd_frac_of_peak": fwd_tf / PEAK_BF16_TFLOPS,
        "bwd_frac_of_peak": (bwd_tf / PEAK_BF16_TFLOPS) if bwd_tf else None,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": swp,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
