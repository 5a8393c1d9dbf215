#!/usr/bin/env python3
"""Throughput of one GPU's share of Ulysses sequence parallelism on MI355X.

One step = the whole hot path over one batch of synthetic input, with every
input already resident in HBM:
  pack Q, K, V (sequence-sharded -> head group)      ulysses_pack_multi
  pack dO                                            ulysses_pack
  causal attention forward                           attn_fwd
  causal attention backward                          attn_bwd
  unpack O (head group -> sequence-sharded)          ulysses_unpack
  unpack dQ, dK, dV                                  ulysses_unpack_multi

Metric: algorithmic causal-attention fwd+bwd TFLOP/s of the step
(14 * D * C * hq FLOP, C = number of causal (query, key) pairs), with the
roofline of the dominant call and the oracle timed on the host as a baseline.
Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3] [--no-side-legs]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for
                                             scaling rocprofv3 byte counters)
       python bench.py --gemm-calibration   (the vendor library's bf16 and fp16
                                             GEMMs, the matrix-unit rate that
                                             this box sustains)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def causal_pairs(N: int, cu) -> int:
    if cu is None:
        return N * (N + 1) // 2
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    return int((lens * (lens + 1) // 2).sum())


def oracle_threads() -> int:
    """Threads for the oracle: every core this process may run on, capped at
    16, the CPU share of one GPU on the boxes this runs on (the host itself
    may show more cores; they belong to the other GPUs' jobs)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def cpu_baseline(cfg, cu, host, budget_s: float):
    """The oracle as it stands, on a bounded sample of the same workload: fp64
    forward+backward for the last R query rows of the head group (every
    visible key), R sized to take about `budget_s` seconds. Returns the
    record and the oracle's result for those rows."""
    from oracle import attn_ref, bf16_bits_to_f64, f32_bits_to_f64, pack_ref

    dec = bf16_bits_to_f64 if cfg.dtype == "bf16" else f32_bits_to_f64
    x = {n: dec(pack_ref(host[n], cfg.group)) for n in ("q", "k", "v", "do")}
    workers = oracle_threads()
    _, start = _doc_starts(cfg.N, cu)

    def run(R):
        rows = np.arange(cfg.N - R, cfg.N)
        t = time.perf_counter()
        res = attn_ref(x["q"], x["k"], x["v"], cfg.scale, cu, do=x["do"], rows=rows, workers=workers)
        dt = time.perf_counter() - t
        pairs = int((rows - start[rows] + 1).sum())
        return dt, pairs, res

    # probe, then size R so that the measured run takes about budget_s (the
    # cost of a row is about proportional to the keys it sees)
    R = min(cfg.N, 64)
    dt, pairs, res = run(R)
    while dt < budget_s / 2 and R < cfg.N:
        R = min(cfg.N, int(R * max(1.5, min(8.0, budget_s / max(dt, 1e-3)))))
        dt, pairs, res = run(R)
    flops = 14 * cfg.D * cfg.hq * pairs
    rate = flops / dt
    full = 14 * cfg.D * cfg.hq * causal_pairs(cfg.N, cu)
    rec = {"value": rate / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "host_cores": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
           "seconds": round(dt, 2),
           "sample": f"fp64 numpy oracle, forward+backward of the last {R} query rows x {cfg.hq} q heads "
                     f"({pairs * cfg.hq:.3g} causal pairs) of workload {cfg.workload}",
           "full_step_seconds_extrapolated": round(full / rate, 1)}
    return rec, res


def parity_of_sample(outs, res, N: int) -> dict:
    """The timed step's outputs against the oracle on the sampled rows: O,
    LSE and dQ of those rows, and dK/dV of the key columns from the first
    sampled row on (only rows at or after a key see it, so the oracle's sums
    over the sampled rows are complete there). Max-abs errors, max |ref|, and
    the worst error relative to max(2e-2, one bf16 ulp of |ref|)."""
    import torch
    rows = res["rows"]
    lo = int(rows[0])
    sel = torch.from_numpy(rows).to(outs["o"].device)

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)
    pairs = {"o": (f64(outs["o"][sel]), res["o"]), "lse": (f64(outs["lse"][:, sel]), res["lse"]),
             "dq": (f64(outs["dq"][sel]), res["dq"]), "dk": (f64(outs["dk"][lo:]), res["dk"][lo:]),
             "dv": (f64(outs["dv"][lo:]), res["dv"][lo:])}
    out = {}
    for name, (got, ref) in pairs.items():
        err = np.abs(got - ref)
        bar = np.maximum(2e-2, np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7))
        out[name] = {"max_err": float(err.max()), "max_abs_ref": float(np.abs(ref).max())}
        if name != "lse":
            out[name]["worst_err_over_bar"] = round(float((err / bar).max()), 4)
    out["elements"] = f"rows {lo}..{N - 1} of O, LSE, dQ; key columns {lo}..{N - 1} of dK, dV"
    return out


# The sources of the attn_bwd call's kernels (and what they include).
BWD_SOURCES = ("attn_bwd.hip", "attn_bwd_dkdv.hip", "bwd_common.hpp", "lds_tile.hpp", "common.hpp", "internal.hpp",
               "workspace.cpp")


def source_digest() -> str:
    """sha256 over the backward's HIP sources and the C header: HBM-traffic
    figures measured with rocprofv3 counters are reported only for the
    sources they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sequence_parallelism_ulysses_amd", "csrc")
    files = [os.path.join(csrc, f) for f in BWD_SOURCES] + [os.path.join(ROOT, "include", "ulysses.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attn_bwd call from profiles/traffic.json (FETCH_SIZE +
    WRITE_SIZE of its launches, scaled by the same counters on a plain copy),
    or None when absent or measured on other sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest():
        return None
    return rec.get("bytes_per_call")


def copy_calibration() -> int:
    """A plain device-to-device copy of 1 GiB, five times."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n, "repeats": 5}}), flush=True)
    return 0


def gemm_rates(sizes=(8192, 16384), dtypes=("bf16", "fp16")) -> dict:
    """TFLOP/s of the vendor library's dense square GEMM (torch.matmul on
    contiguous operands, i.e. hipBLASLt) on this GPU: the matrix-unit rate
    that the chip sustains under a pure MFMA load, a practical ceiling to read
    the attention kernels' rate against (the published peak assumes the
    nominal 2.4 GHz clock, which the chip does not hold under such a load)."""
    import torch
    out = {}
    gen = torch.Generator(device="cuda:0").manual_seed(0)
    for name in dtypes:
        dt = torch.bfloat16 if name == "bf16" else torch.float16
        for n in sizes:
            a = torch.randn(n, n, device="cuda:0", dtype=dt, generator=gen)
            b = torch.randn(n, n, device="cuda:0", dtype=dt, generator=gen)
            reps = max(3, int(2 ** 36 // n ** 3 * 8))
            for _ in range(3):
                c = a @ b
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[f"{name}_n{n}"] = {"ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / ms / 1e9, 1)}
            del a, b, c
    return out


def gemm_calibration() -> int:
    print(json.dumps({"gemm_calibration": gemm_rates()}), flush=True)
    return 0


def fused_qkv_rates(uly, cfg, reps: int) -> dict:
    """The fused-projection variants of the redistribution on this workload's
    shapes: ulysses_pack_qkv from [T, Hq + 2*Hkv, D] shards into the group's
    q/k/v, and ulysses_unpack_qkv back (one launch each instead of three).
    Not part of the step: the workload's shards are separate tensors."""
    import torch
    dev, tdt = "cuda:0", torch.bfloat16
    P, T, D, Hq, Hkv, g = cfg.P, cfg.T, cfg.D, cfg.Hq, cfg.Hkv, cfg.group
    shards = [torch.empty((T, Hq + 2 * Hkv, D), dtype=tdt, device=dev).normal_() for _ in range(P)]
    outs = [torch.empty((P * T, c, D), dtype=tdt, device=dev) for c in (cfg.hq, cfg.hk, cfg.hk)]
    nbytes = 2 * P * T * (cfg.hq + 2 * cfg.hk) * D * 2   # read + write, each once
    res = {}
    for name, fn in (("pack_qkv", lambda: uly.ulysses_pack_qkv(shards, Hq, Hkv, g, *outs)),
                     ("unpack_qkv", lambda: uly.ulysses_unpack_qkv(*outs, Hq, Hkv, g, shards))):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    res["bytes"] = nbytes
    del shards, outs
    torch.cuda.empty_cache()
    return res


def fwd_from_shards_rate(uly, cfg, shards, cu_dev, fwd_flop: int, pack_fwd_ms: float, reps: int) -> dict:
    """attn_fwd_from_shards on the workload's sequence-sharded Q/K/V (no pack
    of Q, K, V before the forward), beside the step's pack + attn_fwd."""
    import torch
    dev = shards["q"][0].device
    o = torch.empty((cfg.N, cfg.hq, cfg.D), dtype=shards["q"][0].dtype, device=dev)
    lse = torch.empty((cfg.hq, cfg.N), dtype=torch.float32, device=dev)

    def run():
        uly.attn_fwd_from_shards(shards["q"], shards["k"], shards["v"], cfg.group, o, lse, cfg.scale, cu_dev)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tf = fwd_flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "pack_qkv_plus_attn_fwd_ms": round(pack_fwd_ms, 4)}


def chunked_rates(uly, cfg, qg, kg, vg, dog, fwd_flop: int, bwd_flop: int, call_ms: dict, reps: int) -> dict:
    """Attention computed ring-style on this GPU: the sequence in P chunks;
    forward = query chunk i against key chunks c < i (attn_fwd, causal = 0)
    and c = i (causal), then attn_merge of the i+1 partial results; backward =
    one attn_bwd_accumulate per chunk pair into float32 gradients (zeroed
    first). Same causal pairs and FLOPs as the single calls; reported beside
    them, not part of the step."""
    import torch
    P, T, hq, hk, D = cfg.P, cfg.T, cfg.hq, cfg.hk, cfg.D
    dev = qg.device
    parts_o = [torch.empty((T, hq, D), dtype=qg.dtype, device=dev) for _ in range(P)]
    parts_l = [torch.empty((hq, T), dtype=torch.float32, device=dev) for _ in range(P)]
    o = torch.empty_like(qg)
    lse = [torch.empty((hq, T), dtype=torch.float32, device=dev) for _ in range(P)]
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk, dv = torch.zeros(qg.shape, **f32), torch.zeros(kg.shape, **f32), torch.zeros(vg.shape, **f32)
    ws = torch.empty(uly.attn_bwd_workspace_size(T, hq, hk, D, qg.dtype), dtype=torch.uint8, device=dev)

    def fwd():
        for i in range(P):
            qi = qg[i * T:(i + 1) * T]
            for c in range(i + 1):
                uly.attn_fwd(qi, kg[c * T:(c + 1) * T], vg[c * T:(c + 1) * T], parts_o[c], parts_l[c],
                             cfg.scale, causal=int(c == i))
            uly.attn_merge(parts_o[:i + 1], parts_l[:i + 1], o[i * T:(i + 1) * T], lse[i])

    def bwd():
        for t in (dq, dk, dv):
            t.zero_()
        for i in range(P):
            r = slice(i * T, (i + 1) * T)
            for c in range(i + 1):
                kc = slice(c * T, (c + 1) * T)
                uly.attn_bwd_accumulate(qg[r], kg[kc], vg[kc], o[r], dog[r], lse[i], dq[r], dk[kc], dv[kc],
                                        cfg.scale, ws, causal=int(c == i))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {"chunks": P, "calls": f"fwd: {P * (P + 1) // 2} attn_fwd + {P} attn_merge; "
                                 f"bwd: {P * (P + 1) // 2} attn_bwd_accumulate (fp32 gradients)"}
    for name, fn, flop, single in (("fwd", fwd, fwd_flop, "attn_fwd"), ("bwd", bwd, bwd_flop, "attn_bwd")):
        ms = timed(fn)
        tf = flop / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     f"vs_single_{single}": round(call_ms[single] / ms, 4)}
    del parts_o, parts_l, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def _doc_starts(N, cu):
    cuv = np.array([0, N]) if cu is None else np.asarray(cu, dtype=np.int64)
    tok = np.arange(N)
    doc = np.searchsorted(cuv, tok, side="right") - 1
    return doc, cuv[doc]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3", help="workload key: c3 (default), c2, c4, c5")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-legs", action="store_true",
                    help="skip the fused-QKV and chunked-forward measurements (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--gemm-calibration", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gemm_calibration:
        return gemm_calibration()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the path on a single GPU; "
              f"--gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        return 2

    import torch
    import sequence_parallelism_ulysses_amd as uly
    import synthetic as syn

    cfg = syn.CONFIGS[args.config]
    if cfg.dtype != "bf16":
        print("bench.py times the bf16 workloads (c2..c5)", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    tdt = torch.bfloat16
    cu = syn.cu_seqlens(cfg)
    cu_dev = None if cu is None else torch.from_numpy(cu).to(dev)

    host, shards = {}, {}
    for n in ("q", "k", "v", "do"):
        # progress on stderr: the million-token inputs take minutes to generate
        print(f"bench: generating {n} shards of {cfg.workload}", file=sys.stderr, flush=True)
        host[n] = syn.all_shards_bits(cfg, n)
        shards[n] = [torch.from_numpy(s.view(np.int16)).to(dev).view(tdt) for s in host[n]]
    N, hq, hk, D, P, T, g = cfg.N, cfg.hq, cfg.hk, cfg.D, cfg.P, cfg.T, cfg.group
    qg = torch.empty((N, hq, D), dtype=tdt, device=dev)
    kg = torch.empty((N, hk, D), dtype=tdt, device=dev)
    vg = torch.empty_like(kg)
    dog = torch.empty_like(qg)
    o = torch.empty_like(qg)
    lse = torch.empty((hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(uly.attn_bwd_workspace_size(N, hq, hk, D, tdt), dtype=torch.uint8, device=dev)
    out_sh = {n: [torch.zeros((T, cfg.heads(n), D), dtype=tdt, device=dev) for _ in range(P)]
              for n in ("o", "dq", "dk", "dv")}

    # Q, K and V are regrouped together after the projections, dQ, dK and dV
    # together after the backward: one launch each (ulysses_pack_multi)
    qkv_sh = [shards["q"], shards["k"], shards["v"]]
    dqkv_sh = [out_sh["dq"], out_sh["dk"], out_sh["dv"]]
    calls = [
        ("pack_qkv", lambda: uly.ulysses_pack_multi(qkv_sh, g, [qg, kg, vg])),
        ("pack_do", lambda: uly.ulysses_pack(shards["do"], g, dog)),
        ("attn_fwd", lambda: uly.attn_fwd(qg, kg, vg, o, lse, cfg.scale, cu_dev)),
        ("attn_bwd", lambda: uly.attn_bwd(qg, kg, vg, o, dog, lse, dq, dk, dv, cfg.scale, ws, cu_dev)),
        ("unpack_o", lambda: uly.ulysses_unpack(o, g, out_sh["o"])),
        ("unpack_dqkv", lambda: uly.ulysses_unpack_multi([dq, dk, dv], g, dqkv_sh)),
    ]

    def step(events=None):
        for i, (_, fn) in enumerate(calls):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # HIP events on the stream the library launches on (torch's current stream)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    call_ms = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
               for i, (name, _) in enumerate(calls)}

    C = causal_pairs(N, cu)
    fwd_flop = 4 * D * C * hq
    bwd_flop = 10 * D * C * hq
    step_flop = fwd_flop + bwd_flop
    value = step_flop / (ms_step * 1e-3) / 1e12

    def pack_bytes(name):
        heads = {"pack_qkv": hq + 2 * hk, "unpack_dqkv": hq + 2 * hk, "pack_do": hq, "unpack_o": hq}[name]
        return 2 * N * heads * D * 2
    details = {}
    for name, ms in call_ms.items():
        if name == "attn_fwd":
            a = fwd_flop / (ms * 1e-3) / 1e12
            details[name] = {"ms": round(ms, 4), "TFLOP/s": round(a, 2), "frac_mfma": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
        elif name == "attn_bwd":
            a = bwd_flop / (ms * 1e-3) / 1e12
            details[name] = {"ms": round(ms, 4), "TFLOP/s": round(a, 2), "frac_mfma": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            a = pack_bytes(name) / (ms * 1e-3) / 1e9
            details[name] = {"ms": round(ms, 4), "GB/s": round(a, 1), "frac_hbm": round(a / HBM_PEAK_GBS, 4)}

    dom = max(("attn_fwd", "attn_bwd"), key=lambda n: call_ms[n])
    dom_flop = bwd_flop if dom == "attn_bwd" else fwd_flop
    achieved = dom_flop / (call_ms[dom] * 1e-3) / 1e12
    roofline = {
        "kernel": dom + (" (prep + convert + dK/dV + reduce + dQ launches)" if dom == "attn_bwd" else ""),
        "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(cfg.workload) if dom == "attn_bwd" else None,
        "per_launch": f"{'10' if dom == 'attn_bwd' else '4'}*D*C*hq = {dom_flop:.4g} FLOP, "
                      f"C = {C} causal pairs, hq = {hq}, D = {D}",
        "avg_launch_ms": round(call_ms[dom], 4),
    }
    pack_total_ms = sum(v for k, v in call_ms.items() if "pack" in k)
    pack_total_bytes = sum(pack_bytes(k) for k in call_ms if "pack" in k)

    line = {
        "metric": "causal attn fwd+bwd TFLOP/s per GPU head group (% MFMA peak); pack GB/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "N": N, "P": P, "tokens_per_shard": T, "q_heads": hq, "kv_heads": hk,
                   "head_dim": D, "causal": True, "documents": None if cu is None else int(len(cu) - 1),
                   "causal_pairs": C, "step_flop": step_flop,
                   "seed": f"numpy SeedSequence({cfg.seed}), one child per tensor (q, k, v, dO) and shard"},
        "frac_mfma_step": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "pack_unpack": {"GB/s": round(pack_total_bytes / (pack_total_ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(pack_total_bytes / (pack_total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "bytes": pack_total_bytes, "ms": round(pack_total_ms, 4)},
        "roofline": roofline,
        "calls": details,
    }
    if not args.no_side_legs:
        line["fused_qkv"] = fused_qkv_rates(uly, cfg, args.steps)
        if cfg.T % 64 == 0:
            line["fwd_from_shards"] = fwd_from_shards_rate(uly, cfg, shards, cu_dev, fwd_flop,
                                                           call_ms["pack_qkv"] + call_ms["attn_fwd"], args.steps)
    if not args.no_side_legs:
        # the same box's vendor bf16 GEMM, as a practical matrix-unit ceiling
        g = gemm_rates(dtypes=("bf16",))
        best = max(v["tflops"] for v in g.values())
        line["vendor_gemm"] = dict(g, step_over_best=round(value / best, 4))
    if cu is None and not args.no_side_legs:
        line["chunked"] = chunked_rates(uly, cfg, qg, kg, vg, dog, fwd_flop, bwd_flop, call_ms,
                                        max(3, args.steps // 4))
    if not args.no_cpu_baseline:
        line["cpu_baseline"], res = cpu_baseline(cfg, cu, host, args.cpu_seconds)
        line["parity_sample"] = parity_of_sample({"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, res, N)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
