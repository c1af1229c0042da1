#!/usr/bin/env python3
"""Benchmark of the tiled attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM: one attn_prefill_fwd for a prefill workload, one
attn_decode_fwd (plan, split kernel and log-sum-exp combine) for the decode
workload. The headline workload is the largest one, the long non-causal bf16
self-attention (B=4, H=16, S_q=S_k=16384, d=128, dense BSHD). W untimed steps
run first, then exactly K steps are timed on the stream the kernels are launched
on, in up to ten repetitions of back-to-back launches, each between two HIP events,
bracketed by device synchronisation: the headline is K steps over their total
time, and the repetitions give the trimmed mean (20% cut at each end), the median,
the spread and a "noisy" flag above 10% spread.

The same JSON line carries the split-KV decode workload (B=32, 32/8 heads, d=128,
bf16, key lengths U[1024, 65536], 16 splits) measured the same way (10 warmup
launches, 10 repetitions of 50), a roofline object for the dominant kernel of each,
the parity of the timed outputs against the fp64 oracle on a sample, the oracle
itself timed on the host cores (cpu_baseline), and the device facts the peaks are
derived from. A failing parity check withholds the value (null) and exits non-zero;
--debug-mismatch N lists the N largest deviations from the oracle, --report PATH
writes the line to a file as well.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Dense fp16/bf16 matrix-core throughput per compute unit and clock on gfx950: each of
# the 4 SIMDs of a CU completes one v_mfma_f32_32x32x16 (2*32*32*16 = 32768 flops) per
# 32 cycles (measured on the device), i.e. 4 * 1024 flops per clock and CU. The peak is
# this times the device's compute units and peak engine clock (2516.6 TFLOP/s for 256
# CUs at 2.4 GHz).
MFMA_FLOP_PER_CLK_CU = 4096
# HBM3E peak of the MI355X as published (8 TB/s). The runtime's memory clock and bus
# width are recorded next to it but do not give the HBM rate reliably.
PEAK_HBM_GBS = 8000.0
TOL = {"f16": 2e-2, "bf16": 4e-2}
TRIM = 0.2
NOISY_SPREAD = 0.10
KERNEL_SOURCES = ["attention_forward_tiled_amd/csrc/prefill.hip",
                  "attention_forward_tiled_amd/csrc/decode.hip",
                  "attention_forward_tiled_amd/csrc/common.hpp",
                  "attention_forward_tiled_amd/build.py"]      # compile flags
HEADLINE = "long_noncausal_bf16_s16384"
DECODE = "splitkv_decode_bf16_64k"

# The headline metric: prefill TFLOP/s (causal flops counted as half) against the dense
# fp16/bf16 MFMA peak, decode KV GB/s against the HBM peak.
METRIC = "attn fwd TFLOP/s (% MFMA peak) for prefill; decode KV GB/s (% HBM peak)"


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def host_facts() -> dict:
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_count": os.cpu_count(), "affinity": affinity, "blas_threads": blas_threads(),
            "machine": platform.machine()}


def rocm_version() -> str:
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            pass
    return ""


def device_facts(torch) -> dict:
    """Device facts from hipDeviceProp_t (through the library) and the derived peaks."""
    from attention_forward_tiled_amd import attn_device_info
    info = attn_device_info(torch.cuda.current_device())
    peak = info["compute_units"] * info["clock_khz"] * 1e3 * MFMA_FLOP_PER_CLK_CU / 1e12
    mem_rate = 2 * info["memory_clock_khz"] * 1e3 * info["memory_bus_bits"] / 8 / 1e9
    return {"name": info["name"], "arch": info["arch"], "compute_units": info["compute_units"],
            "clock_mhz": info["clock_khz"] / 1e3, "memory_clock_mhz": info["memory_clock_khz"] / 1e3,
            "memory_bus_bits": info["memory_bus_bits"], "total_memory_gib": round(info["total_memory"] / 2**30, 1),
            "lds_per_cu": info["lds_per_cu"], "l2_bytes": info["l2_bytes"],
            "hip_runtime_version": info["runtime_version"], "driver_version": info["driver_version"],
            "rocm": rocm_version(), "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
            "peak_mfma_tflops": round(peak, 1),
            "peak_mfma_derivation": f"{info['compute_units']} CUs x {info['clock_khz'] / 1e3:.0f} MHz x "
                                    f"{MFMA_FLOP_PER_CLK_CU} flop/clk/CU (dense fp16/bf16)",
            "peak_hbm_gbs": PEAK_HBM_GBS,
            "hbm_from_runtime_clock_gbs": round(mem_rate, 1)}


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------- workloads

class PrefillWorkload:
    kernel = "prefill_kernel"

    def __init__(self, case, seed):
        import torch
        from attn_workloads import make_prefill_inputs
        from attention_forward_tiled_amd import attn_prefill_fwd
        self.case, self.fn, self.torch = case, attn_prefill_fwd, torch
        # head size 256 without the precise option runs the eight-wave narrow kernel
        if case.head_dim == 256 and not case.precise:
            self.kernel = "prefill_narrow_kernel"
        self.inp = make_prefill_inputs(case, seed)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()  # noqa: E731
        self.q, self.k, self.v = to(self.inp.q), to(self.inp.k), to(self.inp.v)
        self.bt = torch.from_numpy(self.inp.block_table).cuda() if self.inp.block_table is not None else None
        need_lens = self.bt is not None or case.seqlens_k is not None
        self.sl = torch.from_numpy(self.inp.seqlens_k).cuda() if need_lens else None
        odt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[case.o_dtype]
        self.out = torch.full(self.q.shape, float("nan"), dtype=odt, device="cuda")
        # workspace of the tail split, when the library splits this launch (allocated
        # once, outside the timed region); the step is then main items, split units and
        # the combine
        from attention_forward_tiled_amd import attn_prefill_workspace_bytes
        need = attn_prefill_workspace_bytes(self.q, num_heads_kv=case.heads_kv, seqlen_k=case.seqlen_k,
                                            causal=case.causal, layout=case.layout, precise=case.precise)
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        self.tail_split_bytes = need

    def step(self):
        c = self.case
        self.fn(self.q, self.k, self.v, causal=c.causal, block_table=self.bt, seqlens_k=self.sl,
                seqlen_k=c.seqlen_k, layout=c.layout, out=self.out, precise=c.precise,
                kv_splits=0 if self.ws is not None else 1, workspace=self.ws)

    def kernel_only(self):
        return None          # the step is the prefill launch (three kernels with a tail split)

    def work(self):
        return float(self.case.flops_half_convention())

    def unit(self):
        return "TFLOP/s", 1e12

    def config(self):
        c = self.case
        return {"workload": c.name, "batch": c.batch, "heads_q": c.heads_q, "heads_kv": c.heads_kv,
                "seqlen_q": c.seqlen_q, "seqlen_k": c.seqlen_k, "head_dim": c.head_dim,
                "causal": c.causal, "kv": c.kv, "layout": c.layout, "dtype": c.dtype,
                "flops_per_step": self.work(), "flops_exact_per_step": float(c.flops_exact()),
                "flop_convention": "4*d*S_q*S_k*B*Hq, halved when causal",
                "tail_split_workspace_bytes": int(self.tail_split_bytes)}

    def sample_rows(self):
        Sq = self.case.seqlen_q
        if Sq * self.case.batch * self.case.heads_q * self.case.seqlen_k <= 2048 * 2048 * 32:
            return np.arange(Sq)
        n = max(8, int(2048 * 2048 * 32 / (self.case.batch * self.case.heads_q * self.case.seqlen_k)))
        return np.unique(np.linspace(0, Sq - 1, num=min(Sq, n)).astype(np.int64))

    def finite(self):
        return bool(self.torch.isfinite(self.out).all())

    def cpu_sample(self, min_seconds):
        """Oracle on a row sample; returns (value in the metric's unit, seconds, sample text, err)."""
        import oracle
        from attn_workloads import bits_to_f64
        c, inp = self.case, self.inp
        rows = self.sample_rows()
        q = bits_to_f64(inp.q, c.dtype)
        k = bits_to_f64(inp.k, c.dtype)
        v = bits_to_f64(inp.v, c.dtype)
        reps, t_total = 0, 0.0
        while True:
            t0 = time.perf_counter()
            O, _ = oracle.attention(q, k, v, causal=c.causal, layout=c.layout, block_table=inp.block_table,
                                    seqlens_k=inp.seqlens_k, q_index=rows)
            t_total += time.perf_counter() - t0
            reps += 1
            if t_total >= min_seconds or reps >= 50:
                break
        sec = t_total / reps
        # the sample's share of the whole workload's visible (query, key) pairs
        pairs_s = 0
        for L in c.lengths():
            off = L - c.seqlen_q
            vis = np.minimum(L, rows + off + 1) if c.causal else np.full(rows.size, L)
            pairs_s += int(np.maximum(vis, 0).sum())
        frac = pairs_s / max(1, c.visible_pairs())
        value = frac * self.work() / sec / 1e12
        got = self.out.float().cpu().numpy().astype(np.float64)
        got = got[:, rows] if c.layout == "bshd" else got[:, :, rows]
        text = (f"oracle on {rows.size} of {c.seqlen_q} query rows x all {c.batch * c.heads_q} "
                f"(sequence, head) pairs ({100 * frac:.2f}% of the visible pairs), {reps} rep(s)")
        names = ("seq", "row", "head", "col") if c.layout == "bshd" else ("seq", "head", "row", "col")
        maps = tuple(rows if nm == "row" else None for nm in names)
        return value, sec, text, (got, O, names, maps)


class DecodeWorkload:
    kernel = "decode_stream_kernel"

    def __init__(self, case, seed):
        import torch
        from attn_workloads import make_decode_inputs
        from attention_forward_tiled_amd import (attn_decode_fwd, attn_decode_workspace_bytes,
                                                 attn_splitkv_combine)
        self.case, self.fn, self.comb, self.torch = case, attn_decode_fwd, attn_splitkv_combine, torch
        self.inp = make_decode_inputs(case, seed)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()  # noqa: E731
        self.q, self.kc, self.vc = to(self.inp.q), to(self.inp.k_cache), to(self.inp.v_cache)
        self.bt = torch.from_numpy(self.inp.block_table).cuda()
        self.sl = torch.from_numpy(self.inp.seqlens_k).cuda()
        B, Hq, d, S = case.batch, case.heads_q, case.head_dim, case.num_splits
        self.ws = torch.empty(attn_decode_workspace_bytes(B, Hq, S, d), dtype=torch.uint8, device="cuda")
        self.out = torch.full((B, Hq, d), float("nan"), dtype=tdt, device="cuda")
        rows = B * Hq * S
        self.part_o = self.ws[: rows * d * 4].view(torch.float32).view(B, Hq, S, d)
        off = ((rows * d * 4 + 255) // 256) * 256
        self.part_lse = self.ws[off: off + rows * 4].view(torch.float32).view(B, Hq, S)
        self.comb_out = torch.empty_like(self.out)

    def step(self):
        self.fn(self.q, self.kc, self.vc, self.bt, self.sl, max_seqlen_k=self.inp.max_seqlen_k,
                num_splits=self.case.num_splits, out=self.out, workspace=self.ws)

    def kernel_only(self):
        """The step minus the combine: the combine launch alone on the same partials."""
        return lambda: self.comb(self.part_o, self.part_lse, out=self.comb_out)

    def work(self):
        c = self.case
        return float(2 * int(self.inp.seqlens_k.sum()) * c.heads_kv * c.head_dim * 2)

    def unit(self):
        return "GB/s", 1e9

    def config(self):
        c = self.case
        return {"workload": c.name, "batch": c.batch, "heads_q": c.heads_q, "heads_kv": c.heads_kv,
                "head_dim": c.head_dim, "dtype": c.dtype, "num_splits": c.num_splits,
                "seqlens_k_sum": int(self.inp.seqlens_k.sum()), "kv_bytes_per_step": self.work(),
                "byte_convention": "K+V bytes of every valid key, read once per KV head"}

    def finite(self):
        return bool(self.torch.isfinite(self.out).all())

    def cpu_sample(self, min_seconds):
        import oracle
        from attn_workloads import bits_to_f64
        c, inp = self.case, self.inp
        order = np.argsort(inp.seqlens_k)
        seqs = sorted(int(x) for x in order[:: max(1, c.batch // 4)][:4])
        tables, pages = [], []
        for b in seqs:
            n = -(-int(inp.seqlens_k[b]) // 64)
            tables.append(list(range(len(pages), len(pages) + n)))
            pages.extend(int(x) for x in inp.block_table[b, :n])
        table = np.zeros((len(seqs), max(len(t) for t in tables)), dtype=np.int64)
        for i, t in enumerate(tables):
            table[i, :len(t)] = t
        k = bits_to_f64(inp.k_cache[pages], c.dtype)
        v = bits_to_f64(inp.v_cache[pages], c.dtype)
        q = bits_to_f64(inp.q[seqs], c.dtype)
        reps, t_total = 0, 0.0
        while True:
            t0 = time.perf_counter()
            O, _ = oracle.attention(q, k, v, causal=False, block_table=table, seqlens_k=inp.seqlens_k[seqs])
            t_total += time.perf_counter() - t0
            reps += 1
            if t_total >= min_seconds or reps >= 50:
                break
        sec = t_total / reps
        nbytes = 2 * int(inp.seqlens_k[seqs].sum()) * c.heads_kv * c.head_dim * 2
        got = self.out.float().cpu().numpy().astype(np.float64)[seqs]
        text = (f"oracle on {len(seqs)} of {c.batch} sequences (key lengths "
                f"{inp.seqlens_k[seqs].tolist()}), all heads, {reps} rep(s)")
        return nbytes / sec / 1e9, sec, text, (got, O[:, 0], ("seq", "head", "col"), (np.array(seqs), None, None))


def make_workload(name, seed):
    from attn_workloads import CONFIGS, DecodeCase
    case = CONFIGS[name]
    return DecodeWorkload(case, seed) if isinstance(case, DecodeCase) else PrefillWorkload(case, seed)


# ---------------------------------------------------------------------------- timing

def spin_up(fn, ms, torch):
    """Untimed launches of the step for about `ms` of wall time, so that the GPU leaves its
    idle clocks before the warmup steps and the timed region (a cold MI355X needs on the
    order of 100 ms of load; a 60-us step timed after ten warmup launches ran ~18% slow).
    Returns the number of launches."""
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def rep_sizes(steps: int, reps: int):
    """Split `steps` launches into min(reps, steps) back-to-back repetitions of nearly
    equal size (the first ones one larger when it does not divide)."""
    reps = max(1, min(reps, steps))
    base, extra = divmod(steps, reps)
    return [base + (1 if r < extra else 0) for r in range(reps)]


def trimmed_mean(x, cut=TRIM):
    x = np.sort(np.asarray(x, dtype=np.float64))
    k = int(cut * x.size)
    return float(x[k:x.size - k].mean()) if x.size > 2 * k else float(x.mean())


def time_reps(fn, steps, warmup, reps, torch):
    """W untimed launches, then exactly `steps` launches in repetitions, each between two
    HIP events recorded on the stream the launches go to. Returns the mean time per
    launch over all steps and the per-repetition statistics (ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    sizes = rep_sizes(steps, reps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    ev[0].record(stream)
    for r, n in enumerate(sizes):
        for _ in range(n):
            fn()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / n for r, n in enumerate(sizes)]
    total = ev[0].elapsed_time(ev[-1])
    med = float(np.median(per))
    spread = (max(per) - min(per)) / med if med > 0 else 0.0
    stats = {"reps": len(sizes), "launches_per_rep": sizes[0] if len(set(sizes)) == 1 else sizes,
             "trimmed_mean_ms": round(trimmed_mean(per), 6), "median_ms": round(med, 6),
             "min_ms": round(min(per), 6), "max_ms": round(max(per), 6), "spread": round(spread, 4),
             "noisy": bool(spread > NOISY_SPREAD)}
    return total / steps, stats


def roofline(wl, kernel_ms, dev):
    unit, scale = wl.unit()
    achieved = wl.work() / (kernel_ms * 1e-3) / scale
    if unit == "TFLOP/s":
        peak = dev["peak_mfma_tflops"]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        peak = dev["peak_hbm_gbs"]
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                "frac": round(achieved / peak, 4)}
    roof["kernel"] = wl.kernel
    roof["kernel_ms"] = round(kernel_ms, 6)
    roof["traffic"] = load_traffic(wl.case.name)
    return roof


def measure(wl, steps, warmup, reps, spinup_ms, torch, dev):
    """Time one workload; returns (ms per step, rep statistics, roofline, spin-up launches)."""
    spin = spin_up(wl.step, spinup_ms, torch)
    ms, stats = time_reps(wl.step, steps, warmup, reps, torch)
    kernel_ms = ms
    other = wl.kernel_only()
    if other is not None:
        other_ms, _ = time_reps(other, steps, warmup, reps, torch)
        kernel_ms = ms - other_ms
    return ms, stats, roofline(wl, kernel_ms, dev), spin


def worst_samples(got, ref, n, names, maps):
    """The n entries with the largest |got - ref|, worst first: their index along each named
    axis (through `maps` back to the whole output where the sample took a subset) and both
    values."""
    err = np.abs(got - ref)
    out = []
    for f in np.argsort(err, axis=None, kind="stable")[::-1][:n]:
        idx = np.unravel_index(f, err.shape)
        where = {nm: int(m[i]) if m is not None else int(i) for nm, m, i in zip(names, maps, idx)}
        out.append({**where, "got": float(got[idx]), "expected": float(ref[idx]), "abs_err": float(err[idx])})
    return out


def parity_and_baseline(wl, cpu_seconds, no_cpu, debug_mismatch=0):
    """Parity of the timed output on the oracle sample, and the oracle timed on it."""
    unit, _ = wl.unit()
    if not wl.finite():
        return None, {"max_abs_err": None, "pass": False, "checked": "output has NaN/inf (rows left unwritten)"}
    if no_cpu:
        return None, None
    cv, sec, text, (got, ref, names, maps) = wl.cpu_sample(cpu_seconds)
    err = float(np.abs(got - ref).max())
    host = host_facts()
    cpu = {"value": round(cv, 6), "unit": unit, "cores": host["blas_threads"], "kind": "oracle",
           "sample": text, "seconds": round(sec, 3), "host_cpu_count": host["cpu_count"],
           "host_affinity": host["affinity"],
           "cores_meaning": "BLAS threads of the fp64 oracle's matrix products (the rest runs on one thread)"}
    tol = TOL[wl.case.dtype] if not getattr(wl.case, "precise", False) else 1e-4
    parity = {"max_abs_err": err, "tol": tol, "pass": bool(err <= tol),
              "checked": "whole output finite (NaN-filled before the first launch); timed output vs the "
                         "fp64 oracle on the cpu_baseline sample"}
    if debug_mismatch > 0:
        parity["worst"] = worst_samples(got, ref, debug_mismatch, names, maps)
        for w in parity["worst"]:
            print(f"# {wl.case.name} mismatch: {w}", file=sys.stderr, flush=True)
    return cpu, parity


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=10, help="repetitions the timed steps are split into")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--decode-workload", default=DECODE,
                    help="second workload measured into the 'decode' object ('none' to skip)")
    ap.add_argument("--decode-launches", type=int, default=50, help="launches per repetition for it")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="untimed launches before the warmup steps, to bring the clocks up")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (HBM counter calibration)")
    ap.add_argument("--debug-mismatch", type=int, default=0, metavar="N",
                    help="add the N largest deviations from the oracle (index, value, expected) to "
                         "each parity object and print them")
    ap.add_argument("--report", metavar="PATH", help="also write the JSON line, indented, to PATH")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the attention forward here runs on a single "
              f"MI355X and has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = device_facts(torch)

    wl = make_workload(args.workload, args.seed)
    unit, scale = wl.unit()
    print(f"# {args.workload}: first launch", file=sys.stderr, flush=True)
    wl.step()                       # first call: output kept for the parity check
    torch.cuda.synchronize()
    ms, stats, roof, spin = measure(wl, args.steps, args.warmup, args.reps, args.spinup_ms, torch, dev)
    value = wl.work() / (ms * 1e-3) / scale
    print(f"# {args.workload}: {ms:.5f} ms per step", file=sys.stderr, flush=True)

    dec = None
    if args.decode_workload != "none" and args.decode_workload != args.workload:
        dw = make_workload(args.decode_workload, args.seed)
        dw.step()
        torch.cuda.synchronize()
        dms, dstats, droof, _ = measure(dw, args.reps * args.decode_launches, 10, args.reps,
                                        args.spinup_ms, torch, dev)
        dunit, dscale = dw.unit()
        dvalue = dw.work() / (dms * 1e-3) / dscale
        print(f"# {args.decode_workload}: {dms:.5f} ms per step", file=sys.stderr, flush=True)
        dcpu, dpar = parity_and_baseline(dw, 2.0, args.no_cpu_baseline, args.debug_mismatch)
        ok = dpar is None or dpar["pass"]
        dec = {"workload": dw.case.name, "value": round(dvalue, 1) if ok else None, "unit": dunit,
               "ms_per_step": round(dms, 6), "timing": dstats,
               "roofline": droof, "parity": dpar, "cpu_baseline": dcpu, "config": dw.config()}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu, parity = parity_and_baseline(wl, args.cpu_seconds, args.no_cpu_baseline, args.debug_mismatch)
    ok = parity is None or parity["pass"]
    line = {
        "metric": METRIC,
        "value": round(value, 3) if ok else None,
        "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.case.dtype, "data": "synthetic", "seed": args.seed,
        "config": wl.config(), "timing": stats, "spinup": {"ms": args.spinup_ms, "launches": spin},
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "decode": dec, "device": dev,
        "host": host_facts(),
    }
    print(json.dumps(line), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(line, f, indent=1)
    dec_ok = dec is None or dec["parity"] is None or dec["parity"]["pass"]
    return 0 if (ok and dec_ok) else 1


if __name__ == "__main__":
    sys.exit(main())
