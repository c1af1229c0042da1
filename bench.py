#!/usr/bin/env python3
"""Benchmark of the tiled attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM: one attn_prefill_fwd for a prefill workload, one
attn_decode_fwd (split kernel + log-sum-exp combine) for the decode workload.
The default workload is the causal GQA prefill over a paged cache (B=1, 32 query
heads, 8 KV heads, S_q=S_k=2048, d=128, fp16). W untimed steps run first, then
exactly K steps are timed between HIP events on the stream the kernels are
launched on, bracketed by device synchronisation.

Prints one JSON line with the throughput (prefill: TFLOP/s with causal FLOPs
counted as half; decode: K/V GB/s), a roofline object for the dominant kernel,
a parity check of the timed output against the fp64 oracle on a sample, and the
oracle itself timed on the host cores (cpu_baseline).
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
sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2516.6    # 256 CUs x 2.4 GHz x 4096 dense fp16/bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0            # HBM3E
TOL = {"f16": 2e-2, "bf16": 4e-2}
KERNEL_SOURCES = ["attention_forward_tiled_amd/csrc/prefill.hip",
                  "attention_forward_tiled_amd/csrc/decode.hip",
                  "attention_forward_tiled_amd/csrc/common.hpp",
                  "attention_forward_tiled_amd/build.py"]      # compile flags


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
    def __init__(self, case, seed):
        import torch
        from attn_workloads import make_prefill_inputs
        from attention_forward_tiled_amd import attn_prefill_fwd
        self.case, self.fn, self.torch = case, attn_prefill_fwd, torch
        self.inp = make_prefill_inputs(case, seed)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()  # noqa: E731
        self.q, self.k, self.v = to(self.inp.q), to(self.inp.k), to(self.inp.v)
        self.bt = torch.from_numpy(self.inp.block_table).cuda() if self.inp.block_table is not None else None
        need_lens = self.bt is not None or case.seqlens_k is not None
        self.sl = torch.from_numpy(self.inp.seqlens_k).cuda() if need_lens else None
        odt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[case.o_dtype]
        self.out = torch.empty(self.q.shape, dtype=odt, device="cuda")
        self.kernel = "prefill_kernel"

    def step(self):
        c = self.case
        self.fn(self.q, self.k, self.v, causal=c.causal, block_table=self.bt, seqlens_k=self.sl,
                seqlen_k=c.seqlen_k, layout=c.layout, out=self.out, precise=c.precise)

    def work(self):
        return float(self.case.flops_half_convention())

    def unit(self):
        return "TFLOP/s", 1e12

    def config(self):
        c = self.case
        return {"workload": c.name, "batch": c.batch, "heads_q": c.heads_q, "heads_kv": c.heads_kv,
                "seqlen_q": c.seqlen_q, "seqlen_k": c.seqlen_k, "head_dim": c.head_dim,
                "causal": c.causal, "kv": c.kv, "layout": c.layout, "flops_per_step": self.work(),
                "flops_exact_per_step": float(c.flops_exact()),
                "flop_convention": "4*d*S_q*S_k*B*Hq, halved when causal"}

    def sample_rows(self):
        Sq = self.case.seqlen_q
        if Sq * self.case.batch * self.case.heads_q * self.case.seqlen_k <= 2048 * 2048 * 32:
            return np.arange(Sq)
        n = max(8, int(2048 * 2048 * 32 / (self.case.batch * self.case.heads_q * self.case.seqlen_k)))
        return np.unique(np.linspace(0, Sq - 1, num=min(Sq, n)).astype(np.int64))

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
        err = float(np.abs(got - O).max())
        text = (f"oracle on {rows.size} of {c.seqlen_q} query rows x all {c.batch * c.heads_q} "
                f"(sequence, head) pairs ({100 * frac:.1f}% of the visible pairs), {reps} rep(s)")
        return value, sec, text, err


class DecodeWorkload:
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
        self.out = torch.empty((B, Hq, d), dtype=tdt, device="cuda")
        rows = B * Hq * S
        self.part_o = self.ws[: rows * d * 4].view(torch.float32).view(B, Hq, S, d)
        off = ((rows * d * 4 + 255) // 256) * 256
        self.part_lse = self.ws[off: off + rows * 4].view(torch.float32).view(B, Hq, S)
        self.comb_out = torch.empty_like(self.out)
        self.kernel = "decode_stream_kernel"

    def step(self):
        self.fn(self.q, self.kc, self.vc, self.bt, self.sl, max_seqlen_k=self.inp.max_seqlen_k,
                num_splits=self.case.num_splits, out=self.out, workspace=self.ws)

    def combine_step(self):
        self.comb(self.part_o, self.part_lse, out=self.comb_out)

    def work(self):
        c = self.case
        return float(2 * int(self.inp.seqlens_k.sum()) * c.heads_kv * c.head_dim * 2)

    def unit(self):
        return "GB/s", 1e9

    def config(self):
        c = self.case
        return {"workload": c.name, "batch": c.batch, "heads_q": c.heads_q, "heads_kv": c.heads_kv,
                "head_dim": c.head_dim, "num_splits": c.num_splits,
                "seqlens_k_sum": int(self.inp.seqlens_k.sum()), "kv_bytes_per_step": self.work(),
                "byte_convention": "K+V bytes of every valid key, read once per KV head"}

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
        err = float(np.abs(got - O[:, 0]).max())
        text = (f"oracle on {len(seqs)} of {c.batch} sequences (key lengths "
                f"{inp.seqlens_k[seqs].tolist()}), all heads, {reps} rep(s)")
        return nbytes / sec / 1e9, sec, text, err


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
    import time
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def time_steps(fn, steps, warmup, torch):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_causal_paged_f16_s2048")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--spinup-ms", type=float, default=200.0,
                    help="untimed launches before the warmup steps, to bring the clocks up")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (HBM counter calibration)")
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

    wl = make_workload(args.workload, args.seed)
    unit, scale = wl.unit()
    wl.step()                       # first call: output kept for the parity check
    torch.cuda.synchronize()
    spin = spin_up(wl.step, args.spinup_ms, torch)
    ms = time_steps(wl.step, args.steps, args.warmup, torch)
    value = wl.work() / (ms * 1e-3) / scale

    # dominant kernel: the prefill kernel itself, or the decode split kernel (step minus combine)
    kernel_ms = ms
    if isinstance(wl, DecodeWorkload):
        comb_ms = time_steps(wl.combine_step, args.steps, args.warmup, torch)
        kernel_ms = ms - comb_ms
    achieved = wl.work() / (kernel_ms * 1e-3) / scale
    if unit == "TFLOP/s":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = wl.kernel
    roof["kernel_ms"] = round(kernel_ms, 5)
    roof["traffic"] = load_traffic(args.workload)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cv, sec, text, err = wl.cpu_sample(args.cpu_seconds)
        cpu = {"value": round(cv, 6), "unit": unit, "cores": blas_threads(), "kind": "oracle",
               "sample": text, "seconds": round(sec, 3)}
        tol = TOL[wl.case.dtype] if not getattr(wl.case, "precise", False) else 1e-4
        parity = {"max_abs_err": err, "tol": tol, "pass": bool(err <= tol),
                  "checked": "timed output vs the fp64 oracle on the cpu_baseline sample"}

    dtype = wl.case.dtype
    line = {
        "metric": METRIC,
        "value": round(value, 3) if (parity is None or parity["pass"]) else None,
        "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "spinup": {"ms": args.spinup_ms, "launches": spin},
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": wl.config(), "roofline": roof, "cpu_baseline": cpu, "parity": parity,
    }
    print(json.dumps(line), flush=True)
    return 0 if (parity is None or parity["pass"]) else 1


if __name__ == "__main__":
    sys.exit(main())
