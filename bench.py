"""Benchmark of the dual-stream Gated DeltaNet layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-components] [--only fwd|step|serve|conv] [--json-out PATH]

A step is one pass of the layer's hot path over one batch of the headline
workload -- 4 documents x 8192 tokens (prompt 2048, response in blocks of
B = 4), 16 heads, d_k = d_v = 128, bf16 q/k/v with fp32 gates and state:
the dual-stream forward and, once the backward exists, the backward.  Inputs are
resident in HBM before the timed region.  The serving cycle (256 requests x 16
heads, four EVALs + one COMMIT) and the packed ShortConv (32768 tokens, 8
documents, 3x32x128 channels) are timed in the same run and reported under
"components".  Rank 0 prints one JSON line.

Method: "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes),
Overall framework and Key designs items 2-4.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dual-stream GDN tokens/s (H=16,d=128,B=4,L=8K) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

# Algorithmic bytes per (token, head) of the forward at d = 128, bf16 io:
# q, k, v read (3 x 256 B), alpha, beta (8 B), o written (256 B); the noisy
# stream moves the same per response token.  Checkpoints are excluded.
FWD_BYTES_PER_TH = 3 * 256 + 8 + 256
# Algorithmic flops per (token, head), triangular halves only, chunk C:
#   clean 6 d^2 + 5 C d + C^2/3 ;  noisy 4 d^2 + 4 C d + 8 B d
def fwd_flops_per_th(d, C, B, noisy):
    return (4 * d * d + 4 * C * d + 8 * B * d) if noisy else (6 * d * d + 5 * C * d + C * C / 3)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-components", action="store_true")
    p.add_argument("--only", choices=["fwd", "step", "serve", "conv"], default=None)
    p.add_argument("--json-out", default=None)
    return p.parse_args()


class Timer:
    """HIP-event timing of one kernel call on the current stream (the library
    launches on the caller's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.times = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.times.setdefault(name, []).append((s, e))
        return out

    def avg_ms(self, name):
        ev = self.times.get(name, [])
        if not ev:
            return None
        return float(np.mean([s.elapsed_time(e) for s, e in ev]))

    def clear(self):
        self.times = {}


def traffic_for(kernel_file, kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, valid only if
    the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel, {})
    src = os.path.join(ROOT, "gated_deltanet_dual_amd", "csrc", kernel_file)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if rec.get("source_sha") != sha or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_deltanet_dual_amd as g
    from gated_deltanet_dual_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    g.lib()
    timer = Timer(torch)
    bf = torch.bfloat16

    def up(x, to_bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(bf) if to_bf16 else t

    # ------------------------------------------------------------ headline inputs
    log("bench: generating the headline workload (4 x 8192 tokens, H=16, d=128)")
    inp = wl.headline(with_grads=True, round_io=False)
    B, H, d = inp.block_size, inp.H, 128
    T = inp.T
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    X = dict(q=up(inp.q, True), k=up(inp.k, True), v=up(inp.v, True), a=up(inp.alpha), b=up(inp.beta),
             qn=up(inp.qn, True), kn=up(inp.kn, True), vn=up(inp.vn, True), an=up(inp.alpha_n),
             bn=up(inp.beta_n))
    args10 = [X[k] for k in ("q", "k", "v", "a", "b", "qn", "kn", "vn", "an", "bn")]
    o = torch.empty((T, H, d), dtype=bf, device=dev)
    on = torch.empty_like(o)
    hf = torch.empty((vl.num_docs, H, d, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    n_resp = int(sum(inp.cu_seqlens[i + 1] - inp.cu_seqlens[i] - inp.prompt_lens[i]
                     for i in range(vl.num_docs)))
    C = g.chunk_size()

    def step():
        timer.run("gdn_dual_fwd", lambda: g.gdn_dual_fwd(vl, *args10, B, out=(o, on)))

    result = {}
    if args.only in (None, "fwd", "step"):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        timer.clear()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = 1e3 * wall / args.steps
        fwd_ms = timer.avg_ms("gdn_dual_fwd")
        th_total = T * H
        th_resp = n_resp * H
        alg_bytes = FWD_BYTES_PER_TH * (th_total + th_resp)
        alg_flops = (fwd_flops_per_th(d, C, B, False) * th_total + fwd_flops_per_th(d, C, B, True) * th_resp)
        gbs = alg_bytes / (fwd_ms * 1e-3) / 1e9
        tflops = alg_flops / (fwd_ms * 1e-3) / 1e12
        workload = "gdn_dual_fwd 4x8192 p2048 B4 H16 d128 bf16"
        result.update({
            "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded normal q/k/v, L2-normalised q/k, smooth gates)",
            "config": {"workload": "dual-stream GDN layer forward, 4 docs x 8192 tokens, prompt 2048, "
                                   "B=4, H=16, d_k=d_v=128, bf16 io, fp32 gates/state",
                       "global_batch": 4, "seq_len": 8192, "block_size": B, "heads": H, "head_dim": d,
                       "parallelism": "single GPU", "step": "fwd"},
            "roofline": {"kernel": "gdn_dual_fwd_kernel<bf16,128>", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic_for("gdn_fwd.hip", "gdn_dual_fwd_kernel", workload),
                         "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
                         "kernel_ms": fwd_ms, "mfma_alg_tflops": tflops,
                         "mfma_alg_frac": tflops / MFMA_BF16_PEAK_TFLOPS},
        })
        log("bench: fwd %.3f ms/launch, %.1f GB/s alg (%.1f%% of HBM), %.1f TFLOP/s alg"
            % (fwd_ms, gbs, 100 * gbs / HBM_PEAK_GBS, tflops))

    comps = {}
    if not args.no_components and args.only in (None, "serve"):
        comps["serving"] = bench_serving(torch, g, wl, dev, timer, up, args)
    if not args.no_components and args.only in (None, "conv"):
        comps["shortconv"] = bench_conv(torch, g, wl, dev, timer, up, args)
    if comps:
        result["components"] = comps

    if not args.no_cpu_baseline and args.only is None:
        result["cpu_baseline"] = cpu_baseline(inp)

    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def bench_serving(torch, g, wl, dev, timer, up, args):
    """256 requests x 16 heads, fp32 128x128 states, B=4: 4 EVAL + 1 COMMIT per
    cycle.  Three independently seeded pools are rotated so the 256 MiB of live
    state is not served from the 256 MB last-level cache between calls."""
    log("bench: serving cycle (256 req x 16 heads, 4 EVAL + COMMIT)")
    n_rot = 3
    sets = []
    for r in range(n_rot):
        s = wl.serving(seed=4 + 100 * r)
        blocks = [tuple(up(x, i < 3) for i, x in enumerate(blk)) for blk in s.evals + [s.commit]]
        sets.append((up(s.slot_idx), up(s.pool), blocks))
    R, Bs, H, d = 256, 4, 16, 128
    o = torch.empty((R, Bs, H, d), dtype=torch.bfloat16, device=dev)

    def cycle(i):
        slot, pool, blocks = sets[i % n_rot]
        for e in range(4):
            timer.run("eval", lambda: g.block_step(slot, pool, *blocks[e], g.EVAL, o=o))
        timer.run("commit", lambda: g.block_step(slot, pool, *blocks[4], g.COMMIT, o=o))

    for i in range(max(args.warmup, 3)):
        cycle(i)
    torch.cuda.synchronize()
    timer.clear()
    n = max(args.steps, 6)
    t0 = time.perf_counter()
    for i in range(n):
        cycle(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev, cm = timer.avg_ms("eval"), timer.avg_ms("commit")
    state = R * H * d * d * 4
    io_tok = R * Bs * H * (3 * d * 2 + 8 + d * 2)
    ev_bytes, cm_bytes = state + io_tok, 2 * state + io_tok
    return {"workload": "serving block step, 256 requests x 16 heads, fp32 128x128 states, B=4",
            "eval_ms": ev, "commit_ms": cm, "cycle_ms": 1e3 * wall / n,
            "eval_gbs": ev_bytes / (ev * 1e-3) / 1e9, "commit_gbs": cm_bytes / (cm * 1e-3) / 1e9,
            "eval_hbm_frac": ev_bytes / (ev * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "commit_hbm_frac": cm_bytes / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": R * Bs * 5 / (wall / n), "bound": "hbm",
            "alg_bytes": {"eval": ev_bytes, "commit": cm_bytes}}


def bench_conv(torch, g, wl, dev, timer, up, args):
    log("bench: packed ShortConv (32768 tokens, 8 docs, 12288 channels, W=4)")
    p = wl.packed_conv(round_io=False)
    vl = g.Varlen(p["cu_seqlens"], p["prompt_lens"], dev)
    x, xn, w = up(p["x"], True), up(p["xn"], True), up(p["weight"])
    y, yn = torch.empty_like(x), torch.empty_like(x)
    for _ in range(max(args.warmup, 2)):
        g.shortconv_dual(vl, p["block_size"], x, xn, w, out=(y, yn))
    torch.cuda.synchronize()
    timer.clear()
    n = max(args.steps // 2, 5)
    for _ in range(n):
        timer.run("conv", lambda: g.shortconv_dual(vl, p["block_size"], x, xn, w, out=(y, yn)))
    torch.cuda.synchronize()
    ms = timer.avg_ms("conv")
    T, C = x.shape
    n_resp = int(sum(p["cu_seqlens"][i + 1] - p["cu_seqlens"][i] - p["prompt_lens"][i] for i in range(8)))
    alg = 2 * C * (T + n_resp + 2 * T)  # read x (all), xn (response), write y, yn
    return {"workload": "dual ShortConv, 1 packed row of 32768 tokens, 8 docs, 3x32x128 channels, W=4, bf16",
            "ms": ms, "gbs": alg / (ms * 1e-3) / 1e9, "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes": alg, "tokens_per_s": T / (ms * 1e-3), "bound": "hbm"}


def cpu_baseline(inp):
    """The fp64 oracle, as is, on a bounded sample of the same workload: all
    4 documents at full length for 4 of the 16 heads (scaled to the full head
    count in the reported rate)."""
    import oracle
    heads = [0, 1, 2, 3]
    sub = {name: np.ascontiguousarray(getattr(inp, name)[:, heads])
           for name in ("q", "k", "v", "alpha", "beta", "qn", "kn", "vn", "alpha_n", "beta_n")}
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = min(cores, 16)
    # bf16 values as the GPU sees them
    from gated_deltanet_dual_amd.workloads import round_bf16
    for name in ("q", "k", "v", "qn", "kn", "vn"):
        sub[name] = round_bf16(sub[name])
    t0 = time.perf_counter()
    oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, sub["q"], sub["k"], sub["v"], sub["alpha"],
                        sub["beta"], sub["qn"], sub["kn"], sub["vn"], sub["alpha_n"], sub["beta_n"],
                        inp.block_size, threads=threads)
    dt = time.perf_counter() - t0
    T = inp.T
    frac = len(heads) / inp.H
    return {"value": T * frac / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fwd, all 4 docs x 8192 tokens, heads 0-3 of 16 (rate scaled to 16 heads); "
                      "%.1f s on %d threads (%s)" % (dt, threads, platform.processor() or platform.machine())}


if __name__ == "__main__":
    main()
