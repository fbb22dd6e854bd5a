"""Benchmark of the dual-stream Gated DeltaNet layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-components] [--json-out PATH]
                    [--only step|step_sweep|infer|serve|serve_sweep|conv|layer|routes|memory|copy]

A step is one pass of the layer's hot path over one batch of the headline
workload -- 4 documents x 8192 tokens (prompt 2048, response in blocks of
B = 4), 16 heads, d_k = d_v = 128, bf16 q/k/v with fp32 gates and state:
the dual-stream forward (chunk-start states saved) and the backward.  Inputs are
resident in HBM before the timed region.  Also timed in the same run and
reported under "components": the inference forward; the serving cycle (256
requests x 16 heads, four EVALs + one COMMIT), AR-Trust (verify + scatter, and
the replay pair), the serving conv step; the packed ShortConv and its reverse
mode (32768 tokens, 8 documents, 3x32x128 channels); the packed layer
(unfused, fused, training); the masked route against chunk-then-refine at
blocks of 4 to 32; the training step's device memory with every chunk-start
state kept, with stride-4 checkpoints, and with stride-4 checkpoints in windows
of 32 chunks, against the chunk-then-refine forward.  One JSON line is printed.

Method: "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes),
Overall framework and Key designs items 2-4.
"""
from __future__ import annotations

import argparse
import ctypes
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

# Algorithmic bytes per (token, head) at d = 128, bf16 io, fp32 gates; every
# input read once and every output written once; the noisy stream moves the
# same per response token.
#   forward : q, k, v (3 x 256) + alpha, beta (8) + o (256)             = 1032
#   backward: q, k, v, do (4 x 256) + alpha, beta (8)
#             + dq, dk, dv (3 x 256) + dalpha, dbeta (8)                = 1808
# The chunk-start states the training forward saves (fp32 d x d per chunk
# slot) are written once by the forward and read once by the backward.
FWD_BYTES_PER_TH = 3 * 256 + 8 + 256
BWD_BYTES_PER_TH = 4 * 256 + 8 + 3 * 256 + 8
# the backward pre-pass reads q, k, do and the gates of both streams (not v)
# and the six chunk matrices (their live parts, chunk_matrix_bytes), and hands the reverse scan, per (chunk slot,
# head), R (128 x 128 fp32), W (hi + lo bf16), two fragment sets of K and the
# chunk decay; the scan reads that and writes the chunk's end-state adjoint
# (128 x 128 fp32) and K dS' (32 x 128 fp32) for the per-chunk pass
PRE_BYTES_PER_TH = 3 * 256 + 8
PACK_BYTES_PER_SLOT_HEAD = (128 * 128 + 1024 + 2048 + 2048 + 64) * 4
# the same without the two K fragment sets, which the reverse scan takes from
# the forward's hand-over when the backward reuses the forward's workspace
PRE_PACK_BYTES_PER_SLOT_HEAD = (128 * 128 + 1024 + 64) * 4
SCAN_BYTES_PER_SLOT_HEAD = PACK_BYTES_PER_SLOT_HEAD + 128 * 128 * 4 + 32 * 128 * 4
# the forward's preparation pass reads q, k and the gates of both streams and
# v, and writes the six 32 x 32 fp32 chunk matrices and the hand-over; the
# forward scan reads that and writes the chunk-start states; the output pass
# reads the layer's inputs, the six chunk matrices and the chunk-start states
# and writes o, o~ (FWD_BYTES_PER_TH plus the states) (the forward's hand-over
# carries Z = diag(D) T V, 32 x 128 fp32, in place of the backward's 128 x 128 R)
FWD_PACK_BYTES_PER_SLOT_HEAD = (32 * 128 + 1024 + 2048 + 2048 + 64) * 4
FWD_SCAN_BYTES_PER_SLOT_HEAD = FWD_PACK_BYTES_PER_SLOT_HEAD + 128 * 128 * 4

def chunk_matrix_live_bytes(B, has_noisy, C=32):
    """Bytes of one (chunk, head) record of the six C x C fp32 chunk matrices
    (T, T~, Mwo, Mwq, Mwk, Mw~) that are stored and read: the library moves
    only the 64-byte half-rows whose masks can hold a non-zero entry (T, Mwo:
    j <= i; T~: p_i <= j <= i; Mwq, Mwk: j < p_i; Mw~: j in i's block; the
    noisy four not at all in a chunk without response rows)."""
    live = 0
    for mtx in range(6):
        for row in range(C):
            p = row & -B
            for lo in (0, 16):
                if mtx in (0, 2):
                    on = lo <= row
                elif not has_noisy:
                    on = False
                elif mtx == 1:
                    on = lo <= row and lo + 15 >= p
                elif mtx == 5:
                    on = lo <= p + B - 1 and lo + 15 >= p
                else:
                    on = lo < p
                live += 64 if on else 0
    return live


def chunk_matrix_bytes(cu_seqlens, prompt_lens, H, B, C=32):
    """The chunk-matrix bytes one pass writes or reads for a packed batch."""
    per = {nz: chunk_matrix_live_bytes(B, nz, C) for nz in (False, True)}
    tot = 0
    for i in range(len(prompt_lens)):
        n, P = int(cu_seqlens[i + 1] - cu_seqlens[i]), int(prompt_lens[i])
        for c in range((n + C - 1) // C):
            tot += per[(c * C + C > P) and (P < n)]
    return tot * H
PREP_BYTES_PER_TH = 2 * 256 + 8
STEP_KERNELS = ("gdn_fwd_prep_kernel", "gdn_fwd_scan_kernel", "gdn_dual_fwd_kernel",
                "gdn_bwd_pre_kernel", "gdn_bwd_scan_kernel", "gdn_bwd_chunk_kernel")


def fwd_flops_per_th(d, C, B, noisy):
    """Triangular halves only, chunk C: clean 6d^2 + 5Cd + C^2/3, noisy
    4d^2 + 4Cd + 8Bd."""
    return (4 * d * d + 4 * C * d + 8 * B * d) if noisy else (6 * d * d + 5 * C * d + C * C / 3)


def bwd_flops_per_th(d, C, noisy):
    """Contractions of the chunked backward, same rule: clean 16d^2 + 12Cd,
    noisy 10d^2 + 8Cd."""
    return (10 * d * d + 8 * C * d) if noisy else (16 * d * d + 12 * C * d)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-components", action="store_true")
    p.add_argument("--only", choices=["step", "step_sweep", "infer", "serve", "serve_sweep", "conv", "layer", "routes",
                                      "memory", "copy"], default=None,
                   help="run one part only (copy: a plain 1 GiB device copy, the reference "
                        "transfer for HBM byte counters)")
    p.add_argument("--json-out", default=None)
    return p.parse_args()


class Timer:
    """HIP-event timing of one library call on torch's current stream, which
    is the stream the binding passes to the library."""

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


TRAFFIC_SOURCE = ("profiles/traffic.json: rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, calibrated on a 1 GiB "
                  "copy, taken in a separate counter run of this command; reported only while the kernel's "
                  "sources hash to the recorded value (null otherwise)")


def traffic_for(kernel, workload, field="bytes_per_launch"):
    """Calibrated HBM bytes per launch from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain
    1 GiB copy), or another counter-measured field of the same record (the
    MFMA busy percentage), valid only while the kernel's sources are unchanged
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for f in rec["source_files"].split("+"):
        src = os.path.join(ROOT, "gated_deltanet_dual_amd", "csrc", f)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if rec.get("source_sha") != h.hexdigest()[:16]:
        return None
    return rec.get(field)


def device_copy(torch, dev, args):
    """A plain 1 GiB device-to-device copy: 1 GiB read + 1 GiB written per
    launch, the calibration transfer for FETCH_SIZE / WRITE_SIZE."""
    x = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(max(args.steps, 3)):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": x.numel() * 4, "launches": max(args.steps, 3)}), flush=True)


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
    if args.only == "copy":
        device_copy(torch, dev, args)
        return
    g.lib()
    timer = Timer(torch)
    bf = torch.bfloat16

    def up(x, to_bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(bf) if to_bf16 else t

    result = {}
    comps = {}
    need_headline = args.only in (None, "step", "infer")
    if need_headline:
        result, comps, inp = run_headline(torch, g, wl, dev, timer, up, args)
    if not args.no_components and args.only in (None, "serve"):
        comps["serving"] = bench_serving(torch, g, wl, dev, timer, up, args)
    if not args.no_components and args.only in (None, "conv"):
        comps["shortconv"], comps["shortconv_bwd"] = bench_conv(torch, g, wl, dev, timer, up, args)
    if not args.no_components and args.only in (None, "layer"):
        comps["packed_layer"] = bench_packed_layer(torch, g, wl, dev, timer, up, args)
    if args.only == "step_sweep":
        comps["step_sweep"] = bench_step_sweep(torch, g, wl, dev, up, args)
    if args.only == "serve_sweep":
        comps["serving_sweep"] = bench_serving_sweep(torch, g, dev, args)
    if not args.no_components and args.only in (None, "routes"):
        comps["routes"] = bench_routes(torch, g, wl, dev, timer, up, args)
    if not args.no_components and args.only in (None, "memory"):
        comps["memory"] = bench_memory(torch, g, wl, dev, timer, up, args)
    if comps:
        result["components"] = comps

    if not args.no_cpu_baseline and args.only is None:
        result["cpu_baseline"] = cpu_baseline(inp)

    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def run_headline(torch, g, wl, dev, timer, up, args):
    """The headline step (fwd with checkpoints + bwd) and the inference forward."""
    bf = torch.bfloat16
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
    do, don = up(inp.do, True), up(inp.don, True)
    o = torch.empty((T, H, d), dtype=bf, device=dev)
    on = torch.empty_like(o)
    C = g.chunk_size()
    n_slots = T // C + vl.num_docs
    ckpt = torch.empty((n_slots, H, d, d), dtype=torch.float32, device=dev)
    fws = torch.empty((max(g.workspace_bytes(vl, H, d, B, g.BF16), 256),), dtype=torch.uint8, device=dev)
    g.gdn_dual_fwd(vl, *args10, B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
    ws = torch.empty((g.lib().flare_gdn_dual_workspace_size(vl.ref(), ctypes.byref(g._shape(H, d, B, g.BF16)), 1),),
                     dtype=torch.uint8, device=dev)
    grads = g.gdn_dual_bwd(vl, *args10, B, ckpt, do, don, workspace=ws)
    torch.cuda.synchronize()
    n_resp = int(sum(inp.cu_seqlens[i + 1] - inp.cu_seqlens[i] - inp.prompt_lens[i]
                     for i in range(vl.num_docs)))
    th_total, th_resp = T * H, n_resp * H
    ckpt_bytes = n_slots * H * d * d * 4
    n_chunk_heads = H * sum((int(inp.cu_seqlens[i + 1] - inp.cu_seqlens[i]) + C - 1) // C
                            for i in range(vl.num_docs))
    cm_bytes = chunk_matrix_bytes(inp.cu_seqlens, inp.prompt_lens, H, B, C)

    def step():
        g.gdn_dual_fwd(vl, *args10, B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
        g.gdn_dual_bwd(vl, *args10, B, ckpt, do, don, out=grads, workspace=ws, fwd_workspace=fws)

    result = {}
    comps = {}
    if args.only in (None, "step"):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # the timed steps run with the library's per-launch events off; the
        # per-kernel times come from a second, separate pass of as many steps
        t0 = time.perf_counter()
        for _ in range(args.steps):
            timer.run("step", step)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = timer.avg_ms("step")
        g.timing_reset()
        g.timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        g.timing_enable(False)
        kern = {}
        for name in STEP_KERNELS:
            ms, n = g.timing_avg_ms(name)
            kern[name] = {"ms": ms, "launches": n}
        g.timing_reset()
        alg = {
            "gdn_fwd_prep_kernel": PREP_BYTES_PER_TH * (th_total + th_resp) + 256 * th_total
                                   + FWD_PACK_BYTES_PER_SLOT_HEAD * n_chunk_heads + cm_bytes,
            "gdn_fwd_scan_kernel": FWD_SCAN_BYTES_PER_SLOT_HEAD * n_chunk_heads,
            "gdn_dual_fwd_kernel": FWD_BYTES_PER_TH * (th_total + th_resp) + ckpt_bytes + cm_bytes,
            "gdn_bwd_pre_kernel": PRE_BYTES_PER_TH * (th_total + th_resp) + PRE_PACK_BYTES_PER_SLOT_HEAD * n_chunk_heads
                                  + cm_bytes,
            "gdn_bwd_scan_kernel": SCAN_BYTES_PER_SLOT_HEAD * n_chunk_heads,
            "gdn_bwd_chunk_kernel": BWD_BYTES_PER_TH * (th_total + th_resp) + ckpt_bytes,
        }
        fwd_flops = fwd_flops_per_th(d, C, B, False) * th_total + fwd_flops_per_th(d, C, B, True) * th_resp
        bwd_flops = bwd_flops_per_th(d, C, False) * th_total + bwd_flops_per_th(d, C, True) * th_resp
        step_bytes = (FWD_BYTES_PER_TH + BWD_BYTES_PER_TH) * (th_total + th_resp) + 2 * ckpt_bytes
        step_flops = fwd_flops + bwd_flops
        t_roof = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        dom = max(kern, key=lambda k: kern[k]["ms"] or 0.0)
        kms = kern[dom]["ms"]
        gbs = alg[dom] / (kms * 1e-3) / 1e9
        workload = "fwd(ckpt)+bwd 4x8192 p2048 B4 H16 d128 bf16"
        result.update({
            "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded normal q/k/v, L2-normalised q/k, smooth gates, normal upstream grads)",
            "config": {"workload": "dual-stream GDN layer forward (training, chunk-start states saved) + "
                                   "backward, 4 docs x 8192 tokens, prompt 2048, B=4, H=16, d_k=d_v=128, "
                                   "bf16 io, fp32 gates/state",
                       "global_batch": 4, "seq_len": 8192, "block_size": B, "heads": H, "head_dim": d,
                       "parallelism": "single GPU", "step": "fwd+bwd"},
            "roofline": {"kernel": dom, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic_for(dom, workload),
                         "traffic_source": TRAFFIC_SOURCE,
                         "alg_bytes_per_launch": alg[dom], "kernel_ms": kms,
                         "mfma_busy_pct": traffic_for(dom, workload, "mfma_util_pct")},
            "kernels": {k: dict(v, alg_bytes=alg[k],
                                alg_gbs=(alg[k] / (v["ms"] * 1e-3) / 1e9) if v["ms"] else None,
                                mfma_busy_pct=traffic_for(k, workload, "mfma_util_pct"))
                        for k, v in kern.items()},
            "step_roofline": {"alg_bytes": step_bytes, "alg_flops": step_flops, "t_roof_ms": 1e3 * t_roof,
                              "frac": 1e3 * t_roof / ms_step,
                              "hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "mfma_alg_frac": step_flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                              "wall_ms_per_step": 1e3 * wall / args.steps},
        })
        log("bench: step %.3f ms (%s), roofline frac %.3f"
            % (ms_step, ", ".join("%s %.3f ms" % (k, v["ms"] or -1) for k, v in kern.items()),
               1e3 * t_roof / ms_step))

    if not args.no_components and args.only in (None, "infer"):
        comps["fwd_inference"] = bench_infer(torch, g, vl, args10, B, o, on, fws, timer, args,
                                             th_total, th_resp, fwd_flops_per_th(d, C, B, False) * th_total
                                             + fwd_flops_per_th(d, C, B, True) * th_resp)
    return result, comps, inp


def bench_infer(torch, g, vl, args10, B, o, on, fws, timer, args, th_total, th_resp, flops):
    """The forward alone, inference mode (nothing saved)."""
    log("bench: forward, inference mode")
    for _ in range(args.warmup):
        g.gdn_dual_fwd(vl, *args10, B, out=(o, on), want_h_final=False, workspace=fws)
    torch.cuda.synchronize()
    timer.clear()
    for _ in range(args.steps):
        timer.run("infer", lambda: g.gdn_dual_fwd(vl, *args10, B, out=(o, on), want_h_final=False, workspace=fws))
    torch.cuda.synchronize()
    ms = timer.avg_ms("infer")
    alg = FWD_BYTES_PER_TH * (th_total + th_resp)
    return {"workload": "dual-stream GDN forward, inference, 4 x 8192 tokens, B=4, H=16, d=128, bf16",
            "ms": ms, "tokens_per_s": vl.total_tokens / (ms * 1e-3), "alg_bytes": alg, "alg_flops": flops,
            "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_alg_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def bench_serving(torch, g, wl, dev, timer, up, args):
    """256 requests x 16 heads, fp32 128x128 states, B=4.  EVAL and COMMIT are
    each timed alone with three independently seeded pools rotated call by
    call, so no timed call finds its 256 MiB of states in the 256 MB
    last-level cache (the reported eval/commit figures); the serving cycle (4
    EVAL + 1 COMMIT on one pool set, sets rotated per cycle) is timed as a
    whole, and within it EVALs 2-4 may find the states still cached."""
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
            g.block_step(slot, pool, *blocks[e], g.EVAL, o=o)
        g.block_step(slot, pool, *blocks[4], g.COMMIT, o=o)

    n = max(args.steps, 6)
    # cold calls: consecutive calls read different pools (3 x 256 MiB)
    for i in range(max(args.warmup, 3)):
        slot, pool, blocks = sets[i % n_rot]
        g.block_step(slot, pool, *blocks[0], g.EVAL, o=o)
    torch.cuda.synchronize()
    timer.clear()
    for i in range(3 * n):
        slot, pool, blocks = sets[i % n_rot]
        timer.run("eval", lambda: g.block_step(slot, pool, *blocks[i % 4], g.EVAL, o=o))
    for i in range(3 * n):
        slot, pool, blocks = sets[i % n_rot]
        timer.run("commit", lambda: g.block_step(slot, pool, *blocks[4], g.COMMIT, o=o))
    torch.cuda.synchronize()
    ev, cm = timer.avg_ms("eval"), timer.avg_ms("commit")
    for i in range(max(args.warmup, 3)):
        cycle(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        cycle(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same cycle captured once per pool set as a HIP graph (the library
    # launches on torch's current stream, so torch's capture records it) and
    # replayed: the launch gaps between the five kernels go away
    def plain_cycle(i):  # no timing events inside a capture
        slot, pool, blocks = sets[i % n_rot]
        for e in range(4):
            g.block_step(slot, pool, *blocks[e], g.EVAL, o=o)
        g.block_step(slot, pool, *blocks[4], g.COMMIT, o=o)

    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plain_cycle(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(n_rot):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            plain_cycle(r)
        graphs.append(gph)
    torch.cuda.synchronize()
    for i in range(max(args.warmup, 3)):
        graphs[i % n_rot].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        graphs[i % n_rot].replay()
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - t0
    del graphs
    state = R * H * d * d * 4
    io_tok = R * Bs * H * (3 * d * 2 + 8 + d * 2)
    ev_bytes, cm_bytes = state + io_tok, 2 * state + io_tok

    # AR-Trust: verify K = 4 drafted tokens (the state after each kept as a
    # candidate), then scatter the accepted one; accepted counts ~ U{0..K},
    # seeded, on the device
    K = Bs
    cand = torch.empty((R, K, H, d, d), dtype=torch.float32, device=dev)
    gen = np.random.default_rng(45)
    acc = [up(gen.integers(0, K + 1, R).astype(np.int32)) for _ in range(n_rot)]
    n_acc = [int(np.count_nonzero(a.cpu().numpy())) for a in acc]

    def ar_cycle(i):
        slot, pool, blocks = sets[i % n_rot]
        timer.run("verify", lambda: g.gdn_verify(slot, pool, *blocks[4], o=o, cand=cand))
        timer.run("scatter", lambda: g.gdn_scatter(slot, acc[i % n_rot], cand, pool))

    for i in range(max(args.warmup, 3)):
        ar_cycle(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        ar_cycle(i)
    torch.cuda.synchronize()
    ar_wall = time.perf_counter() - t0
    vf, sc = timer.avg_ms("verify"), timer.avg_ms("scatter")

    # the replay form of the same rollback: the causal outputs without
    # candidates, then the COMMIT of each accepted prefix (same counts)
    def replay_cycle(i):
        slot, pool, blocks = sets[i % n_rot]
        timer.run("verify_out", lambda: g.gdn_verify_outputs(slot, pool, *blocks[4], o=o))
        timer.run("commit_prefix", lambda: g.gdn_commit_prefix(slot, pool, *blocks[4], acc[i % n_rot]))

    for i in range(max(args.warmup, 3)):
        replay_cycle(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        replay_cycle(i)
    torch.cuda.synchronize()
    rp_wall = time.perf_counter() - t0
    vo, cp = timer.avg_ms("verify_out"), timer.avg_ms("commit_prefix")

    # the same EVAL / COMMIT with the ShortConv in front: raw bf16 projections,
    # W = 4 clean histories per slot, SiLU, q/k L2 norm
    Wc = 4
    crng = np.random.default_rng(46)
    cws = [up(crng.uniform(-0.5, 0.5, (H * d, Wc)).astype(np.float32)) for _ in range(3)]
    caches = [torch.randn((512, Wc - 1, 3, H * d), generator=torch.Generator(device=dev).manual_seed(47 + r),
                          device=dev).to(torch.bfloat16) for r in range(n_rot)]

    def conv_cycle(i):
        slot, pool, blocks = sets[i % n_rot]
        for e in range(4):
            timer.run("eval_conv", lambda: g.block_step_conv(slot, pool, caches[i % n_rot], cws, *blocks[e], g.EVAL,
                                                             activation=1, o=o))
        timer.run("commit_conv", lambda: g.block_step_conv(slot, pool, caches[i % n_rot], cws, *blocks[4], g.COMMIT,
                                                           activation=1, o=o))

    for i in range(max(args.warmup, 3)):
        conv_cycle(i)
    torch.cuda.synchronize()
    for i in range(n):
        conv_cycle(i)
    torch.cuda.synchronize()
    evc, cmc = timer.avg_ms("eval_conv"), timer.avg_ms("commit_conv")
    hist = R * H * (Wc - 1) * 3 * d * 2  # the histories read (and written back by COMMIT)
    evc_bytes, cmc_bytes = ev_bytes + hist, cm_bytes + 2 * hist
    vf_bytes = state + io_tok + K * state  # pool read, block io, K candidate states written
    sc_bytes = 2 * float(np.mean(n_acc)) * H * d * d * 4  # accepted candidates read, slots written
    # the prefix commit reads and writes the slots with an accepted token, and
    # the drafted block's io
    cp_bytes = 2 * float(np.mean(n_acc)) * H * d * d * 4 + io_tok
    return {"workload": "serving block step, 256 requests x 16 heads, fp32 128x128 states, B=4",
            "eval_ms": ev, "commit_ms": cm, "timing": "eval/commit: each call alone, pools rotated per call "
                                                      "(states never in the last-level cache)",
            "cycle_ms": 1e3 * wall / n,
            "eval_gbs": ev_bytes / (ev * 1e-3) / 1e9, "commit_gbs": cm_bytes / (cm * 1e-3) / 1e9,
            "eval_hbm_frac": ev_bytes / (ev * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "commit_hbm_frac": cm_bytes / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": R * Bs * 5 / (wall / n), "bound": "hbm",
            "graph_cycle_ms": 1e3 * graph_wall / n, "graph_tokens_per_s": R * Bs * 5 / (graph_wall / n),
            "alg_bytes": {"eval": ev_bytes, "commit": cm_bytes, "verify": vf_bytes, "scatter": sc_bytes},
            "with_conv": {"eval_ms": evc, "commit_ms": cmc, "eval_gbs": evc_bytes / (evc * 1e-3) / 1e9,
                          "commit_gbs": cmc_bytes / (cmc * 1e-3) / 1e9,
                          "eval_hbm_frac": evc_bytes / (evc * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "commit_hbm_frac": cmc_bytes / (cmc * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "alg_bytes": {"eval": evc_bytes, "commit": cmc_bytes}},
            "ar_trust": {"verify_ms": vf, "scatter_ms": sc, "cycle_ms": 1e3 * ar_wall / n,
                         "verify_gbs": vf_bytes / (vf * 1e-3) / 1e9, "scatter_gbs": sc_bytes / (sc * 1e-3) / 1e9,
                         "verify_hbm_frac": vf_bytes / (vf * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "scatter_hbm_frac": sc_bytes / (sc * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "drafted_tokens_per_s": R * K / (ar_wall / n),
                         "replay": {"verify_outputs_ms": vo, "commit_prefix_ms": cp, "cycle_ms": 1e3 * rp_wall / n,
                                    "verify_outputs_gbs": ev_bytes / (vo * 1e-3) / 1e9,
                                    "commit_prefix_gbs": cp_bytes / (cp * 1e-3) / 1e9,
                                    "alg_bytes": {"verify_outputs": ev_bytes, "commit_prefix": cp_bytes},
                                    "drafted_tokens_per_s": R * K / (rp_wall / n)}}}


CONV_WORKLOAD = "packed conv 32768 tokens 8 docs 12288 ch W4 bf16"


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
    fwd = {"workload": "dual ShortConv, 1 packed row of 32768 tokens, 8 docs, 3x32x128 channels, W=4, bf16",
           "ms": ms, "gbs": alg / (ms * 1e-3) / 1e9, "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "alg_bytes": alg, "tokens_per_s": T / (ms * 1e-3), "bound": "hbm",
           "traffic": traffic_for("shortconv_dual_kernel", CONV_WORKLOAD)}
    # ---- reverse mode on the same inputs; output gradients ~ N(0, 1) drawn on
    # the device from a seeded generator
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    dy = torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16)
    dyn = torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16)
    W = w.shape[1]
    dx, dxn = torch.empty_like(x), torch.empty_like(x)
    dw = torch.empty((C, W), dtype=torch.float32, device=dev)
    db = torch.empty((C,), dtype=torch.float32, device=dev)
    ws = torch.empty((g.shortconv_dual_bwd_workspace_bytes(vl, p["block_size"], C, W),), dtype=torch.uint8,
                     device=dev)

    def bwd():
        return g.shortconv_dual_bwd(vl, p["block_size"], x, xn, w, dy, dyn, workspace=ws, out=(dx, dxn, dw, db))

    for _ in range(max(args.warmup, 2)):
        bwd()
    torch.cuda.synchronize()
    for _ in range(n):
        timer.run("conv_bwd", bwd)
    torch.cuda.synchronize()
    bms = timer.avg_ms("conv_bwd")
    # read x, dy (all rows), xn, dyn (response rows); write dx, dxn
    balg = 2 * C * (4 * T + 2 * n_resp)
    bwd_d = {"workload": "dual ShortConv reverse mode, same row and shape, bf16 (dx, dx~, dweight, dbias)",
             "ms": bms, "gbs": balg / (bms * 1e-3) / 1e9, "hbm_frac": balg / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "alg_bytes": balg, "tokens_per_s": T / (bms * 1e-3), "bound": "hbm",
             "traffic": traffic_for("shortconv_dual_bwd_kernel", CONV_WORKLOAD)}
    return fwd, bwd_d


def bench_packed_layer(torch, g, wl, dev, timer, up, args):
    """The layer's whole input side on the packed row (32768 tokens, 8 docs,
    32 heads x 128, W=4, bf16): ShortConv on q, k, v of both streams, q/k L2
    norm, dual GDN.  Unfused: three flare_shortconv_dual calls, then the GDN
    forward with its q/k L2 flag.  Fused: flare_qkv_prologue, then the GDN
    forward without flags.  Conv in the loads: flare_gdn_dual_fwd_conv, the
    ShortConv formed where the GDN kernels load their rows (no rows written).
    Training: the fused forward with chunk-start states, the GDN backward and
    the prologue's reverse mode."""
    log("bench: packed layer (32768 tokens, 8 docs, 32 heads x 128, ShortConv W=4 + L2 + dual GDN)")
    bf = torch.bfloat16
    p = wl.packed_conv(round_io=False)
    B, H, d = p["block_size"], p["H"], p["d"]
    vl = g.Varlen(p["cu_seqlens"], p["prompt_lens"], dev)
    x, xn, w = up(p["x"], True), up(p["xn"], True), up(p["weight"])
    T, C3 = x.shape
    C = C3 // 3
    xs = [x[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    xns = [xn[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    ws_ = [w[s * C:(s + 1) * C].contiguous() for s in range(3)]
    del x, xn
    gates = [up(p[k]) for k in ("alpha", "beta", "alpha_n", "beta_n")]
    ys, yns = [torch.empty_like(t) for t in xs], [torch.empty_like(t) for t in xs]
    hv = lambda t: t.view(T, H, d)
    o = torch.empty((T, H, d), dtype=bf, device=dev)
    on = torch.empty_like(o)
    fws = torch.empty((max(g.workspace_bytes(vl, H, d, B, g.BF16, g.QK_L2NORM),
                           g.workspace_bytes(vl, H, d, B, g.BF16), 256),), dtype=torch.uint8, device=dev)

    def gdn_args(q, k, v, qn, kn, vn):
        return [hv(q), hv(k), hv(v), gates[0], gates[1], hv(qn), hv(kn), hv(vn), gates[2], gates[3]]

    def unfused():
        for s in range(3):
            g.shortconv_dual(vl, B, xs[s], xns[s], ws_[s], out=(ys[s], yns[s]))
        g.gdn_dual_fwd(vl, *gdn_args(*ys, *yns), B, flags=g.QK_L2NORM, out=(o, on), want_h_final=False,
                       workspace=fws)

    def fused():
        g.qkv_prologue(vl, B, d, xs, xns, ws_, out=(ys, yns))
        g.gdn_dual_fwd(vl, *gdn_args(*ys, *yns), B, out=(o, on), want_h_final=False, workspace=fws)

    def conv_in_load():  # the ShortConv formed where the GDN kernels load q, k, v: no rows written
        g.gdn_dual_fwd_conv(vl, xs, xns, ws_, *gates, B, activation=0, flags=g.QK_L2NORM, out=(o, on),
                            want_h_final=False, workspace=fws)

    n = max(args.steps // 2, 3)
    res = {}
    for name, fn in (("unfused_fwd", unfused), ("fused_fwd", fused), ("conv_in_load_fwd", conv_in_load)):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        for _ in range(n):
            timer.run(name, fn)
        torch.cuda.synchronize()
        res[name] = timer.avg_ms(name)
    # training: fused prologue -> GDN forward with states -> GDN backward -> prologue reverse mode
    Cs = g.chunk_size()
    ckpt = torch.empty((T // Cs + vl.num_docs, H, d, d), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(33)
    do = torch.randn((T, H, d), generator=gen, device=dev).to(bf)
    don = torch.randn((T, H, d), generator=gen, device=dev).to(bf)
    bws = torch.empty((g.lib().flare_gdn_dual_workspace_size(vl.ref(), ctypes.byref(g._shape(H, d, B, g.BF16)), 1),),
                      dtype=torch.uint8, device=dev)
    pws = torch.empty((g.qkv_prologue_bwd_workspace_bytes(vl, B, H, d, ws_[0].shape[1]),), dtype=torch.uint8,
                      device=dev)
    g.qkv_prologue(vl, B, d, xs, xns, ws_, out=(ys, yns))
    g.gdn_dual_fwd(vl, *gdn_args(*ys, *yns), B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
    grads = g.gdn_dual_bwd(vl, *gdn_args(*ys, *yns), B, ckpt, do, don, workspace=bws, fwd_workspace=fws)
    dxs, dxns = [torch.empty_like(t) for t in xs], [torch.empty_like(t) for t in xs]
    dws = [torch.empty_like(t) for t in ws_]
    flat = lambda t: t.view(T, H * d)

    def train():
        g.qkv_prologue(vl, B, d, xs, xns, ws_, out=(ys, yns))
        g.gdn_dual_fwd(vl, *gdn_args(*ys, *yns), B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
        g.gdn_dual_bwd(vl, *gdn_args(*ys, *yns), B, ckpt, do, don, out=grads, workspace=bws, fwd_workspace=fws)
        g.qkv_prologue_bwd(vl, B, d, xs, xns, ws_, [flat(grads[k]) for k in ("dq", "dk", "dv")],
                           [flat(grads[k]) for k in ("dqn", "dkn", "dvn")], workspace=pws, out=(dxs, dxns, dws))

    for _ in range(max(args.warmup, 1)):
        train()
    torch.cuda.synchronize()
    for _ in range(n):
        timer.run("train", train)
    torch.cuda.synchronize()
    res["train"] = timer.avg_ms("train")
    out = {"workload": "packed row 32768 tokens, 8 docs, H=32, d=128, B=4, ShortConv W=4 on q/k/v + q/k L2 + dual GDN, bf16"}
    for k, ms in res.items():
        out[k] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3)}
    out["fused_speedup_fwd"] = res["unfused_fwd"] / res["fused_fwd"]
    out["conv_in_load_speedup_fwd"] = res["unfused_fwd"] / res["conv_in_load_fwd"]
    # one pass of the projections: x (all rows) and x~ (response rows) read, o, o~ written
    n_resp = int(sum(p["cu_seqlens"][i + 1] - p["cu_seqlens"][i] - p["prompt_lens"][i] for i in range(vl.num_docs)))
    out["conv_in_load_fwd"]["layer_io_bytes"] = 3 * H * d * 2 * (T + n_resp) + 2 * H * d * 2 * (T + n_resp)
    return out




def bench_step_sweep(torch, g, wl, dev, up, args):
    """The headline step (forward with chunk-start states, backward) at the same
    32768 tokens packed as 4 x 8192, 8 x 4096, 32 x 1024, 128 x 256, 2 x 16384
    and one document of 32768 (prompt a quarter of each document, B = 4, 16 heads,
    d = 128, bf16), with per-kernel times.  Not part of the default run."""
    log("bench: training step against the packing of 32768 tokens")
    H, d, B = 16, 128, 4
    out = {"workload": "dual-stream GDN fwd (states) + bwd, 32768 tokens in N documents, H=16, d=128, B=4, bf16"}
    for ndoc, L in ((4, 8192), (8, 4096), (32, 1024), (128, 256), (2, 16384), (1, 32768)):
        inp = wl.gdn_inputs([L] * ndoc, [L // 4] * ndoc, H, d, d, B, seed=5, with_grads=True, round_io=False)
        a10 = [up(inp.q, True), up(inp.k, True), up(inp.v, True), up(inp.alpha), up(inp.beta), up(inp.qn, True),
               up(inp.kn, True), up(inp.vn, True), up(inp.alpha_n), up(inp.beta_n)]
        do, don = up(inp.do, True), up(inp.don, True)
        vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
        T = inp.T
        o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
        on = torch.empty_like(o)
        ckpt = torch.empty((T // g.chunk_size() + ndoc, H, d, d), dtype=torch.float32, device=dev)
        fws = torch.empty((max(g.workspace_bytes(vl, H, d, B, g.BF16), 256),), dtype=torch.uint8, device=dev)
        ws = torch.empty((g.lib().flare_gdn_dual_workspace_size(vl.ref(), ctypes.byref(g._shape(H, d, B, g.BF16)),
                                                                 1),), dtype=torch.uint8, device=dev)
        g.gdn_dual_fwd(vl, *a10, B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
        grads = g.gdn_dual_bwd(vl, *a10, B, ckpt, do, don, workspace=ws, fwd_workspace=fws)

        def step():
            g.gdn_dual_fwd(vl, *a10, B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
            g.gdn_dual_bwd(vl, *a10, B, ckpt, do, don, out=grads, workspace=ws, fwd_workspace=fws)

        for _ in range(max(args.warmup, 2)):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(args.steps, 5)
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        row = {"ms": ms, "tokens_per_s": T / (ms * 1e-3)}
        # per-kernel times from a separate pass with the library's events on
        g.timing_reset()
        g.timing_enable(True)
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        for k in STEP_KERNELS:
            row[k] = g.timing_avg_ms(k)[0]
        g.timing_enable(False)
        out["%dx%d" % (ndoc, L)] = row
        del a10, do, don, o, on, ckpt, fws, ws, grads
        torch.cuda.empty_cache()
    return out


def bench_serving_sweep(torch, g, dev, args):
    """The serving step's efficiency against the number of requests (64 to
    2048 requests x 16 heads, d = 128, B = 4, bf16): EVAL and COMMIT each
    timed alone over three rotating pools of 2R random fp32 states, so no
    call finds its states in the last-level cache.  Not part of the default
    run."""
    log("bench: serving step against the request count")
    H, d, B = 16, 128, 4
    out = {"workload": "serving block step, R requests x 16 heads, fp32 128x128 states, B=4, bf16, uncached pools"}
    for R in (64, 128, 256, 512, 1024, 2048):
        sets = []
        for r in range(3):
            gen = torch.Generator(device=dev)
            gen.manual_seed(10 + r)
            pool = torch.randn((2 * R, H, d, d), generator=gen, device=dev) / d ** 0.5
            slot = torch.randperm(2 * R, device=dev)[:R].to(torch.int32)
            blk = [torch.randn((R, B, H, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(3)]
            a = torch.rand((R, B, H), generator=gen, device=dev) * 0.15 + 0.85
            b = torch.rand((R, B, H), generator=gen, device=dev) * 0.8 + 0.1
            sets.append((slot, pool, blk, a, b))
        o = torch.empty((R, B, H, d), dtype=torch.bfloat16, device=dev)
        row = {}
        state = R * H * d * d * 4
        io = R * B * H * (3 * d * 2 + 8 + d * 2)
        for mode, name in ((g.EVAL, "eval"), (g.COMMIT, "commit")):
            call = lambda s_: g.block_step(s_[0], s_[1], *s_[2], s_[3], s_[4], mode, o=o)
            for i in range(3):
                call(sets[i % 3])
            torch.cuda.synchronize()
            ev = []
            for i in range(max(args.steps, 12)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call(sets[i % 3])
                e1.record()
                ev.append((e0, e1))
            torch.cuda.synchronize()
            ms = float(np.mean([x.elapsed_time(y) for x, y in ev]))
            alg = (state if mode == g.EVAL else 2 * state) + io
            row[name + "_us"] = 1e3 * ms
            row[name + "_gbs"] = alg / (ms * 1e-3) / 1e9
        out["R%d" % R] = row
        del sets
        torch.cuda.empty_cache()
    return out


def bench_routes(torch, g, wl, dev, timer, up, args):
    """The two ways to give every noisy block its clean boundary state, at the
    dual workload (4 x 4096 tokens, prompt 1024, H=16, d=128, bf16), blocks of
    4 to 32: the masked route (flare_gdn_dual_fwd: boundary states rebuilt on
    chip from chunk-start states, none stored) against chunk-then-refine
    (flare_gdn_dual_fwd_route1: every boundary state stored, then every noisy
    block refined from it).  Both inference forwards; route I also writes the
    chunk-start states it needs."""
    log("bench: masked route vs chunk-then-refine, 4 x 4096 tokens, H=16, d=128, B = 4..32")
    bf = torch.bfloat16
    out = {"workload": "dual-stream GDN forward, 4 x 4096 tokens (prompt 1024), H=16, d=128, bf16"}
    n = max(args.steps // 2, 3)
    for B in (4, 8, 16, 32):
        inp = wl.dual_bf16(block_size=B)
        H, d, T = inp.H, 128, inp.T
        vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
        a10 = [up(inp.q, True), up(inp.k, True), up(inp.v, True), up(inp.alpha), up(inp.beta),
               up(inp.qn, True), up(inp.kn, True), up(inp.vn, True), up(inp.alpha_n), up(inp.beta_n)]
        o = torch.empty((T, H, d), dtype=bf, device=dev)
        on = torch.empty_like(o)
        fws = torch.empty((max(g.workspace_bytes(vl, H, d, B, g.BF16), 256),), dtype=torch.uint8, device=dev)
        shp = g._shape(H, d, B, g.BF16)
        r1_bytes = int(g.lib().flare_gdn_route1_workspace_size(vl.ref(), ctypes.byref(shp)))
        rws = torch.empty((r1_bytes,), dtype=torch.uint8, device=dev)
        ckpt = torch.empty((T // g.chunk_size() + vl.num_docs, H, d, d), dtype=torch.float32, device=dev)
        masked = lambda: g.gdn_dual_fwd(vl, *a10, B, out=(o, on), want_h_final=False, workspace=fws)
        route1 = lambda: g.gdn_dual_fwd_route1(vl, *a10, B, out=(o, on), ckpt=ckpt, workspace=rws,
                                               want_h_final=False)
        row = {}
        for name, fn in (("masked", masked), ("route1", route1)):
            for _ in range(max(args.warmup, 1)):
                fn()
            torch.cuda.synchronize()
            key = "%s_B%d" % (name, B)
            for _ in range(n):
                timer.run(key, fn)
            torch.cuda.synchronize()
            row[name + "_ms"] = timer.avg_ms(key)
        row["route1_workspace_bytes"] = r1_bytes
        row["masked_workspace_bytes"] = int(fws.numel())
        row["route1_over_masked"] = row["route1_ms"] / row["masked_ms"]
        out["B%d" % B] = row
        del a10, o, on, fws, rws, ckpt
        torch.cuda.empty_cache()
    return out


def bench_memory(torch, g, wl, dev, timer, up, args):
    """Device memory of one training step at the headline shape (4 x 8192,
    prompt 2048, B = 4, H = 16, d = 128, bf16), over what the inputs, output
    gradients, outputs and gradients already hold: the step's intermediates
    (checkpoints, workspaces), as torch's peak allocation.  Modes: one pass
    with every chunk-start state kept and the forward's workspace kept for the
    backward (the timed step); stride-4 checkpoints in one pass (the backward
    rebuilds the other states; the forward's workspace freed after it);
    stride-4 checkpoints with both passes in windows of 32 chunks; and the
    chunk-then-refine route's forward, which stores every block-boundary
    state.  Each mode's step time alongside (buffers allocated outside the
    timed region)."""
    log("bench: training-step memory, one pass vs strided checkpoints and windows vs route I")
    bf = torch.bfloat16
    inp = wl.headline(with_grads=True, round_io=False)
    B, H, d, T = inp.block_size, inp.H, 128, inp.T
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    a10 = [up(inp.q, True), up(inp.k, True), up(inp.v, True), up(inp.alpha), up(inp.beta),
           up(inp.qn, True), up(inp.kn, True), up(inp.vn, True), up(inp.alpha_n), up(inp.beta_n)]
    do, don = up(inp.do, True), up(inp.don, True)
    del inp
    o = torch.empty((T, H, d), dtype=bf, device=dev)
    on = torch.empty_like(o)
    grads = {"dq": torch.empty_like(o), "dk": torch.empty_like(o), "dv": torch.empty_like(o),
             "dalpha": torch.empty_like(a10[3]), "dbeta": torch.empty_like(a10[3]),
             "dqn": torch.empty_like(o), "dkn": torch.empty_like(o), "dvn": torch.empty_like(o),
             "dalpha_n": torch.empty_like(a10[3]), "dbeta_n": torch.empty_like(a10[3]), "dh0": None}
    u8 = lambda n: torch.empty((max(int(n), 256),), dtype=torch.uint8, device=dev)

    def ckpt_buf(stride):
        return torch.empty((g.ckpt_slots(vl, H, d, B, g.BF16, stride), H, d, d), dtype=torch.float32, device=dev)

    def train(stride, window, keep_fws, bufs=None):
        """One fwd + bwd; with bufs=None every intermediate is allocated here,
        in the order a training framework holds them, and freed when dead."""
        ck = bufs["ck"] if bufs else ckpt_buf(stride)
        fws = bufs["fws"] if bufs else u8(g.workspace_bytes(vl, H, d, B, g.BF16, window=window))
        g.gdn_dual_fwd(vl, *a10, B, out=(o, on), ckpt=ck, want_h_final=False, workspace=fws, ckpt_stride=stride,
                       window=window)
        if not keep_fws and not bufs:
            del fws
            fws = None
        bws = bufs["bws"] if bufs else u8(g.workspace_bytes(vl, H, d, B, g.BF16, for_bwd=True, stride=stride,
                                                            window=window))
        g.gdn_dual_bwd(vl, *a10, B, ck, do, don, out=grads, workspace=bws, ckpt_stride=stride, window=window,
                       fwd_workspace=fws if keep_fws else None)

    modes = {"one_pass_all_states": (1, 0, True), "one_pass_stride4": (4, 0, False),
             "window32_stride4": (4, 32, False)}
    out = {"workload": "training step (dual forward + backward), 4 x 8192 tokens, prompt 2048, B=4, H=16, d=128, "
                       "bf16; bytes above inputs, output gradients, outputs and gradients"}
    n = max(args.steps // 2, 3)
    for name, (stride, window, keep) in modes.items():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        train(stride, window, keep)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        bufs = {"ck": ckpt_buf(stride), "fws": u8(g.workspace_bytes(vl, H, d, B, g.BF16, window=window)),
                "bws": u8(g.workspace_bytes(vl, H, d, B, g.BF16, for_bwd=True, stride=stride, window=window))}
        for _ in range(max(args.warmup, 1)):
            train(stride, window, keep, bufs)
        torch.cuda.synchronize()
        for _ in range(n):
            timer.run("mem_" + name, lambda: train(stride, window, keep, bufs))
        torch.cuda.synchronize()
        out[name] = {"ckpt_stride": stride, "window_chunks": window, "peak_bytes": int(peak),
                     "ckpt_bytes": int(bufs["ck"].numel() * 4), "fwd_workspace_bytes": int(bufs["fws"].numel()),
                     "bwd_workspace_bytes": int(bufs["bws"].numel()), "ms": timer.avg_ms("mem_" + name)}
        del bufs
    # chunk-then-refine: its forward alone stores every block-boundary state
    shp = g._shape(H, d, B, g.BF16)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    ck = ckpt_buf(1)
    rws = u8(g.lib().flare_gdn_route1_workspace_size(vl.ref(), ctypes.byref(shp)))
    g.gdn_dual_fwd_route1(vl, *a10, B, out=(o, on), ckpt=ck, workspace=rws, want_h_final=False)
    torch.cuda.synchronize()
    n_blocks = sum((8192 - 2048 + B - 1) // B for _ in range(4))
    out["route1_forward"] = {"peak_bytes": int(torch.cuda.max_memory_allocated(dev) - base),
                             "block_states_bytes": n_blocks * H * d * d * 4, "workspace_bytes": int(rws.numel()),
                             "ckpt_bytes": int(ck.numel() * 4)}
    del ck, rws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp):
    """The fp64 oracle, as is, on the same step: forward then backward of the
    whole headline batch (4 documents x 8192 tokens, all 16 heads), on the
    bf16-rounded values the GPU sees, threads over (document, head)."""
    import oracle
    from gated_deltanet_dual_amd.workloads import round_bf16
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = min(cores, 16)
    x = {n: getattr(inp, n) for n in ("q", "k", "v", "alpha", "beta", "qn", "kn", "vn", "alpha_n", "beta_n",
                                      "do", "don")}
    for n in ("q", "k", "v", "qn", "kn", "vn", "do", "don"):
        x[n] = round_bf16(x[n])
    clean = [x[n] for n in ("q", "k", "v", "alpha", "beta")]
    noisy = [x[n] for n in ("qn", "kn", "vn", "alpha_n", "beta_n")]
    t0 = time.perf_counter()
    oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *clean, *noisy, inp.block_size, threads=threads)
    t1 = time.perf_counter()
    oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *clean, *noisy, inp.block_size, x["do"], x["don"],
                        threads=threads)
    t2 = time.perf_counter()
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": inp.T / (t2 - t0), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole step: fp64 forward (%.1f s) + backward (%.1f s) of 4 docs x 8192 tokens, "
                      "16 heads, %d threads on %s" % (t1 - t0, t2 - t1, threads, cpu)}


if __name__ == "__main__":
    main()
