"""Benchmark: backward TFLOPS on selected blocks for 64-token block-sparse attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3|4] [--no-cpu-baseline]

One step runs the whole path once over one batch of synthetic input already resident in HBM:
invert_indices (q2k -> k2q), the forward (o, lse), and the backward chain (preprocess; index stage =
work order; kv-major dK/dV kernel; q-major dQ kernel with the dQ scale/convert fused). Every stage is
bracketed by HIP events on the stream it runs on (torch's current stream, which the binding passes).

  value       = selected-block FLOPs of the backward / time of the backward chain, where
                selected-block FLOPs = pairs * 5 GEMMs * 2*64*64*128 (the FastVideo commit
                message's "TFLOPS on selected blocks", kernels-only window: preprocess -> order ->
                main -> postprocess);
  ms_per_step = mean time of a whole step (invert + forward + backward);
  roofline    = the dominant backward kernel, bwd_dkdv_kernel (kv-major dK/dV): its algorithmic
                FLOPs (4 GEMMs of 2*64*64*128 per selected pair: S, dP, dV, dK) / its mean launch
                duration measured with HIP events on its stream, against the MI355X dense bf16 MFMA
                peak (2.5 PFLOP/s). `traffic` is the bytes per launch that rocprofv3's FETCH_SIZE and
                WRITE_SIZE counters gave (scaled by a plain copy's reading), taken from the committed
                summary in profiles/ while the kernel's sources still hash to the value recorded
                there, else null;
  cpu_baseline= the float64 CPU oracle's backward on a bounded sample of the same workload.

The headline workload is B=1 H=8 S=32768 D=128, 25 % density (default); --workload 4 selects
S=65536 at 12.5 % density. The line also carries, under `secondary`, the other headline workload
and the 524288-token workload (the library's default dQ mode, 2 steps after 1 warm-up; --no-524k
skips it).
`api_backward_ms` times the public V.backward() on its defaults (inverting q2k, default dQ mode,
outputs and workspace from torch's caching allocator), i.e. invert + backward chain, each call
right after a forward as in a step.
--workload 5 times the 524288-token case alone (the library's default dQ mode unless --dq-mode
says otherwise; use few steps, e.g. --steps 3 --warmup 1: a step is a few seconds).
--chunk-blocks sets the backward's chunk width (with the spill: one chunk's dS tiles at a time).
Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "bwd TFLOPS on selected blocks, B=1 H=8 D=128 S=32k/65k; % bf16 MFMA peak"
GEMM_FLOP = 2 * 64 * 64 * 128      # one 64x64x128 GEMM
FLOP_PER_PAIR = 5 * GEMM_FLOP       # the selected-block FLOP count of the backward
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
WORKLOAD_TEXT = {
    3: "VSA 64-token block-sparse attention backward, B=1 H=8 S=32768 D=128 bf16, 25% density "
       "(top-k 128 of 512 kv blocks per q block), all blocks full, o/lse from the GPU forward",
    4: "VSA 64-token block-sparse attention backward, B=1 H=8 S=65536 D=128 bf16, 12.5% density "
       "(top-k 128 of 1024 kv blocks per q block), all blocks full, device work order",
    5: "VSA 64-token block-sparse attention backward, B=1 H=8 S=524288 D=128 bf16, 25% density "
       "(top-k 2048 of 8192 kv blocks per q block), last kv block 40 valid tokens, inputs "
       "0.5*N(0,1)",
}
# (batch, heads, seqlen, q2k row width) of the 524288-token workload, for the default dQ mode
WORKLOAD_SHAPE = {5: (1, 8, 524288, 2048)}


PROFILE = {3: "profiles/backward_S32768_H8_topk128of512.md"}
# the kernel and its launch (grid, work order) from include/vsa.h and vsa_api.hip
KERNEL_SOURCES = ("bwd_dkdv.hip", "vsa_device.h", "vsa_kernels.h", "vsa_api.hip", "../../include/vsa.h")


def counter_traffic(workload, kernel="bwd_dkdv_kernel"):
    """Bytes per launch of `kernel` from the committed rocprofv3 summary, or None when there is no
    summary for this workload or the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, PROFILE.get(workload, "-"))
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.normpath(os.path.join(ROOT, "block_sparse_attention_attn_amd", "csrc", n)),
                  "rb") as f:
            h.update(f.read())
    section, traffic, sha = None, None, None
    for line in open(path):
        if line.startswith("### "):
            section = line[4:].strip()
        elif section == kernel and line.startswith("- traffic_bytes_per_launch:"):
            traffic = int(line.split(":")[1])
        elif section == kernel and line.startswith("- source_sha256:"):
            sha = line.split(":")[1].split()[0]
    return traffic if sha == h.hexdigest() else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_workload(n, steps, warmup, dq_mode, api_steps=0, chunk_blocks=0):
    import torch

    import block_sparse_attention_attn_amd as V
    import workloads

    dev = "cuda:0"
    c = workloads.config(n)
    pairs = c.pairs
    q, k, v, do = (t.to(dev) for t in (c.q, c.k, c.v, c.do))
    idx, num, vbs = c.q2k_idx.to(dev), c.q2k_num.to(dev), c.vbs.to(dev)
    # buffers allocated once; every step rewrites them
    o = torch.empty_like(q)
    lse = torch.empty(c.B, c.H, c.S, dtype=torch.float32, device=dev)
    k2q_idx = torch.empty(c.B, c.H, c.nb, c.nb, dtype=torch.int32, device=dev)
    k2q_num = torch.empty(c.B, c.H, c.nb, dtype=torch.int32, device=dev)
    inv_ws = torch.empty(V.invert_workspace_bytes(c.B, c.H, c.nb, c.nb), dtype=torch.uint8,
                         device=dev)
    plan = V.BwdPlan(do, q, k, v, o, lse, k2q_idx, k2q_num, vbs, q2k_idx=idx, q2k_num=num,
                     dq_mode=dq_mode, chunk_blocks=chunk_blocks)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        V.invert_indices(idx, num, c.nb, workspace=inv_ws, out=(k2q_idx, k2q_num))
        if ev is not None:
            ev[1].record()
        V.forward(q, k, v, idx, num, vbs, out=(o, lse))
        if ev is not None:
            ev[2].record()
        for i, s in enumerate((plan.PREPROCESS, plan.INDEX, plan.DKDV, plan.DQ)):
            plan.stage(s)
            if ev is not None:
                ev[3 + i].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    def span(e, a, b):
        return [x[a].elapsed_time(x[b]) for x in e]

    invert = span(evs, 0, 1)
    fwd = span(evs, 1, 2)
    bwd = span(evs, 2, 6)
    pre, index, dkdv, dq = (span(evs, 2 + i, 3 + i) for i in range(4))
    total = t_start.elapsed_time(t_end) / steps
    res = dict(
        workload=n, pairs=pairs, ms_per_step=total, wall_s=wall,
        bwd_ms=statistics.mean(bwd), bwd_ms_median=statistics.median(bwd),
        invert_ms=statistics.mean(invert), fwd_ms=statistics.mean(fwd),
        pre_ms=statistics.mean(pre), index_ms=statistics.mean(index),
        dkdv_ms=statistics.mean(dkdv), dkdv_ms_median=statistics.median(dkdv),
        dq_ms=statistics.mean(dq), dq_ms_median=statistics.median(dq))
    res["bwd_tflops"] = pairs * FLOP_PER_PAIR / (res["bwd_ms"] * 1e-3) / 1e12
    # executed MFMA work: 4 GEMMs per pair in the dK/dV kernel; 3 in the recomputing dQ kernel,
    # 1 in the spill one, which reads 8 KiB of dS per pair from HBM
    spill = dq_mode == V.DQ_SPILL
    # a chunked spill (spill mode whose kv-major kernel runs in chunks) runs the dQ launches inside
    # the DKDV stage, after each chunk's kv-major launch: dkdv_ms then covers both kernels
    cb = chunk_blocks if chunk_blocks != 0 else (V.CHUNK_BLOCKS if c.nb >= V.CHUNK_MIN_KV_BLOCKS
                                                 else 0)
    res["dq_in_dkdv_stage"] = spill and 0 < cb < c.nb
    if res["dq_in_dkdv_stage"]:
        res["dkdv_dq_tflops"] = pairs * 5 * GEMM_FLOP / (res["dkdv_ms"] * 1e-3) / 1e12
    else:
        res["dkdv_tflops"] = pairs * 4 * GEMM_FLOP / (res["dkdv_ms"] * 1e-3) / 1e12
        res["dq_tflops"] = pairs * (1 if spill else 3) * GEMM_FLOP / (res["dq_ms"] * 1e-3) / 1e12
        if spill:
            res["dq_ds_read_GBps"] = pairs * 8192 / (res["dq_ms"] * 1e-3) / 1e9
    res["fwd_tflops"] = pairs * 2 * GEMM_FLOP / (res["fwd_ms"] * 1e-3) / 1e12
    del plan
    torch.cuda.empty_cache()
    if api_steps:
        # the public entry a caller uses, on its defaults: inverts q2k, picks the dQ mode
        # (default_dq_mode) and allocates outputs and workspace through torch's caching
        # allocator. Each call follows a forward, as the backward chain does in a step, and the
        # events bracket the call alone (its inversion included).
        for _ in range(2):
            V.backward(do, q, k, v, o, lse, idx, num, vbs)
        torch.cuda.synchronize()
        api = []
        for _ in range(api_steps):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            V.forward(q, k, v, idx, num, vbs, out=(o, lse))
            a0.record()
            V.backward(do, q, k, v, o, lse, idx, num, vbs)
            a1.record()
            api.append((a0, a1))
        torch.cuda.synchronize()
        res["api_backward_ms"] = statistics.mean(a0.elapsed_time(a1) for a0, a1 in api)
        res["api_dq_mode"] = "spill" if V.default_dq_mode(c.B, c.H, c.S, idx.shape[-1]) == V.DQ_SPILL \
            else "recompute"
        torch.cuda.empty_cache()
    return res, c


def cpu_baseline(c, budget_s=15.0):
    """The oracle's backward, q block by q block of head 0, until ~budget_s of CPU work."""
    import numpy as np
    from oracle import vsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    Q, K, V_, DO = (O.f64(t[0, 0]) for t in (c.q, c.k, c.v, c.do))
    idx = c.q2k_idx[:1, :1]
    num = c.q2k_num[:1, :1]
    done_pairs = 0
    blocks = 0
    t0 = time.perf_counter()
    while blocks < c.nb and (time.perf_counter() - t0 < budget_s or blocks < 4):
        keys = O.kept_keys(idx, num, c.vbs, 0, 0, blocks)
        rows = slice(blocks * 64, (blocks + 1) * 64)
        O.qblock_backward(Q[rows], DO[rows], K[keys], V_[keys], c.sm_scale)
        done_pairs += int(num[0, 0, blocks])
        blocks += 1
    dt = time.perf_counter() - t0
    return dict(value=done_pairs * FLOP_PER_PAIR / dt / 1e12, unit="TFLOPS", cores=int(threads),
                kind="oracle",
                sample=f"float64 numpy oracle backward (recomputing each q block's softmax) over q "
                       f"blocks 0..{blocks - 1} of head 0 of the same workload: {done_pairs} "
                       f"selected pairs in {dt:.1f} s; BLAS threads {threads}, "
                       f"os.cpu_count()={os.cpu_count()}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=(3, 4, 5))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-524k", action="store_true",
                    help="skip the 524288-token secondary leg (about a minute, mostly input "
                         "generation)")
    ap.add_argument("--dq-mode", choices=("spill", "recompute"), default=None,
                    help="dQ from dS tiles the dK/dV kernel spills to the workspace (8 KiB per "
                         "pair), or recomputed from Q, K, V, dO; default: spill, and for "
                         "--workload 5 the library's default_dq_mode")
    ap.add_argument("--chunk-blocks", type=int, default=0,
                    help="the backward's chunk_blocks (0: the library's choice, < 0: no chunks); "
                         "with chunks the spill holds one chunk's dS tiles")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (a known byte count for "
                         "scaling hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path: the work shards over (batch, head) with no exchange", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read, 268435456 bytes written")
        del src, dst
    log(f"[bench] workload {args.workload}: steps={args.steps} warmup={args.warmup}")
    import block_sparse_attention_attn_amd as V
    if args.dq_mode is None:
        if args.workload == 5:
            c5 = WORKLOAD_SHAPE[5]
            mode = V.default_dq_mode(*c5, chunk_blocks=args.chunk_blocks, device="cuda:0")
        else:
            mode = V.DQ_SPILL
    else:
        mode = V.DQ_SPILL if args.dq_mode == "spill" else V.DQ_RECOMPUTE
    res, case = run_workload(args.workload, args.steps, args.warmup, mode,
                             api_steps=10 if args.workload != 5 else 0,
                             chunk_blocks=args.chunk_blocks)
    log(f"[bench] {json.dumps(res)}")
    secondary = None
    if not args.no_secondary and args.workload != 5:
        secondary = []
        others = [4 if args.workload == 3 else 3]
        if not args.no_524k:
            others.append(5)
        for other in others:
            log(f"[bench] secondary workload {other}")
            if other == 5:  # a step takes about 1.6 s; the library's default dQ mode
                mode2 = V.default_dq_mode(*WORKLOAD_SHAPE[5], device="cuda:0")
                r2, _ = run_workload(5, 2, 1, mode2)
            else:
                mode2 = mode
                r2, _ = run_workload(other, max(5, args.steps // 2), max(2, args.warmup // 2), mode)
            log(f"[bench] {json.dumps(r2)}")
            secondary.append(dict(
                workload=WORKLOAD_TEXT[other], steps=2 if other == 5 else max(5, args.steps // 2),
                bwd_tflops=round(r2["bwd_tflops"], 2), bwd_ms=round(r2["bwd_ms"], 4),
                fwd_ms=round(r2["fwd_ms"], 4), dkdv_ms=round(r2["dkdv_ms"], 4),
                dq_ms=round(r2["dq_ms"], 4),
                dq_mode="spill" if mode2 == V.DQ_SPILL else "recompute",
                frac_of_peak=round(r2["bwd_tflops"] / PEAK_BF16_TFLOPS, 4)))
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(case)
        log(f"[bench] cpu {json.dumps(cpu)}")

    # the dominant kernel; with a chunked spill its stage also holds the dQ launches
    achieved = res["dkdv_tflops"] if "dkdv_tflops" in res else res["dkdv_dq_tflops"]
    line = {
        "metric": METRIC,
        "value": round(res["bwd_tflops"], 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT[args.workload],
            "global_batch": case.B,
            "seq_len": case.S,
            "heads": case.H,
            "head_dim": 128,
            "selected_pairs": res["pairs"],
            "dq_mode": "spill" if mode == V.DQ_SPILL else "recompute",
            "chunk_blocks": args.chunk_blocks,
            "parallelism": "none (1 GPU)",
        },
        "frac_of_peak": round(res["bwd_tflops"] / PEAK_BF16_TFLOPS, 4),
        "breakdown_ms": {k: round(res[k], 4) for k in ("invert_ms", "fwd_ms", "pre_ms", "index_ms",
                                                      "dkdv_ms", "dq_ms", "bwd_ms")},
        "api_backward_ms": round(res["api_backward_ms"], 4) if "api_backward_ms" in res else None,
        "api_dq_mode": res.get("api_dq_mode"),
        "roofline": {
            "kernel": "bwd_dkdv_kernel" if "dkdv_tflops" in res
                      else "bwd_dkdv_kernel + bwd_dq_spill_kernel (chunked spill, 5 GEMMs)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": counter_traffic(args.workload),
            "traffic_unit": "bytes per launch (FETCH_SIZE x copy factor + WRITE_SIZE)",
        },
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
