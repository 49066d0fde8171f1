#!/usr/bin/env python3
"""Benchmark of one GPU's share of the Ulysses sequence-parallel hot path.

Workload (video-DiT share): world Q/K/V [B=1, S=32760, H=40, D=128] bf16,
seeded synthetic N(0,1) with Q scaled by 1/sqrt(128), SP degree P = 8
(token ranges 8 x 4095, head groups 8 x 5). One step is rank 0's share of the
path, every row of it:

  ranges   token / head boundaries (host)
  pack     rank 0's token shard [1, 4095, 40, 128] of Q, K and V into the 8
           head-group blocks [1, 32760, 5, 128] (the data rank 0 sends in the
           first all-to-all; the other ranks' rows were placed beforehand)
  attn     non-causal attention over the full sequence on block 0 (h = 5)
  unpack   rank 0's rows of the 8 output blocks back to [1, 4095, 40, 128]

value = attention flops of a step (4 * S^2 * D * h = 2.7474e12) / step time.
Also reported: the attention kernel alone (HIP events around each launch on
the launch stream), and the world-tensor pack / unpack bandwidth of the full
[1, 32760, 40, 128] tensor (read + write bytes / time, buffers rotated so
the 256 MB last-level cache cannot serve repeats).

cpu_baseline: the float64 CPU oracle on a bounded sample of query rows of
the same attention, on every host core this process may use.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + % MFMA peak at S=32760,h=5,D=128; pack/unpack GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def cpu_baseline(q, k, v, h0, S, D, target_s):
    """Time the oracle (float64 NumPy, process pool over host cores) on a
    sample of query rows of heads [0, h0); returns the cpu_baseline object."""
    from oracle import attention as A
    from ulysses_sequence_attention_amd import synth

    qf, kf, vf = (synth.bf16_bits_to_f32(np.ascontiguousarray(x[:, :, :h0])).astype(np.float64)
                  for x in (q, k, v))
    cores = A.host_cores()
    rng = np.random.default_rng(123)
    # calibrate on one core
    t0 = time.perf_counter()
    A.attention_rows(qf, kf, vf, 0, 0, np.arange(64))
    per_row = (time.perf_counter() - t0) / 64
    n = int(max(64, min(S, target_s * cores / (per_row * h0))))
    rows = {(0, hd): np.sort(rng.choice(S, n, replace=False)) for hd in range(h0)}
    t0 = time.perf_counter()
    A.attention_parallel(qf, kf, vf, rows_per_head=rows, workers=cores)
    wall = time.perf_counter() - t0
    flops = 4.0 * S * D * n * h0
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} query rows x {h0} heads of the S={S}, D={D} attention "
                      f"({flops:.3e} flop, {wall:.1f} s wall, float64 NumPy, "
                      f"{cores} worker processes x 1 BLAS thread)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--relayout-reps", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-relayout-bw", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not "
              "supported (the multi-GPU exchange is not part of this build)", file=sys.stderr)
        sys.exit(2)

    import ulysses_sequence_attention_amd as usp
    from ulysses_sequence_attention_amd import synth

    w = synth.WORKLOADS["video_dit_share"]
    B, S, H, D, P = w.B, w.S, w.H, w.D, w.P
    print(f"[bench] drawing inputs {B}x{S}x{H}x{D} bf16", file=sys.stderr, flush=True)
    q, k, v = synth.draw_workload(w)
    tb = usp.usp_balanced_ranges(S, P)
    hb = usp.usp_balanced_ranges(H, P)
    h0, len0 = hb[1] - hb[0], tb[1] - tb[0]
    attn_flops = 4.0 * B * h0 * S * S * D

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(q, k, v, h0, S, D, args.cpu_seconds)

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    world = [bf(x) for x in (q, k, v)]
    del q, k, v
    shard = [x[:, tb[0]:tb[1]].contiguous() for x in world]
    blocks = [[torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=torch.bfloat16, device=dev)
               for j in range(P)] for _ in range(3)]
    for x, bl in zip(world, blocks):   # every rank's rows, as received in the exchange
        usp.usp_pack_seq_to_heads(x, bl)
    oblocks = [torch.zeros((B, S, hb[j + 1] - hb[j], D), dtype=torch.bfloat16, device=dev)
               for j in range(P)]
    oshard = torch.empty((B, len0, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        for x, bl in zip(shard, blocks):
            usp.usp_pack_seq_to_heads(x, bl, rank=0)
        if ev is not None:
            ev[0].record()
        usp.usp_attention_fwd(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0])
        if ev is not None:
            ev[1].record()
        usp.usp_unpack_heads_to_seq(oblocks, oshard, rank=0)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12

    rel = {}
    if not args.skip_relayout_bw:
        # world pack / unpack of the full [1, 32760, 40, 128] tensor, 3 rotating buffer sets
        print("[bench] world pack/unpack bandwidth", file=sys.stderr, flush=True)
        nbytes = B * S * H * D * 2
        srcs = [world[0]] + [torch.empty_like(world[0]).copy_(world[0]) for _ in range(2)]
        dsts = [[torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=torch.bfloat16, device=dev)
                 for j in range(P)] for _ in range(3)]
        for name, fn in (("pack", lambda i: usp.usp_pack_seq_to_heads(srcs[i % 3], dsts[i % 3])),
                         ("unpack", lambda i: usp.usp_unpack_heads_to_seq(dsts[i % 3], srcs[i % 3]))):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(args.relayout_reps):
                fn(i)
            b_.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b_) / args.relayout_reps
            gbs = 2.0 * nbytes / (ms * 1e-3) / 1e9
            rel[name] = {"us": ms * 1e3, "GB/s": gbs, "frac_peak": gbs / PEAK_HBM_GBS,
                         "bytes_rw": 2 * nbytes}

    out = {
        "metric": METRIC,
        "value": attn_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "video_dit_share", "B": B, "S": S, "H": H, "h": h0, "D": D,
                   "P": P, "rank": 0,
                   "step": "pack rank-0 shard of q,k,v -> attention on head group 0 over "
                           "the full sequence -> unpack rank-0 rows"},
        "attention": {"ms": attn_ms, "TFLOP/s": attn_tflops,
                      "frac_peak": attn_tflops / PEAK_BF16_TFLOPS, "flop": attn_flops},
        "relayout_world": rel,
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
