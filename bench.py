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
  attn     non-causal attention over the full sequence on block 0 (h = 5),
           usp_attention_fwd_ws with its workspace allocated beforehand
  unpack   rank 0's rows of the 8 output blocks back to [1, 4095, 40, 128]

The attention of usp_attention_fwd (no workspace; the same bits) is timed
on its own as well and reported as "attention_no_workspace", and
usp_attention_fwd_gqa (with a workspace) on rank 0's share of the grouped
video-DiT workload (40 query heads over 8 K/V heads: 5 query heads and one
K/V head per rank) as "attention_gqa". "rows_world" reports the model-boundary
row movements at the same share's hidden size ([1, 32760, 5120] bf16 over 8
ranks, world mode): scatter and gather (read + write of the tensor) and the
reduce-scatter of 8 partials (8 reads + 1 write), buffers rotated like the
relayouts'. "ring" reports one rank's ring pass of Ulysses+Ring on the
video-DiT sequence over a 4 (Ulysses) x 2 (ring) grid: ring block 0, head
group 0 (10 heads, 16380 query rows) attends to its own K/V block and then to
ring block 1's (usp_attention_fwd_block, fp32 outputs and lse), and
usp_attention_merge folds the two into the bf16 output; its flops are
4 * Sq * S * D * h = 2.7474e12. The second block's attention runs on a
second stream (its own workspace), as a ring would launch it on arrival, and
the fold waits for it; the one-stream pass is reported beside it. "chunked" times usp_attention_fwd_chunked on
the long-sequence share (B=1, S=131072, h=8, D=128, 3 head-chunk passes of
3/3/2 heads; 7.04e13 flop), and usp_attention_fwd_chunked_ws (workspace
sized for the 3-head pass), next to the single-shot usp_attention_fwd on the
same inputs (all the same bits). "two_phase" runs the same step as the
head-chunked two-phase exchange: for each chunk of the 5 heads (2/2/1), pack
rank 0's rows of those heads of Q, K and V (usp_pack_seq_to_heads_chunk),
attention on those heads of block 0, unpack them
(usp_unpack_heads_to_seq_chunk; "relayout_world" also times one such chunk
of the world tensor alone, heads [0, 2) of every group). Pipelined, a
chunk's pack for the next step and its unpack for this step run on the
second stream as soon as this step's attention of that chunk is done, under
the attention of the following chunks; "serial_*" runs the same phases on
one stream. The output is checked bitwise against the single-shot step.

Steps run pipelined: step i + 1's pack and step i's unpack are issued on a
second stream (default priority) so that they run under the attention of the
neighbouring step (the relayout waves fit beside the attention workgroups on
a CU), with two sets of head and output blocks and stream-ordered events that
keep each step's pack before its attention and its unpack after it. Every
step still does all of its work; the timed region holds exactly K packs, K
attention calls and K unpacks, and the output is checked bitwise against a
serial step. The same steps run serially (one stream) are reported as
"step_serial", with per-kernel HIP events.

value = attention flops of a step (4 * S^2 * D * h = 2.7474e12) / step time.
Also reported: each kernel alone (HIP events around each launch on the
launch stream), the world-tensor pack / unpack bandwidth of the full
[1, 32760, 40, 128] tensor (read + write bytes / time, buffers rotated so the
256 MB last-level cache cannot serve repeats), and a plain device copy of
1 GiB as the practical HBM reference.

cpu_baseline: the float64 CPU oracle on a bounded sample of query rows of
the same attention, on every host core this process may use.

roofline: the attention call (usp_attention_fwd_ws: the key-half flash
kernel, then the merge kernel) is the dominant step; ``achieved`` is its
flops over its event-timed duration.
roofline.traffic: HBM bytes per attention call from rocprofv3 FETCH_SIZE /
WRITE_SIZE counter runs (both kernels), each scaled by what the counter reads
for the plain copy kernel of known size in the same run (``--pmc-summary``);
reported only while the attention source is the one the counters were taken
on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
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
ATTN_SRC = os.path.join(ROOT, "ulysses_sequence_attention_amd", "csrc", "attn_bf16.hip")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "attn_video_dit_share_traffic.json")
COPY_BYTES = 1 << 30


def source_digest(path=ATTN_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def cpu_baseline(q, k, v, h0, S, D, target_s):
    """Time the oracle (float64 NumPy, process pool over host cores) on a
    sample of query rows of heads [0, h0); returns the cpu_baseline object."""
    from oracle import attention as A
    from ulysses_sequence_attention_amd import synth

    qf, kf, vf = (synth.bf16_bits_to_f32(np.ascontiguousarray(x[:, :, :h0])).astype(np.float64)
                  for x in (q, k, v))
    cores = A.host_cores()
    rng = np.random.default_rng(123)
    # calibrate on one core (512 rows, so that copying the head's K/V planes
    # weighs little), then size the sample for about target_s of wall time
    t0 = time.perf_counter()
    A.attention_rows(qf, kf, vf, 0, 0, np.arange(512))
    per_row = (time.perf_counter() - t0) / 512
    n = int(max(64, min(S, target_s * cores / (per_row * h0))))
    rows = {(0, hd): (np.arange(S) if n >= S else np.sort(rng.choice(S, n, replace=False)))
            for hd in range(h0)}
    t0 = time.perf_counter()
    A.attention_parallel(qf, kf, vf, rows_per_head=rows, workers=cores)
    wall = time.perf_counter() - t0
    flops = 4.0 * S * D * n * h0
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"all {S} query rows" if n >= S else f"{n} query rows") +
                      f" x {h0} heads of the S={S}, D={D} attention "
                      f"({flops:.3e} flop, {wall:.1f} s wall, float64 NumPy, "
                      f"{cores} worker processes x 1 BLAS thread)"}


def stored_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("traffic_bytes_per_launch")


def kernel_kind(name):
    """Short name of a kernel of this benchmark from its rocprofv3 name."""
    return ("attention" if "attn_bf16_kernel<128, 8, 1, 2," in name else
            "attention_groups" if "attn_bf16_kernel<128, 8, 2, 1," in name else
            "merge" if "attn_merge_halves" in name else
            "copy" if "copyBuffer" in name else
            "pack" if "relayout_kernel<true>" in name else
            "unpack" if "relayout_kernel<false>" in name else None)


def read_pmc(dirs):
    """rocprofv3 --pmc CSVs under ``dirs`` -> {(kind, counter): {dispatch: value}},
    each value summed over the counter's instances (SEs, SIMDs, channels)."""
    per = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    kind = kernel_kind(r["Kernel_Name"])
                    if kind is None:
                        continue
                    key = (kind, r["Counter_Name"])
                    per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                    per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
                    if "End_Timestamp" in r:
                        per.setdefault((kind, "_duration_ns"), {})[r["Dispatch_Id"]] = (
                            float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
                    for col in ("VGPR_Count", "Accum_VGPR_Count", "LDS_Block_Size", "Workgroup_Size"):
                        if col in r:
                            per.setdefault((kind, "_" + col), {})[r["Dispatch_Id"]] = float(r[col])
    return per


# per-dispatch algorithmic flops of the video-DiT share's attention (all of it
# runs in the key-half kernel; the merge does no matrix work)
ATTN_FLOPS = 4.0 * 5 * 32760 * 32760 * 128


def sq_summary(dirs, out_txt):
    """Summarise rocprofv3 --pmc runs of SQ/GRBM counters of this benchmark:
    per-kernel mean per dispatch of every counter, and for the attention
    kernel the matrix flops the counters imply against the algorithmic
    flops, the matrix-core busy fraction and the LDS figures."""
    per = read_pmc(dirs)
    avg = {k: float(np.mean(list(v.values()))) for k, v in per.items()}
    lines = [f"# kernel source: attn_bf16.hip sha256 {source_digest()}", "",
             "kernel           counter                          mean/dispatch  dispatches"]
    for (kind, ctr), val in sorted(avg.items()):
        if kind == "copy":
            continue
        lines.append(f"{kind:16s} {ctr:32s} {val:14.6g}  {len(per[(kind, ctr)])}")
    a = {c: v for (k, c), v in avg.items() if k == "attention"}
    if a:
        lines.append("")
        lines.append("attention kernel (usp_attention_fwd_ws key-half walk), derived:")
        dur = a.get("_duration_ns")
        if dur:
            lines.append(f"  duration {dur / 1e3:.1f} us per dispatch under the profiler "
                         f"(counters serialise dispatches)")
        mops = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops is not None:
            lines.append(f"  matrix flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = {mops * 512:.4e} "
                         f"against {ATTN_FLOPS:.4e} algorithmic ({mops * 512 / ATTN_FLOPS:.4f}x)")
        n_mfma = a.get("SQ_INSTS_MFMA")
        if n_mfma is not None:
            lines.append(f"  MFMA instructions {n_mfma:.4e} x 32768 flop (32x32x16) = "
                         f"{n_mfma * 32768:.4e} ({n_mfma * 32768 / ATTN_FLOPS:.4f}x algorithmic)")
        busy, gui = a.get("SQ_VALU_MFMA_BUSY_CYCLES"), a.get("GRBM_GUI_ACTIVE")
        if busy is not None and gui:
            # GRBM_GUI_ACTIVE counts each XCD's active cycles (8 instances):
            # the kernel's cycles are gui / 8; 1024 SIMDs
            cyc = gui / 8
            lines.append(f"  GRBM_GUI_ACTIVE / 8 XCDs = {cyc:.4e} cycles"
                         + (f" (= {cyc / (dur * 1e-9) / 1e9:.3f} GHz over the dispatch)" if dur else ""))
            lines.append(f"  matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) = "
                         f"{busy / (1024 * cyc):.3f}")
        coex = a.get("SQ_VALU_MFMA_COEXEC_CYCLES")
        if coex is not None and busy:
            lines.append(f"  VALU issued while the matrix core is busy: {coex / busy:.3f} of busy cycles")
        if a.get("SQ_INSTS_LDS") and a.get("SQ_INSTS_MFMA"):
            lines.append(f"  LDS instructions per MFMA: {a['SQ_INSTS_LDS'] / a['SQ_INSTS_MFMA']:.3f}")
        if a.get("SQ_INSTS_LDS_LOAD_BANDWIDTH") is not None and n_mfma:
            lb = a["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64
            lines.append(f"  LDS bytes loaded {lb:.4e} = {lb / n_mfma:.0f} B per MFMA")
        bc, act = a.get("SQ_LDS_BANK_CONFLICT"), a.get("SQ_LDS_IDX_ACTIVE")
        if bc is not None and act:
            lines.append(f"  LDS bank-conflict cycles / LDS active cycles = {bc / act:.4f}")
        if a.get("SQ_INSTS_VALU_TRANS_F32") is not None:
            lines.append(f"  transcendental VALU instructions {a['SQ_INSTS_VALU_TRANS_F32']:.4e} "
                         f"(one exp2 per score: {5 * 32760 * 32760 / 64:.4e} wave instructions)")
    text = "\n".join(lines)
    print(text)
    if out_txt:
        with open(out_txt, "w") as f:
            f.write(text + "\n")


def pmc_summary(dirs, out_json):
    """Parse rocprofv3 --pmc counter CSVs (FETCH_SIZE and WRITE_SIZE runs of
    this benchmark) into per-kernel KiB per dispatch, calibrate both counters
    on the plain copy kernel (COPY_BYTES read and written per dispatch), and
    write the attention kernel's HBM traffic per launch to ``out_json``."""
    per = read_pmc(dirs)
    # the runtime's copy kernel also serves small copies (a clone, a compare):
    # calibrate on the 1 GiB copies only, the dispatches of at least half the
    # largest count
    for key in [k for k in per if k[0] == "copy"]:
        mx = max(per[key].values())
        per[key] = {d: v for d, v in per[key].items() if v >= 0.5 * mx}
    avg = {k: float(np.mean(list(v.values()))) for k, v in per.items()}
    lines = ["kernel     counter      KiB/dispatch  dispatches"]
    for (kind, ctr), val in sorted(avg.items()):
        lines.append(f"{kind:10s} {ctr:12s} {val:12.1f}  {len(per[(kind, ctr)])}")
    f_copy = avg.get(("copy", "FETCH_SIZE"))
    w_copy = avg.get(("copy", "WRITE_SIZE"))
    ff = COPY_BYTES / (f_copy * 1024) if f_copy else None
    fw = COPY_BYTES / (w_copy * 1024) if w_copy else None
    lines.append(f"copy calibration ({COPY_BYTES} B read and written per dispatch): "
                 f"FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}" if ff and fw else
                 "copy calibration missing")
    res = {"source_sha256": source_digest(), "fetch_factor": ff, "write_factor": fw}
    for kind in ("attention", "merge", "attention_groups", "pack", "unpack"):
        f_k, w_k = avg.get((kind, "FETCH_SIZE")), avg.get((kind, "WRITE_SIZE"))
        if f_k is not None and w_k is not None and ff and fw:
            rb, wb = f_k * 1024 * ff, w_k * 1024 * fw
            res[kind] = {"read_bytes": rb, "write_bytes": wb}
            lines.append(f"{kind}: HBM read {rb / 1e6:.1f} MB + write {wb / 1e6:.1f} MB per "
                         f"dispatch (calibrated)")
    if "attention" in res:
        # one usp_attention_fwd_ws call = one key-half flash dispatch + one merge
        res["traffic_bytes_per_launch"] = sum(
            res[k]["read_bytes"] + res[k]["write_bytes"] for k in ("attention", "merge")
            if k in res)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--relayout-reps", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-relayout-bw", action="store_true")
    ap.add_argument("--skip-gqa", action="store_true", help="skip the grouped-head attention timing")
    ap.add_argument("--skip-rows", action="store_true", help="skip the row-movement timings")
    ap.add_argument("--skip-ring", action="store_true", help="skip the Ulysses+Ring pass timing")
    ap.add_argument("--skip-chunked", action="store_true", help="skip the head-chunked timing")
    ap.add_argument("--skip-two-phase", action="store_true",
                    help="skip the two-phase (per head chunk) step timing")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 counter runs of this benchmark and exit")
    ap.add_argument("--pmc-sq", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 SQ/GRBM counter runs of this benchmark and exit")
    ap.add_argument("--pmc-out", metavar="FILE", help="text file for --pmc-sq's summary")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args.pmc_summary, TRAFFIC_JSON)
        return
    if args.pmc_sq:
        sq_summary(args.pmc_sq, args.pmc_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not "
              "supported: it runs on one GPU (the multi-GPU exchange is not implemented)", file=sys.stderr)
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

    def ev():
        return torch.cuda.Event(enable_timing=True)

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
    ws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, h0, D) // 4,
                     dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(e=None):
        if e is not None:
            e[0].record()
        for x, bl in zip(shard, blocks):
            usp.usp_pack_seq_to_heads(x, bl, rank=0)
        if e is not None:
            e[1].record()
        usp.usp_attention_fwd_ws(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0], ws)
        if e is not None:
            e[2].record()
        usp.usp_unpack_heads_to_seq(oblocks, oshard, rank=0)
        if e is not None:
            e[3].record()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    print(f"[bench] timing {args.steps} serial steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    pack_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    unpack_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    elem = 2  # bf16
    share_bytes = 2 * B * len0 * H * D * elem   # one tensor, read + write

    # the same steps pipelined: two sets of head and output blocks, the
    # relayouts on a second stream (default priority) under the neighbouring
    # steps' attention; stream-ordered events keep every step's pack before its
    # attention and its unpack after it, and no set is rewritten while read
    print("[bench] pipelined steps", file=sys.stderr, flush=True)
    main_s = torch.cuda.current_stream()
    io_s = torch.cuda.Stream()
    bsets = [blocks, [[torch.empty_like(t) for t in bl] for bl in blocks]]
    for x, bl in zip(world, bsets[1]):   # every rank's rows in the second set too
        usp.usp_pack_seq_to_heads(x, bl)
    osets = [oblocks, [torch.zeros_like(t) for t in oblocks]]
    ev_pack = [torch.cuda.Event() for _ in range(2)]
    ev_attn = [torch.cuda.Event() for _ in range(2)]
    ev_unp = [torch.cuda.Event() for _ in range(2)]
    for e in ev_attn + ev_unp:
        e.record(main_s)

    def p_pack(i):
        st = i % 2
        io_s.wait_event(ev_attn[st])      # set st was last read by attention i - 2
        for x, bl in zip(shard, bsets[st]):
            usp.usp_pack_seq_to_heads(x, bl, rank=0, stream=io_s)
        ev_pack[st].record(io_s)

    def p_attn(i):
        st = i % 2
        main_s.wait_event(ev_pack[st])
        main_s.wait_event(ev_unp[st])     # output set st was last read by unpack i - 2
        usp.usp_attention_fwd_ws(bsets[st][0][0], bsets[st][1][0], bsets[st][2][0], osets[st][0],
                                 ws, stream=main_s)
        ev_attn[st].record(main_s)

    def p_unpack(i):
        st = i % 2
        io_s.wait_event(ev_attn[st])
        usp.usp_unpack_heads_to_seq(osets[st], oshard, rank=0, stream=io_s)
        ev_unp[st].record(io_s)

    def pipelined(n, start=None):
        if start is not None:
            io_s.wait_event(start)
        p_pack(0)
        for i in range(n):
            p_attn(i)
            if i + 1 < n:
                p_pack(i + 1)
            p_unpack(i)
        main_s.wait_event(ev_unp[(n - 1) % 2])

    pipelined(args.warmup)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} pipelined steps", file=sys.stderr, flush=True)
    a, b_ = ev(), ev()
    a.record(main_s)
    pipelined(args.steps, start=a)
    b_.record(main_s)
    torch.cuda.synchronize()
    pipe_ms = a.elapsed_time(b_) / args.steps
    # the pipelined steps must leave exactly what a serial step leaves
    pipe_out = oshard.clone()
    step()
    torch.cuda.synchronize()
    if not torch.equal(pipe_out, oshard):
        raise RuntimeError("pipelined steps produced a different output than a serial step")
    del bsets[1], osets[1], pipe_out

    # the two-phase exchange on the same share: per head chunk (2/2/1 of the
    # 5 heads), pack rank 0's rows of the chunk's heads, attention on them,
    # unpack them. Overlapped: the next chunk's pack and this chunk's unpack
    # run on the second stream under the attention (they touch other heads).
    two_phase = None
    if not args.skip_two_phase:
        print("[bench] two-phase steps", file=sys.stderr, flush=True)
        kc = usp.usp_head_chunk_ranges(h0, 3)
        ch = [(kc[c], kc[c + 1]) for c in range(len(kc) - 1)]
        ws_c = torch.empty(usp.usp_attention_workspace_bytes(
            usp.USP_BF16, B, S, max(hi - lo for lo, hi in ch), D) // 4, dtype=torch.float32, device=dev)
        e_cp = [torch.cuda.Event() for _ in ch]
        e_ca = [torch.cuda.Event() for _ in ch]

        def tp_pack(c, stream):
            for x, bl in zip(shard, blocks):
                usp.usp_pack_seq_to_heads_chunk(x, bl, ch[c][0], ch[c][1], rank=0, stream=stream)

        def tp_attn(c):
            usp.usp_attention_fwd_ws(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0], ws_c,
                                     head_lo=ch[c][0], head_hi=ch[c][1], stream=main_s)

        def tp_unpack(c, stream):
            usp.usp_unpack_heads_to_seq_chunk(oblocks, oshard, ch[c][0], ch[c][1], rank=0,
                                              stream=stream)

        def tp_serial():
            for c in range(len(ch)):
                tp_pack(c, main_s)
                tp_attn(c)
                tp_unpack(c, main_s)

        e_cu = [torch.cuda.Event() for _ in ch]
        for e in e_ca + e_cu:
            e.record(main_s)

        def tp_pipelined(n):
            # chunk c of step i + 1 is packed, and chunk c of step i unpacked,
            # as soon as step i's attention of chunk c is done (it has read
            # those heads and written its output), i.e. under the attention
            # of the following chunks; an attention of chunk c waits for the
            # pack of its own step and the unpack of the previous one
            io_s.wait_stream(main_s)
            for c in range(len(ch)):
                io_s.wait_event(e_ca[c])
                tp_pack(c, io_s)
                e_cp[c].record(io_s)
            for i in range(n):
                for c in range(len(ch)):
                    main_s.wait_event(e_cp[c])
                    main_s.wait_event(e_cu[c])
                    tp_attn(c)
                    e_ca[c].record(main_s)
                for c in range(len(ch)):
                    io_s.wait_event(e_ca[c])
                    if i + 1 < n:
                        tp_pack(c, io_s)
                        e_cp[c].record(io_s)
                    tp_unpack(c, io_s)
                    e_cu[c].record(io_s)
            main_s.wait_stream(io_s)

        def tp_serial_n(n):
            for _ in range(n):
                tp_serial()

        tp = {}
        for name, fn in (("serial", tp_serial_n), ("pipelined", tp_pipelined)):
            fn(args.warmup)
            torch.cuda.synchronize()
            a, b_ = ev(), ev()
            a.record(main_s)
            fn(args.steps)
            b_.record(main_s)
            torch.cuda.synchronize()
            tp[name] = a.elapsed_time(b_) / args.steps
            got = oshard.clone()
            step()
            torch.cuda.synchronize()
            if not torch.equal(got, oshard):
                raise RuntimeError(f"two-phase ({name}) steps differ from a single-shot step")
        two_phase = {"chunks": kc, "ms_per_step": tp["pipelined"],
                     "TFLOP/s": attn_flops / (tp["pipelined"] * 1e-3) / 1e12,
                     "serial_ms_per_step": tp["serial"],
                     "serial_TFLOP/s": attn_flops / (tp["serial"] * 1e-3) / 1e12,
                     "how": "per head chunk: pack rank-0 rows of its heads (q, k, v) -> "
                            "attention on its heads of block 0 -> unpack; pipelined: a chunk's "
                            "pack for the next step and unpack for this step on a second stream "
                            "as soon as this step's attention of that chunk is done",
                     "bitwise_equal_single_shot": True}
        del ws_c

    # usp_attention_fwd (no workspace) on the same block, for comparison
    print("[bench] attention without workspace", file=sys.stderr, flush=True)
    for _ in range(3):
        usp.usp_attention_fwd(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0])
    reps = max(3, args.steps // 10)
    a, b_ = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        usp.usp_attention_fwd(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0])
    b_.record()
    torch.cuda.synchronize()
    nows_ms = a.elapsed_time(b_) / reps

    # grouped K/V heads: rank 0's share of the grouped video-DiT workload
    gqa = None
    if not args.skip_gqa:
        print("[bench] attention with grouped K/V heads", file=sys.stderr, flush=True)
        gw = synth.WORKLOADS["gqa_video_share"]
        gq, gk, gv = synth.draw_workload(gw)
        ghq = usp.usp_balanced_ranges(gw.H, gw.P)
        ghk = usp.usp_balanced_ranges(gw.kv_heads, gw.P)
        q0 = bf(gq[:, :, ghq[0]:ghq[1]])
        k0, v0 = (bf(x[:, :, ghk[0]:ghk[1]]) for x in (gk, gv))
        del gq, gk, gv
        o0 = torch.empty_like(q0)
        gh, ghkv = ghq[1] - ghq[0], ghk[1] - ghk[0]
        gws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, gw.B, gw.S, gh, gw.D) // 4,
                          dtype=torch.float32, device=dev)
        for _ in range(3):
            usp.usp_attention_fwd_gqa(q0, k0, v0, o0, ws=gws)
        a, b_ = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            usp.usp_attention_fwd_gqa(q0, k0, v0, o0, ws=gws)
        b_.record()
        torch.cuda.synchronize()
        g_ms = a.elapsed_time(b_) / reps
        g_flops = 4.0 * gw.B * gh * gw.S * gw.S * gw.D
        gqa = {"workload": "gqa_video_share", "h": gh, "h_kv": ghkv, "S": gw.S, "D": gw.D,
               "ms": g_ms, "TFLOP/s": g_flops / (g_ms * 1e-3) / 1e12,
               "entry": "usp_attention_fwd_gqa (workspace)"}
        del q0, k0, v0, o0, gws

    # one rank's Ulysses+Ring pass: two key blocks, then the merge
    ring = None
    if not args.skip_ring:
        print("[bench] Ulysses+Ring pass", file=sys.stderr, flush=True)
        rw = synth.WORKLOADS["video_dit_ring"]
        rq, rk, rv = (bf(x) for x in synth.draw_workload(rw))
        rT = usp.usp_balanced_ranges(rw.S, rw.ring)
        rc = usp.usp_balanced_ranges(rw.H, rw.P)
        rh = rc[1] - rc[0]

        def head_group0(x, i):
            bl = [torch.empty((rw.B, rT[i + 1] - rT[i], rc[j + 1] - rc[j], rw.D),
                              dtype=torch.bfloat16, device=dev) for j in range(rw.P)]
            usp.usp_pack_seq_to_heads(x[:, rT[i]:rT[i + 1]], bl)
            return bl[0]

        qr = head_group0(rq, 0)
        kvr = [(head_group0(rk, i), head_group0(rv, i)) for i in range(rw.ring)]
        del rq, rk, rv
        Sq = rT[1] - rT[0]
        rws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, rw.B, Sq, rh, rw.D) // 4,
                          dtype=torch.float32, device=dev)
        o_acc = torch.empty((rw.B, Sq, rh, rw.D), dtype=torch.float32, device=dev)
        o_blk = torch.empty_like(o_acc)
        l_acc = torch.empty((rw.B, rh, Sq), dtype=torch.float32, device=dev)
        l_blk = torch.empty_like(l_acc)
        o_out = torch.empty((rw.B, Sq, rh, rw.D), dtype=torch.bfloat16, device=dev)
        order = [0] + [(0 - i) % rw.ring for i in range(1, rw.ring)]

        def ring_pass(e=None):
            if e is not None:
                e[0].record()
            usp.usp_attention_fwd_block(qr, *kvr[order[0]], o_acc, lse=l_acc, ws=rws)
            for n, i in enumerate(order[1:]):
                usp.usp_attention_fwd_block(qr, *kvr[i], o_blk, lse=l_blk, ws=rws)
                if e is not None:
                    e[1].record()
                last = n == len(order) - 2
                usp.usp_attention_merge(o_acc, l_acc, o_blk, l_blk, o_out if last else o_acc,
                                        None if last else l_acc)
            if e is not None:
                e[2].record()

        for _ in range(3):
            ring_pass()
        revs = [[ev() for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            ring_pass(revs[i])
        torch.cuda.synchronize()
        r_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in revs]))
        m_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in revs]))
        serial_out = o_out.clone()

        # the same pass with the other blocks' attention on a second stream
        # (each with its own workspace and output buffers): a ring delivers
        # the next block long before the current one is done, so its launch
        # can fill the CUs the current launch leaves idle at its tail; the
        # folds stay in ring order on the first stream
        side = torch.cuda.Stream()
        rws2 = torch.empty_like(rws)
        o_b2 = [o_blk, torch.empty_like(o_blk)]
        l_b2 = [l_blk, torch.empty_like(l_blk)]
        ev_blk = [torch.cuda.Event() for _ in range(2)]
        ev_fold = [torch.cuda.Event() for _ in range(2)]
        main_r = torch.cuda.current_stream()

        def ring_pass_2s():
            start = torch.cuda.Event()
            start.record(main_r)
            side.wait_event(start)
            for e in ev_fold:
                e.record(main_r)
            usp.usp_attention_fwd_block(qr, *kvr[order[0]], o_acc, lse=l_acc, ws=rws, stream=main_r)
            for n, i in enumerate(order[1:]):
                bset = n % 2
                side.wait_event(ev_fold[bset])   # buffer set read by the fold two blocks back
                usp.usp_attention_fwd_block(qr, *kvr[i], o_b2[bset], lse=l_b2[bset], ws=rws2,
                                            stream=side)
                ev_blk[bset].record(side)
                main_r.wait_event(ev_blk[bset])
                last = n == len(order) - 2
                usp.usp_attention_merge(o_acc, l_acc, o_b2[bset], l_b2[bset],
                                        o_out if last else o_acc, None if last else l_acc,
                                        stream=main_r)
                ev_fold[bset].record(main_r)

        for _ in range(3):
            ring_pass_2s()
        torch.cuda.synchronize()
        a2, b2 = ev(), ev()
        a2.record()
        for _ in range(reps):
            ring_pass_2s()
        b2.record()
        torch.cuda.synchronize()
        r2_ms = a2.elapsed_time(b2) / reps
        if not torch.equal(serial_out, o_out):
            raise RuntimeError("the two-stream ring pass changed the output")
        r_flops = 4.0 * rw.B * rh * Sq * rw.S * rw.D
        m_bytes = rw.B * Sq * rh * rw.D * (4 + 4 + 2) + 2 * rw.B * rh * Sq * 4
        ring = {"workload": "video_dit_ring", "grid": f"{rw.P} ulysses x {rw.ring} ring",
                "rank": "ring block 0, head group 0", "h": rh, "Sq": Sq, "S": rw.S, "D": rw.D,
                "ms": r2_ms, "TFLOP/s": r_flops / (r2_ms * 1e-3) / 1e12,
                "frac_peak": r_flops / (r2_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "flop": r_flops,
                "one_stream_ms": r_ms, "one_stream_TFLOP/s": r_flops / (r_ms * 1e-3) / 1e12,
                "merge_us": m_ms * 1e3, "merge_GB/s": m_bytes / (m_ms * 1e-3) / 1e9,
                "entry": "usp_attention_fwd_block (workspace) x 2 + usp_attention_merge; the "
                         "second block on a second stream (one_stream: all on one stream)"}
        del qr, kvr, rws, rws2, o_acc, o_blk, l_acc, l_blk, o_out, o_b2, l_b2, serial_out

    # head-chunked passes on the long-sequence share, against single shot
    chunked = None
    if not args.skip_chunked:
        print("[bench] head-chunked passes (S=131072)", file=sys.stderr, flush=True)
        cw = synth.WORKLOADS["long_chunked"]
        cq, ck, cv = (bf(x) for x in synth.draw_workload(cw))
        co = torch.empty_like(cq)
        c_flops = 4.0 * cw.B * cw.H * cw.S * cw.S * cw.D
        cmax = -(-cw.H // cw.chunks)   # heads of the largest pass
        cws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, cw.B, cw.S, cmax, cw.D) // 4,
                          dtype=torch.float32, device=dev)
        times = {}
        for name, fn in (("chunked", lambda: usp.usp_attention_fwd_chunked(cq, ck, cv, co, cw.chunks)),
                         ("chunked_ws", lambda: usp.usp_attention_fwd_chunked_ws(cq, ck, cv, co, cw.chunks,
                                                                                 cws)),
                         ("single_shot", lambda: usp.usp_attention_fwd(cq, ck, cv, co))):
            fn()
            torch.cuda.synchronize()
            a, b_ = ev(), ev()
            a.record()
            for _ in range(3):
                fn()
            b_.record()
            torch.cuda.synchronize()
            times[name] = a.elapsed_time(b_) / 3
        chunked = {"workload": "long_chunked", "h": cw.H, "S": cw.S, "D": cw.D,
                   "chunks": usp.usp_head_chunk_ranges(cw.H, cw.chunks), "flop": c_flops,
                   "ms": times["chunked"], "TFLOP/s": c_flops / (times["chunked"] * 1e-3) / 1e12,
                   "ws_ms": times["chunked_ws"],
                   "ws_TFLOP/s": c_flops / (times["chunked_ws"] * 1e-3) / 1e12,
                   "single_shot_ms": times["single_shot"],
                   "single_shot_TFLOP/s": c_flops / (times["single_shot"] * 1e-3) / 1e12,
                   "entry": "usp_attention_fwd_chunked (3 passes; ws: usp_attention_fwd_chunked_ws) "
                            "vs usp_attention_fwd"}
        del cq, ck, cv, co, cws

    # plain device copy of 1 GiB: practical HBM reference and counter calibration
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b_ = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(4):
        dst.copy_(src)
    b_.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * COPY_BYTES / (a.elapsed_time(b_) / 4 * 1e-3) / 1e9
    del src, dst

    rows_bw = {}
    if not args.skip_rows:
        print("[bench] model-boundary row movements", file=sys.stderr, flush=True)
        W = H * D
        tbr = usp.usp_balanced_ranges(S, P)
        nbytes = B * S * W * elem
        fulls = [torch.randn((B, S, W), device=dev).to(torch.bfloat16) for _ in range(3)]
        shard_sets = [[torch.empty((B, tbr[r + 1] - tbr[r], W), dtype=torch.bfloat16, device=dev)
                       for r in range(P)] for _ in range(3)]
        partials = [torch.randn((B, S, W), device=dev).to(torch.bfloat16) for _ in range(P)]

        def timed(fn, reps):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b_ = ev(), ev()
            a.record()
            for i in range(reps):
                fn(i)
            b_.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b_) / reps

        for name, fn, moved in (
                ("scatter", lambda i: usp.usp_scatter_rows(fulls[i % 3], shard_sets[i % 3]), 2 * nbytes),
                ("gather", lambda i: usp.usp_gather_rows(shard_sets[i % 3], fulls[i % 3]), 2 * nbytes),
                ("reduce_scatter", lambda i: usp.usp_reduce_scatter_rows(partials, shard_sets[i % 3]),
                 (P + 1) * nbytes)):
            ms = timed(fn, args.relayout_reps)
            gbs = moved / (ms * 1e-3) / 1e9
            rows_bw[name] = {"us": ms * 1e3, "GB/s": gbs, "frac_peak": gbs / PEAK_HBM_GBS,
                             "bytes": moved}
        rows_bw["shape"] = {"B": B, "S": S, "W": W, "P": P, "dtype": "bf16"}
        del fulls, shard_sets, partials

    rel = {}
    if not args.skip_relayout_bw:
        # world pack / unpack of the full [1, 32760, 40, 128] tensor, 3 rotating buffer sets
        print("[bench] world pack/unpack bandwidth", file=sys.stderr, flush=True)
        nbytes = B * S * H * D * elem
        srcs = [world[0]] + [torch.empty_like(world[0]).copy_(world[0]) for _ in range(2)]
        dsts = [[torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=torch.bfloat16, device=dev)
                 for j in range(P)] for _ in range(3)]
        for name, fn in (("pack", lambda i: usp.usp_pack_seq_to_heads(srcs[i % 3], dsts[i % 3])),
                         ("unpack", lambda i: usp.usp_unpack_heads_to_seq(dsts[i % 3], srcs[i % 3]))):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b_ = ev(), ev()
            a.record()
            for i in range(args.relayout_reps):
                fn(i)
            b_.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b_) / args.relayout_reps
            gbs = 2.0 * nbytes / (ms * 1e-3) / 1e9
            rel[name] = {"us": ms * 1e3, "GB/s": gbs, "frac_peak": gbs / PEAK_HBM_GBS,
                         "frac_of_copy": gbs / copy_gbs, "bytes_rw": 2 * nbytes}
        # one two-phase chunk of the same tensor: heads [0, 2) of each group of 5
        cb = nbytes * 2 // h0
        for name, fn in (("pack_chunk", lambda i: usp.usp_pack_seq_to_heads_chunk(
                              srcs[i % 3], dsts[i % 3], 0, 2)),
                         ("unpack_chunk", lambda i: usp.usp_unpack_heads_to_seq_chunk(
                              dsts[i % 3], srcs[i % 3], 0, 2))):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b_ = ev(), ev()
            a.record()
            for i in range(args.relayout_reps):
                fn(i)
            b_.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b_) / args.relayout_reps
            gbs = 2.0 * cb / (ms * 1e-3) / 1e9
            rel[name] = {"us": ms * 1e3, "GB/s": gbs, "frac_peak": gbs / PEAK_HBM_GBS,
                         "frac_of_copy": gbs / copy_gbs, "bytes_rw": 2 * cb,
                         "heads": "[0, 2) of each group of 5"}

    out = {
        "metric": METRIC,
        "value": attn_flops / (pipe_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pipe_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "video_dit_share", "B": B, "S": S, "H": H, "h": h0, "D": D,
                   "P": P, "rank": 0,
                   "step": "pack rank-0 shard of q,k,v -> attention on head group 0 over "
                           "the full sequence -> unpack rank-0 rows; relayouts of neighbouring "
                           "steps on a second stream under the attention"},
        "attention": {"ms": attn_ms, "TFLOP/s": attn_tflops,
                      "frac_peak": attn_tflops / PEAK_BF16_TFLOPS, "flop": attn_flops,
                      "entry": "usp_attention_fwd_ws"},
        "attention_no_workspace": {"ms": nows_ms,
                                   "TFLOP/s": attn_flops / (nows_ms * 1e-3) / 1e12,
                                   "entry": "usp_attention_fwd"},
        "attention_gqa": gqa,
        "ring": ring,
        "chunked": chunked,
        "two_phase": two_phase,
        "step_serial": {"ms_per_step": ms_step,
                        "TFLOP/s": attn_flops / (ms_step * 1e-3) / 1e12,
                        "how": "the same steps on one stream: pack, attention, unpack"},
        "step_pack_qkv": {"us": pack_ms * 1e3,
                          "GB/s": 3 * share_bytes / (pack_ms * 1e-3) / 1e9},
        "step_unpack_o": {"us": unpack_ms * 1e3,
                          "GB/s": share_bytes / (unpack_ms * 1e-3) / 1e9},
        "relayout_world": rel,
        "rows_world": rows_bw,
        "copy_reference_GB/s": copy_gbs,
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(),
                     "kernel": "usp_attention_fwd_ws: attn_bf16_kernel (key halves) + "
                               "attn_merge_halves"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
