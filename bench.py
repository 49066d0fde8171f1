#!/usr/bin/env python3
"""Benchmark of one GPU's share of the Ulysses sequence-parallel hot path.

Workload (video-DiT share): world Q/K/V [B=1, S=32760, H=40, D=128] bf16,
seeded synthetic N(0,1) with Q scaled by 1/sqrt(128), SP degree P = 8
(token ranges 8 x 4095, head groups 8 x 5). One step is rank 0's share of the
path, every row of it:

  ranges   token / head boundaries (host)
  pack     rank 0's token shard [1, 4095, 40, 128] of Q, K and V into the 8
           head-group blocks [1, 32760, 5, 128], the three tensors in one
           launch (usp_pack_seq_to_heads_planes: the data rank 0 sends in the
           first all-to-all; the other ranks' rows were placed beforehand)
  attn     non-causal attention over the full sequence on block 0 (h = 5),
           usp_attention_fwd_ws with its workspace allocated beforehand
  unpack   rank 0's rows of the 8 output blocks back to [1, 4095, 40, 128]

Steps run pipelined: step i + 1's pack and step i's unpack are issued on a
second stream (default priority) so that they run under the attention of the
neighbouring step, with two sets of head and output blocks and stream-ordered
events that keep each step's pack before its attention and its unpack after
it. Every step does all of its work; the timed region holds exactly K packs,
K attention calls and K unpacks, and the output is checked bitwise against a
serial step. The same steps on one stream are "step_serial", with HIP events
around each part of every step (median, minimum and mean per part).

value = attention flops of a step (4 * S^2 * D * h = 2.7474e12) / step time.

Also measured, each with HIP events around every call on its stream (median
and minimum reported; buffers rotated past the 256 MB last-level cache where
a leg says "cold"):
  * usp_attention_fwd (no workspace), usp_attention_fwd_noalloc (static
    scratch) and the same attention with softmax scale 1 instead of
    1/sqrt(D) (the other reading of "Q scaled by 1/sqrt(D)"; ungraded: its
    error against the oracle on sampled rows is reported beside it);
  * the other workloads' full worlds, pack -> attention of every head group
    -> unpack: ViT-L/16 (B=32, S=577, H=16, D=64, P=4; HBM-warm and cold)
    and the indivisible long sequence (B=2, S=65537, H=12, D=64, P=4, 1% of
    K rows x 8);
  * usp_attention_fwd_gqa on rank 0's share of the grouped video-DiT
    workload; one rank's Ulysses+Ring pass (video-DiT over 4 x 2 ranks: two
    key blocks, then the merge; the second block on a second stream with
    whole key walks, and on one stream with the block call); the head-chunked passes on the long
    sequence (B=1, S=131072, h=8, 3/3/2) against single shot; the same step
    as the two-phase exchange (per head chunk 2/2/1: pack, attention,
    unpack); the world relayouts of the [1, 32760, 40, 128] tensor (one
    tensor, and q, k, v in one launch; whole groups and one head chunk) and
    rank 0's share of them (pack of q, k, v; unpack of one tensor), these
    also timed back to back (mean of calls between two events: the launch
    and event overhead of a 16 us call is a sixth of it); the
    model-boundary row movements at [1, 32760, 5120]; a 1 GiB device copy as
    the practical HBM reference.

cpu_baseline: the float64 CPU oracle, per configuration and part, on every
host core this process may use (attention in a process pool, one BLAS thread
per worker; pack/unpack index loops single-threaded): ``value`` is the
video-DiT share's attention on a sample of its rows.

roofline: the attention call (usp_attention_fwd_ws: the key-half flash
kernel, then the merge kernel) is the dominant step; ``achieved`` is its
flops over its mean event-timed duration in the serial steps.
roofline.traffic: HBM bytes per attention call from rocprofv3 FETCH_SIZE /
WRITE_SIZE counter runs (both kernels), each scaled by what the counter reads
for the plain copy kernel of known size in the same run (``--pmc-summary``);
reported only while the attention source is the one the counters were taken
on. roofline.legs repeats every leg's headline figure in compact form.
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
# groups of legs besides the step (--legs selects some, e.g. for a profiler run)
LEG_GROUPS = ("single", "gqa", "ring", "chunked", "two_phase", "worlds", "relayout", "rows")


def source_digest(path=ATTN_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    for key, kind in (("attn_bf16_kernel<128, 8, 1, 2, 64, true>", "attention"),
                      ("attn_bf16_kernel<128, 8, 1, 2, 64, false>", "attention_f32out"),
                      ("attn_bf16_kernel<128, 8, 2, 1, 64, true>", "attention_groups"),
                      ("attn_bf16_kernel<128, 8, 2, 1, 64, false>", "attention_groups_f32out"),
                      ("attn_bf16_kernel<128, 8, 1, 1, 64, true>", "attention_whole"),
                      ("attn_bf16_kernel<128, 8, 1, 1, 64, false>", "attention_whole_f32out"),
                      ("attn_merge_halves<128, true>", "merge"),
                      ("attn_merge_halves<128, false>", "merge_f32out"),
                      ("copyBuffer", "copy"),
                      ("relayout_kernel<true>", "pack"), ("relayout_kernel<false>", "unpack"),
                      ("relayout_chunk_kernel<true>", "pack_chunk"),
                      ("relayout_chunk_kernel<false>", "unpack_chunk"),
                      ("lse_merge_kernel", "lse_merge")):
        if key in name:
            return kind
    return None


def read_pmc(dirs, by_grid=False):
    """rocprofv3 --pmc CSVs under ``dirs`` -> {(kind, counter): {dispatch: value}},
    each value summed over the counter's instances (SEs, SIMDs, channels);
    with ``by_grid`` the kind carries the dispatch's thread count,
    "kind[threads]"."""
    per = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    kind = kernel_kind(r["Kernel_Name"])
                    if kind is None:
                        continue
                    if by_grid:
                        kind = f"{kind}[{int(r['Grid_Size'])}]"
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
        busy, sqb = a.get("SQ_VALU_MFMA_BUSY_CYCLES"), a.get("SQ_BUSY_CYCLES")
        if busy is not None and sqb:
            # SQ_BUSY_CYCLES sums the busy cycles of the 32 shader engines: a
            # dispatch that keeps every engine busy lasts sqb / 32 cycles
            cyc = sqb / 32
            lines.append(f"  SQ_BUSY_CYCLES / 32 engines = {cyc:.4e} cycles"
                         + (f" (= {cyc / (dur * 1e-9) / 1e9:.3f} GHz over the dispatch)" if dur else ""))
            lines.append(f"  matrix cores: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs = {busy / 1024:.4e} cycles "
                         f"= {busy / (1024 * cyc):.3f} of the dispatch ({busy / 1024 / (n_mfma / 1024):.1f} "
                         f"cycles per MFMA)" if n_mfma else "")
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


def copy_factors(per):
    """Calibration of FETCH_SIZE and WRITE_SIZE (KiB per dispatch) on the
    1 GiB copies: bytes per KiB counted, read and write."""
    # the runtime's copy kernel also serves small copies (a clone, a compare):
    # calibrate on the 1 GiB copies only, the dispatches of at least half the
    # largest count
    cp = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        v = per.get(("copy", ctr))
        if v:
            mx = max(v.values())
            cp[ctr] = float(np.mean([x for x in v.values() if x >= 0.5 * mx]))
    ff = COPY_BYTES / (cp["FETCH_SIZE"] * 1024) if cp.get("FETCH_SIZE") else None
    fw = COPY_BYTES / (cp["WRITE_SIZE"] * 1024) if cp.get("WRITE_SIZE") else None
    return ff, fw


def relayout_pmc_summary(dirs, out_txt):
    """HBM bytes per dispatch of the relayout kernels from FETCH_SIZE and
    WRITE_SIZE runs of this benchmark, per launch shape (thread count), with
    the algorithmic bytes each way: every thread moves one 16-byte chunk, so
    threads x 16 B (the last workgroup's idle threads aside)."""
    ff, fw = copy_factors(read_pmc(dirs))
    per = read_pmc(dirs, by_grid=True)
    lines = [f"copy calibration ({COPY_BYTES} B read and written per dispatch): "
             f"FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}" if ff and fw else "copy calibration missing",
             "",
             f"{'dispatch (kernel[threads])':42s} {'n':>3s} {'alg MB each way':>15s} "
             f"{'HBM read MB':>11s} {'HBM write MB':>12s}"]
    kinds = sorted({k for k, c in per if k.split("[")[0] in ("pack", "unpack", "pack_chunk", "unpack_chunk")},
                   key=lambda k: (k.split("[")[0], -int(k.split("[")[1][:-1])))
    for k in kinds:
        f_k, w_k = per.get((k, "FETCH_SIZE")), per.get((k, "WRITE_SIZE"))
        if not f_k or not w_k or not ff or not fw:
            continue
        threads = int(k.split("[")[1][:-1])
        rb = float(np.mean(list(f_k.values()))) * 1024 * ff
        wb = float(np.mean(list(w_k.values()))) * 1024 * fw
        lines.append(f"{k:42s} {len(f_k):3d} {threads * 16 / 1e6:15.1f} {rb / 1e6:11.1f} {wb / 1e6:12.1f}")
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
    ff, fw = copy_factors(per)
    for key in [k for k in per if k[0] == "copy"]:
        mx = max(per[key].values())
        per[key] = {d: v for d, v in per[key].items() if v >= 0.5 * mx}
    avg = {k: float(np.mean(list(v.values()))) for k, v in per.items()}
    lines = ["kernel     counter      KiB/dispatch  dispatches"]
    for (kind, ctr), val in sorted(avg.items()):
        lines.append(f"{kind:10s} {ctr:12s} {val:12.1f}  {len(per[(kind, ctr)])}")
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


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def oracle_parts(data, target_s):
    """Time the oracle (float64 NumPy) on the workloads of this benchmark, per
    configuration and part, on every host core this process may use (the
    attention in a process pool with one BLAS thread per worker; the
    pack/unpack index loops single-threaded, as written). Returns the
    cpu_baseline object: ``value`` is the video-DiT share's attention."""
    from oracle import attention as A
    from oracle import relayout as X
    from ulysses_sequence_attention_amd import synth

    cores = A.host_cores()
    parts = {}

    def f64(x, heads=None):
        x = x if heads is None else x[:, :, heads[0]:heads[1]]
        if x.dtype == np.uint16:
            return synth.bf16_bits_to_f32(np.ascontiguousarray(x)).astype(np.float64)
        return np.ascontiguousarray(x, dtype=np.float64)

    def attn(name, q, k, v, rows_per_head, scale=None, note=""):
        B, S, h, D = q.shape
        n = sum(len(r) for r in rows_per_head.values())
        t0 = time.perf_counter()
        A.attention_parallel(q, k, v, scale=scale, rows_per_head=rows_per_head, workers=cores)
        wall = time.perf_counter() - t0
        flops = 4.0 * D * k.shape[1] * n
        parts[name] = {"wall_s": round(wall, 3), "GFLOP/s": flops / wall / 1e9, "flop": flops,
                       "rows": n, "of_rows": B * S * h, "note": note}
        return flops / wall

    rng = np.random.default_rng(123)

    def sample(S, n):
        return np.arange(S) if n >= S else np.sort(rng.choice(S, n, replace=False))

    # the video-DiT share (heads 0-4 of the world tensor): a sample sized for
    # about target_s of wall time, calibrated on one core
    q, k, v = data["video_dit_share"]
    h0, S = 5, q.shape[1]
    qf, kf, vf = (f64(x, (0, h0)) for x in (q, k, v))
    t0 = time.perf_counter()
    A.attention_rows(qf, kf, vf, 0, 0, np.arange(512))
    per_row = (time.perf_counter() - t0) / 512
    n = int(max(64, min(S, target_s * cores / (per_row * h0))))
    value = attn("attention_video_dit_share", qf, kf, vf,
                 {(0, hd): sample(S, n) for hd in range(h0)},
                 note="rows sampled per head" if n < S else "every row")
    del qf, kf, vf
    # the world pack and unpack of the video-DiT q tensor, index loops
    t0 = time.perf_counter()
    blocks = X.pack_seq_to_heads(q, 8)
    t_pack = time.perf_counter() - t0
    t0 = time.perf_counter()
    X.unpack_heads_to_seq(blocks, q.shape[2])
    t_unpack = time.perf_counter() - t0
    del blocks
    moved = 2.0 * q.nbytes
    parts["pack_world_video_dit"] = {"wall_s": round(t_pack, 3), "GB/s": moved / t_pack / 1e9,
                                     "bytes_rw": moved, "note": "single-threaded index loops"}
    parts["unpack_world_video_dit"] = {"wall_s": round(t_unpack, 3), "GB/s": moved / t_unpack / 1e9,
                                       "bytes_rw": moved, "note": "single-threaded index loops"}
    # the other configurations' attention (every group of the world)
    q, k, v = data["vit_l16"]
    qf, kf, vf = (f64(x) for x in (q, k, v))
    attn("attention_vit_l16", qf, kf, vf,
         {(b, hd): np.arange(q.shape[1]) for b in range(q.shape[0]) for hd in range(q.shape[2])},
         note="every row of all 16 heads")
    q, k, v = data["indivisible_long"]
    qf, kf, vf = (f64(x) for x in (q, k, v))
    attn("attention_indivisible_long", qf, kf, vf,
         {(b, hd): sample(q.shape[1], 256) for b in range(q.shape[0]) for hd in range(q.shape[2])},
         note="256 rows sampled per (batch, head)")
    q, k, v = data["long_chunked"]
    qf, kf, vf = (f64(x) for x in (q, k, v))
    attn("attention_long_chunked", qf, kf, vf,
         {(0, hd): sample(q.shape[1], 96) for hd in range(q.shape[2])},
         note="96 rows sampled per head")
    q, k, v = data["tiny_fp32"]
    qf, kf, vf = (f64(x) for x in (q, k, v))
    attn("attention_tiny_fp32", qf, kf, vf,
         {(0, hd): np.arange(q.shape[1]) for hd in range(q.shape[2])}, note="every row")
    s = parts["attention_video_dit_share"]
    return {"value": value / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"{s['rows']} of {s['of_rows']} rows (5 heads) of the S=32760 D=128 share, "
                      f"{s['wall_s']:.1f} s, fp64 NumPy, {cores} procs",
            "parts": parts}

def short_kernel_name(name):
    """A readable name for a kernel of this benchmark in a trace."""
    kind = kernel_kind(name)
    if kind:
        return {"attention": "attn_bf16_kernel<D=128, key halves> (fwd_ws)",
                "attention_f32out": "attn_bf16_kernel<D=128, key halves, f32 out>",
                "attention_groups": "attn_bf16_kernel<D=128, key groups> (fwd)",
                "attention_groups_f32out": "attn_bf16_kernel<D=128, key groups, f32 out>",
                "attention_whole": "attn_bf16_kernel<D=128, whole walks>",
                "attention_whole_f32out": "attn_bf16_kernel<D=128, whole walks, f32 out>",
                "merge": "attn_merge_halves<D=128>",
                "merge_f32out": "attn_merge_halves<D=128, f32 out>",
                "copy": "__amd_rocclr_copyBuffer",
                "pack": "relayout_kernel<pack>", "unpack": "relayout_kernel<unpack>",
                "pack_chunk": "relayout_chunk_kernel<pack>",
                "unpack_chunk": "relayout_chunk_kernel<unpack>",
                "lse_merge": "lse_merge_kernel"}[kind]
    n = name.replace("void ", "").replace("usp::(anonymous namespace)::", "")
    return n[:56]


def trace_summary(dirs, out_txt, warmup, steps):
    """Summarise a rocprofv3 --kernel-trace run of this benchmark: calls and
    average / minimum / maximum duration per kernel, and the key-half
    attention kernel's durations per call; the serial steps' timed calls are
    dispatches warmup + 1 .. warmup + steps of that kernel (and of the
    merge), whose mean is compared with the events of the same run."""
    rows = []
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            with open(path) as f:
                rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per, per_grid = {}, {}
    for r in rows:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        name = short_kernel_name(r["Kernel_Name"])
        per.setdefault(name, []).append(us)
        wgs = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) * int(r["Grid_Size_Y"]) * \
            int(r["Grid_Size_Z"])
        per_grid.setdefault((name, wgs), []).append(us)
    total = sum(sum(v) for v in per.values())
    lines = [f"# kernel source: attn_bf16.hip sha256 {source_digest()}", "",
             f"{'kernel':56s} {'workgroups':>10s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
             f"{'max_us':>9s} {'pct':>6s}"]
    for (name, wgs), v in sorted(per_grid.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name:56s} {wgs:10d} {len(v):6d} {np.mean(v):9.1f} {min(v):9.1f} {max(v):9.1f} "
                     f"{100 * sum(v) / total:6.2f}")
    lines += ["", "durations in dispatch order (us), for the library's kernels with at most 400 dispatches "
                  "of one launch shape:"]
    for (name, wgs), v in sorted(per_grid.items(), key=lambda kv: -sum(kv[1])):
        if len(v) <= 400 and ("attn" in name or "relayout" in name or "merge" in name):
            lines.append(f"  {name} [{wgs} workgroups]: " + " ".join(f"{x:.1f}" for x in v))
    att = per.get(short_kernel_name("attn_bf16_kernel<128, 8, 1, 2, 64, true>"), [])
    mrg = per.get(short_kernel_name("attn_merge_halves<128, true>"), [])
    lines += ["", "key-half attn_bf16_kernel durations per call (us), in order: " +
              " ".join(f"{x:.0f}" for x in att)]
    if len(att) >= warmup + steps and len(mrg) >= warmup + steps:
        a = float(np.mean(att[warmup:warmup + steps]))
        m = float(np.mean(mrg[warmup:warmup + steps]))
        lines.append(f"serial steps' timed calls ({steps} after {warmup} warmup): attn_bf16_kernel "
                     f"{a:.1f} us + attn_merge_halves {m:.1f} us = {a + m:.1f} us per call")
        # the step's relayouts: rank 0's pack of q, k, v and unpack of o, one
        # dispatch each per step, in the same order as the attention
        share = [(k, v) for k, v in per_grid.items() if k[0] in ("relayout_kernel<pack>", "relayout_kernel<unpack>")
                 and len(v) == len(att)]
        for (name, wgs), v in sorted(share):
            x = float(np.mean(v[warmup:warmup + steps]))
            lines.append(f"serial steps' timed calls: {name} [{wgs} workgroups] {x:.1f} us "
                         f"(minimum {min(v[warmup:warmup + steps]):.1f})")
    # ring passes: from the start of the earlier of the two block attention
    # dispatches before each log-sum-exp merge to that merge's end (on two
    # streams the blocks run at once, so their durations do not add up)
    spans, attn_rows = [], []
    for r in rows:
        name = short_kernel_name(r["Kernel_Name"])
        if name.startswith("attn_bf16_kernel"):
            attn_rows.append(r)
        elif name == "lse_merge_kernel" and len(attn_rows) >= 2:
            t0 = min(int(x["Start_Timestamp"]) for x in attn_rows[-2:])
            spans.append((int(r["End_Timestamp"]) - t0) / 1e3)
    if spans:
        lines += ["", "ring passes, kernel time from the first block's start to the merge's end (us), in "
                      "order: " + " ".join(f"{x:.1f}" for x in spans)]
    text = "\n".join(lines)
    print(text)
    if out_txt:
        with open(out_txt, "w") as f:
            f.write(text + "\n")


class Timer:
    """HIP events around every call of a leg on one stream; summary in ms."""

    def __init__(self, torch, stream=None):
        self.torch, self.stream, self.ev = torch, stream, []

    def __call__(self, fn, *args, **kw):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s = self.stream or t.cuda.current_stream()
        a.record(s)
        fn(*args, **kw)
        b.record(s)
        self.ev.append((a, b))

    def summary(self):
        self.torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in self.ev])
        return {"median_ms": float(np.median(ms)), "min_ms": float(ms.min()),
                "mean_ms": float(ms.mean()), "calls": int(len(ms))}


_SPIN = {"cycles_per_ms": None}


def queue_ahead(torch, host_ms):
    """Queue a GPU spin of about ``host_ms`` + 1 ms (capped at 250 ms) in
    front of work about to be enqueued. The calls timed behind it then find
    the GPU busy and run back to back, so the events around a short call
    measure the GPU's time for it, not the host's argument marshalling and
    launch (which for a 16 us relayout is longer than the kernel)."""
    if _SPIN["cycles_per_ms"] is None:
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(4_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN["cycles_per_ms"] = 4_000_000 / max(a.elapsed_time(b), 1e-3)
    ms = min(host_ms + 1.0, 250.0)
    torch.cuda._sleep(int(ms * _SPIN["cycles_per_ms"]))


def host_ms_per_call(torch, fn, warm):
    """Warm-up calls of ``fn(i)``; returns the host's enqueue time and the
    GPU's time per call (ms)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    t0 = time.perf_counter()
    for i in range(warm):
        fn(i)
    host = (time.perf_counter() - t0) * 1e3 / max(warm, 1)
    b.record()
    torch.cuda.synchronize()
    return host, a.elapsed_time(b) / max(warm, 1)


def top_up_warmup(torch, fn, gpu, done, target_ms=100.0, cap=400):
    """More untimed calls of ``fn(i)`` after ``done`` warm-up calls of ``gpu``
    ms each, until about ``target_ms`` of GPU work (at most ``cap`` calls): a
    leg that follows another workload is timed once the clock has settled on
    its own."""
    for i in range(done, min(cap, int(target_ms / max(gpu, 1e-3)))):
        fn(i)


def spin_if_host_bound(torch, host, gpu, calls):
    """Queue a spin ahead of ``calls`` timed calls when the host's enqueue
    time per call is not well below the GPU's (short calls); long calls keep
    the GPU busy by themselves and are timed without one (a spin idles all
    but one CU, and the clock then starts the first timed call lower)."""
    if host > 0.5 * gpu:
        queue_ahead(torch, 1.5 * host * calls)


def timed(torch, fn, reps, warm=3):
    """Median / minimum / mean of ``reps`` calls of ``fn(i)`` after ``warm``
    (and more, up to about 0.1 s of GPU work), each between two HIP events;
    short calls are issued behind a GPU spin (queue_ahead)."""
    host, gpu = host_ms_per_call(torch, fn, warm)
    top_up_warmup(torch, fn, gpu, warm)
    spin_if_host_bound(torch, host, gpu, reps)
    t = Timer(torch)
    for i in range(reps):
        t(fn, i)
    return t.summary()


def back_to_back(torch, fn, reps, warm=3):
    """Mean per call of ``reps`` calls of ``fn(i)`` issued back to back
    between two HIP events (no event between calls) behind a GPU spin, in ms."""
    host, gpu = host_ms_per_call(torch, fn, warm)
    top_up_warmup(torch, fn, gpu, warm)
    spin_if_host_bound(torch, host, gpu, reps)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="minimum untimed warm-up time before the timed steps")
    ap.add_argument("--relayout-reps", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle's video-DiT attention sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-legs", action="store_true",
                    help="time only the video-DiT step (for profiler runs)")
    ap.add_argument("--legs", metavar="LIST",
                    help="comma-separated leg groups to run besides the step (default: all): "
                         + ",".join(LEG_GROUPS))
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 counter runs of this benchmark and exit")
    ap.add_argument("--pmc-sq", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 SQ/GRBM counter runs of this benchmark and exit")
    ap.add_argument("--pmc-out", metavar="FILE", help="text file for --pmc-sq's summary")
    ap.add_argument("--pmc-relayout", nargs="+", metavar="DIR",
                    help="summarise FETCH_SIZE / WRITE_SIZE runs of the relayout legs and exit "
                         "(text to --pmc-out)")
    ap.add_argument("--trace-summary", nargs="+", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace run of this benchmark and exit "
                         "(with the run's --steps and --warmup)")
    ap.add_argument("--trace-out", metavar="FILE", help="text file for --trace-summary")
    ap.add_argument("--trace-json", metavar="FILE",
                    help="the traced run's JSON line (gives its warm-up and timed step counts)")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args.pmc_summary, TRAFFIC_JSON)
        return
    if args.pmc_relayout:
        relayout_pmc_summary(args.pmc_relayout, args.pmc_out)
        return
    if args.pmc_sq:
        sq_summary(args.pmc_sq, args.pmc_out)
        return
    if args.trace_summary:
        warm, steps = args.warmup, args.steps
        if args.trace_json:  # the traced run's own output: its warm-up and timed steps
            with open(args.trace_json) as f:
                run = json.loads(f.read().strip().splitlines()[-1])
            warm, steps = run["config"]["warmup_steps_done"], run["steps"]
        trace_summary(args.trace_summary, args.trace_out, warm, steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not "
              "supported: it runs on one GPU (the multi-GPU exchange is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import ulysses_sequence_attention_amd as usp
    from ulysses_sequence_attention_amd import synth

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    w = synth.WORKLOADS["video_dit_share"]
    B, S, H, D, P = w.B, w.S, w.H, w.D, w.P
    legs_on = not args.skip_legs
    chosen = None if args.legs is None else set(args.legs.split(","))
    if chosen is not None and not chosen <= set(LEG_GROUPS):
        raise SystemExit(f"--legs: unknown group(s) {sorted(chosen - set(LEG_GROUPS))}; "
                         f"known: {','.join(LEG_GROUPS)}")

    def on(group):
        return legs_on and (chosen is None or group in chosen)
    names = ["video_dit_share"] + (["vit_l16", "indivisible_long", "long_chunked", "tiny_fp32"]
                                   if legs_on or not args.no_cpu_baseline else [])
    data = {}
    for name in names:
        say(f"drawing {name}")
        data[name] = synth.draw_workload(synth.WORKLOADS[name])
    tb = usp.usp_balanced_ranges(S, P)
    hb = usp.usp_balanced_ranges(H, P)
    h0, len0 = hb[1] - hb[0], tb[1] - tb[0]
    attn_flops = 4.0 * B * h0 * S * S * D

    cpu = None
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle, per configuration and part)")
        cpu = oracle_parts(data, args.cpu_seconds)

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    def blocks_of(Bx, Sx, hbx, Dx, dtype=torch.bfloat16):
        return [torch.empty((Bx, Sx, hbx[j + 1] - hbx[j], Dx), dtype=dtype, device=dev)
                for j in range(len(hbx) - 1)]

    world = [bf(x) for x in data["video_dit_share"]]
    shard = [x[:, tb[0]:tb[1]].contiguous() for x in world]
    blocks = [blocks_of(B, S, hb, D) for _ in range(3)]
    usp.usp_pack_seq_to_heads_planes(world, blocks)   # every rank's rows, as received
    oblocks = [torch.zeros_like(t) for t in blocks[0]]
    oshard = torch.empty((B, len0, H, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, h0, D),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(e=None):
        if e is not None:
            e[0].record()
        usp.usp_pack_seq_to_heads_planes(shard, blocks, rank=0)
        if e is not None:
            e[1].record()
        usp.usp_attention_fwd_ws(blocks[0][0], blocks[1][0], blocks[2][0], oblocks[0], ws)
        if e is not None:
            e[2].record()
        usp.usp_unpack_heads_to_seq(oblocks, oshard, rank=0)
        if e is not None:
            e[3].record()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # warm-up: W steps, and more until the GPU has been busy for
    # --warmup-seconds (a fresh process's first attention calls run up to 25%
    # slower while the shader clock ramps up); none of it is timed
    say(f"warmup {args.warmup} steps (at least {args.warmup_seconds} s)")
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t0 < args.warmup_seconds:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    say(f"timing {args.steps} serial steps")
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    def part(i0, i1):
        ms = np.array([e[i0].elapsed_time(e[i1]) for e in evs])
        return {"median_ms": float(np.median(ms)), "min_ms": float(ms.min()), "mean_ms": float(ms.mean()),
                "calls": int(len(ms))}

    t_pack, t_attn, t_unpack = part(0, 1), part(1, 2), part(2, 3)
    attn_tflops = tflops(attn_flops, t_attn["mean_ms"])
    share_bytes = 2 * B * len0 * H * D * 2   # one tensor's shard, read + write

    # the same steps pipelined (see the module docstring)
    say("pipelined steps")
    main_s = torch.cuda.current_stream()
    io_s = torch.cuda.Stream()
    bsets = [blocks, [[torch.empty_like(t) for t in bl] for bl in blocks]]
    usp.usp_pack_seq_to_heads_planes(world, bsets[1])
    osets = [oblocks, [torch.zeros_like(t) for t in oblocks]]
    ev_pack = [torch.cuda.Event() for _ in range(2)]
    ev_attn = [torch.cuda.Event() for _ in range(2)]
    ev_unp = [torch.cuda.Event() for _ in range(2)]
    for e in ev_attn + ev_unp:
        e.record(main_s)

    def p_pack(i):
        st = i % 2
        io_s.wait_event(ev_attn[st])      # set st was last read by attention i - 2
        usp.usp_pack_seq_to_heads_planes(shard, bsets[st], rank=0, stream=io_s)
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

    t0 = time.perf_counter()
    n_pwarm = 0
    while n_pwarm < args.warmup or time.perf_counter() - t0 < args.warmup_seconds / 2:
        pipelined(max(args.warmup, 4))
        torch.cuda.synchronize()
        n_pwarm += max(args.warmup, 4)
    say(f"timing {args.steps} pipelined steps")
    a, b_ = ev(), ev()
    a.record(main_s)
    pipelined(args.steps, start=a)
    b_.record(main_s)
    torch.cuda.synchronize()
    pipe_ms = a.elapsed_time(b_) / args.steps
    pipe_out = oshard.clone()
    step()
    torch.cuda.synchronize()
    if not torch.equal(pipe_out, oshard):
        raise RuntimeError("pipelined steps produced a different output than a serial step")
    del bsets[1], osets[1], pipe_out

    legs = {}
    out_extra = {}
    reps = max(5, args.steps // 4)
    blk0 = (blocks[0][0], blocks[1][0], blocks[2][0])
    if legs_on:
        if on("single"):
            say("attention without workspace / without allocation / softmax scale 1")
            legs["attn_no_workspace"] = timed(torch, lambda i: usp.usp_attention_fwd(*blk0, oblocks[0]), reps)
            legs["attn_noalloc"] = timed(torch, lambda i: usp.usp_attention_fwd_noalloc(*blk0, oblocks[0]),
                                         reps)
            o_s1 = torch.empty((B, S, h0, D), dtype=torch.float32, device=dev)
            legs["attn_scale1"] = timed(torch, lambda i: usp.usp_attention_fwd_ws(*blk0, o_s1, ws, scale=1.0),
                                        reps)
            # the scale-1 reading against the oracle on sampled rows (ungraded)
            from oracle import attention as A
            rows = np.sort(np.random.default_rng(7).choice(S, 48, replace=False))
            qh, kh, vh = (synth.bf16_bits_to_f32(np.ascontiguousarray(x[:, :, :h0])).astype(np.float64)
                          for x in data["video_dit_share"])
            got = o_s1.cpu().numpy().astype(np.float64)
            dmax, num, den = 0.0, 0.0, 0.0
            for hd in range(h0):
                ref, _ = A.attention_rows(qh, kh, vh, 0, hd, rows, scale=1.0)
                d = got[0, rows, hd] - ref
                dmax = max(dmax, float(np.abs(d).max()))
                num += float((d * d).sum())
                den += float((ref * ref).sum())
            legs["attn_scale1"].update({"max_abs": dmax, "rel_frob": (num / den) ** 0.5,
                                        "rows_checked": 48 * h0})
            del o_s1, qh, kh, vh

        if on("gqa"):
            # grouped K/V heads: rank 0's share of the grouped video-DiT workload
            say("attention with grouped K/V heads")
            gw = synth.WORKLOADS["gqa_video_share"]
            gq, gk, gv = synth.draw_workload(gw)
            ghq = usp.usp_balanced_ranges(gw.H, gw.P)
            ghk = usp.usp_balanced_ranges(gw.kv_heads, gw.P)
            q0 = bf(gq[:, :, ghq[0]:ghq[1]])
            k0, v0 = (bf(x[:, :, ghk[0]:ghk[1]]) for x in (gk, gv))
            del gq, gk, gv
            o0 = torch.empty_like(q0)
            gh = ghq[1] - ghq[0]
            gws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, gw.B, gw.S, gh, gw.D),
                              dtype=torch.uint8, device=dev)
            legs["attn_gqa"] = timed(torch, lambda i: usp.usp_attention_fwd_gqa(q0, k0, v0, o0, ws=gws), reps)
            legs["attn_gqa"]["flop"] = 4.0 * gw.B * gh * gw.S * gw.S * gw.D
            del q0, k0, v0, o0, gws

        if on("ring"):
            # one rank's Ulysses+Ring pass: two key blocks, then the merge
            say("Ulysses+Ring pass")
            rw = synth.WORKLOADS["video_dit_ring"]
            rq, rk, rv = (bf(x) for x in synth.draw_workload(rw))
            rT = usp.usp_balanced_ranges(rw.S, rw.ring)
            rc = usp.usp_balanced_ranges(rw.H, rw.P)
            rh = rc[1] - rc[0]

            def head_group0(x, i):
                bl = blocks_of(rw.B, rT[i + 1] - rT[i], rc, rw.D)
                usp.usp_pack_seq_to_heads(x[:, rT[i]:rT[i + 1]].contiguous(), bl)
                return bl[0]

            qr = head_group0(rq, 0)
            kvr = [(head_group0(rk, i), head_group0(rv, i)) for i in range(rw.ring)]
            del rq, rk, rv
            Sq = rT[1] - rT[0]
            rws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, rw.B, Sq, rh, rw.D),
                              dtype=torch.uint8, device=dev)
            rws2 = torch.empty_like(rws)
            o_acc = torch.empty((rw.B, Sq, rh, rw.D), dtype=torch.float32, device=dev)
            l_acc = torch.empty((rw.B, rh, Sq), dtype=torch.float32, device=dev)
            o_b2 = [torch.empty_like(o_acc) for _ in range(2)]
            l_b2 = [torch.empty_like(l_acc) for _ in range(2)]
            o_out = torch.empty((rw.B, Sq, rh, rw.D), dtype=torch.bfloat16, device=dev)
            order = [0] + [(0 - i) % rw.ring for i in range(1, rw.ring)]
            side = torch.cuda.Stream()
            ev_blk = [torch.cuda.Event() for _ in range(2)]
            ev_fold = [torch.cuda.Event() for _ in range(2)]

            def ring_pass(i, two_streams=True):
                # two streams: the later blocks' attention on a second stream (a ring
                # delivers a block long before the one before it is done), whole key
                # walks so the two launches fill each other's last rounds; one stream:
                # the block call, whose key halves fill a launch's last round alone.
                # Folds in ring order on the first stream.
                ms_ = torch.cuda.current_stream()
                st2 = side if two_streams else ms_
                start = torch.cuda.Event()
                start.record(ms_)
                st2.wait_event(start)
                for e in ev_fold:
                    e.record(ms_)

                def block(kv, o_, l_, ws_, st_):
                    if two_streams:
                        usp.usp_attention_fwd_block_whole(qr, *kv, o_, lse=l_, stream=st_)
                    else:
                        usp.usp_attention_fwd_block(qr, *kv, o_, lse=l_, ws=ws_, stream=st_)
                block(kvr[order[0]], o_acc, l_acc, rws, ms_)
                for n, blk in enumerate(order[1:]):
                    s2 = n % 2
                    st2.wait_event(ev_fold[s2])
                    block(kvr[blk], o_b2[s2], l_b2[s2], rws2 if two_streams else rws, st2)
                    ev_blk[s2].record(st2)
                    ms_.wait_event(ev_blk[s2])
                    last = n == len(order) - 2
                    usp.usp_attention_merge(o_acc, l_acc, o_b2[s2], l_b2[s2], o_out if last else o_acc,
                                            None if last else l_acc, stream=ms_)
                    ev_fold[s2].record(ms_)

            legs["ring_one_stream"] = timed(torch, lambda i: ring_pass(i, False), reps)
            legs["ring"] = timed(torch, ring_pass, reps)
            two = o_out.clone()
            # the same whole-walk launches serialised on one stream: the same bits
            ms_ = torch.cuda.current_stream()
            usp.usp_attention_fwd_block_whole(qr, *kvr[order[0]], o_acc, lse=l_acc, stream=ms_)
            for blk in order[1:]:
                usp.usp_attention_fwd_block_whole(qr, *kvr[blk], o_b2[0], lse=l_b2[0], stream=ms_)
                usp.usp_attention_merge(o_acc, l_acc, o_b2[0], l_b2[0], o_out if blk == order[-1] else o_acc,
                                        None if blk == order[-1] else l_acc, stream=ms_)
            torch.cuda.synchronize()
            if not torch.equal(two, o_out):
                raise RuntimeError("the two-stream ring pass changed the output")
            legs["ring"]["flop"] = 4.0 * rw.B * rh * Sq * rw.S * rw.D
            del qr, kvr, rws, rws2, o_acc, l_acc, o_b2, l_b2, o_out, two

        if on("chunked"):
            # head-chunked passes on the long-sequence share, against single shot
            say("head-chunked passes (S=131072)")
            cw = synth.WORKLOADS["long_chunked"]
            cq, ck, cv = (bf(x) for x in data["long_chunked"])
            co = torch.empty_like(cq)
            cmax = -(-cw.H // cw.chunks)
            cws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, cw.B, cw.S, cmax, cw.D),
                              dtype=torch.uint8, device=dev)
            fws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, cw.B, cw.S, cw.H, cw.D),
                              dtype=torch.uint8, device=dev)
            c_flops = 4.0 * cw.B * cw.H * cw.S * cw.S * cw.D
            for name, fn in (("chunked", lambda i: usp.usp_attention_fwd_chunked(cq, ck, cv, co, cw.chunks)),
                             ("chunked_ws", lambda i: usp.usp_attention_fwd_chunked_ws(cq, ck, cv, co,
                                                                                       cw.chunks, cws)),
                             ("single_shot", lambda i: usp.usp_attention_fwd(cq, ck, cv, co)),
                             ("single_shot_ws", lambda i: usp.usp_attention_fwd_ws(cq, ck, cv, co, fws))):
                legs["long_" + name] = timed(torch, fn, 3, warm=1)
                legs["long_" + name]["flop"] = c_flops
            del cq, ck, cv, co, cws, fws

        if on("two_phase"):
            # the two-phase exchange on the same share: per head chunk (2/2/1 of
            # the 5 heads), pack rank 0's rows of the chunk's heads (q, k, v in one
            # launch), attention on them, unpack them. Overlapped: a chunk's pack
            # for the next step and its unpack for this step go to the second
            # stream as soon as this step's attention of that chunk is done.
            say("two-phase steps")
            kc = usp.usp_head_chunk_ranges(h0, 3)
            ch = [(kc[c], kc[c + 1]) for c in range(len(kc) - 1)]
            ws_c = torch.empty(usp.usp_attention_workspace_bytes(
                usp.USP_BF16, B, S, max(hi - lo for lo, hi in ch), D), dtype=torch.uint8, device=dev)
            e_cp = [torch.cuda.Event() for _ in ch]
            e_ca = [torch.cuda.Event() for _ in ch]
            e_cu = [torch.cuda.Event() for _ in ch]
            for e in e_ca + e_cu:
                e.record(main_s)

            def tp_pack(c, stream):
                usp.usp_pack_seq_to_heads_planes(shard, blocks, rank=0, head_lo=ch[c][0],
                                                 head_hi=ch[c][1], stream=stream)

            def tp_attn(c):
                usp.usp_attention_fwd_ws(*blk0, oblocks[0], ws_c, head_lo=ch[c][0], head_hi=ch[c][1],
                                         stream=main_s)

            def tp_unpack(c, stream):
                usp.usp_unpack_heads_to_seq_chunk(oblocks, oshard, ch[c][0], ch[c][1], rank=0,
                                                  stream=stream)

            def tp_serial(n):
                for _ in range(n):
                    for c in range(len(ch)):
                        tp_pack(c, main_s)
                        tp_attn(c)
                        tp_unpack(c, main_s)

            def tp_pipelined(n):
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

            for name, fn in (("two_phase_serial", tp_serial), ("two_phase", tp_pipelined)):
                fn(args.warmup)
                torch.cuda.synchronize()
                a, b_ = ev(), ev()
                a.record(main_s)
                fn(args.steps)
                b_.record(main_s)
                torch.cuda.synchronize()
                legs[name] = {"mean_ms": a.elapsed_time(b_) / args.steps, "steps": args.steps,
                              "flop": attn_flops}
                got = oshard.clone()
                step()
                torch.cuda.synchronize()
                if not torch.equal(got, oshard):
                    raise RuntimeError(f"{name} steps differ from a single-shot step")
            del ws_c

        if on("worlds"):
            # the other workloads' whole worlds: pack q, k, v -> attention of every
            # head group -> unpack, with each part timed
            def world_leg(name, sets):
                wl = synth.WORKLOADS[name]
                tbw = usp.usp_balanced_ranges(wl.S, wl.P)
                hbw = usp.usp_balanced_ranges(wl.H, wl.P)
                del tbw
                host = data[name]
                sets_ = []
                for si in range(sets):
                    qkv = [bf(x) for x in host]
                    bl = [blocks_of(wl.B, wl.S, hbw, wl.D) for _ in range(3)]
                    ob = blocks_of(wl.B, wl.S, hbw, wl.D)
                    out = torch.empty((wl.B, wl.S, wl.H, wl.D), dtype=torch.bfloat16, device=dev)
                    wsw = torch.empty(usp.usp_attention_workspace_bytes(
                        usp.USP_BF16, wl.B, wl.S, max(hbw[j + 1] - hbw[j] for j in range(wl.P)), wl.D),
                        dtype=torch.uint8, device=dev)
                    sets_.append((qkv, bl, ob, out, wsw))
                flops = 4.0 * wl.B * wl.H * wl.S * wl.S * wl.D
                tw = [Timer(torch) for _ in range(4)]

                def run(i):
                    qkv, bl, ob, out, wsw = sets_[i % sets]
                    tw[0](usp.usp_pack_seq_to_heads_planes, qkv, bl)
                    a_ = torch.cuda.Event(enable_timing=True)
                    a_.record()
                    for j in range(wl.P):
                        usp.usp_attention_fwd_ws(bl[0][j], bl[1][j], bl[2][j], ob[j], wsw)
                    b2 = torch.cuda.Event(enable_timing=True)
                    b2.record()
                    tw[1].ev.append((a_, b2))
                    tw[2](usp.usp_unpack_heads_to_seq, ob, out)

                host, gpu = host_ms_per_call(torch, run, 3)
                top_up_warmup(torch, run, gpu, 3)
                tw = [Timer(torch) for _ in range(4)]
                n = max(6, reps)
                spin_if_host_bound(torch, host, gpu, n)
                whole = Timer(torch)
                for i in range(n):
                    whole(run, i)
                pk, at, up, wh = tw[0].summary(), tw[1].summary(), tw[2].summary(), whole.summary()
                res = {"B": wl.B, "S": wl.S, "H": wl.H, "D": wl.D, "P": wl.P, "flop": flops,
                       "buffer_sets": sets, "pack_qkv": pk, "attention": at, "unpack": up, "step": wh,
                       "attention_TFLOP/s": tflops(flops, at["median_ms"]),
                       "attention_frac": tflops(flops, at["median_ms"]) / PEAK_BF16_TFLOPS,
                       "step_TFLOP/s": tflops(flops, wh["median_ms"]),
                       "pack_qkv_GB/s": gbs(3 * 2 * wl.B * wl.S * wl.H * wl.D * 2, pk["median_ms"]),
                       "unpack_GB/s": gbs(2 * wl.B * wl.S * wl.H * wl.D * 2, up["median_ms"])}
                del sets_
                return res

            say("ViT-L/16 world (warm, then cold)")
            out_extra["vit_l16_world"] = {"warm": world_leg("vit_l16", 1), "cold": world_leg("vit_l16", 3)}
            say("indivisible long world")
            out_extra["indivisible_long_world"] = world_leg("indivisible_long", 1)

    # plain device copy of 1 GiB: practical HBM reference and counter calibration
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp = timed(torch, lambda i: dst.copy_(src), 4, warm=2)
    copy_gbs = gbs(2.0 * COPY_BYTES, cp["median_ms"])
    del src, dst

    rel = {}
    rows_bw = {}
    if legs_on:
        if on("relayout"):
            say("world relayout bandwidth")
            nbytes = B * S * H * D * 2
            sets = [[world[t]] + [torch.empty_like(world[t]).copy_(world[t]) for _ in range(2)]
                    for t in range(3)]   # per tensor, three rotating copies
            dsts = [[blocks_of(B, S, hb, D) for _ in range(3)] for _ in range(3)]
            cb = 2 * (nbytes * 2 // h0)   # heads [0, 2) of every group of 5, read + write

            def rl(name, fn, moved):
                r = timed(torch, fn, args.relayout_reps)
                r.update({"GB/s": gbs(moved, r["median_ms"]), "GB/s_min_time": gbs(moved, r["min_ms"]),
                          "frac_peak": gbs(moved, r["median_ms"]) / PEAK_HBM_GBS, "bytes_rw": moved})
                rel[name] = r

            rl("pack", lambda i: usp.usp_pack_seq_to_heads(sets[0][i % 3], dsts[0][i % 3]), 2 * nbytes)
            rl("unpack", lambda i: usp.usp_unpack_heads_to_seq(dsts[0][i % 3], sets[0][i % 3]), 2 * nbytes)
            rl("pack_qkv", lambda i: usp.usp_pack_seq_to_heads_planes(
                [sets[t][i % 3] for t in range(3)], [dsts[t][i % 3] for t in range(3)]), 6 * nbytes)
            rl("pack_chunk", lambda i: usp.usp_pack_seq_to_heads_chunk(sets[0][i % 3], dsts[0][i % 3], 0, 2),
               cb)
            rl("unpack_chunk", lambda i: usp.usp_unpack_heads_to_seq_chunk(dsts[0][i % 3], sets[0][i % 3],
                                                                           0, 2), cb)
            rl("pack_chunk_qkv", lambda i: usp.usp_pack_seq_to_heads_planes(
                [sets[t][i % 3] for t in range(3)], [dsts[t][i % 3] for t in range(3)], head_lo=0,
                head_hi=2), 3 * cb)
            # rank 0's share, as in the step (one call moves one shard per
            # tensor): per call with events, and back to back; sources and
            # destinations rotate over 9 sets (377 MB of blocks)
            len0 = tb[1] - tb[0]
            shares = [[torch.empty((B, len0, H, D), dtype=torch.bfloat16, device=dev).normal_()
                       for _ in range(3)] for _ in range(3)]
            sb = 2 * B * len0 * H * D * 2
            share_legs = (
                ("pack_qkv_rank0", lambda i: usp.usp_pack_seq_to_heads_planes(
                    [shares[t][i % 3] for t in range(3)], [dsts[t][(i + t) % 3] for t in range(3)], rank=0),
                 3 * sb),
                ("unpack_rank0", lambda i: usp.usp_unpack_heads_to_seq(
                    dsts[i % 9 // 3][i % 3], shares[i % 9 // 3][i % 3], rank=0), sb))
            for name, fn, moved in share_legs:
                rl(name, fn, moved)
                ms_b2b = back_to_back(torch, fn, args.relayout_reps)
                rel[name].update({"back_to_back_ms": ms_b2b, "GB/s_back_to_back": gbs(moved, ms_b2b),
                                  "frac_peak_back_to_back": gbs(moved, ms_b2b) / PEAK_HBM_GBS})
            del shares
            for r in rel.values():
                r["frac_of_copy"] = r["GB/s"] / copy_gbs
            del sets, dsts

        if on("rows"):
            say("model-boundary row movements")
            W = H * D
            nb = B * S * W * 2
            fulls = [torch.randn((B, S, W), device=dev).to(torch.bfloat16) for _ in range(3)]
            shard_sets = [[torch.empty((B, tb[r + 1] - tb[r], W), dtype=torch.bfloat16, device=dev)
                           for r in range(P)] for _ in range(3)]
            partials = [torch.randn((B, S, W), device=dev).to(torch.bfloat16) for _ in range(P)]
            for name, fn, moved in (
                    ("scatter", lambda i: usp.usp_scatter_rows(fulls[i % 3], shard_sets[i % 3]), 2 * nb),
                    ("gather", lambda i: usp.usp_gather_rows(shard_sets[i % 3], fulls[i % 3]), 2 * nb),
                    ("reduce_scatter", lambda i: usp.usp_reduce_scatter_rows(partials, shard_sets[i % 3]),
                     (P + 1) * nb)):
                r = timed(torch, fn, args.relayout_reps)
                r.update({"GB/s": gbs(moved, r["median_ms"]), "frac_peak": gbs(moved, r["median_ms"]) /
                          PEAK_HBM_GBS, "bytes": moved})
                rows_bw[name] = r
            rows_bw["shape"] = {"B": B, "S": S, "W": W, "P": P, "dtype": "bf16"}
            del fulls, shard_sets, partials

    # compact per-leg figures (also kept inside the roofline object)
    summary = {"attn_video_dit_share": {"TFLOP/s": attn_tflops, "frac": attn_tflops / PEAK_BF16_TFLOPS,
                                        "median_ms": t_attn["median_ms"], "min_ms": t_attn["min_ms"]},
               "step_pack_qkv_rank0": {"GB/s": gbs(3 * share_bytes, t_pack["median_ms"]),
                                       "frac": gbs(3 * share_bytes, t_pack["median_ms"]) / PEAK_HBM_GBS},
               "step_unpack_o_rank0": {"GB/s": gbs(share_bytes, t_unpack["median_ms"]),
                                       "frac": gbs(share_bytes, t_unpack["median_ms"]) / PEAK_HBM_GBS}}
    for name, r in legs.items():
        f = r.get("flop", attn_flops)
        ms = r.get("median_ms", r["mean_ms"])
        summary[name] = {"TFLOP/s": tflops(f, ms), "frac": tflops(f, ms) / PEAK_BF16_TFLOPS,
                         "median_ms": ms}
        if "max_abs" in r:
            summary[name].update({"max_abs": r["max_abs"], "rel_frob": r["rel_frob"]})
    for name, r in out_extra.items():
        for tag, rr in ([("", r)] if "flop" in r else [("_" + k, v) for k, v in r.items()]):
            summary[name + tag] = {"attn_TFLOP/s": rr["attention_TFLOP/s"],
                                   "attn_frac": rr["attention_frac"],
                                   "step_TFLOP/s": rr["step_TFLOP/s"],
                                   "pack_qkv_GB/s": rr["pack_qkv_GB/s"], "unpack_GB/s": rr["unpack_GB/s"]}
    for name, r in rel.items():
        summary["relayout_" + name] = {"GB/s": r["GB/s"], "frac": r["frac_peak"]}
        if "GB/s_back_to_back" in r:
            summary["relayout_" + name].update({"GB/s_back_to_back": r["GB/s_back_to_back"],
                                                "frac_back_to_back": r["frac_peak_back_to_back"]})
    for name in ("scatter", "gather", "reduce_scatter"):
        if name in rows_bw:
            summary["rows_" + name] = {"GB/s": rows_bw[name]["GB/s"], "frac": rows_bw[name]["frac_peak"]}

    out = {
        "metric": METRIC,
        "value": tflops(attn_flops, pipe_ms),
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
                   "P": P, "rank": 0, "warmup_steps_done": n_warm,
                   "step": "pack rank-0 shard of q,k,v -> attention on head group 0 -> unpack "
                           "rank-0 rows; pipelined on two streams"},
        "attention": dict(t_attn, **{"TFLOP/s": attn_tflops, "frac_peak": attn_tflops / PEAK_BF16_TFLOPS,
                                     "flop": attn_flops, "entry": "usp_attention_fwd_ws"}),
        "step_serial": {"ms_per_step": ms_step, "TFLOP/s": tflops(attn_flops, ms_step),
                        "pack_qkv": t_pack, "attention": t_attn, "unpack_o": t_unpack},
        "step_pack_qkv": dict(t_pack, **{"GB/s": gbs(3 * share_bytes, t_pack["median_ms"])}),
        "step_unpack_o": dict(t_unpack, **{"GB/s": gbs(share_bytes, t_unpack["median_ms"])}),
        "legs": legs,
        "configs": out_extra,
        "relayout_world": rel,
        "rows_world": rows_bw,
        "copy_reference_GB/s": copy_gbs,
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(),
                     "kernel": "usp_attention_fwd_ws: attn_bf16_kernel + attn_merge_halves",
                     "median_ms": t_attn["median_ms"], "min_ms": t_attn["min_ms"],
                     "mean_ms": t_attn["mean_ms"], "legs": summary},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
