"""The hot path under HIP graph capture. Given a caller workspace the library
neither allocates nor synchronizes, so a whole step — pack of Q, K, V,
attention of every head group, unpack — can be captured once and
replayed. Each replay follows new inputs copied into the captured buffers
and eager work on the device, and is compared bit for bit with the same step
run eagerly."""
import pytest

import ulysses_sequence_attention_amd as usp
from ulysses_sequence_attention_amd import synth

from gpu_util import DEV, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("phases", [False, True])
def test_step_replays_from_a_captured_graph(phases):
    """phases: the two-phase form of the same step (per head chunk 2/2 of the
    4 heads of a group: pack, attention, unpack), whose replays must also
    equal the eager single-shot step."""
    import torch
    w = synth.WORKLOADS["vit_l16"]            # B=32, S=577, H=16, D=64, P=4
    B, S, H, D, P = w.B, w.S, w.H, w.D, w.P
    hb = usp.usp_balanced_ranges(H, P)
    bf = torch.bfloat16
    qkv = [torch.empty((B, S, H, D), dtype=bf, device=DEV) for _ in range(3)]
    blocks = [[torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=bf, device=DEV) for j in range(P)]
              for _ in range(3)]
    oblocks = [torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=bf, device=DEV) for j in range(P)]
    out = torch.empty((B, S, H, D), dtype=bf, device=DEV)
    hmax = max(hb[j + 1] - hb[j] for j in range(P))
    ws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, hmax, D) // 4,
                     dtype=torch.float32, device=DEV)

    def step():
        for x, bl in zip(qkv, blocks):
            usp.usp_pack_seq_to_heads(x, bl)
        for j in range(P):
            usp.usp_attention_fwd_ws(blocks[0][j], blocks[1][j], blocks[2][j], oblocks[j], ws)
        usp.usp_unpack_heads_to_seq(oblocks, out)

    def step_phases():
        for lo, hi in ((0, 2), (2, 4)):
            for x, bl in zip(qkv, blocks):
                usp.usp_pack_seq_to_heads_chunk(x, bl, lo, hi)
            for j in range(P):
                usp.usp_attention_fwd_ws(blocks[0][j], blocks[1][j], blocks[2][j], oblocks[j], ws,
                                         head_lo=lo, head_hi=hi)
            usp.usp_unpack_heads_to_seq_chunk(oblocks, out, lo, hi)

    captured = step_phases if phases else step
    assert usp.usp_head_chunk_ranges(hb[1] - hb[0], 2) == [0, 2, 4]

    def load(seed):
        for dst, src in zip(qkv, synth.draw_qkv(B, S, H, D, seed)):
            dst.copy_(to_dev(src, synth.BF16))

    load(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up outside the capture
        captured()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    log(f"capture pack -> attention x4 -> unpack (ViT-L/16 world){' in head-chunk phases' if phases else ''}")
    with torch.cuda.graph(graph):
        captured()
    torch.cuda.synchronize()
    for i, seed in enumerate((101, 102, 103)):
        load(seed)
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)
        log(f"graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        del junk
        log(f"eager step {i}")
        step()
        torch.cuda.synchronize()
        assert torch.equal(got, out), f"replay {i} differs from the eager step"
        assert not torch.isnan(got.float()).any()


def test_default_attention_under_capture():
    """usp_attention_fwd given no workspace, captured into a graph: while the
    stream is capturing the call takes nothing from the library's pool and
    runs the key-group kernel (1000 keys at D = 128 split in halves). Every
    replay, with new inputs copied in and eager work between, equals the
    eager call (which takes its workspace from the pool) bit for bit."""
    import torch
    B, S, h, D = 1, 1000, 4, 128
    q, k, v = (torch.empty((B, S, h, D), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    o = torch.empty((B, S, h, D), dtype=torch.float32, device=DEV)

    def load(seed):
        for dst, src in zip((q, k, v), synth.draw_qkv(B, S, h, D, seed)):
            dst.copy_(to_dev(src, synth.BF16))

    load(200)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up outside the capture
        usp.usp_attention_fwd(q, k, v, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    log("capture usp_attention_fwd without a workspace")
    with torch.cuda.graph(graph):
        usp.usp_attention_fwd(q, k, v, o)
    torch.cuda.synchronize()
    for i, seed in enumerate((201, 202, 203)):
        load(seed)
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)
        log(f"graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        got = o.clone()
        del junk
        log(f"eager call {i}")
        usp.usp_attention_fwd(q, k, v, o)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), o.view(torch.int32)), f"replay {i}"
