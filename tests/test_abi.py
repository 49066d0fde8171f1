"""The C ABI on the host (no GPU): exports, host range logic, argument checks.

Every call here returns before any device work: host-only range functions,
and invalid arguments that the library must reject without launching."""
import ctypes
import os
import subprocess

import pytest

import ulysses_sequence_attention_amd as usp
from oracle import ranges as R

L = usp.lib()
FAKE = 0x10000  # 16-byte aligned address that is never dereferenced


def test_exports_every_declared_symbol():
    declared = usp.header_symbols()
    assert len(declared) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", usp._binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(L, name)


def test_version():
    assert "gfx950" in usp.usp_version()


def test_host_ranges_match_oracle():
    for total in range(1, 80):
        for parts in range(1, min(total, 70) + 1):
            assert usp.usp_balanced_ranges(total, parts) == R.balanced_ranges(total, parts)
    for total, parts in [(32760, 8), (65537, 4), (131072, 7), (2**40 + 3, 64)]:
        assert usp.usp_balanced_ranges(total, parts) == R.balanced_ranges(total, parts)


def test_head_chunks_match_oracle():
    for heads in range(1, 40):
        for chunks in range(1, heads + 1):
            try:
                ref = R.head_chunk_ranges(heads, chunks)
            except ValueError:
                with pytest.raises(usp.UspError) as e:
                    usp.usp_head_chunk_ranges(heads, chunks)
                assert e.value.status == -1
                continue
            assert usp.usp_head_chunk_ranges(heads, chunks) == ref


@pytest.mark.parametrize("total,parts", [(3, 4), (5, 0), (0, 1), (-1, 1)])
def test_range_errors(total, parts):
    with pytest.raises(usp.UspError) as e:
        usp.usp_balanced_ranges(total, parts)
    assert e.value.status == -1
    assert usp.usp_last_error()


def _pack(seq=FAKE, blk=(FAKE,), dt=1, B=1, S=8, H=4, D=64, P=1, rank=-1):
    arr = (ctypes.c_void_p * max(len(blk), 1))(*blk)
    return L.usp_pack_seq_to_heads(seq, arr, dt, B, S, H, D, P, rank, None)


def _unpack(seq=FAKE, blk=(FAKE,), dt=1, B=1, S=8, H=4, D=64, P=1, rank=-1):
    arr = (ctypes.c_void_p * max(len(blk), 1))(*blk)
    return L.usp_unpack_heads_to_seq(arr, seq, dt, B, S, H, D, P, rank, None)


@pytest.mark.parametrize("fn", [_pack, _unpack])
@pytest.mark.parametrize("kw,status", [
    (dict(P=0), -1), (dict(P=65, blk=(FAKE,) * 65, H=65, S=65), -1),
    (dict(S=2, P=3, blk=(FAKE,) * 3), -1), (dict(H=2, P=3, blk=(FAKE,) * 3), -1),
    (dict(rank=1), -1), (dict(B=0), -2), (dict(D=0), -2), (dict(dt=7), -3),
    (dict(D=4), -4), (dict(dt=0, D=2), -4), (dict(seq=FAKE + 8), -4),
    (dict(blk=(FAKE + 4,)), -4), (dict(seq=None), -1), (dict(blk=(None,)), -1),
    (dict(B=2**40, S=2**40), -2),
])
def test_relayout_rejects(fn, kw, status):
    assert fn(**kw) == status
    assert usp.usp_last_error()


def _pack_chunk(seq=FAKE, blk=(FAKE, FAKE), dt=1, B=1, S=8, H=4, D=64, P=2, rank=-1, lo=0, hi=1):
    arr = (ctypes.c_void_p * max(len(blk), 1))(*blk)
    return L.usp_pack_seq_to_heads_chunk(seq, arr, dt, B, S, H, D, P, rank, lo, hi, None)


def _unpack_chunk(seq=FAKE, blk=(FAKE, FAKE), dt=1, B=1, S=8, H=4, D=64, P=2, rank=-1, lo=0, hi=1):
    arr = (ctypes.c_void_p * max(len(blk), 1))(*blk)
    return L.usp_unpack_heads_to_seq_chunk(arr, seq, dt, B, S, H, D, P, rank, lo, hi, None)


@pytest.mark.parametrize("fn", [_pack_chunk, _unpack_chunk])
@pytest.mark.parametrize("kw,status", [
    # the whole-group checks
    (dict(P=0), -1), (dict(S=1), -1), (dict(rank=2), -1), (dict(B=0), -2), (dict(dt=7), -3),
    (dict(D=4), -4), (dict(seq=FAKE + 8), -4), (dict(blk=(FAKE, None)), -1),
    # the chunk: equal groups, non-empty, inside a group of H / P heads
    (dict(H=5), -1), (dict(lo=1, hi=1), -1), (dict(lo=0, hi=3), -1), (dict(lo=-1), -1),
    (dict(lo=2, hi=1), -1),
])
def test_chunk_relayout_rejects(fn, kw, status):
    assert fn(**kw) == status
    assert usp.usp_last_error()


def _attn(q=FAKE, k=FAKE, v=FAKE, o=FAKE, i=1, out=0, B=1, S=16, h=2, D=64, lo=0, hi=2,
          scale=0.0, lse=None):
    return L.usp_attention_fwd(q, k, v, o, i, out, B, S, h, D, lo, hi, scale, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(h=0, hi=0), -1), (dict(lo=1, hi=1), -1),
    (dict(lo=0, hi=3), -1), (dict(lo=-1), -1), (dict(B=0), -2), (dict(S=0), -2),
    (dict(i=5), -3), (dict(out=5), -3), (dict(i=0, out=1), -3), (dict(D=96), -5),
    (dict(i=0, D=48), -5), (dict(k=FAKE + 2), -4), (dict(lse=FAKE + 2), -4),
])
def test_attention_rejects(kw, status):
    assert _attn(**kw) == status
    assert usp.usp_last_error()


def _ws_bytes(i, B, S, heads, D):
    out = ctypes.c_size_t(12345)
    st = L.usp_attention_workspace_bytes(i, B, S, heads, D, ctypes.byref(out))
    return st, out.value


def test_workspace_bytes():
    # two key halves x 256-row tiles x (D unnormalised O + 1 maximum + 2 row sums) fp32
    assert _ws_bytes(1, 1, 32760, 5, 128) == (0, 128 * 5 * 2 * 256 * 131 * 4)
    assert _ws_bytes(1, 2, 257, 3, 64) == (0, 2 * 3 * 2 * 2 * 256 * 67 * 4)
    assert _ws_bytes(1, 1, 1, 1, 64) == (0, 2 * 256 * 67 * 4)
    assert _ws_bytes(0, 1, 1000, 4, 64) == (0, 0)  # fp32 inputs need none
    assert usp.usp_attention_workspace_bytes(usp.USP_BF16, 1, 512, 2, 128) == 2 * 2 * 2 * 256 * 131 * 4
    assert L.usp_attention_workspace_bytes(1, 1, 16, 2, 64, None) == -1
    assert _ws_bytes(1, 0, 16, 2, 64)[0] == -2
    assert _ws_bytes(1, 1, 16, 0, 64)[0] == -2
    assert _ws_bytes(7, 1, 16, 2, 64)[0] == -3


def _attn_ws(ws=FAKE, nbytes=1 << 40, q=FAKE, i=1, out=0, B=1, S=16, h=2, D=64, lo=0, hi=2):
    return L.usp_attention_fwd_ws(q, FAKE, FAKE, FAKE, i, out, B, S, h, D, lo, hi, 0.0, None, ws,
                                  nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), -1), (dict(ws=FAKE + 4), -4), (dict(nbytes=1000), -1),
    (dict(nbytes=2 * 2 * 256 * 67 * 4 - 1), -1), (dict(q=None), -1), (dict(D=96), -5),
    (dict(lo=0, hi=3), -1),
])
def test_attention_ws_rejects(kw, status):
    assert _attn_ws(**kw) == status
    assert usp.usp_last_error()


def _planes(n=2, seq=True, blk=True, bad_plane=None, P=3, H=6, lo=0, hi=0):
    seqs = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    blks = (ctypes.c_void_p * (4 * P))(*([FAKE] * (4 * P)))
    if bad_plane is not None:
        seqs[bad_plane] = FAKE + 4
    return L.usp_pack_seq_to_heads_planes(n, seqs if seq else None, blks if blk else None, 1, 1, 64,
                                          H, 64, P, -1, lo, hi, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), -1), (dict(n=5), -1), (dict(seq=False), -1), (dict(blk=False), -1),
    (dict(bad_plane=1), -4),            # the second plane's tensor is misaligned
    (dict(H=7, lo=0, hi=1), -1),         # head-chunk phase with ragged groups
    (dict(lo=1, hi=1), -1),              # empty head chunk
    (dict(P=0), -1),
])
def test_planes_reject(kw, status):
    assert _planes(**kw) == status
    assert usp.usp_last_error()


def test_planes_binding_rejects_mismatched_planes():
    import torch
    a = torch.empty((1, 8, 6, 64), dtype=torch.bfloat16)
    b = torch.empty((1, 8, 6, 64), dtype=torch.float32)
    blocks = [[torch.empty((1, 8, 2, 64), dtype=torch.bfloat16) for _ in range(3)]] * 2
    with pytest.raises(ValueError):
        usp.usp_pack_seq_to_heads_planes([a, b], blocks)
    with pytest.raises(ValueError):
        usp.usp_pack_seq_to_heads_planes([a], blocks)


def _attn_na(q=FAKE, i=1, out=0, B=1, S=16, h=2, D=64, lo=0, hi=2):
    return L.usp_attention_fwd_noalloc(q, FAKE, FAKE, FAKE, i, out, B, S, h, D, lo, hi, 0.0, None,
                                       None)


@pytest.mark.parametrize("kw,status", [
    # beyond the static scratch: 2 x 16384 rows x 8 heads at D = 128 (268 MB > 192 MiB),
    # rejected from the sizes alone, before any device call
    (dict(B=2, S=16384, h=8, D=128, hi=8), -1),
    (dict(q=None), -1), (dict(D=96), -5), (dict(lo=1, hi=1), -1), (dict(i=7), -3),
])
def test_noalloc_rejects(kw, status):
    assert _attn_na(**kw) == status
    msg = usp.usp_last_error()
    assert msg
    if kw.get("B") == 2:
        assert "scratch" in msg and str(192 << 20) in msg


def test_noalloc_scratch_limit_in_header():
    text = open(usp._binding.HEADER).read()
    assert "#define USP_NOALLOC_SCRATCH_BYTES (192u << 20)" in text
    # the video-DiT share (B = 1, S = 32760, 5 heads, D = 128) fits
    assert _ws_bytes(1, 1, 32760, 5, 128)[1] <= 192 << 20


def test_chunked_rejects():
    f = L.usp_attention_fwd_chunked
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, 5, 64, 0.0, None, 4, None) == -1  # empty chunk
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, 5, 64, 0.0, None, 6, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, 5, 64, 0.0, None, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, 5, 80, 0.0, None, 2, None) == -5


def test_single_hip_runtime_in_process():
    # libusp must share PyTorch's HIP runtime: a second libamdhip64 copy in the
    # process leaves PyTorch on a runtime it was not built for.
    import os
    usp.lib()
    with open(f"/proc/{os.getpid()}/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def _attn_gqa(h=4, hkv=2, lo=0, hi=4, ws=None, nbytes=0, D=64):
    return L.usp_attention_fwd_gqa(FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, h, hkv, D, lo, hi, 0.0,
                                   None, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hkv=0), -1), (dict(hkv=3), -1), (dict(hkv=5, h=4), -1), (dict(h=6, hkv=4, hi=6), -1),
    (dict(ws=FAKE + 4, nbytes=1 << 30), -4), (dict(ws=FAKE, nbytes=100), -1), (dict(D=80), -5),
])
def test_attention_gqa_rejects(kw, status):
    assert _attn_gqa(**kw) == status
    assert usp.usp_last_error()


def _rows(fn, full=FAKE, ptrs=(FAKE, FAKE), dt=1, B=1, S=8, W=64, P=2, rank=-1, parts=None):
    arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    if fn == "scatter":
        return L.usp_scatter_rows(full, arr, dt, B, S, W, P, rank, None)
    if fn == "gather":
        return L.usp_gather_rows(arr, full, dt, B, S, W, P, None)
    parr = (ctypes.c_void_p * max(len(parts or ptrs), 1))(*(parts or ptrs))
    return L.usp_reduce_scatter_rows(parr, arr, dt, B, S, W, P, rank, None)


@pytest.mark.parametrize("fn", ["scatter", "gather", "reduce"])
@pytest.mark.parametrize("kw,status", [
    (dict(P=0), -1), (dict(P=65, ptrs=(FAKE,) * 65, S=65), -1), (dict(S=1), -1),
    (dict(B=0), -2), (dict(W=0), -2), (dict(dt=7), -3), (dict(W=4), -4), (dict(dt=0, W=2), -4),
    (dict(ptrs=(FAKE, FAKE + 8)), -4), (dict(ptrs=(FAKE, None)), -1), (dict(B=2**40, S=2**40), -2),
])
def test_rows_reject(fn, kw, status):
    assert _rows(fn, **kw) == status
    assert usp.usp_last_error()


def test_rows_reject_rank_and_full():
    assert _rows("scatter", rank=2) == -1
    assert _rows("reduce", rank=2) == -1
    assert _rows("scatter", full=None) == -1
    assert _rows("gather", full=FAKE + 4) == -4
    assert _rows("reduce", parts=(FAKE, None)) == -1


def _attn_block(q=FAKE, k=FAKE, Sq=16, Sk=40, h=4, hkv=2, lo=0, hi=4, ws=None, nbytes=0, D=64,
                i=1, out=0):
    return L.usp_attention_fwd_block(q, k, FAKE, FAKE, i, out, 1, Sq, Sk, h, hkv, D, lo, hi, 0.0,
                                     None, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Sk=0), -2), (dict(Sq=0), -2), (dict(Sk=2**31), -2), (dict(hkv=3), -1),
    (dict(lo=2, hi=2), -1), (dict(k=None), -1), (dict(k=FAKE + 8), -4), (dict(D=80), -5),
    (dict(i=0, out=1), -3), (dict(ws=FAKE + 4, nbytes=1 << 30), -4),
    (dict(ws=FAKE, nbytes=2 * 256 * 67 * 4 * 4 - 1), -1),
])
def test_attention_block_rejects(kw, status):
    assert _attn_block(**kw) == status
    assert usp.usp_last_error()


def _attn_block_whole(q=FAKE, k=FAKE, Sq=16, Sk=40, h=4, hkv=2, lo=0, hi=4, D=64, i=1, out=0,
                      lse=None):
    return L.usp_attention_fwd_block_whole(q, k, FAKE, FAKE, i, out, 1, Sq, Sk, h, hkv, D, lo, hi,
                                           0.0, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Sk=0), -2), (dict(Sq=0), -2), (dict(Sk=2**31), -2), (dict(hkv=3), -1),
    (dict(hkv=0), -1), (dict(lo=2, hi=2), -1), (dict(hi=5), -1), (dict(k=None), -1),
    (dict(q=None), -1), (dict(k=FAKE + 8), -4), (dict(lse=FAKE + 2), -4), (dict(D=80), -5),
    (dict(i=1, D=32), -5), (dict(i=0, out=1), -3), (dict(i=5), -3), (dict(out=3), -3),
])
def test_attention_block_whole_rejects(kw, status):
    assert _attn_block_whole(**kw) == status
    assert usp.usp_last_error()


def _merge(oa=FAKE, la=FAKE, ob=FAKE + 256, lb=FAKE + 512, o=FAKE + 1024, lse=None, out=0, B=1,
           S=16, h=2, D=64, lo=0, hi=2):
    return L.usp_attention_merge(oa, la, ob, lb, o, lse, out, B, S, h, D, lo, hi, None)


@pytest.mark.parametrize("kw,status", [
    (dict(oa=None), -1), (dict(lb=None), -1), (dict(o=None), -1), (dict(h=0, hi=0), -1),
    (dict(lo=2, hi=2), -1), (dict(hi=3), -1), (dict(B=0), -2), (dict(S=0), -2), (dict(out=4), -3),
    (dict(D=48), -5), (dict(D=256), -5), (dict(oa=FAKE + 8), -4), (dict(o=FAKE + 4), -4),
    (dict(la=FAKE + 2), -4), (dict(lse=FAKE + 1), -4), (dict(out=1, o=FAKE), -1),
    (dict(out=1, o=FAKE + 256), -1), (dict(B=2**40, S=2**20), -2),
])
def test_attention_merge_rejects(kw, status):
    assert _merge(**kw) == status
    assert usp.usp_last_error()


def test_chunked_ws_rejects():
    f = L.usp_attention_fwd_chunked_ws
    need = 2 * 256 * 67 * 4 * 3   # S = 16, D = 64: one tile per head, largest pass 3 heads
    args = (FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 16, 5, 64, 0.0, None)
    assert f(*args, 2, None, need, None) == -1           # no workspace
    assert f(*args, 2, FAKE + 4, need, None) == -4       # misaligned
    assert f(*args, 2, FAKE, need - 1, None) == -1       # below the largest pass
    assert f(*args, 4, FAKE, need, None) == -1           # 5 heads in 4 chunks leaves one empty
    assert f(*args[:9], 80, *args[10:], 2, FAKE, need, None) == -5  # D = 80
    assert usp.usp_last_error()


def test_c_consumer_links_against_this_library():
    """The plain C consumer of the ABI resolves libusp to this package's build
    and the HIP runtime, with no PyTorch library (linking only, no GPU)."""
    import os
    binp = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "usp_abi_check")
    assert os.path.exists(binp), "run __graft_entry__.build() first"
    out = subprocess.run(["ldd", binp], capture_output=True, text=True, check=True).stdout
    libs = {line.split()[0]: line for line in out.splitlines() if "=>" in line}
    assert os.path.realpath(usp._binding.LIB_PATH) in os.path.realpath(libs["libusp.so"].split("=>")[1].split()[0])
    assert "libamdhip64.so.7" in libs and "not found" not in libs["libamdhip64.so.7"]
    assert not any("torch" in line for line in libs.values())


def test_binding_fails_loudly_without_the_library():
    """No fallback path: with libusp.so absent the binding raises instead of
    computing anything (checked in a fresh process)."""
    import subprocess
    import sys
    code = ("import ulysses_sequence_attention_amd._binding as b\n"
            "b._LIB = None\n"
            "b.LIB_PATH = '/nonexistent/libusp.so'\n"
            "try:\n"
            "    b.usp_balanced_ranges(10, 3)\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    print('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.stdout.startswith("raised") and "is missing" in r.stdout, r.stdout + r.stderr
