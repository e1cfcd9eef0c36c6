"""The C-ABI library on the host: it loads, exports every entry point the header
declares, and rejects invalid arguments before any HIP call (CPU only; no call
here reaches a kernel launch)."""
import os
import re
import subprocess

import pytest

import long_context_causal_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

# fake, well-separated, 256-byte-aligned device addresses: never dereferenced
Q, K, V, O, LSE, SQ, SK = (n << 40 for n in range(1, 8))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=LSE, B=1, Hq=16, Hkv=4, Lq=512, Lk=512, D=256, q_offset=0,
            seg_q=None, seg_k=None, causal=1, dtype=gqa.GQA_F32, stream=None)


def call(**over):
    a = dict(GOOD)
    a.update(over)
    return gqa.fwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Lq"], a["Lk"],
                       a["D"], a["q_offset"], a["seg_q"], a["seg_k"], a["causal"], a["dtype"], a["stream"])


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int64_t|int|const char\s*\*)\s*(gqa_attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(gqa.EXPORTS)
    lib = gqa.load_library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gqa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(gqa_attn_\w+)", out))
    assert set(names) <= exported
    # and nothing else: the kernels, launchers and helpers stay internal
    functions = set(re.findall(r"\s[TW]\s(\S+)", out))
    assert functions == exported, sorted(functions - exported)[:5]


def test_version_and_strerror():
    assert gqa.version() == (1, 8)
    msgs = [gqa.strerror(c) for c in range(8)]
    assert len(set(msgs)) == 8 and msgs[0] == "success"
    assert "unknown" in gqa.strerror(99)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(Lq=0), 2), (dict(Lk=-1), 2), (dict(D=0), 2),
    (dict(Hq=16, Hkv=3), 2), (dict(q_offset=-1), 2), (dict(seg_q=SQ), 2), (dict(seg_k=SK), 2),
    (dict(D=128), 3), (dict(dtype=3), 3), (dict(dtype=-1), 3), (dict(Hq=65, Hkv=1), 3), (dict(Hq=256, Hkv=2), 3),
    (dict(Lq=1 << 31), 3), (dict(Lk=1 << 31), 3),
    (dict(q=Q + 2), 4), (dict(k=K + 8), 4), (dict(v=V + 4), 4), (dict(o=O + 2), 4), (dict(lse=LSE + 2), 4),
    (dict(seg_q=SQ + 2, seg_k=SK), 4),
    (dict(o=Q + 4096), 6), (dict(o=K), 6), (dict(lse=O + 64), 6), (dict(lse=V), 6),
    # o or lse over the segment ids, which every workgroup reads while others write
    (dict(seg_q=SQ, seg_k=SK, o=SQ - 4096), 6), (dict(seg_q=SQ, seg_k=SK, o=SK + 256), 6),
    (dict(seg_q=SQ, seg_k=SK, lse=SQ + 4), 6), (dict(seg_q=SQ, seg_k=SK, lse=SK - 64), 6),
])
def test_fwd_rejects_before_launch(over, code):
    assert call(**over) == code


@pytest.mark.parametrize("over,code", [
    (dict(o1=None), 1), (dict(lse=None), 1), (dict(rows=0), 2), (dict(D=0), 2), (dict(D=12), 3),
    (dict(dtype=5), 3), (dict(o1=O + 8), 4), (dict(lse2=LSE + 2), 4), (dict(o=Q + 16), 6),
    (dict(lse=SQ + 4), 6), (dict(o=K + 512), 6),
    # the merged lse over o1 or o2, which other rows still read
    (dict(lse=Q + 64), 6), (dict(lse=K + 1024), 6),
])
def test_merge_rejects_before_launch(over, code):
    a = dict(o1=Q, lse1=SQ, o2=K, lse2=SK, o=O, lse=LSE, rows=100, D=256, dtype=gqa.GQA_F32, stream=None)
    a.update(over)
    assert gqa.merge_raw(a["o1"], a["lse1"], a["o2"], a["lse2"], a["o"], a["lse"], a["rows"], a["D"],
                         a["dtype"], a["stream"]) == code


DO, DQ, DK, DV, DEL = (n << 40 for n in range(8, 13))
BWD_GOOD = dict(q=Q, k=K, v=V, o=O, lse=LSE, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DEL, B=1, Hq=16, Hkv=4,
                Lq=512, Lk=512, D=256, q_offset=0, seg_q=None, seg_k=None, causal=1, dtype=gqa.GQA_F32,
                stream=None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1), (dict(dout=None), 1), (dict(dq=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1), (dict(delta=None), 1),
    (dict(B=0), 2), (dict(Lq=0), 2), (dict(Hq=16, Hkv=3), 2), (dict(q_offset=-1), 2), (dict(seg_q=SQ), 2),
    (dict(D=128), 3), (dict(dtype=7), 3), (dict(Hq=130, Hkv=2), 3), (dict(Lq=(1 << 21) + 1), 3),
    (dict(Lk=(1 << 21) + 1), 3),
    (dict(dout=DO + 4), 4), (dict(dq=DQ + 8), 4), (dict(dk=DK + 2), 4), (dict(delta=DEL + 2), 4),
    (dict(dq=Q), 6), (dict(dq=DO + 256), 6), (dict(dk=V), 6), (dict(dv=DK), 6), (dict(delta=LSE), 6),
    (dict(delta=DQ + 1024), 6), (dict(dv=O + 1024), 6), (dict(seg_q=DQ + 64, seg_k=SK), 6),
    (dict(seg_q=SQ, seg_k=DEL), 6),
])
def test_bwd_rejects_before_launch(over, code):
    a = dict(BWD_GOOD)
    a.update(over)
    assert gqa.bwd_raw(*(a[n] for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta", "B", "Hq",
                                         "Hkv", "Lq", "Lk", "D", "q_offset", "seg_q", "seg_k", "causal",
                                         "dtype", "stream"))) == code


WS = 13 << 40
SPLIT_GOOD = dict(GOOD, n_split=8, workspace=WS, workspace_bytes=1 << 30)


def call_split(**over):
    a = dict(SPLIT_GOOD)
    a.update(over)
    return gqa.fwd_split_raw(*(a[n] for n in ("q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Lq", "Lk", "D",
                                              "q_offset", "seg_q", "seg_k", "causal", "dtype", "n_split",
                                              "workspace", "workspace_bytes", "stream")))


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(Lq=0), 2), (dict(D=128), 3), (dict(q=Q + 2), 4), (dict(o=K), 6),
    (dict(n_split=0), 3), (dict(n_split=1025), 3), (dict(workspace=None), 1),
    (dict(workspace_bytes=8 * 16 * 512 * 257 * 4 - 1), 7), (dict(workspace=WS + 4), 4),
    (dict(workspace=Q + 4096), 6), (dict(workspace=LSE - 1024), 6),
])
def test_fwd_split_rejects_before_launch(over, code):
    assert call_split(**over) == code


def call_noalloc(**over):
    a = dict(GOOD, n_split=0)
    a.update(over)
    return gqa.fwd_split_noalloc_raw(*(a[n] for n in ("q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Lq", "Lk", "D",
                                                      "q_offset", "seg_q", "seg_k", "causal", "dtype", "n_split",
                                                      "stream")))


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(Lq=0), 2), (dict(D=128), 3), (dict(q=Q + 2), 4), (dict(o=K), 6),
    (dict(n_split=-1), 3), (dict(n_split=1025), 3),
    # partials beyond the static scratch: 64 rows x 16 heads x 1024 splits x 257 fp32 = 1.08 GB
    (dict(Lq=64, Lk=65536, n_split=1024), 7),
    (dict(Lq=512, Lk=65536, n_split=8), 7),
])
def test_fwd_split_noalloc_rejects_before_launch(over, code):
    assert call_noalloc(**over) == code


def test_split_workspace_and_count():
    # workspace: n_split * B * Hq * Lq * (D + 1) fp32 values
    assert gqa.split_workspace(2, 16, 100, 256, 8) == 8 * 2 * 16 * 100 * 257 * 4
    assert gqa.split_workspace(1, 16, 100, 256, 0) == 0
    # one decode row over 60,926 keys (bf16 decode kernel, 32-key tiles): 4
    # workgroups without splits, so the count aims at 256 workgroups: 64
    # ranges of >= 4 tiles
    assert gqa.split_count(1, 16, 4, 1, 60926, gqa.GQA_BF16) == 64
    # the 30k fp32 forward already launches 3,808 workgroups
    assert gqa.split_count(1, 16, 4, 30468, 30468, gqa.GQA_F32) == 1
    # short keys: at most a quarter of the tile count (fp32 decode kernel:
    # 1000 keys = 63 tiles of 16)
    assert gqa.split_count(1, 16, 4, 1, 1000, gqa.GQA_F32) == 15
    # fp32 rows past the decode bound (32 positions) take the long-block
    # kernel's 32-key tiles: 32 rows = one block of 4 workgroups, 1000 keys =
    # 32 tiles, at most 8 ranges
    assert gqa.split_count(1, 16, 4, 32, 1000, gqa.GQA_F32) == 8
    # 16-bit decode shapes (Lq < 32) count the decode kernel's workgroups: row
    # blocks of 64 packed (head, position) rows per KV head. 16 heads per KV
    # head x 31 positions = 496 rows = 8 blocks: 32 workgroups per split, so 8
    # splits fill 256; 16 decode rows (64 rows, one block): 64 splits
    assert gqa.split_count(1, 64, 4, 31, 60926, gqa.GQA_BF16) == 8
    assert gqa.split_count(1, 16, 4, 16, 60926, gqa.GQA_F16) == 64
    assert gqa.split_count(1, 16, 4, 16, 60926, gqa.GQA_F32) == 64
    # 32-key tiles: 200 keys = 7 tiles, at most a quarter of them (1)
    assert gqa.split_count(1, 16, 4, 16, 200, gqa.GQA_BF16) == 1
    assert gqa.split_count(1, 16, 4, 16, 260, gqa.GQA_BF16) == 2
    # 16-key tiles (fp32): 200 keys = 13 tiles, a quarter of them (3)
    assert gqa.split_count(1, 16, 4, 16, 200, gqa.GQA_F32) == 3
    # group sizes that are not powers of two: a workgroup takes the largest of
    # 4, 2 and 1 heads that divides the group. 3 heads: 1 head x 4 blocks of
    # 32 positions, so 100 rows are one block x 4 KV heads x 3 head chunks =
    # 12 workgroups and 22 splits; 6 heads: 2 heads x 64 positions, 2 blocks
    # x 4 x 3 = 24 workgroups and 11 splits
    assert gqa.split_count(1, 12, 4, 100, 60926, gqa.GQA_BF16) == 22
    assert gqa.split_count(1, 24, 4, 100, 60926, gqa.GQA_BF16) == 11


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 16, 8, 256)
    k = torch.zeros(1, 4, 8, 256)
    with pytest.raises(ValueError):
        gqa.fwd(q, k, k)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "long_context_causal_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "oracle_attn" not in text, f


# id-range index (gqa_attn_seg_index) and the indexed forward and backward
QI, KI = 14 << 40, 15 << 40


def test_seg_index_bytes():
    assert gqa.seg_index_bytes(1, 131072) == 131072 // 16 * 8
    assert gqa.seg_index_bytes(3, 17) == 3 * 2 * 8  # a partial last block of one id
    assert gqa.seg_index_bytes(0, 16) == 0 and gqa.seg_index_bytes(1, 0) == 0


@pytest.mark.parametrize("over,code", [
    (dict(seg=None), 1), (dict(index=None), 1), (dict(B=0), 2), (dict(L=-3), 2), (dict(L=1 << 31), 3),
    (dict(B=1 << 24), 3), (dict(seg=SQ + 2), 4), (dict(index=QI + 4), 4), (dict(index_bytes=8 * 63 - 1), 7),
    (dict(index=SQ + 256), 6), (dict(index=SQ - 64), 6),
])
def test_seg_index_rejects_before_launch(over, code):
    a = dict(seg=SQ, B=1, L=1000, index=QI, index_bytes=8 * 64, stream=None)
    a.update(over)
    assert gqa.seg_index_raw(a["seg"], a["B"], a["L"], a["index"], a["index_bytes"], a["stream"]) == code


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(Lq=0), 2), (dict(D=128), 3),
    # an index without segment ids, misaligned, or under an output
    (dict(seg_q=None, seg_k=None), 2), (dict(seg_q=None, seg_k=None, seg_q_index=None), 2),
    (dict(seg_q_index=QI + 4), 4), (dict(seg_k_index=KI + 2), 4),
    (dict(o=QI - 4096), 6), (dict(lse=KI + 8), 6), (dict(lse=KI - 64), 6),
])
def test_fwd_indexed_rejects_before_launch(over, code):
    a = dict(GOOD, seg_q=SQ, seg_k=SK, seg_q_index=QI, seg_k_index=KI)
    a.update(over)
    assert gqa.fwd_indexed_raw(*(a[n] for n in ("q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Lq", "Lk", "D",
                                                "q_offset", "seg_q", "seg_k", "seg_q_index", "seg_k_index",
                                                "causal", "dtype", "stream"))) == code


@pytest.mark.parametrize("over,code", [
    (dict(dq=None), 1), (dict(seg_q=None, seg_k=None), 2), (dict(seg_k_index=KI + 4), 4),
    (dict(dq=QI - 64), 6), (dict(delta=KI + 16), 6), (dict(dk=QI - 1024), 6),
])
def test_bwd_indexed_rejects_before_launch(over, code):
    a = dict(BWD_GOOD, seg_q=SQ, seg_k=SK, seg_q_index=QI, seg_k_index=KI)
    a.update(over)
    assert gqa.bwd_indexed_raw(*(a[n] for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta", "B",
                                                "Hq", "Hkv", "Lq", "Lk", "D", "q_offset", "seg_q", "seg_k",
                                                "seg_q_index", "seg_k_index", "causal", "dtype",
                                                "stream"))) == code
