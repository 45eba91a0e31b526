"""C-ABI host logic, without a GPU: the library loads, exports every symbol
include/attn.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import attention_flash_attn_prefill_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["attn_status_string", "attn_prefill", "attn_paged_decode",
                            "attn_paged_decode_workspace_size", "attn_paged_decode_num_splits",
                            "attn_prefill_gqa", "attn_paged_decode_gqa",
                            "attn_paged_decode_gqa_workspace_size",
                            "attn_paged_decode_gqa_num_splits", "attn_extend",
                            "attn_prefill_fp8", "attn_prefill_lse", "attn_prefill_bwd",
                            "attn_prefill_bwd_workspace_size",
                            "attn_paged_decode_gqa_noalloc", "attn_prefill_splitkv",
                            "attn_prefill_splitkv_num_splits",
                            "attn_prefill_splitkv_workspace_size", "attn_extend_splitkv",
                            "attn_extend_splitkv_num_splits",
                            "attn_extend_splitkv_workspace_size"])
    assert set(names) == set(attn.SIGNATURES)


def test_header_constants_match_binding():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    consts = {n: int(v, 0) for n, v in re.findall(r"\b(ATTN_[A-Z0-9_]+)\s*=\s*(0x[0-9a-fA-F]+|\d+)",
                                                  src)}
    assert len(consts) == 10
    for name, value in consts.items():
        assert getattr(attn, name) == value, name


def test_library_exports_every_declared_symbol():
    lib = attn.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings():
    assert attn.attn_status_string(0) == "ok"
    for s in range(1, 5):
        assert attn.attn_status_string(s) not in ("ok", "unknown status")
    assert attn.attn_status_string(99) == "unknown status"


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=1, Sq=16, Skv=16, D=128, layout=0, dtype=0,
             causal=0, scale=0.1, stream=0)
    a.update(kw)
    return attn.attn_prefill(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), attn.ATTN_E_INVALID),
    (dict(Sq=-3), attn.ATTN_E_INVALID),
    (dict(layout=2), attn.ATTN_E_INVALID),
    (dict(dtype=7), attn.ATTN_E_INVALID),
    (dict(dtype=0x200), attn.ATTN_E_INVALID),
    (dict(dtype=attn.ATTN_OUT_F32 | 2), attn.ATTN_E_INVALID),
    (dict(dtype=attn.ATTN_OUT_F32 | attn.ATTN_BF16, D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(scale=float("nan")), attn.ATTN_E_INVALID),
    (dict(scale=float("inf")), attn.ATTN_E_INVALID),
    (dict(scale=-0.5), attn.ATTN_E_INVALID),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(D=256), attn.ATTN_E_UNSUPPORTED),
    (dict(D=0), attn.ATTN_E_INVALID),
    (dict(q=None), attn.ATTN_E_INVALID),
    (dict(o=None), attn.ATTN_E_INVALID),
    (dict(k=None), attn.ATTN_E_INVALID),
    (dict(q=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(v=FAKE + 2), attn.ATTN_E_INVALID),
    (dict(layout=1, H=1 << 20, Sq=4096, Skv=4096), attn.ATTN_E_UNSUPPORTED),  # 32-bit offsets
    (dict(layout=1, H=1 << 17, Sq=2, Skv=2), attn.ATTN_E_UNSUPPORTED),  # in-tile byte offsets
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0),
                                dict(B=0, q=None, k=None, v=None, o=None),
                                dict(Sq=0, q=None, o=None)])
def test_prefill_empty_is_a_noop(kw):
    assert _prefill(**kw) == attn.ATTN_OK


def _prefill_gqa(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=8, H_kv=2, Sq=16, Skv=16, D=128, layout=0,
             dtype=0, causal=0, scale=0.1, stream=0)
    a.update(kw)
    return attn.attn_prefill_gqa(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=3), attn.ATTN_E_INVALID),       # 3 does not divide 8
    (dict(H_kv=0), attn.ATTN_E_INVALID),
    (dict(H_kv=-1), attn.ATTN_E_INVALID),
    (dict(H_kv=16), attn.ATTN_E_INVALID),      # more KV heads than query heads
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(k=None), attn.ATTN_E_INVALID),
    (dict(layout=1, H=1 << 16, H_kv=1 << 16, Sq=4096, Skv=4096), attn.ATTN_E_UNSUPPORTED),
])
def test_prefill_gqa_validation(kw, status):
    assert _prefill_gqa(**kw) == status


def test_prefill_gqa_empty_is_a_noop():
    assert _prefill_gqa(H=0, H_kv=0, q=None, k=None, v=None, o=None) == attn.ATTN_OK
    assert _prefill_gqa(Sq=0) == attn.ATTN_OK


def _prefill_lse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=8, H_kv=2, Sq=16, Skv=16, D=128,
             layout=0, dtype=0, causal=0, scale=0.1, stream=0)
    a.update(kw)
    return attn.attn_prefill_lse(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=FAKE + 2), attn.ATTN_E_INVALID),   # lse must be 4-byte aligned
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(o=None), attn.ATTN_E_INVALID),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(dtype=9), attn.ATTN_E_INVALID),
])
def test_prefill_lse_validation(kw, status):
    assert _prefill_lse(**kw) == status


def test_prefill_lse_empty_is_a_noop():
    assert _prefill_lse(Sq=0, q=None, o=None, lse=None) == attn.ATTN_OK


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dO=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1,
             H=8, H_kv=2, Sq=16, Skv=16, D=128, layout=0, dtype=0, causal=0, scale=0.1,
             workspace=FAKE, workspace_bytes=1 << 20, stream=0)
    a.update(kw)
    return attn.attn_prefill_bwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), attn.ATTN_E_INVALID),
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(H_kv=0), attn.ATTN_E_INVALID),
    (dict(layout=2), attn.ATTN_E_INVALID),
    (dict(dtype=7), attn.ATTN_E_INVALID),
    (dict(scale=float("nan")), attn.ATTN_E_INVALID),
    (dict(scale=-1.0), attn.ATTN_E_INVALID),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(D=0), attn.ATTN_E_INVALID),
    (dict(dO=None), attn.ATTN_E_INVALID),
    (dict(lse=None), attn.ATTN_E_INVALID),
    (dict(dq=None), attn.ATTN_E_INVALID),
    (dict(dk=None), attn.ATTN_E_INVALID),
    (dict(dv=None), attn.ATTN_E_INVALID),
    (dict(dq=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(lse=FAKE + 2), attn.ATTN_E_INVALID),
    (dict(workspace=None), attn.ATTN_E_WORKSPACE),
    (dict(workspace_bytes=2 * 16 * 8 * 4 - 4), attn.ATTN_E_WORKSPACE),
    (dict(workspace=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(layout=1, H=1 << 20, H_kv=1 << 20, Sq=4096, Skv=4096, workspace_bytes=1 << 40),
     attn.ATTN_E_UNSUPPORTED),                   # 32-bit in-head offsets
    (dict(layout=1, H=1 << 17, H_kv=1 << 17, Sq=2, Skv=2, workspace_bytes=1 << 40),
     attn.ATTN_E_UNSUPPORTED),                   # in-tile byte offsets
    (dict(B=1 << 20, H=1 << 10, H_kv=1 << 10, Sq=1 << 10, Skv=1 << 10, workspace_bytes=1 << 62),
     attn.ATTN_E_UNSUPPORTED),                   # grid sizes
])
def test_prefill_bwd_validation(kw, status):
    assert _bwd(**kw) == status


def test_prefill_bwd_empty_is_a_noop():
    none = dict(q=None, k=None, v=None, o=None, dO=None, lse=None, dq=None, dk=None, dv=None,
                workspace=None, workspace_bytes=0)
    assert _bwd(B=0, **none) == attn.ATTN_OK
    assert _bwd(Sq=0, Skv=0, **none) == attn.ATTN_OK


def test_prefill_bwd_workspace_size():
    # two fp32 per query row, each array rounded up to 256 bytes
    assert attn.attn_prefill_bwd_workspace_size(2, 32, 8192) == 2 * (2 * 32 * 8192 * 4)
    assert attn.attn_prefill_bwd_workspace_size(1, 1, 3) == 512
    assert attn.attn_prefill_bwd_workspace_size(0, 4, 4) == 0
    assert attn.attn_prefill_bwd_workspace_size(-1, 4, 4) == 0


def _decode_gqa(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE, seq_lens=FAKE, o=FAKE, B=4,
             H=32, H_kv=8, D=128, page_size=16, num_pages=64, max_pages_per_seq=8, dtype=0,
             scale=0.1, workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return attn.attn_paged_decode_gqa(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=5), attn.ATTN_E_INVALID),
    (dict(H_kv=0), attn.ATTN_E_INVALID),
    (dict(H_kv=64), attn.ATTN_E_INVALID),
    (dict(page_size=32), attn.ATTN_E_UNSUPPORTED),
    (dict(workspace_bytes=64), attn.ATTN_E_WORKSPACE),
    (dict(dtype=attn.ATTN_OUT_F32 | 5), attn.ATTN_E_INVALID),
])
def test_decode_gqa_validation(kw, status):
    assert _decode_gqa(**kw) == status


def test_gqa_split_plan_and_workspace():
    # attn_paged_decode is the H_kv = H case
    assert attn.attn_paged_decode_gqa_num_splits(64, 32, 32, 512, 16) == \
        attn.attn_paged_decode_num_splits(64, 32, 512, 16)
    assert attn.attn_paged_decode_gqa_workspace_size(64, 32, 32, 128, 512, 16) == \
        attn.attn_paged_decode_workspace_size(64, 32, 128, 512, 16)
    # (work ranges, tokens per range at least).  The batch's tiles are cut
    # into at most 2048 equal ranges (one resident wave each; 1024 for groups
    # of 16 or more query heads, whose partials are larger), each covering at
    # least min(group, 32) / 2 tiles of 32 tokens, clamped to [4, 8], so a
    # range's partial rows (one per query of the group) stay a small share of
    # its K/V and its start a small share of its time
    assert attn.attn_paged_decode_gqa_num_splits(64, 32, 32, 512, 16) == (2048, 128)
    assert attn.attn_paged_decode_gqa_num_splits(64, 32, 8, 512, 16) == (2048, 128)
    assert attn.attn_paged_decode_gqa_num_splits(256, 32, 1, 512, 16) == (1024, 256)
    assert attn.attn_paged_decode_gqa_num_splits(64, 32, 2, 512, 16) == (1024, 256)
    assert attn.attn_paged_decode_gqa_num_splits(64, 64, 8, 512, 16) == (2048, 128)
    assert attn.attn_paged_decode_gqa_num_splits(1, 8, 1, 512, 16) == (64, 128)
    assert attn.attn_paged_decode_gqa_num_splits(2, 64, 1, 100, 16) == (25, 256)
    assert attn.attn_paged_decode_gqa_num_splits(4, 6, 4, 8, 16) == (0, 0)
    # partial rows for every (range, line) pair a call can touch: at most
    # ranges + lines of them, min(group, 32) rows of D + 1 floats each
    lines = 64 * 8
    ws = attn.attn_paged_decode_gqa_workspace_size(64, 32, 8, 128, 512, 16)
    assert ws >= (2048 + lines) * 4 * 129 * 4 + (64 + 3) * 4
    assert attn.attn_paged_decode_gqa_workspace_size(4, 8, 2, 96, 8, 16) == 0
    # token positions must fit 32 bits
    assert attn.attn_paged_decode_gqa_num_splits(1, 8, 1, 1 << 27, 16) == (0, 0)


def _decode(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE, seq_lens=FAKE, o=FAKE, B=4,
             H=8, D=128, page_size=16, num_pages=64, max_pages_per_seq=8, dtype=0, scale=0.1,
             workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return attn.attn_paged_decode(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), attn.ATTN_E_INVALID),
    (dict(page_size=8), attn.ATTN_E_UNSUPPORTED),
    (dict(page_size=0), attn.ATTN_E_INVALID),
    (dict(D=80), attn.ATTN_E_UNSUPPORTED),
    (dict(dtype=3), attn.ATTN_E_INVALID),
    (dict(dtype=attn.ATTN_OUT_F32 | 0x400), attn.ATTN_E_INVALID),
    (dict(scale=float("nan")), attn.ATTN_E_INVALID),
    (dict(num_pages=0), attn.ATTN_E_INVALID),
    (dict(max_pages_per_seq=0), attn.ATTN_E_INVALID),
    (dict(page_table=None), attn.ATTN_E_INVALID),
    (dict(seq_lens=FAKE + 2), attn.ATTN_E_INVALID),
    (dict(k_cache=FAKE + 4), attn.ATTN_E_INVALID),
    (dict(workspace=None), attn.ATTN_E_WORKSPACE),
    (dict(workspace_bytes=16), attn.ATTN_E_WORKSPACE),
    (dict(B=1 << 28), attn.ATTN_E_UNSUPPORTED),  # B * H past 32-bit indexing
])
def test_decode_validation(kw, status):
    assert _decode(**kw) == status


def test_decode_empty_is_a_noop():
    assert _decode(B=0, q=None, o=None) == attn.ATTN_OK
    assert _decode(H=0) == attn.ATTN_OK


def test_split_plan_and_workspace():
    # one line per (sequence, head): 64 x 32 lines of up to 256 tiles, cut
    # into at most 2048 ranges of at least 4 tiles (128 tokens)
    n, tps = attn.attn_paged_decode_num_splits(64, 32, 512, 16)
    assert (n, tps) == (2048, 128)
    ws = attn.attn_paged_decode_workspace_size(64, 32, 128, 512, 16)
    slots = n + 64 * 32  # (range, line) pairs a call can touch
    assert ws >= slots * 129 * 4 + (64 + 3) * 4
    # fewer ranges when the batch cannot hold 2048 of at least 4 tiles
    assert attn.attn_paged_decode_num_splits(1, 1, 8, 16) == (1, 128)
    assert attn.attn_paged_decode_num_splits(1, 32, 512, 16) == (2048, 128)
    assert attn.attn_paged_decode_num_splits(1, 4, 64, 16) == (32, 128)
    assert attn.attn_paged_decode_num_splits(4, 8, 8, 7) == (0, 0)
    assert attn.attn_paged_decode_workspace_size(4, 8, 96, 8, 16) == 0


def test_no_cpu_fallback(tmp_path):
    with pytest.raises(ImportError):
        attn.load_library(str(tmp_path / "missing.so"))


def _extend(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE,
             prefix_lens=FAKE, qo_start=FAKE, o=FAKE, B=4, H=8, H_kv=2, D=128, total_tokens=100,
             max_extend_len=64, page_size=16, num_pages=64, max_pages_per_seq=8, dtype=1,
             scale=0.1, stream=0)
    a.update(kw)
    return attn.attn_extend(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(max_extend_len=-1), attn.ATTN_E_INVALID),
    (dict(total_tokens=-1), attn.ATTN_E_INVALID),
    (dict(D=32), attn.ATTN_E_UNSUPPORTED),
    (dict(page_size=8), attn.ATTN_E_UNSUPPORTED),
    (dict(qo_start=None), attn.ATTN_E_INVALID),
    (dict(qo_start=FAKE + 2), attn.ATTN_E_INVALID),
    (dict(k_cache=None), attn.ATTN_E_INVALID),          # a prefix may exist
    (dict(num_pages=0), attn.ATTN_E_INVALID),
    (dict(q=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(max_extend_len=1 << 20, H=64, H_kv=8), attn.ATTN_E_UNSUPPORTED),
    # key positions (prefix plus new tokens) must stay below 2^31
    (dict(max_pages_per_seq=1 << 27), attn.ATTN_E_UNSUPPORTED),
    (dict(max_pages_per_seq=(1 << 27) - 4, max_extend_len=64), attn.ATTN_E_UNSUPPORTED),
])
def test_extend_validation(kw, status):
    assert _extend(**kw) == status
    # the split form checks its arguments the same way, before the workspace
    assert _extend_split(**kw) == status


def _extend_split(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE,
             prefix_lens=FAKE, qo_start=FAKE, o=FAKE, B=1, H=8, H_kv=2, D=128, total_tokens=300,
             max_extend_len=300, page_size=16, num_pages=512, max_pages_per_seq=250, dtype=1,
             scale=0.1, workspace=FAKE, workspace_bytes=1 << 40, stream=0)
    a.update(kw)
    return attn.attn_extend_splitkv(**a)


@pytest.mark.parametrize("kw,status", [
    # this batch splits: a workspace is required, big enough, 16-byte aligned
    (dict(workspace=None), attn.ATTN_E_WORKSPACE),
    (dict(workspace_bytes=1024), attn.ATTN_E_WORKSPACE),
    (dict(workspace=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
])
def test_extend_splitkv_validation(kw, status):
    assert _extend_split(**kw) == status


def test_extend_splitkv_empty_is_a_noop():
    assert _extend_split(B=0, q=None, k=None, v=None, o=None, qo_start=None, workspace=None,
                         workspace_bytes=0) == attn.ATTN_OK
    assert _extend_split(max_extend_len=0, workspace=None, workspace_bytes=0) == attn.ATTN_OK


def test_extend_splitkv_plan_and_workspace():
    f, w = attn.attn_extend_splitkv_num_splits, attn.attn_extend_splitkv_workspace_size
    # a 512-token chunk after up to 32k prefix tokens, H32/8: 8 head groups x
    # 8 query tiles of 64 rows = 64 units; 4 splits fill the 256 CUs once
    assert f(1, 32, 8, 128, 512, 512, 2048) == 4
    assert w(1, 32, 8, 128, 512, 512, 2048) == 4 * (512 * 32 * 128 * 4 + 512 * 32 * 4)
    # a ragged batch of 8 long sequences already fills the GPU: no split
    assert f(8, 32, 8, 128, 8192, 1872, 366) == 1
    assert w(8, 32, 8, 128, 8192, 1872, 366) == 0
    # fewer than 16 key tiles (no prefix, 300 new tokens): no split
    assert f(1, 8, 2, 128, 300, 300, 0) == 1
    # nothing to compute: one split, no workspace; invalid sizes: 0
    assert f(0, 8, 2, 128, 300, 300, 8) == 1
    assert w(0, 8, 2, 128, 300, 300, 8) == 0
    assert f(1, 8, 3, 128, 300, 300, 8) == 0
    assert f(1, 8, 2, 80, 300, 300, 8) == 0
    assert f(1, 8, 2, 128, -1, 300, 8) == 0
    assert w(1, 8, 2, 128, 300, 300, -1) == 0


def test_extend_empty_is_a_noop():
    assert _extend(B=0, q=None, k=None, v=None, o=None, qo_start=None) == attn.ATTN_OK
    assert _extend(max_extend_len=0) == attn.ATTN_OK
    assert _extend(total_tokens=0) == attn.ATTN_OK


def _prefill_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=4, H_kv=2, Sq=16, Skv=16, D=128, layout=0,
             out_dtype=0, causal=0, scale=0.1, q_descale=0.01, k_descale=0.01, v_descale=0.01,
             stream=0)
    a.update(kw)
    return attn.attn_prefill_fp8(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q_descale=float("nan")), attn.ATTN_E_INVALID),
    (dict(v_descale=-1.0), attn.ATTN_E_INVALID),
    (dict(k_descale=float("inf")), attn.ATTN_E_INVALID),
    (dict(out_dtype=2), attn.ATTN_E_INVALID),
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(D=256), attn.ATTN_E_UNSUPPORTED),
    (dict(layout=3), attn.ATTN_E_INVALID),
    (dict(k=FAKE + 1), attn.ATTN_E_INVALID),
])
def test_prefill_fp8_validation(kw, status):
    assert _prefill_fp8(**kw) == status


def test_prefill_fp8_empty_is_a_noop():
    assert _prefill_fp8(Sq=0, q=None, o=None) == attn.ATTN_OK


def _decode_noalloc(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, page_table=FAKE, seq_lens=FAKE, o=FAKE, B=4,
             H=32, H_kv=8, D=128, page_size=16, num_pages=64, max_pages_per_seq=8, dtype=0,
             scale=0.1, stream=0)
    a.update(kw)
    return attn.attn_paged_decode_gqa_noalloc(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=5), attn.ATTN_E_INVALID),
    (dict(page_size=32), attn.ATTN_E_UNSUPPORTED),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(q=None), attn.ATTN_E_INVALID),
    (dict(o=FAKE + 8), attn.ATTN_E_INVALID),
    (dict(scale=float("nan")), attn.ATTN_E_INVALID),
    (dict(B=0), attn.ATTN_OK),
    # partials beyond the library's 32 MiB array: refused before any HIP call
    (dict(B=4096, H=32, H_kv=32, max_pages_per_seq=512), attn.ATTN_E_WORKSPACE),
    (dict(B=2048, H=32, H_kv=1, max_pages_per_seq=512), attn.ATTN_E_WORKSPACE),
])
def test_decode_noalloc_validation(kw, status):
    assert _decode_noalloc(**kw) == status


def test_decode_noalloc_limit_matches_workspace_size():
    """The sizes the no-allocation decode accepts are exactly those whose
    workspace fits ATTN_DECODE_SCRATCH_BYTES; the bench's decode workloads fit."""
    cap = attn.ATTN_DECODE_SCRATCH_BYTES
    assert cap == 32 << 20
    for B, H, H_kv, mp in [(64, 32, 32, 512), (64, 32, 8, 512), (256, 32, 1, 512)]:
        assert 0 < attn.attn_paged_decode_gqa_workspace_size(B, H, H_kv, 128, mp, 16) <= cap
    big = attn.attn_paged_decode_gqa_workspace_size(4096, 32, 32, 128, 512, 16)
    assert big > cap


def _splitkv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=8, H_kv=8, Sq=128, Skv=32768, D=128,
             layout=0, dtype=0, causal=0, scale=0.1, workspace=FAKE, workspace_bytes=1 << 40,
             stream=0)
    a.update(kw)
    return attn.attn_prefill_splitkv(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=3), attn.ATTN_E_INVALID),
    (dict(layout=2), attn.ATTN_E_INVALID),
    (dict(D=96), attn.ATTN_E_UNSUPPORTED),
    (dict(scale=-1.0), attn.ATTN_E_INVALID),
    (dict(q=None), attn.ATTN_E_INVALID),
    (dict(o=FAKE + 4), attn.ATTN_E_INVALID),
    # this shape splits: a workspace is required, big enough, 16-byte aligned
    (dict(workspace=None), attn.ATTN_E_WORKSPACE),
    (dict(workspace_bytes=1024), attn.ATTN_E_WORKSPACE),
    (dict(workspace=FAKE + 8), attn.ATTN_E_INVALID),
])
def test_prefill_splitkv_validation(kw, status):
    assert _splitkv(**kw) == status


def test_prefill_splitkv_empty_is_a_noop():
    assert _splitkv(Sq=0, q=None, o=None, workspace=None, workspace_bytes=0) == attn.ATTN_OK


def test_prefill_splitkv_plan_and_workspace():
    # 8 heads x 1 query tile = 8 workgroups over 512 key tiles: 32 splits of
    # 16 tiles fill the 256 CUs once (64 would take two rounds of 8 tiles,
    # the same time plus twice the partials)
    assert attn.attn_prefill_splitkv_num_splits(1, 8, 128, 32768, 128) == 32
    rows = 1 * 8 * 128
    assert attn.attn_prefill_splitkv_workspace_size(1, 8, 128, 32768, 128) == \
        32 * (rows * 128 * 4 + rows * 4)
    # a 512-query, 32-head chunk against 32k keys: 64 items x 4 splits = 256
    assert attn.attn_prefill_splitkv_num_splits(1, 32, 512, 32768, 128) == 4
    # 100 items: 5 splits (500 workgroups, two per CU) beat 2 (one round of
    # 200, 78% of the CUs) and 3 (300: a second round of 44)
    assert attn.attn_prefill_splitkv_num_splits(1, 25, 1024, 16384, 128) == 5
    # 240 items nearly fill the CUs: no split is modelled faster than any
    assert attn.attn_prefill_splitkv_num_splits(1, 40, 1536, 16384, 128) == 1
    assert attn.attn_prefill_splitkv_workspace_size(1, 40, 1536, 16384, 128) == 0
    # keys too few to split twice (under 16 key tiles): no split, no workspace
    assert attn.attn_prefill_splitkv_num_splits(1, 8, 128, 960, 128) == 1
    assert attn.attn_prefill_splitkv_workspace_size(1, 8, 128, 960, 128) == 0
    assert attn.attn_prefill_splitkv_num_splits(1, 8, 128, 1000, 128) == 2
    # a grid of two workgroups per CU already: no split
    assert attn.attn_prefill_splitkv_num_splits(4, 32, 4096, 4096, 128) == 1
    # splits limited by the keys: 20 tiles -> 2 splits of 10
    assert attn.attn_prefill_splitkv_num_splits(1, 1, 64, 1280, 64) == 2
    # D = 64 tiles hold 128 query rows and a CU holds three workgroups: 64
    # items x 12 splits = 768
    assert attn.attn_prefill_splitkv_num_splits(1, 32, 256, 65536, 64) == 12
    # ... but with few key tiles per split the per-workgroup cost wins: two
    # per CU (21 splits of 15 tiles), not three (32 of 10)
    assert attn.attn_prefill_splitkv_num_splits(1, 8, 300, 20000, 64) == 21
    assert attn.attn_prefill_splitkv_num_splits(1, 8, 128, 32768, 80) == 0
    assert attn.attn_prefill_splitkv_workspace_size(-1, 8, 128, 32768, 128) == 0
