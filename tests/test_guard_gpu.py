"""Out-of-bounds write checks: every output is a view into the middle of a
larger buffer whose guard regions (64 KiB on each side) hold a sentinel bit
pattern; after the call the guards must be untouched and every element of
the view written (the view starts as NaN).  Ragged shapes, both layouts,
causal and not, every entry point that writes device memory."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

GUARD_BYTES = 64 * 1024
SENTINEL = 0x5A  # byte pattern of the guard regions


def _guarded(shape, dtype):
    """(buffer, view): the view is a contiguous tensor of `shape` in the middle
    of a uint8 buffer with GUARD_BYTES of sentinel on each side, NaN-filled
    (0xFF bytes for an integer view: a workspace)."""
    elem = torch.empty((), dtype=dtype).element_size()
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((GUARD_BYTES * 2 + n * elem,), SENTINEL, dtype=torch.uint8, device="cuda")
    view = buf[GUARD_BYTES:GUARD_BYTES + n * elem].view(dtype).view(shape)
    view.fill_(float("nan") if dtype.is_floating_point else 0xFF)
    return buf, view


def _check(buf, view, what):
    torch.cuda.synchronize()
    lo = buf[:GUARD_BYTES]
    hi = buf[buf.numel() - GUARD_BYTES:]
    assert bool((lo == SENTINEL).all()), f"{what}: write before the output"
    assert bool((hi == SENTINEL).all()), f"{what}: write past the output"
    assert bool(torch.isfinite(view.float()).all()), f"{what}: output not fully written"


@pytest.mark.parametrize("Sq,Skv", [(77, 300), (300, 77), (257, 257), (1, 65)])
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,H,H_kv", [(128, 3, 3), (64, 2, 2), (128, 8, 2)])
def test_prefill_and_lse_stay_in_bounds(gpu_lib, Sq, Skv, layout, causal, D, H, H_kv):
    attn = gpu_lib
    q, k, v = workloads.prefill_inputs(2, H, Sq, Skv, D, "bf16", layout, seed=Sq + 3 * D,
                                       h_kv=H_kv)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    print(f"[case] guard prefill Sq{Sq} Skv{Skv} {layout} causal={causal} D{D} H{H}/{H_kv}",
          flush=True)
    buf, o = _guarded(tuple(q.shape), torch.bfloat16)
    lbuf, lse = _guarded((2, H, Sq), torch.float32)
    attn.prefill_with_lse(qg, kg, vg, causal=causal, layout=layout, out=o, lse=lse)
    _check(buf, o, "prefill o")
    # a row that sees no key holds LSE -inf, so the check is that no row is
    # left NaN, not that every row is finite
    torch.cuda.synchronize()
    assert bool((lbuf[:GUARD_BYTES] == SENTINEL).all()) and \
        bool((lbuf[lbuf.numel() - GUARD_BYTES:] == SENTINEL).all()), "lse written out of bounds"
    assert not bool(torch.isnan(lse).any()), "lse row not written"
    buf32, o32 = _guarded(tuple(q.shape), torch.float32)
    attn.prefill(qg, kg, vg, causal=causal, layout=layout, out=o32)
    _check(buf32, o32, "prefill fp32 o")


@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2), (32, 1)])
def test_decode_stays_in_bounds(gpu_lib, H, H_kv):
    attn = gpu_lib
    b = workloads.paged_decode_inputs(B=5, H=H, D=128, page_size=16, num_pages=200, seed=H,
                                      seq_lens=[1, 0, 700, 33, 1500], h_kv=H_kv)
    g = {n: getattr(b, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    print(f"[case] guard decode H{H}/{H_kv}", flush=True)
    buf, o = _guarded(tuple(b.q.shape), torch.float16)
    need = attn.attn_paged_decode_gqa_workspace_size(5, H, H_kv, 128, b.max_pages_per_seq, 16)
    wbuf, ws = _guarded((need,), torch.uint8)
    attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"], out=o,
                      workspace=ws)
    _check(buf, o, "decode o")
    torch.cuda.synchronize()
    assert bool((wbuf[:GUARD_BYTES] == SENTINEL).all()) and \
        bool((wbuf[wbuf.numel() - GUARD_BYTES:] == SENTINEL).all()), "workspace overrun"


def test_extend_stays_in_bounds(gpu_lib):
    attn = gpu_lib
    batch = workloads.extend_inputs(4, 8, 128, [40, 0, 500, 17], [100, 33, 0, 260], "bf16",
                                    seed=98, h_kv=2)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache", "page_table",
                                              "prefix_lens", "qo_start")}
    print("[case] guard extend", flush=True)
    buf, o = _guarded(tuple(batch.q.shape), torch.bfloat16)
    attn.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                g["prefix_lens"], g["qo_start"], out=o)
    _check(buf, o, "extend o")


@pytest.mark.parametrize("layout,causal", [("BSHD", True), ("BHSD", False)])
def test_backward_stays_in_bounds(gpu_lib, layout, causal):
    attn = gpu_lib
    q, k, v, do = workloads.backward_inputs(2, 8, 190, 333, 128, "bf16", layout, amp=0.5,
                                            seed=99, h_kv=2)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.prefill_with_lse(qg, kg, vg, causal=causal, layout=layout)
    print(f"[case] guard backward {layout} causal={causal}", flush=True)
    bq, dq = _guarded(tuple(q.shape), torch.bfloat16)
    bk, dk = _guarded(tuple(k.shape), torch.bfloat16)
    bv, dv = _guarded(tuple(v.shape), torch.bfloat16)
    need = attn.attn_prefill_bwd_workspace_size(2, 8, 190)
    bw, ws = _guarded((need,), torch.uint8)
    attn.prefill_backward(qg, kg, vg, o, dog, lse, causal=causal, layout=layout, dq=dq, dk=dk,
                          dv=dv, workspace=ws)
    _check(bq, dq, "dq")
    _check(bk, dk, "dk")
    _check(bv, dv, "dv")
    torch.cuda.synchronize()
    assert bool((bw[:GUARD_BYTES] == SENTINEL).all()) and \
        bool((bw[bw.numel() - GUARD_BYTES:] == SENTINEL).all()), "workspace overrun"


@pytest.mark.parametrize("layout,causal", [("BHSD", False), ("BSHD", True)])
def test_prefill_splitkv_stays_in_bounds(gpu_lib, layout, causal):
    attn = gpu_lib
    B, H, H_kv, Sq, Skv, D = 1, 4, 2, 77, 2100, 128
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "bf16", layout, seed=97, h_kv=H_kv)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    assert attn.attn_prefill_splitkv_num_splits(B, H, Sq, Skv, D) > 1
    print(f"[case] guard split-kv prefill {layout} causal={causal}", flush=True)
    buf, o = _guarded(tuple(q.shape), torch.bfloat16)
    need = attn.attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D)
    wbuf, ws = _guarded((need,), torch.uint8)
    attn.prefill_splitkv(qg, kg, vg, causal=causal, layout=layout, out=o, workspace=ws)
    _check(buf, o, "split-kv o")
    torch.cuda.synchronize()
    assert bool((wbuf[:GUARD_BYTES] == SENTINEL).all()) and \
        bool((wbuf[wbuf.numel() - GUARD_BYTES:] == SENTINEL).all()), "workspace overrun"


def test_extend_splitkv_stays_in_bounds(gpu_lib):
    attn = gpu_lib
    pl, el = [1300, 0, 2500, 17], [100, 33, 0, 150]
    batch = workloads.extend_inputs(4, 8, 128, pl, el, "bf16", seed=98, h_kv=2)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache",
                                              "page_table", "prefix_lens", "qo_start")}
    T, H, D = batch.q.shape
    args = (4, H, 2, D, T, max(el), batch.page_table.shape[1])
    assert attn.attn_extend_splitkv_num_splits(*args) > 1
    print("[case] guard split-kv extend", flush=True)
    buf, o = _guarded(tuple(batch.q.shape), torch.bfloat16)
    wbuf, ws = _guarded((attn.attn_extend_splitkv_workspace_size(*args),), torch.uint8)
    attn.extend_splitkv(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                        g["prefix_lens"], g["qo_start"], out=o, workspace=ws)
    _check(buf, o, "split-kv extend o")
    torch.cuda.synchronize()
    assert bool((wbuf[:GUARD_BYTES] == SENTINEL).all()) and \
        bool((wbuf[wbuf.numel() - GUARD_BYTES:] == SENTINEL).all()), "workspace overrun"
