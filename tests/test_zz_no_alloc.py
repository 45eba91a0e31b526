"""attn_paged_decode_gqa_noalloc (partials in the library's own device array)
against attn_paged_decode_gqa with a caller workspace, through the C ABI:
bitwise equal on two calls in a row, the second with a smaller input, and
within the oracle's bar."""
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu


def _both(attn, batch, scale):
    B, H, D = batch.q.shape
    H_kv = batch.k_cache.shape[2]
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    need = attn.attn_paged_decode_gqa_workspace_size(B, H, H_kv, D, batch.max_pages_per_seq,
                                                     batch.page_size)
    assert 0 < need <= attn.ATTN_DECODE_SCRATCH_BYTES
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o_ws = torch.full_like(g["q"], float("nan"))
    o_na = torch.full_like(g["q"], float("nan"))
    args = (g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"])
    sizes = (B, H, H_kv, D, batch.page_size, batch.num_pages, batch.max_pages_per_seq)
    code = attn.ATTN_BF16 if batch.q.dtype == torch.bfloat16 else attn.ATTN_F16
    print(f"[case] decode noalloc B{B} H{H}/{H_kv} D{D} {batch.q.dtype} need={need}", flush=True)
    st = attn.attn_paged_decode_gqa(*args, o_ws, *sizes, code, scale, ws, need)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    st = attn.attn_paged_decode_gqa_noalloc(*args, o_na, *sizes, code, scale)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    return o_ws.cpu(), o_na.cpu()


def test_decode_noalloc_matches_workspace_form_twice(gpu_lib):
    attn = gpu_lib
    big = workloads.decode_config(7)  # B64, 32 query heads over 8 KV heads, 16-token pages
    o_ws, o_na = _both(attn, big, big.meta["scale"])
    assert torch.isfinite(o_na.float()).all()
    assert torch.equal(o_na, o_ws)
    # a smaller batch through the same array (one head per KV head, bf16)
    small = workloads.paged_decode_inputs(B=5, H=8, D=128, dtype="bf16", page_size=16,
                                          num_pages=300, seq_lens=[1, 700, 16, 2000, 33], seed=9)
    o_ws, o_na = _both(attn, small, 0.09)
    assert torch.equal(o_na, o_ws)
    ref = oracle.paged_decode(small.q, small.k_cache, small.v_cache, small.page_table,
                              small.seq_lens, scale=0.09)
    assert_parity(o_na.double().numpy(), ref, "noalloc decode, second (smaller) call")


def test_decode_noalloc_on_a_side_stream(gpu_lib):
    """A non-default stream of the current device is accepted; the result is
    bitwise the workspace form's."""
    attn = gpu_lib
    b = workloads.paged_decode_inputs(B=3, H=8, D=64, dtype="f16", page_size=16, num_pages=64,
                                      seq_lens=[5, 300, 17], seed=10, h_kv=2)
    g = {n: getattr(b, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    ref = attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                            scale=0.125)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o = torch.full_like(g["q"], float("nan"))
    print("[case] decode noalloc on a side stream", flush=True)
    with torch.cuda.stream(side):
        st = attn.attn_paged_decode_gqa_noalloc(g["q"], g["k_cache"], g["v_cache"],
                                                g["page_table"], g["seq_lens"], o, 3, 8, 2, 64,
                                                16, 64, b.max_pages_per_seq, attn.ATTN_F16, 0.125,
                                                stream=side)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_decode_noalloc_refuses_oversized(gpu_lib):
    attn = gpu_lib
    q = torch.zeros((4096, 32, 128), dtype=torch.float16, device="cuda")
    kc = torch.zeros((8, 16, 32, 128), dtype=torch.float16, device="cuda")
    pt = torch.zeros((4096, 512), dtype=torch.int32, device="cuda")
    sl = torch.ones((4096,), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    st = attn.attn_paged_decode_gqa_noalloc(q, kc, kc, pt, sl, o, 4096, 32, 32, 128, 16, 8, 512,
                                            attn.ATTN_F16, 0.1)
    assert st == attn.ATTN_E_WORKSPACE
