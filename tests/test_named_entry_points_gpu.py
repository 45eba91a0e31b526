"""The two entry points the C ABI is built around, attn_prefill and
attn_paged_decode, called directly through ctypes with raw device pointers
and sizes (no convenience wrapper), on the tiny prefill, the causal BSHD 8k
prefill and the paged-decode workloads.  Each result is written into a
NaN-prefilled buffer, compared with the fp64 oracle over the whole tensor,
and checked bitwise against the grouped-query entry points (attn_prefill_gqa,
attn_paged_decode_gqa with H_kv = H) that the other tests drive."""
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import MAX_ABS_TOL, REL_FRO_TOL, assert_parity

pytestmark = pytest.mark.gpu


def _dims(q, k, layout):
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        Skv = k.shape[2]
    else:
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
    return B, H, Sq, Skv, D


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, 3])
def test_attn_prefill_direct(gpu_lib, cfg, progress):
    attn = gpu_lib
    q, k, v, m = workloads.prefill_config(cfg)
    B, H, Sq, Skv, D = _dims(q, k, m["layout"])
    code = attn.ATTN_BF16 if m["dtype"] == "bf16" else attn.ATTN_F16
    layout = attn.LAYOUTS[m["layout"]]
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o = whole.nan_like(qg)
    print(f"[case] attn_prefill direct, {m['name']}", flush=True)
    st = attn.attn_prefill(qg, kg, vg, o, B, H, Sq, Skv, D, layout, code, m["causal"], m["scale"])
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    o_gqa = whole.nan_like(qg)
    st = attn.attn_prefill_gqa(qg, kg, vg, o_gqa, B, H, H, Sq, Skv, D, layout, code,
                               m["causal"], m["scale"])
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    o, o_gqa = o.cpu(), o_gqa.cpu()
    assert torch.equal(o, o_gqa)
    kw = dict(causal=m["causal"], scale=m["scale"], layout=m["layout"])
    res = whole.compare(whole.prefill_units(q, k, v, ["o"], **kw), {"o": o},
                        progress=progress)["o"]
    print(f"[parity] attn_prefill {m['name']} (whole tensor): {res}", flush=True)
    assert res.nonfinite == 0
    assert res.max_abs <= MAX_ABS_TOL and res.rel_fro <= REL_FRO_TOL, res


@pytest.mark.timeout(600)
def test_attn_paged_decode_direct(gpu_lib):
    """The paged-decode workload through attn_paged_decode with a
    caller-sized workspace; the cache's free slots hold NaN, which must not
    leak into O."""
    attn = gpu_lib
    fill = float("nan")
    batch = workloads.decode_config(4, fill=fill)
    B, H, D = batch.q.shape
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    need = attn.attn_paged_decode_workspace_size(B, H, D, batch.max_pages_per_seq,
                                                 batch.page_size)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o = whole.nan_like(g["q"])
    print(f"[case] attn_paged_decode direct, {batch.meta['name']} fill={fill}", flush=True)
    st = attn.attn_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                                g["seq_lens"], o, B, H, D, batch.page_size, batch.num_pages,
                                batch.max_pages_per_seq, attn.ATTN_F16, batch.meta["scale"], ws,
                                need)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    # too small a workspace is refused before any launch
    assert attn.attn_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                                  g["seq_lens"], o, B, H, D, batch.page_size, batch.num_pages,
                                  batch.max_pages_per_seq, attn.ATTN_F16, batch.meta["scale"],
                                  ws, need - 1) == attn.ATTN_E_WORKSPACE
    o_gqa = attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"],
                              g["seq_lens"], scale=batch.meta["scale"])
    torch.cuda.synchronize()
    o, o_gqa = o.cpu(), o_gqa.cpu()
    assert torch.equal(o, o_gqa)
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, scale=batch.meta["scale"])
    assert_parity(o.double().numpy(), ref, f"attn_paged_decode {batch.meta['name']} fill={fill}")
