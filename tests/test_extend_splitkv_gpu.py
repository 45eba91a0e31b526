"""GPU parity of attn_extend_splitkv (extend attention with each unit's keys
-- its paged prefix tiles, then its new tokens' tiles -- split over
workgroups and merged by log-sum-exp) against the fp64 oracle, on batches
whose grids are too small to fill the GPU: one or a few sequences with long
prefixes (chunked prefill of a long prompt).  Also: NaN in the cache's free
slots, in the output buffer and in the workspace; the fp32 output; run-to-run
determinism; the rows attn_extend leaves alone (invalid row ranges, rows past
max_extend_len) left alone here too; a rejected prefix page still making its
sequence NaN; bitwise attn_extend when the plan does not split; and a
512-token chunk after a 32k-token prefix compared over the whole output."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import assert_parity

pytestmark = pytest.mark.gpu


def _gpu(batch):
    return {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache",
                                                 "page_table", "prefix_lens", "qo_start")}


def _splits(attn, batch, max_extend_len=None):
    T, H, D = batch.q.shape
    el = (batch.qo_start[1:] - batch.qo_start[:-1]).tolist()
    mx = max(el) if max_extend_len is None else max_extend_len
    return attn.attn_extend_splitkv_num_splits(len(el), H, batch.k.shape[1], D, T, mx,
                                               batch.page_table.shape[1]), mx


def _run(attn, batch, out=None, out_dtype=None, max_extend_len=None, fill_ws=True, g=None):
    g = _gpu(batch) if g is None else g
    T, H, D = batch.q.shape
    n, mx = _splits(attn, batch, max_extend_len)
    need = attn.attn_extend_splitkv_workspace_size(len(batch.prefix_lens), H, batch.k.shape[1], D,
                                                   T, mx, batch.page_table.shape[1])
    ws = torch.full((max(need, 1),), 0xFF if fill_ws else 0, dtype=torch.uint8, device="cuda")
    o = attn.extend_splitkv(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                            g["prefix_lens"], g["qo_start"], max_extend_len=mx, out=out,
                            out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return o, n


CASES = [  # B, H, H_kv, D, dtype, prefix_lens, extend_lens
    (1, 8, 2, 128, "bf16", [4000], [300]),          # four heads per workgroup
    (1, 6, 1, 128, "f16", [5000], [200]),           # one head per workgroup
    (2, 8, 8, 64, "f16", [1500, 37], [400, 129]),   # D 64, ragged, a prefix of 37
    (3, 8, 2, 128, "f16", [0, 4100, 999], [65, 1, 256]),  # no prefix, one new token
    (1, 4, 4, 64, "bf16", [2049], [64]),            # prefix ending one past a page
]


def _ids(c):
    B, H, H_kv, D, dtype, pl, el = c
    return f"B{B}H{H}-{H_kv}D{D}{dtype}P{'-'.join(map(str, pl))}E{'-'.join(map(str, el))}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_extend_splitkv_parity(gpu_lib, case):
    attn = gpu_lib
    B, H, H_kv, D, dtype, pl, el = case
    batch = workloads.extend_inputs(B, H, D, pl, el, dtype, seed=300 + sum(pl) % 97 + D,
                                    h_kv=H_kv, fill=float("nan"))
    n, _ = _splits(attn, batch)
    print(f"[case] extend splitkv {_ids(case)} splits {n}", flush=True)
    assert n > 1, n  # every case here splits
    g = _gpu(batch)
    out = torch.full(batch.q.shape, float("nan"), dtype=batch.q.dtype, device="cuda")
    o, _ = _run(attn, batch, out=out, g=g)
    o2, _ = _run(attn, batch, fill_ws=False, g=g)
    assert torch.isfinite(o.float()).all(), "rows unwritten, or NaN from a free cache slot"
    assert torch.equal(o, o2)
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start)
    assert_parity(o.double().cpu().numpy(), ref, f"extend splitkv {_ids(case)}")
    o32, _ = _run(attn, batch, out_dtype=torch.float32, g=g)
    # the fp32 output: only the kernels' own error (fp16 P, fp32 sums)
    assert_parity(o32.double().cpu().numpy(), ref, f"extend splitkv fp32 {_ids(case)}",
                  max_abs_tol=3e-3, rel_fro_tol=5e-4)
    assert torch.equal(o32.to(o.dtype), o)


def test_extend_splitkv_without_split_is_extend(gpu_lib):
    """A batch whose plan has one split (too few key tiles) is attn_extend,
    bitwise, with no workspace."""
    attn = gpu_lib
    batch = workloads.extend_inputs(2, 8, 128, [300, 0], [300, 200], "bf16", seed=310, h_kv=2)
    n, _ = _splits(attn, batch)
    assert n == 1
    g = _gpu(batch)
    print("[case] extend splitkv no split", flush=True)
    a = attn.extend_splitkv(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                            g["prefix_lens"], g["qo_start"])
    b = attn.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                    g["prefix_lens"], g["qo_start"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_extend_splitkv_bad_page_gives_nan(gpu_lib):
    """A live prefix page id outside the pool makes its sequence's rows NaN
    (the split holding that tile passes NaN to the merge); the other
    sequences are unaffected.  The pool sits one page into a padded
    allocation, so the id one past the pool stays inside it."""
    attn = gpu_lib
    batch = workloads.extend_inputs(3, 8, 128, [1200, 3000, 900], [40, 70, 20], "f16", seed=311,
                                    h_kv=2)
    P = batch.k_cache.shape[0]
    table = batch.page_table.clone()
    table[1, 150] = P          # token 2400 of sequence 1's prefix
    pad = (P + 2,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    g = _gpu(batch)
    g["k_cache"], g["v_cache"], g["page_table"] = k_pad[1:P + 1], v_pad[1:P + 1], table.cuda()
    n, _ = _splits(attn, batch)
    print(f"[case] extend splitkv bad page, splits {n}", flush=True)
    assert n > 1
    o, _ = _run(attn, batch, g=g)
    o = o.float().cpu()
    s = batch.qo_start.tolist()
    assert torch.isnan(o[s[1]:s[2]]).all()
    good = list(range(s[0], s[1])) + list(range(s[2], s[3]))
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, seqs=[0, 2])
    assert_parity(o[good].double().numpy(), ref[good], "extend splitkv, valid pages")


@pytest.mark.parametrize("bad", ["past_end", "negative"])
def test_extend_splitkv_leaves_rows_alone(gpu_lib, bad):
    """Rows attn_extend does not write stay as the caller left them: those of
    a sequence with an invalid row range and those past max_extend_len."""
    attn = gpu_lib
    pl, el = [2000, 1500, 3000, 500], [90, 40, 120, 60]
    batch = workloads.extend_inputs(4, 8, 128, pl, el, "bf16", seed=312, h_kv=2)
    g = _gpu(batch)
    T = batch.q.shape[0]
    starts = batch.qo_start.clone()
    if bad == "past_end":
        starts[4] = T + 3
        skipped = [3]
    else:
        starts[2] = -1
        skipped = [1, 2]
    g["qo_start"] = starts.cuda()
    out = torch.full(batch.q.shape, 7.0, dtype=batch.q.dtype, device="cuda")
    n, _ = _splits(attn, batch, max_extend_len=64)
    print(f"[case] extend splitkv invalid range {bad}, max_extend_len 64, splits {n}", flush=True)
    assert n > 1
    _run(attn, batch, out=out, max_extend_len=64, g=g)
    o = out.cpu()
    s = batch.qo_start.tolist()
    for b in skipped:
        assert torch.all(o[s[b]:s[b + 1]] == 7.0), f"sequence {b} (invalid range) was written"
    seqs = [b for b in range(4) if b not in skipped]
    for b in seqs:
        assert torch.all(o[s[b] + min(el[b], 64):s[b + 1]] == 7.0), f"sequence {b} past 64"
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, seqs=seqs)
    rows = [r for b in seqs for r in range(s[b], s[b] + min(el[b], 64))]
    assert_parity(o[rows].double().numpy(), ref[rows], f"extend splitkv around {bad}")


def test_extend_splitkv_no_cache_null_pointers(gpu_lib):
    """max_pages_per_seq = 0 with the cache, page table and prefix lengths
    NULL: causal attention over the new tokens, split."""
    attn = gpu_lib
    el = [1500, 700]
    batch = workloads.extend_inputs(2, 8, 128, [0, 0], el, "bf16", seed=313, h_kv=2)
    T, H, D = batch.q.shape
    q, k, v = batch.q.cuda(), batch.k.cuda(), batch.v.cuda()
    starts = batch.qo_start.cuda()
    n = attn.attn_extend_splitkv_num_splits(2, H, 2, D, T, max(el), 0)
    need = attn.attn_extend_splitkv_workspace_size(2, H, 2, D, T, max(el), 0)
    print(f"[case] extend splitkv no cache (NULL pointers), splits {n}", flush=True)
    assert n > 1
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o = torch.full_like(q, float("nan"))
    st = attn.attn_extend_splitkv(q, k, v, None, None, None, None, starts, o, 2, H, 2, D, T,
                                  max(el), 16, 0, 0, attn.ATTN_BF16, 1 / np.sqrt(D), ws, need)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start)
    assert torch.isfinite(o.float()).all()
    assert_parity(o.double().cpu().numpy(), ref, "extend splitkv without a cache")


@pytest.mark.timeout(600)
def test_extend_splitkv_chunk_whole(gpu_lib, progress):
    """A 512-token chunk after a 32768-token paged prefix (H32/8, D128, bf16),
    the shape of one step of chunked prefill: split, NaN-prefilled output,
    compared with the oracle over the whole output."""
    attn = gpu_lib
    batch = workloads.extend_inputs(1, 32, 128, [32768], [512], "bf16", seed=314, h_kv=8)
    n, _ = _splits(attn, batch)
    print(f"[case] extend splitkv 512 after 32k, splits {n}", flush=True)
    assert n > 1
    out = whole.nan_like(batch.q)
    o, _ = _run(attn, batch, out=out)
    o = o.cpu()
    st = whole.compare(whole.extend_units(batch, ["o"], scale=1 / np.sqrt(128)), {"o": o},
                       progress=progress)["o"]
    print(f"[parity] extend splitkv chunk (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0
    assert st.max_abs <= 1e-2 and st.rel_fro <= 2e-3, st
