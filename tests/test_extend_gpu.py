"""GPU parity of extend attention (attn_extend: new tokens after a paged
prefix) through the C ABI against the fp64 oracle; same bar as prefill."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import MAX_ABS_TOL, REL_FRO_TOL, assert_parity

pytestmark = pytest.mark.gpu


def _gpu(batch):
    return {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache",
                                                 "page_table", "prefix_lens", "qo_start")}


def _run(attn, batch, **kw):
    g = _gpu(batch)
    print(f"[case] extend B{len(batch.prefix_lens)} H{batch.q.shape[1]}/{batch.k.shape[1]} "
          f"D{batch.q.shape[2]} {batch.q.dtype} prefix={batch.prefix_lens.tolist()[:6]} "
          f"starts={batch.qo_start.tolist()[:7]}", flush=True)
    o = attn.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                    g["prefix_lens"], g["qo_start"], **kw)
    torch.cuda.synchronize()
    return o.cpu()


def _ref(batch, **kw):
    return oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                         batch.page_table, batch.prefix_lens, batch.qo_start, **kw)


CASES = [  # (prefix_lens, extend_lens)
    ([0, 1, 15, 16, 17, 63, 64, 65], [1, 2, 17, 64, 65, 100, 255, 256]),
    ([300, 1000, 0], [700, 5, 513]),
    ([128, 4096], [1, 300]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("H,H_kv", [(8, 8), (8, 2), (6, 1), (16, 2), (32, 1)])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (128, "f16"), (64, "f16"), (64, "bf16")])
def test_extend_parity_nan_poisoned(gpu_lib, case, H, H_kv, D, dtype):
    pl, el = CASES[case]
    batch = workloads.extend_inputs(len(pl), H, D, pl, el, dtype, seed=80 + case + H_kv + D,
                                    h_kv=H_kv, fill=float("nan"))
    o = _run(gpu_lib, batch)
    assert torch.isfinite(o.float()).all(), "NaN from a free cache slot leaked into O"
    assert_parity(o.double().numpy(), _ref(batch), f"extend case {case} H{H}/{H_kv} D{D} {dtype}")


def test_extend_without_prefix_equals_causal_prefill_bitwise(gpu_lib):
    el = [300, 77]
    batch = workloads.extend_inputs(2, 8, 128, [0, 0], el, "bf16", seed=90, h_kv=2)
    o = _run(gpu_lib, batch)
    for b in range(2):
        r0, r1 = int(batch.qo_start[b]), int(batch.qo_start[b + 1])
        ref = gpu_lib.prefill(batch.q[None, r0:r1].cuda(), batch.k[None, r0:r1].cuda(),
                              batch.v[None, r0:r1].cuda(), causal=True, layout="BSHD")
        torch.cuda.synchronize()
        assert torch.equal(o[r0:r1], ref[0].cpu()), f"sequence {b}"


def test_extend_equals_prefill_on_concatenated_kv_bitwise(gpu_lib):
    """With a prefix of whole 64-key tiles, extend walks the same tiles as a
    bottom-right causal prefill over prefix + new keys."""
    P, E = 256, 190
    batch = workloads.extend_inputs(1, 4, 128, [P], [E], "f16", seed=91, h_kv=4)
    o = _run(gpu_lib, batch)
    tok = torch.arange(P)
    pages = batch.page_table[0].long()[tok // 16]
    kk = torch.cat([batch.k_cache[pages, tok % 16], batch.k])[None]
    vv = torch.cat([batch.v_cache[pages, tok % 16], batch.v])[None]
    ref = gpu_lib.prefill(batch.q[None].cuda(), kk.cuda(), vv.cuda(), causal=True, layout="BSHD")
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0].cpu())


def test_extend_out_f32(gpu_lib):
    batch = workloads.extend_inputs(3, 8, 128, [40, 0, 500], [100, 33, 260], "bf16", seed=92,
                                    h_kv=2)
    o32 = _run(gpu_lib, batch, out_dtype=torch.float32)
    o16 = _run(gpu_lib, batch)
    assert_parity(o32.double().numpy(), _ref(batch), "extend out_f32", max_abs_tol=3e-3,
                  rel_fro_tol=5e-4)
    assert torch.equal(o32.to(o16.dtype), o16)


def test_extend_bad_page_id_gives_nan(gpu_lib):
    batch = workloads.extend_inputs(3, 4, 128, [40, 100, 20], [30, 20, 10], "f16", seed=93,
                                    num_pages=64)
    P = batch.k_cache.shape[0]
    table = batch.page_table.clone()
    table[1, 2] = P            # a live prefix page of sequence 1: one past the pool
    table[0, 5] = P + 500      # past sequence 0's prefix: never read
    batch.page_table = table
    pad = (P + 2,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    g = _gpu(batch)
    print("[case] extend bad page id", flush=True)
    o = gpu_lib.extend(g["q"], g["k"], g["v"], k_pad[1:P + 1], v_pad[1:P + 1], g["page_table"],
                       g["prefix_lens"], g["qo_start"]).float().cpu()
    torch.cuda.synchronize()
    s = batch.qo_start.tolist()
    assert torch.isnan(o[s[1]:s[2]]).all()
    good = list(range(s[0], s[1])) + list(range(s[2], s[3]))
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        torch.where(table >= P, torch.zeros_like(table), table),
                        batch.prefix_lens, batch.qo_start, seqs=[0, 2])
    assert_parity(o[good].double().numpy(), ref[good], "extend sequences with valid pages")


def test_extend_negative_page_id_gives_nan(gpu_lib):
    # A negative page id is outside [0, num_pages) too.  The pool sits one page
    # into a padded allocation, so an id of -1 stays inside it even if it were
    # dereferenced; the most negative id runs only once -1 is rejected.
    batch = workloads.extend_inputs(3, 4, 128, [40, 100, 20], [30, 20, 10], "f16", seed=95,
                                    num_pages=64)
    P = batch.k_cache.shape[0]
    pad = (P + 2,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    g = _gpu(batch)
    s = batch.qo_start.tolist()
    good = list(range(s[0], s[1])) + list(range(s[2], s[3]))
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, seqs=[0, 2])
    for bad in (-1, -(1 << 31)):
        table = batch.page_table.clone()
        table[1, 2] = bad      # a live prefix page of sequence 1
        print(f"[case] extend page id {bad}", flush=True)
        o = gpu_lib.extend(g["q"], g["k"], g["v"], k_pad[1:P + 1], v_pad[1:P + 1],
                           table.cuda(), g["prefix_lens"], g["qo_start"]).float().cpu()
        torch.cuda.synchronize()
        assert torch.isnan(o[s[1]:s[2]]).all(), f"page id {bad} was not rejected"
        assert_parity(o[good].double().numpy(), ref[good], "extend sequences with valid pages")


def test_extend_rows_past_max_extend_len_untouched(gpu_lib):
    batch = workloads.extend_inputs(2, 4, 64, [10, 20], [40, 100], "f16", seed=94)
    g = _gpu(batch)
    out = torch.full(batch.q.shape, 7.0, dtype=batch.q.dtype, device="cuda")
    print("[case] extend max_extend_len 64", flush=True)
    gpu_lib.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                   g["prefix_lens"], g["qo_start"], max_extend_len=64, out=out)
    torch.cuda.synchronize()
    o = out.cpu()
    ref = _ref(batch)
    rows = list(range(0, 40)) + list(range(40, 104))
    assert_parity(o[rows].double().numpy(), ref[rows], "rows within max_extend_len")
    assert torch.all(o[104:140] == 7.0)


@pytest.mark.timeout(600)
def test_extend_gqa_b8_whole(gpu_lib, progress):
    """The ragged extend batch at full size: NaN-prefilled output, every
    sequence's rows against the oracle."""
    batch = workloads.extend_config(9)
    scale = batch.meta["scale"]
    out = whole.nan_like(batch.q)
    o = _run(gpu_lib, batch, scale=scale, out=out)
    st = whole.compare(whole.extend_units(batch, ["o"], scale=scale), {"o": o},
                       progress=progress)["o"]
    print(f"[parity] {batch.meta['name']} (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0, f"{st.nonfinite} elements not written (or not finite)"
    assert st.max_abs <= MAX_ABS_TOL and st.rel_fro <= REL_FRO_TOL, f"{batch.meta['name']}: {st}"


def _permuted(batch, perm):
    """The same sequences in another batch order: new-token rows regrouped,
    prefix lengths and page-table rows moved with them, the cache unchanged."""
    s = batch.qo_start.tolist()
    rows = [r for b in perm for r in range(s[b], s[b + 1])]
    lens = [s[b + 1] - s[b] for b in perm]
    starts = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    return workloads.ExtendBatch(q=batch.q[rows], k=batch.k[rows], v=batch.v[rows],
                                 k_cache=batch.k_cache, v_cache=batch.v_cache,
                                 page_table=batch.page_table[perm].contiguous(),
                                 prefix_lens=batch.prefix_lens[perm].contiguous(),
                                 qo_start=starts, page_size=batch.page_size, meta=batch.meta)


@pytest.mark.parametrize("H,H_kv", [(32, 8), (8, 8)])
def test_extend_sequence_order_independent_bitwise(gpu_lib, H, H_kv):
    """Batches of up to 64 sequences are taken longest work unit first across
    the batch (a unit is a sequence's query tile, worth its prefix plus causal
    keys; ties by batch index): any batch order, with tied, empty and long
    prefixes and sequences without new tokens, gives each sequence bitwise the
    same rows, and those rows match the oracle."""
    pl = [700, 0, 700, 65, 3000, 700, 1, 0, 1500, 64, 700, 2999]
    el = [40, 300, 0, 129, 64, 1, 256, 17, 90, 200, 33, 5]
    batch = workloads.extend_inputs(len(pl), H, 128, pl, el, "bf16", seed=95 + H, h_kv=H_kv)
    perm = [4, 10, 1, 7, 2, 11, 0, 9, 5, 3, 8, 6]
    o = _run(gpu_lib, batch)
    o2 = _run(gpu_lib, _permuted(batch, perm))
    s = batch.qo_start.tolist()
    rows = [r for b in perm for r in range(s[b], s[b + 1])]
    assert torch.equal(o2, o[rows])
    assert_parity(o.double().numpy(), _ref(batch), f"extend ranked batch H{H}/{H_kv}")


def test_extend_many_sequences(gpu_lib):
    """More than 64 sequences (the plain work order) and 64 exactly (the
    largest ranked batch), against the oracle on a spread of sequences."""
    rng = np.random.default_rng(96)
    for B in (64, 90):
        pl = rng.integers(0, 600, B).tolist()
        el = rng.integers(0, 70, B).tolist()
        batch = workloads.extend_inputs(B, 8, 128, pl, el, "f16", seed=96 + B, h_kv=2)
        o = _run(gpu_lib, batch)
        seqs = list(range(0, B, 7)) + [B - 1]
        ref = _ref(batch, seqs=seqs)
        s = batch.qo_start.tolist()
        rows = [r for b in seqs for r in range(s[b], s[b + 1])]
        assert_parity(o[rows].double().numpy(), ref[rows], f"extend B{B} ({len(seqs)} sequences)")


@pytest.mark.parametrize("B", [2, 64])
def test_extend_no_cache_null_pointers_equals_causal_prefill_bitwise(gpu_lib, B):
    """max_pages_per_seq = 0 with k_cache, v_cache, page_table and prefix_lens
    all NULL (the header allows it when there is no prefix): every sequence's
    rows are bitwise those of causal prefill over its new tokens.  B = 2 and
    B = 64 take the longest-first work order, which then reads no prefix
    length."""
    attn = gpu_lib
    rng = np.random.default_rng(97 + B)
    el = [300, 77] if B == 2 else rng.integers(0, 90, B).tolist()
    batch = workloads.extend_inputs(B, 8, 128, [0] * B, el, "bf16", seed=97 + B, h_kv=2)
    T, H, D = batch.q.shape
    H_kv = batch.k.shape[1]
    q, k, v = batch.q.cuda(), batch.k.cuda(), batch.v.cuda()
    starts = batch.qo_start.cuda()
    o = torch.full_like(q, float("nan"))
    print(f"[case] extend B{B} no cache (NULL pointers, max_pages_per_seq 0)", flush=True)
    st = attn.attn_extend(q, k, v, None, None, None, None, starts, o, B, H, H_kv, D, T,
                          max(el), 16, 0, 0, attn.ATTN_BF16, 1 / np.sqrt(D))
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize()
    o = o.cpu()
    assert torch.isfinite(o.float()).all(), "rows left unwritten"
    s = batch.qo_start.tolist()
    for b in range(B):
        if s[b + 1] == s[b]:
            continue
        ref = attn.prefill(q[None, s[b]:s[b + 1]].contiguous(), k[None, s[b]:s[b + 1]].contiguous(),
                           v[None, s[b]:s[b + 1]].contiguous(), causal=True, layout="BSHD")
        torch.cuda.synchronize()
        assert torch.equal(o[s[b]:s[b + 1]], ref[0].cpu()), f"sequence {b}"


@pytest.mark.parametrize("B", [6, 70])
@pytest.mark.parametrize("bad", ["past_end", "negative"])
def test_extend_invalid_row_range_skipped(gpu_lib, B, bad):
    """A sequence whose row range is invalid (it ends past total_tokens, or a
    start is negative) is not computed: its rows keep the caller's values,
    and every other sequence is still right (B = 6 takes the longest-first
    order, B = 70 the plain one)."""
    rng = np.random.default_rng(98 + B)
    pl = rng.integers(0, 300, B).tolist()
    el = rng.integers(1, 90, B).tolist()
    batch = workloads.extend_inputs(B, 8, 128, pl, el, "bf16", seed=98 + B, h_kv=2)
    g = _gpu(batch)
    T = batch.q.shape[0]
    starts = batch.qo_start.clone()
    if bad == "past_end":
        starts[B] = T + 3
        skipped = [B - 1]
    else:
        starts[2] = -1
        skipped = [1, 2]
    out = torch.full(batch.q.shape, 7.0, dtype=batch.q.dtype, device="cuda")
    print(f"[case] extend B{B} invalid range {bad}", flush=True)
    gpu_lib.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                   g["prefix_lens"], starts.cuda(), max_extend_len=max(el), out=out)
    torch.cuda.synchronize()
    o = out.cpu()
    s = batch.qo_start.tolist()
    for b in skipped:
        assert torch.all(o[s[b]:s[b + 1]] == 7.0), f"sequence {b} (invalid range) was written"
    seqs = [b for b in range(B) if b not in skipped]
    ref = _ref(batch, seqs=seqs)
    rows = [r for b in seqs for r in range(s[b], s[b + 1])]
    assert_parity(o[rows].double().numpy(), ref[rows], f"extend B{B} around an invalid range")
