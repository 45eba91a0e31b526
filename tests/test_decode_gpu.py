"""GPU parity of attn_paged_decode (through the C ABI) against the fp64 oracle.

The oracle gathers each sequence's K/V through the page table explicitly.
Full-size workload: every (sequence, head) output is compared.  Edge cases:
sequence lengths around page (16), tile (32) and range boundaries,
NaN-poisoned unused cache slots, bitwise invariance under a page-pool
permutation and under a wider page table, a single sequence in short ranges.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu


def _to_gpu(batch):
    return {k: getattr(batch, k).cuda() for k in ("q", "k_cache", "v_cache", "page_table",
                                                 "seq_lens")}


def _run(attn, batch, scale=None, page_table=None, out=None):
    print(f"[case] decode B{batch.q.shape[0]} H{batch.q.shape[1]} D{batch.q.shape[2]} "
          f"{batch.q.dtype} pages{batch.num_pages} lens={batch.seq_lens.tolist()[:8]}...",
          flush=True)
    g = _to_gpu(batch)
    if page_table is not None:
        g["page_table"] = page_table.cuda()
    o = attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                          scale=scale, out=out)
    torch.cuda.synchronize()
    return o.cpu()


def _ref(batch, scale=None):
    return oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                               batch.seq_lens, scale=scale)


EDGE_LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 1000, 4096, 8191, 8192]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_edge_lengths_nan_poisoned(gpu_lib, D, dtype):
    H = 6
    batch = workloads.paged_decode_inputs(B=len(EDGE_LENS), H=H, D=D, dtype=dtype, page_size=16,
                                          num_pages=2048, max_seq=8192, seed=D + len(dtype),
                                          seq_lens=EDGE_LENS, fill=float("nan"))
    o = _run(gpu_lib, batch)
    assert torch.isfinite(o.float()).all(), "NaN from an unused cache slot leaked into O"
    assert_parity(o.double().numpy(), _ref(batch), f"edge lengths D{D} {dtype}")


def test_decode_one_long_among_short(gpu_lib):
    lens = [1] * 20 + [8192] + [3] * 11
    batch = workloads.paged_decode_inputs(B=len(lens), H=8, D=128, page_size=16, num_pages=1024,
                                          seed=12, seq_lens=lens)
    assert_parity(_run(gpu_lib, batch).double().numpy(), _ref(batch), "one long among short")


def test_decode_pool_permutation_bitwise(gpu_lib):
    batch = workloads.paged_decode_inputs(B=16, H=8, D=128, page_size=16, num_pages=4096,
                                          max_seq=3000, seed=21)
    moved = workloads.permute_pool(batch, seed=99)
    a = _run(gpu_lib, batch)
    b = _run(gpu_lib, moved)
    assert torch.equal(a, b)
    assert_parity(a.double().numpy(), _ref(batch), "pool permutation")


def test_decode_wide_page_table_changes_nothing(gpu_lib):
    """Widening the page table (unused columns, holding an id past the pool)
    leaves O bitwise the same: the work ranges are cut from the actual
    lengths on the device, not from the table's width, and the unused
    columns are never read."""
    attn = gpu_lib
    batch = workloads.paged_decode_inputs(B=32, H=8, D=128, page_size=16, num_pages=8192,
                                          max_seq=4096, seed=31)
    wide = torch.full((32, 4096), batch.num_pages + 7, dtype=torch.int32)
    wide[:, :batch.max_pages_per_seq] = batch.page_table
    a = _run(attn, batch)
    b = _run(attn, batch, page_table=wide)
    assert torch.equal(a, b)
    assert_parity(b.double().numpy(), _ref(batch), "wide page table")


def test_decode_scale(gpu_lib):
    batch = workloads.paged_decode_inputs(B=4, H=4, D=64, page_size=16, num_pages=256,
                                          max_seq=700, seed=41)
    for scale in (0.0, 0.05, 0.4):
        assert_parity(_run(gpu_lib, batch, scale=scale).double().numpy(),
                      _ref(batch, scale=scale), f"scale {scale}")


def test_decode_paged_b64_full_size(gpu_lib):
    """Every (sequence, head) of the paged-decode workload, written into a
    NaN-prefilled output."""
    batch = workloads.decode_config(4)
    out = torch.full(tuple(batch.q.shape), float("nan"), dtype=batch.q.dtype, device="cuda")
    o = _run(gpu_lib, batch, scale=batch.meta["scale"], out=out)
    ref = _ref(batch, scale=batch.meta["scale"])
    assert_parity(o.double().numpy(), ref, f"{batch.meta['name']} (all sequences and heads)")


@pytest.mark.parametrize("dtype,amp", [("f16", 6.0), ("bf16", 8.0)])
def test_decode_large_logits(gpu_lib, dtype, amp):
    """Large q and k make the running max jump between batches and splits."""
    batch = workloads.paged_decode_inputs(B=12, H=8, D=128, dtype=dtype, page_size=16,
                                          num_pages=4096, min_seq=1, max_seq=4000, seed=41,
                                          amp=amp)
    # V at std 1/3 keeps |O| < 2, where rounding O to bf16 costs < 4e-3.
    batch.v_cache = (batch.v_cache.float() / (3 * amp)).to(batch.v_cache.dtype)
    o = _run(gpu_lib, batch)
    assert_parity(o.double().numpy(), _ref(batch), f"decode amp {amp} {dtype}")


def test_decode_small_batch_short_ranges(gpu_lib):
    """One sequence of 3000 tokens over four heads: 376 tiles in ranges of the
    fewest tiles the plan allows (4), some of them crossing from one head's
    line to the next."""
    batch = workloads.paged_decode_inputs(B=1, H=4, D=64, page_size=16, num_pages=700,
                                          seq_lens=[3000], max_pages_per_seq=640, seed=42)
    n, tps = gpu_lib.attn_paged_decode_num_splits(1, 4, 640, 16)
    assert (n, tps) == (320, 128)
    o = _run(gpu_lib, batch)
    assert_parity(o.double().numpy(), _ref(batch), "B1 short ranges")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_out_f32(gpu_lib, dtype):
    attn = gpu_lib
    batch = workloads.paged_decode_inputs(B=len(EDGE_LENS), H=4, D=128, dtype=dtype,
                                          page_size=16, num_pages=2048, max_seq=8192, seed=61,
                                          seq_lens=EDGE_LENS)
    g = _to_gpu(batch)
    print(f"[case] decode out_f32 {dtype}", flush=True)
    args = (g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"])
    o32 = attn.paged_decode(*args, out_dtype=torch.float32)
    o16 = attn.paged_decode(*args)
    torch.cuda.synchronize()
    # With an fp32 output only the rounding of P to fp16 for the P.V product
    # (2^-11 relative per weight) and fp32 accumulation remain: the bar of the
    # grouped-query fp32-output test.
    assert_parity(o32.double().cpu().numpy(), _ref(batch), f"decode out_f32 {dtype}",
                  max_abs_tol=3e-3, rel_fro_tol=5e-4)
    if dtype == "bf16":
        # both outputs come from the same fp32 partials: the default output is
        # the fp32 one rounded
        assert torch.equal(o32.to(o16.dtype), o16)
    else:
        # fp16 inputs and output keep the partials in fp16, rounded once
        # more than for the fp32 output
        assert_parity(o16.double().cpu().numpy(), o32.double().cpu().numpy(),
                      "decode fp16 output against the fp32 output", max_abs_tol=2e-3,
                      rel_fro_tol=5e-4)


def test_decode_rejects_bad_page_ids_on_device(gpu_lib):
    """Page ids outside [0, num_pages) among a sequence's live pages make its
    output NaN; other sequences are unaffected.  The cache is a view into a
    buffer with one spare page on each side, so even a missed check would
    read allocated memory (and fail the NaN assertion) rather than fault."""
    attn = gpu_lib
    lens = [40, 100, 33, 200, 17, 64]
    batch = workloads.paged_decode_inputs(B=6, H=4, D=128, page_size=16, num_pages=300,
                                          seq_lens=lens, max_pages_per_seq=16, seed=62)
    P = batch.num_pages
    table = batch.page_table.clone()
    table[1, 0] = P          # first page of sequence 1: one past the pool
    table[3, 7] = -1         # a middle page of sequence 3
    table[4, 5] = P + 1000   # past sequence 4's live pages: never read, no effect
    print("[case] decode bad page ids", flush=True)
    pad_shape = (P + 2,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad_shape, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad_shape, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    k_view, v_view = k_pad[1:P + 1], v_pad[1:P + 1]
    assert k_view.is_contiguous() and k_view.shape[0] == P
    o = attn.paged_decode(batch.q.cuda(), k_view, v_view, table.cuda(),
                          batch.seq_lens.cuda()).float().cpu()
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all() and torch.isnan(o[3]).all()
    good = [0, 2, 4, 5]
    assert torch.isfinite(o[good]).all()
    ref = _ref(batch)
    assert_parity(o[good].double().numpy(), ref[good], "sequences with valid pages")


def test_decode_many_sequences(gpu_lib):
    """70000 short sequences (more than a 16-bit grid dimension holds), two
    heads, lengths 0-40: every row is written (NaN-prefilled output), empty
    sequences give 0, and sampled sequences match the oracle."""
    r = np.random.default_rng(5)
    lens = r.integers(0, 41, 70000).tolist()
    pages = sum(-(-n // 16) for n in lens)
    batch = workloads.paged_decode_inputs(B=70000, H=2, D=64, dtype="f16", page_size=16,
                                          num_pages=pages + 16, seq_lens=lens,
                                          max_pages_per_seq=3, seed=77)
    out = torch.full(tuple(batch.q.shape), float("nan"), dtype=batch.q.dtype, device="cuda")
    o = _run(gpu_lib, batch, out=out)
    assert torch.isfinite(o.float()).all()
    empty = [b for b, n in enumerate(lens) if n == 0]
    assert torch.count_nonzero(o[empty]) == 0
    idx = list(range(0, 70000, 117)) + list(range(69990, 70000))
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, batch_indices=idx)
    assert_parity(o[idx].double().numpy(), ref, "decode 70000 sequences (sampled)")
