"""GPU parity of grouped-query / multi-query attention (H_kv < H) through the
C ABI against the fp64 oracle, for prefill (attn_prefill_gqa) and paged
decode (attn_paged_decode_gqa).  Same bar as the multi-head tests: max-abs
<= 1e-2 and relative Frobenius <= 2e-3; with an fp32 output, 3e-3 and 5e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import MAX_ABS_TOL, REL_FRO_TOL, assert_parity

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.double().cpu().numpy()


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("H,H_kv", [(8, 2), (12, 3), (8, 1), (64, 8)])
@pytest.mark.parametrize("dtype,layout,causal", [("f16", "BHSD", False), ("bf16", "BSHD", True),
                                                 ("bf16", "BHSD", True), ("f16", "BSHD", False)])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gqa(gpu_lib, H, H_kv, dtype, layout, causal, D):
    Sq, Skv = (150, 333) if H <= 12 else (70, 90)
    q, k, v = workloads.prefill_inputs(2, H, Sq, Skv, D, dtype, layout, seed=H + H_kv + D,
                                       h_kv=H_kv)
    print(f"[case] prefill_gqa H{H}/{H_kv} D{D} {dtype} {layout} causal={causal}", flush=True)
    o = gpu_lib.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, causal=causal, layout=layout)
    assert_parity(_f64(o), ref, f"prefill gqa H{H}/{H_kv} D{D} {dtype} {layout} causal={causal}")


def test_prefill_gqa_equals_repeated_kv_bitwise(gpu_lib):
    """Grouped K/V give bitwise the result of the same K/V repeated per query head."""
    q, k, v = workloads.prefill_inputs(2, 8, 300, 300, 128, "bf16", "BHSD", seed=71, h_kv=2)
    print("[case] prefill_gqa vs repeated kv", flush=True)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o_g = gpu_lib.prefill(qg, kg, vg, causal=True)
    o_r = gpu_lib.prefill(qg, kg.repeat_interleave(4, dim=1).contiguous(),
                          vg.repeat_interleave(4, dim=1).contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_r)


@pytest.mark.timeout(900)
def test_prefill_gqa_causal_bshd_8k_whole(gpu_lib, progress):
    """The grouped-query causal 8k workload at full size, NaN-prefilled
    output, compared with the oracle over the whole tensor."""
    q, k, v, m = workloads.prefill_config(6)
    print(f"[case] prefill {m['name']} whole tensor", flush=True)
    kw = dict(causal=m["causal"], scale=m["scale"], layout=m["layout"])
    qg = q.cuda()
    o = gpu_lib.prefill(qg, k.cuda(), v.cuda(), out=whole.nan_like(qg), **kw)
    torch.cuda.synchronize()
    outs = {"o": o.cpu()}
    st = whole.compare(whole.prefill_units(q, k, v, ["o"], **kw), outs, progress=progress)["o"]
    print(f"[parity] {m['name']} (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0, f"{st.nonfinite} elements not written (or not finite)"
    assert st.max_abs <= MAX_ABS_TOL and st.rel_fro <= REL_FRO_TOL, f"{m['name']}: {st}"


# ------------------------------------------------------------------- decode

EDGE_LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 1000, 4096, 8191, 8192]


def _decode(attn, batch, **kw):
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    o = attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"], **kw)
    torch.cuda.synchronize()
    return o.cpu()


def _ref(batch):
    return oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                               batch.seq_lens)


@pytest.mark.parametrize("H,H_kv", [(8, 4), (8, 2), (32, 8), (32, 1), (64, 1), (40, 5)])
@pytest.mark.parametrize("D,dtype", [(128, "f16"), (128, "bf16"), (64, "f16"), (64, "bf16")])
def test_decode_gqa_edge_lengths_nan_poisoned(gpu_lib, H, H_kv, D, dtype):
    batch = workloads.paged_decode_inputs(B=len(EDGE_LENS), H=H, D=D, dtype=dtype, page_size=16,
                                          num_pages=2048, max_seq=8192, seed=H + H_kv + D,
                                          seq_lens=EDGE_LENS, fill=float("nan"), h_kv=H_kv)
    print(f"[case] decode_gqa H{H}/{H_kv} D{D} {dtype} edge lengths", flush=True)
    o = _decode(gpu_lib, batch)
    assert torch.isfinite(o.float()).all(), "NaN from an unused cache slot leaked into O"
    assert_parity(_f64(o), _ref(batch), f"decode gqa H{H}/{H_kv} D{D} {dtype}")


def test_decode_gqa_out_f32_and_rounding(gpu_lib):
    batch = workloads.paged_decode_inputs(B=len(EDGE_LENS), H=16, D=128, dtype="bf16",
                                          page_size=16, num_pages=2048, max_seq=8192, seed=72,
                                          seq_lens=EDGE_LENS, h_kv=4)
    print("[case] decode_gqa out_f32", flush=True)
    o32 = _decode(gpu_lib, batch, out_dtype=torch.float32)
    o16 = _decode(gpu_lib, batch)
    assert_parity(_f64(o32), _ref(batch), "decode gqa out_f32", max_abs_tol=3e-3,
                  rel_fro_tol=5e-4)
    assert torch.equal(o32.to(o16.dtype), o16)


def test_decode_gqa_pool_permutation_bitwise(gpu_lib):
    batch = workloads.paged_decode_inputs(B=16, H=16, D=128, page_size=16, num_pages=4096,
                                          max_seq=4000, seed=73, h_kv=2)
    moved = workloads.permute_pool(batch, seed=9)
    print("[case] decode_gqa pool permutation", flush=True)
    assert torch.equal(_decode(gpu_lib, batch), _decode(gpu_lib, moved))


def test_decode_gqa_bad_page_ids(gpu_lib):
    lens = [40, 100, 33, 200]
    batch = workloads.paged_decode_inputs(B=4, H=8, D=128, page_size=16, num_pages=300,
                                          seq_lens=lens, max_pages_per_seq=16, seed=74, h_kv=2)
    P = batch.num_pages
    table = batch.page_table.clone()
    table[1, 3] = P          # a middle page of sequence 1
    table[3, 0] = -1         # first page of sequence 3
    table[2, 6] = P + 99     # past sequence 2's live pages: never read
    print("[case] decode_gqa bad page ids", flush=True)
    pad = (P + 2,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    o = gpu_lib.paged_decode(batch.q.cuda(), k_pad[1:P + 1], v_pad[1:P + 1], table.cuda(),
                             batch.seq_lens.cuda()).float().cpu()
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all() and torch.isnan(o[3]).all()
    assert_parity(_f64(o[[0, 2]]), _ref(batch)[[0, 2]], "gqa sequences with valid pages")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [7, 8])
def test_decode_gqa_full_size_whole(gpu_lib, cfg, progress):
    """Grouped- and multi-query decode workloads at full size: NaN-prefilled
    output, every (sequence, head) compared with the oracle."""
    batch = workloads.decode_config(cfg)
    print(f"[case] decode config {cfg} {batch.meta['name']} whole tensor", flush=True)
    out = whole.nan_like(batch.q)
    o = _decode(gpu_lib, batch, scale=batch.meta["scale"], out=out)
    st = whole.compare(whole.decode_units(batch, ["o"], scale=batch.meta["scale"]), {"o": o},
                       progress=progress)["o"]
    print(f"[parity] {batch.meta['name']} (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0, f"{st.nonfinite} elements not written (or not finite)"
    assert st.max_abs <= MAX_ABS_TOL and st.rel_fro <= REL_FRO_TOL, f"config {cfg}: {st}"


# Grouped-query decode cuts the batch's 32-token tiles (line after line, a
# line = one sequence's tiles for one KV head) into equal ranges, one wave
# each; a range may end inside a line and run on into the next ones.  These
# cases put range ends everywhere: inside lines, on line and sequence
# boundaries, past empty sequences.

def _lens_batch(lens, H, H_kv, seed, D=128, dtype="f16", **kw):
    pages = sum(-(-max(n, 0) // 16) for n in lens)
    return workloads.paged_decode_inputs(B=len(lens), H=H, D=D, dtype=dtype, page_size=16,
                                         num_pages=pages + 64, seq_lens=lens, seed=seed,
                                         h_kv=H_kv, **kw)


@pytest.mark.parametrize("H,H_kv", [(8, 2), (32, 1), (64, 1)])
def test_decode_gqa_ranges_mixed_lengths(gpu_lib, H, H_kv):
    """700 sequences (more than one pass of the length scan) mixing empty,
    one-token, page-edge and long ones: every head against the oracle, and
    O = 0 exactly for the empty sequences."""
    rng = np.random.default_rng(H + H_kv)
    lens = rng.choice([0, 1, 16, 17, 33, 100, 512, 513, 2000], size=700).tolist()
    batch = _lens_batch(lens, H, H_kv, seed=75 + H)
    print(f"[case] decode_gqa ranges H{H}/{H_kv} B700 mixed lengths", flush=True)
    o = _decode(gpu_lib, batch)
    live = [b for b, n in enumerate(lens) if n > 0]
    empty = [b for b, n in enumerate(lens) if n == 0]
    assert empty and torch.count_nonzero(o[empty]) == 0
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, batch_indices=live)
    assert_parity(_f64(o[live]), ref, f"decode gqa ranges H{H}/{H_kv} mixed lengths")


@pytest.mark.parametrize("lens,H,H_kv", [([60000], 32, 1), ([0, 37000, 0], 64, 1),
                                         ([5, 30000], 16, 2)])
def test_decode_gqa_ranges_long_sequences(gpu_lib, lens, H, H_kv):
    """Few long sequences: one line spread over many ranges (up to a hundred
    partials merged per head), two query chunks per KV head (group 64)."""
    batch = _lens_batch(lens, H, H_kv, seed=76 + H, dtype="bf16")
    print(f"[case] decode_gqa ranges H{H}/{H_kv} long {lens}", flush=True)
    o = _decode(gpu_lib, batch)
    live = [b for b, n in enumerate(lens) if n > 0]
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, batch_indices=live)
    assert_parity(_f64(o[live]), ref, f"decode gqa ranges long {lens}")
    assert torch.count_nonzero(o[[b for b, n in enumerate(lens) if n == 0]]) == 0


@pytest.mark.parametrize("lens,H,H_kv,dtype", [([9000, 3, 40000], 3, 1, "f16"),
                                               ([9000, 3, 40000], 6, 2, "bf16"),
                                               ([5000, 100, 8192, 1, 17], 3, 3, "f16")])
def test_decode_combine_row_groups(gpu_lib, lens, H, H_kv, dtype):
    """The combines merge eight (sequence, head) rows per workgroup: B*H not a
    multiple of eight leaves the last workgroup part empty, and long
    sequences give a row more partials than one batch of loads holds (fp16
    partials 16 at a time, fp32 ones 8)."""
    assert (len(lens) * H) % 8 != 0
    batch = _lens_batch(lens, H, H_kv, seed=81 + H, dtype=dtype)
    print(f"[case] decode combine rows B{len(lens)} H{H}/{H_kv} {dtype} {lens}", flush=True)
    o = _decode(gpu_lib, batch)
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens)
    assert_parity(_f64(o), ref, f"decode combine rows B{len(lens)} H{H}/{H_kv} {dtype}")


def test_decode_gqa_ranges_workspace_reused(gpu_lib):
    """The range metadata is rewritten by every call: a workspace used for a
    batch of long sequences, then for the same sizes with mostly empty ones,
    gives bitwise what a fresh workspace gives."""
    attn = gpu_lib
    long_b = _lens_batch([4000] * 24, 32, 4, seed=77)
    short_lens = [0] * 24
    short_lens[5], short_lens[17] = 70, 1
    short_b = workloads.paged_decode_inputs(B=24, H=32, D=128, page_size=16,
                                            num_pages=long_b.num_pages, seq_lens=short_lens,
                                            max_pages_per_seq=long_b.max_pages_per_seq, seed=78,
                                            h_kv=4)
    need = attn.attn_paged_decode_gqa_workspace_size(24, 32, 4, 128, long_b.max_pages_per_seq, 16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    print("[case] decode_gqa ranges workspace reuse", flush=True)
    _decode(attn, long_b, workspace=ws)
    again = _decode(attn, short_b, workspace=ws)
    fresh = _decode(attn, short_b)
    assert torch.equal(again, fresh)
    ref = oracle.paged_decode(short_b.q, short_b.k_cache, short_b.v_cache, short_b.page_table,
                              short_b.seq_lens, batch_indices=[5, 17])
    assert_parity(_f64(fresh[[5, 17]]), ref, "decode gqa after workspace reuse")


def test_decode_gqa_ranges_bad_page_in_long_sequence(gpu_lib):
    """A bad page id deep inside a sequence that spans several ranges makes
    every head of that sequence NaN and leaves the others exact."""
    lens = [3000, 9000, 20, 5000]
    batch = _lens_batch(lens, 32, 1, seed=79, max_pages_per_seq=600)
    P = batch.num_pages
    table = batch.page_table.clone()
    table[1, 400] = P + 3  # one past the pool, plus 3: inside the padding below
    # The pool sits one page into an allocation with five spare pages, so a
    # missed device-side check would read allocated memory (and fail the
    # asserts) rather than fault.
    pad = (P + 5,) + tuple(batch.k_cache.shape[1:])
    k_pad = torch.zeros(pad, dtype=batch.k_cache.dtype, device="cuda")
    v_pad = torch.zeros(pad, dtype=batch.v_cache.dtype, device="cuda")
    k_pad[1:P + 1].copy_(batch.k_cache)
    v_pad[1:P + 1].copy_(batch.v_cache)
    print("[case] decode_gqa ranges bad page in a long sequence", flush=True)
    g = {n: getattr(batch, n).cuda() for n in ("q", "seq_lens")}
    o = gpu_lib.paged_decode(g["q"], k_pad[1:P + 1], v_pad[1:P + 1], table.cuda(),
                             g["seq_lens"]).float().cpu()
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all()
    assert torch.isfinite(o[[0, 2, 3]]).all()
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, batch_indices=[0, 2, 3])
    assert_parity(_f64(o[[0, 2, 3]]), ref, "gqa sequences around the bad one")
