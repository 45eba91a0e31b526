"""Seeded input generators: shapes, determinism, page-pool bookkeeping (CPU only)."""
import math

import numpy as np
import torch

import workloads


def test_prefill_config_shapes_and_determinism():
    q, k, v, meta = workloads.prefill_config(1)
    assert q.shape == (1, 2, 128, 64) and q.dtype == torch.float16
    assert meta["scale"] == 1 / 8
    q2, _, _, _ = workloads.prefill_config(1)
    assert torch.equal(q, q2)
    q3, k3, v3 = workloads.prefill_inputs(2, 3, 5, 7, 8, "bf16", "BSHD", amp=0.5, seed=3)
    assert q3.shape == (2, 5, 3, 8) and k3.shape == (2, 7, 3, 8) and k3.dtype == torch.bfloat16


def test_amp_and_rounding():
    g = torch.Generator().manual_seed(9)
    raw = torch.randn((1, 1, 4, 8), generator=g)
    q, _, _ = workloads.prefill_inputs(1, 1, 4, 4, 8, "bf16", "BHSD", amp=0.5, seed=9)
    assert torch.equal(q, (raw * 0.5).to(torch.bfloat16))


def test_paged_batch_layout():
    b = workloads.paged_decode_inputs(B=5, H=2, D=8, page_size=16, num_pages=64, seed=4,
                                      seq_lens=[1, 16, 17, 33, 64])
    assert b.page_table.dtype == torch.int32 and b.seq_lens.dtype == torch.int32
    used = []
    for i, n in enumerate(b.seq_lens.tolist()):
        npg = math.ceil(n / 16)
        used += b.page_table[i, :npg].tolist()
    assert len(set(used)) == len(used), "a page is shared between sequences"
    assert all(0 <= p < 64 for p in used)
    # unused page-table entries point at a page that holds no live token
    unused = b.meta["unused_page"]
    assert unused not in used
    assert torch.count_nonzero(b.k_cache[unused]) == 0


def test_decode_config_statistics():
    b = workloads.decode_config(4)
    assert b.q.shape == (64, 32, 128) and b.k_cache.shape == (65536, 16, 32, 128)
    lens = b.seq_lens.numpy()
    assert lens.min() >= 1 and lens.max() <= 8192
    assert b.page_table.shape == (64, 512)
    live = int(lens.sum())
    assert b.meta["n_live_tokens"] == live


def test_pool_permutation_keeps_sequences():
    b = workloads.paged_decode_inputs(B=3, H=1, D=4, page_size=16, num_pages=16, seed=2,
                                      seq_lens=[5, 20, 40])
    m = workloads.permute_pool(b, seed=1)
    for i, n in enumerate(b.seq_lens.tolist()):
        t = torch.arange(n)
        a = b.k_cache[b.page_table[i].long()[t // 16], t % 16]
        c = m.k_cache[m.page_table[i].long()[t // 16], t % 16]
        assert torch.equal(a, c)
