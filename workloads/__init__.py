"""Seeded synthetic inputs shared by the attention kernels' tests, the bench and the oracle.

This module holds no attention arithmetic.  It only draws random numbers,
rounds them to the storage dtype, and does the page-pool bookkeeping that lays
each sequence's tokens out in a paged KV cache.  Both sides of every parity
check (the HIP library and the CPU oracle) take their inputs from here.

Recipe (the same for every shape):

* ``torch.Generator().manual_seed(seed)`` on the CPU;
* float32 ``randn`` in the tensor's own memory layout, drawn in the order
  q, k, v; multiplied by ``amp``; rounded to fp16/bf16 with round-to-nearest-even
  (torch's ``.to``);
* paged decode draws, in order: ``seq_lens`` (integers, uniform on
  ``[min_seq, max_seq]`` inclusive), a permutation of the page pool, q, then K
  and V for the live tokens in (sequence, token) order.  Sequence ``b`` takes
  the next ``ceil(seq_len_b / page_size)`` pages of the permutation, so no page
  is shared.  Cache slots that hold no live token are filled with ``fill``
  (0 for the benchmark, NaN for the robustness tests).  Page-table entries past
  a sequence's last page point at page ``unused_page`` (a page that holds no
  live token when the pool has one), and are never meant to be read.

The workloads mirror the LLM-shaped attention of the pages (Llama-2-13B-like
heads, long causal contexts, a paged decode batch); their public benchmark
suite is not available here, so these seeded tensors stand in for it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}

# Prefill workloads, keyed by the config number used throughout the repository.
PREFILL_CONFIGS = {
    1: dict(name="tiny-mha-d64", B=1, H=2, Sq=128, Skv=128, D=64, dtype="f16",
            layout="BHSD", causal=False, amp=1.0, scale=1.0 / 8.0),
    2: dict(name="llama2-13b-prefill", B=4, H=40, Sq=4096, Skv=4096, D=128, dtype="f16",
            layout="BHSD", causal=False, amp=1.0, scale=None),
    3: dict(name="causal-bshd-8k", B=2, H=32, Sq=8192, Skv=8192, D=128, dtype="bf16",
            layout="BSHD", causal=True, amp=0.5, scale=None),
    5: dict(name="long-causal-32k", B=1, H=64, Sq=32768, Skv=32768, D=128, dtype="bf16",
            layout="BHSD", causal=True, amp=1.0, scale=None),
    # Grouped-query attention (four query heads per KV head), otherwise shaped
    # like the causal 8k workload.
    6: dict(name="gqa-causal-bshd-8k", B=2, H=32, H_kv=8, Sq=8192, Skv=8192, D=128,
            dtype="bf16", layout="BSHD", causal=True, amp=0.5, scale=None),
    # FP8 (e4m3fn, per-tensor descales) inputs in the headline shape; O in fp16.
    10: dict(name="fp8-llama2-13b-prefill", B=4, H=40, Sq=4096, Skv=4096, D=128, dtype="fp8",
             layout="BHSD", causal=False, amp=1.0, scale=None, out_dtype="f16"),
    # One 512-token chunk of a long prompt against its 32k keys so far
    # (bottom-right causal), run through the split-KV prefill: 64 workgroups
    # unsplit, too few for 256 CUs.
    13: dict(name="chunk-prefill-512-at-32k", B=1, H=32, H_kv=8, Sq=512, Skv=32768, D=128,
             dtype="bf16", layout="BSHD", causal=True, amp=1.0, scale=None, splitkv=True),
}

# Backward workloads: the gradients of the causal 8k BSHD prefill (a training
# step's attention), with dO drawn like the inputs.
BACKWARD_CONFIGS = {
    11: dict(name="bwd-causal-bshd-8k", B=2, H=32, Sq=8192, Skv=8192, D=128, dtype="bf16",
             layout="BSHD", causal=True, amp=0.5, amp_do=1.0, scale=None),
    # The same with four query heads per KV head.
    12: dict(name="bwd-gqa-causal-bshd-8k", B=2, H=32, H_kv=8, Sq=8192, Skv=8192, D=128,
             dtype="bf16", layout="BSHD", causal=True, amp=0.5, amp_do=1.0, scale=None),
}

# Paged decode workload.
DECODE_CONFIGS = {
    4: dict(name="paged-decode-b64", B=64, H=32, D=128, dtype="f16", page_size=16,
            num_pages=65536, min_seq=1, max_seq=8192),
    # Grouped-query (8 KV heads for 32 query heads) and multi-query (1 KV head)
    # decode over the same length mix.
    7: dict(name="gqa-paged-decode-b64", B=64, H=32, H_kv=8, D=128, dtype="f16",
            page_size=16, num_pages=65536, min_seq=1, max_seq=8192),
    8: dict(name="mqa-paged-decode-b256", B=256, H=32, H_kv=1, D=128, dtype="f16",
            page_size=16, num_pages=131072, min_seq=1, max_seq=8192),
}


# Extend (chunked prefill after a cached prefix): a batch of sequences, each
# with a cached prefix and a chunk of new tokens.
EXTEND_CONFIGS = {
    9: dict(name="extend-gqa-b8", B=8, H=32, H_kv=8, D=128, dtype="bf16", page_size=16,
            min_prefix=0, max_prefix=8192, min_extend=256, max_extend=2048),
    # one step of chunked prefill through the paged cache: a 512-token chunk
    # of a long prompt after its first 32768 tokens, through attn_extend_splitkv
    14: dict(name="chunk-extend-512-at-32k", B=1, H=32, H_kv=8, D=128, dtype="bf16",
             page_size=16, min_prefix=32768, max_prefix=32768, min_extend=512, max_extend=512,
             splitkv=True),
}


def default_scale(D: int) -> float:
    """Softmax scale used when a workload names none: 1/sqrt(head_dim)."""
    return 1.0 / math.sqrt(D)


def layout_shape(B: int, H: int, S: int, D: int, layout: str) -> tuple:
    if layout == "BHSD":
        return (B, H, S, D)
    if layout == "BSHD":
        return (B, S, H, D)
    raise ValueError(f"unknown layout {layout!r}")


def _draw(shape, g, amp, dtype):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if amp != 1.0:
        x.mul_(amp)
    return x.to(DTYPES[dtype])


def device_normal(shape, dtype="f16", seed=0, device="cuda", amp=1.0, chunk=1 << 28):
    """Seeded N(0,1) * amp rounded (RNE) to ``dtype``, drawn on ``device`` by a
    device generator seeded with ``seed``: for tensors of billions of
    elements, too large to draw on the host and copy.  float32 draws in chunks
    of ``chunk`` elements, in memory order."""
    out = torch.empty(shape, dtype=DTYPES[dtype], device=device)
    g = torch.Generator(device=device).manual_seed(seed)
    flat = out.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device)
        if amp != 1.0:
            x.mul_(amp)
        flat[i:i + n].copy_(x)
        del x
    return out


def prefill_inputs(B, H, Sq, Skv, D, dtype="f16", layout="BHSD", amp=1.0, seed=0, h_kv=None):
    """Seeded q, k, v (CPU tensors in ``layout``), drawn q then k then v.
    k and v have ``h_kv`` heads (default H)."""
    g = torch.Generator().manual_seed(seed)
    hk = H if h_kv is None else h_kv
    q = _draw(layout_shape(B, H, Sq, D, layout), g, amp, dtype)
    k = _draw(layout_shape(B, hk, Skv, D, layout), g, amp, dtype)
    v = _draw(layout_shape(B, hk, Skv, D, layout), g, amp, dtype)
    return q, k, v


def backward_inputs(B, H, Sq, Skv, D, dtype="f16", layout="BHSD", amp=1.0, amp_do=1.0, seed=0,
                    h_kv=None):
    """Seeded q, k, v, dO: q, k, v exactly as ``prefill_inputs`` draws them for
    the same seed, then dO (shaped like q, N(0,1) * amp_do) from the same
    generator."""
    g = torch.Generator().manual_seed(seed)
    hk = H if h_kv is None else h_kv
    q = _draw(layout_shape(B, H, Sq, D, layout), g, amp, dtype)
    k = _draw(layout_shape(B, hk, Skv, D, layout), g, amp, dtype)
    v = _draw(layout_shape(B, hk, Skv, D, layout), g, amp, dtype)
    do = _draw(layout_shape(B, H, Sq, D, layout), g, amp_do, dtype)
    return q, k, v, do


def backward_config(cfg: int):
    """(q, k, v, dO, meta) for one of the numbered backward workloads, seeded with its number."""
    c = dict(BACKWARD_CONFIGS[cfg])
    q, k, v, do = backward_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                  c["layout"], c["amp"], c["amp_do"], seed=cfg,
                                  h_kv=c.get("H_kv"))
    c.setdefault("H_kv", c["H"])
    if c["scale"] is None:
        c["scale"] = default_scale(c["D"])
    c["seed"] = cfg
    return q, k, v, do, c


FP8_MAX = 448.0  # largest finite e4m3fn value


def quantize_fp8(x: torch.Tensor):
    """Per-tensor e4m3fn quantisation: descale = amax / 448, codes = RNE(x / descale).
    Returns (codes as torch.float8_e4m3fn, descale as a Python float)."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = amax / FP8_MAX if amax > 0 else 1.0
    return (x / descale).to(torch.float8_e4m3fn), descale


def prefill_inputs_fp8(B, H, Sq, Skv, D, layout="BHSD", amp=1.0, seed=0, h_kv=None):
    """Seeded e4m3fn q, k, v with per-tensor descales: float32 N(0,1)*amp drawn
    as in ``prefill_inputs`` (q, then k, then v), each quantised by
    ``quantize_fp8``.  Returns (q8, k8, v8, (q_descale, k_descale, v_descale))."""
    g = torch.Generator().manual_seed(seed)
    hk = H if h_kv is None else h_kv
    out, scales = [], []
    for heads, S in ((H, Sq), (hk, Skv), (hk, Skv)):
        x = torch.randn(layout_shape(B, heads, S, D, layout), generator=g, dtype=torch.float32)
        if amp != 1.0:
            x.mul_(amp)
        c, d = quantize_fp8(x)
        out.append(c)
        scales.append(d)
    return out[0], out[1], out[2], tuple(scales)


def prefill_config(cfg: int):
    """(q, k, v, meta) for one of the numbered prefill workloads, seeded with its number."""
    c = dict(PREFILL_CONFIGS[cfg])
    if c["dtype"] == "fp8":
        q, k, v, c["descales"] = prefill_inputs_fp8(c["B"], c["H"], c["Sq"], c["Skv"], c["D"],
                                                    c["layout"], c["amp"], seed=cfg,
                                                    h_kv=c.get("H_kv"))
    else:
        q, k, v = prefill_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                 c["layout"], c["amp"], seed=cfg, h_kv=c.get("H_kv"))
    c.setdefault("H_kv", c["H"])
    if c["scale"] is None:
        c["scale"] = default_scale(c["D"])
    c["seed"] = cfg
    return q, k, v, c


@dataclass
class PagedBatch:
    q: torch.Tensor            # [B, H, D]
    k_cache: torch.Tensor      # [num_pages, page_size, H_kv, D]
    v_cache: torch.Tensor      # [num_pages, page_size, H_kv, D]
    page_table: torch.Tensor   # [B, max_pages_per_seq] int32
    seq_lens: torch.Tensor     # [B] int32
    page_size: int
    meta: dict = field(default_factory=dict)

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])


def _np_bits_dtype(dtype):
    return np.uint16  # fp16 and bf16 are both 2-byte; stored as raw bits


def paged_decode_inputs(B, H, D, dtype="f16", page_size=16, num_pages=65536,
                        min_seq=1, max_seq=8192, seed=0, fill=0.0, seq_lens=None,
                        amp=1.0, max_pages_per_seq=None, h_kv=None):
    """Seeded paged-decode batch (CPU tensors).

    ``seq_lens`` may be given explicitly (a list of ints); otherwise it is drawn
    uniformly from ``[min_seq, max_seq]``.  The cache is allocated with
    ``numpy.zeros`` (lazily mapped) unless ``fill`` is nonzero/NaN, so an 8 GiB
    pool costs host memory only for its live pages.
    """
    g = torch.Generator().manual_seed(seed)
    if seq_lens is None:
        lens = torch.randint(min_seq, max_seq + 1, (B,), generator=g, dtype=torch.int64)
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int64)
        assert lens.numel() == B
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, -(-max(max_seq, int(lens.max()) if B else 1) // page_size))
    pages_needed = [(-(-int(n) // page_size)) for n in lens.tolist()]
    assert all(p <= max_pages_per_seq for p in pages_needed), "sequence longer than the page table"
    total_pages = sum(pages_needed)
    assert total_pages <= num_pages, "page pool too small for the batch"
    perm = torch.randperm(num_pages, generator=g)
    unused_page = int(perm[total_pages]) if total_pages < num_pages else int(perm[0])

    page_table = torch.full((B, max_pages_per_seq), unused_page, dtype=torch.int32)
    cursor = 0
    for b, npg in enumerate(pages_needed):
        page_table[b, :npg] = perm[cursor:cursor + npg].to(torch.int32)
        cursor += npg

    hk = H if h_kv is None else h_kv
    q = _draw((B, H, D), g, amp, dtype)
    n_live = int(lens.sum())
    k_live = _draw((n_live, hk, D), g, amp, dtype)
    v_live = _draw((n_live, hk, D), g, amp, dtype)

    shape = (num_pages, page_size, hk, D)
    tdt = DTYPES[dtype]
    if fill == 0.0 and not math.isnan(fill):
        k_np = np.zeros(shape, dtype=np.uint16)
        v_np = np.zeros(shape, dtype=np.uint16)
    else:
        bits = int(torch.tensor([fill], dtype=tdt).view(torch.int16).item()) & 0xFFFF
        k_np = np.full(shape, bits, dtype=np.uint16)
        v_np = np.full(shape, bits, dtype=np.uint16)

    # Scatter live tokens: token t of sequence b -> (page_table[b, t // page_size], t % page_size).
    kb = k_live.view(torch.int16).numpy().view(np.uint16)
    vb = v_live.view(torch.int16).numpy().view(np.uint16)
    cursor = 0
    for b, n in enumerate(lens.tolist()):
        if n == 0:
            continue
        t = np.arange(n)
        pages = page_table[b].numpy()[t // page_size]
        slots = t % page_size
        k_np[pages, slots] = kb[cursor:cursor + n]
        v_np[pages, slots] = vb[cursor:cursor + n]
        cursor += n

    k_cache = torch.from_numpy(k_np).view(torch.int16).view(tdt)
    v_cache = torch.from_numpy(v_np).view(torch.int16).view(tdt)
    meta = dict(B=B, H=H, H_kv=hk, D=D, dtype=dtype, page_size=page_size, num_pages=num_pages,
                seed=seed, fill=fill, n_live_tokens=n_live, unused_page=unused_page)
    return PagedBatch(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                      seq_lens=lens.to(torch.int32), page_size=page_size, meta=meta)


@dataclass
class ExtendBatch:
    q: torch.Tensor            # [T, H, D], new tokens of all sequences, packed
    k: torch.Tensor            # [T, H_kv, D]
    v: torch.Tensor            # [T, H_kv, D]
    k_cache: torch.Tensor      # [num_pages, page_size, H_kv, D] (the prefixes)
    v_cache: torch.Tensor
    page_table: torch.Tensor   # [B, max_pages_per_seq] int32
    prefix_lens: torch.Tensor  # [B] int32
    qo_start: torch.Tensor     # [B + 1] int32, new tokens of b at rows qo_start[b] ..
    page_size: int
    meta: dict = field(default_factory=dict)

    @property
    def max_extend_len(self) -> int:
        return int((self.qo_start[1:] - self.qo_start[:-1]).max()) if len(self.qo_start) > 1 else 0


def extend_inputs(B, H, D, prefix_lens, extend_lens, dtype="f16", page_size=16, num_pages=None,
                  seed=0, h_kv=None, amp=1.0, fill=0.0):
    """Seeded extend batch (CPU tensors): the prefixes are a paged-decode batch
    (``paged_decode_inputs`` with seq_lens = prefix_lens, same seed); the new
    tokens' q, k, v are then drawn from a generator seeded ``seed + 7919``, in
    the order q, k, v, packed token-major."""
    prefix_lens = [int(x) for x in prefix_lens]
    extend_lens = [int(x) for x in extend_lens]
    assert len(prefix_lens) == B and len(extend_lens) == B
    hk = H if h_kv is None else h_kv
    pages = sum(-(-p // page_size) for p in prefix_lens)
    if num_pages is None:
        num_pages = max(1, 2 * pages)
    max_pages = max(1, -(-max(prefix_lens + [1]) // page_size))
    pre = paged_decode_inputs(B, H, D, dtype, page_size, num_pages, seed=seed, fill=fill,
                              seq_lens=prefix_lens, amp=amp, max_pages_per_seq=max_pages,
                              h_kv=hk)
    g = torch.Generator().manual_seed(seed + 7919)
    T = sum(extend_lens)
    q = _draw((T, H, D), g, amp, dtype)
    k = _draw((T, hk, D), g, amp, dtype)
    v = _draw((T, hk, D), g, amp, dtype)
    starts = torch.tensor([0] + list(np.cumsum(extend_lens)), dtype=torch.int32)
    meta = dict(B=B, H=H, H_kv=hk, D=D, dtype=dtype, page_size=page_size, num_pages=num_pages,
                seed=seed, total_tokens=T)
    return ExtendBatch(q=q, k=k, v=v, k_cache=pre.k_cache, v_cache=pre.v_cache,
                       page_table=pre.page_table, prefix_lens=pre.seq_lens, qo_start=starts,
                       page_size=page_size, meta=meta)


def extend_config(cfg: int):
    """ExtendBatch for one of the numbered extend workloads, seeded with its number:
    prefix and extend lengths drawn uniformly (inclusive) from their ranges."""
    c = dict(EXTEND_CONFIGS[cfg])
    g = torch.Generator().manual_seed(cfg)
    plen = torch.randint(c["min_prefix"], c["max_prefix"] + 1, (c["B"],), generator=g).tolist()
    elen = torch.randint(c["min_extend"], c["max_extend"] + 1, (c["B"],), generator=g).tolist()
    batch = extend_inputs(c["B"], c["H"], c["D"], plen, elen, c["dtype"], c["page_size"],
                          seed=cfg, h_kv=c.get("H_kv"))
    batch.meta.update(name=c["name"], scale=default_scale(c["D"]), config=cfg)
    return batch


def decode_config(cfg: int, fill=0.0):
    """PagedBatch for one of the numbered decode workloads, seeded with its number."""
    c = dict(DECODE_CONFIGS[cfg])
    batch = paged_decode_inputs(c["B"], c["H"], c["D"], c["dtype"], c["page_size"],
                                c["num_pages"], c["min_seq"], c["max_seq"], seed=cfg, fill=fill,
                                h_kv=c.get("H_kv"))
    batch.meta.update(name=c["name"], scale=default_scale(c["D"]), config=cfg)
    return batch


def permute_pool(batch: PagedBatch, seed: int) -> PagedBatch:
    """The same logical batch with its pages moved to other pool slots.

    Page p of the pool moves to slot ``perm[p]`` and the page table is
    remapped accordingly, so every sequence still sees the same tokens.
    """
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(batch.num_pages, generator=g)
    k = torch.empty_like(batch.k_cache)
    v = torch.empty_like(batch.v_cache)
    k[perm] = batch.k_cache
    v[perm] = batch.v_cache
    table = perm[batch.page_table.long()].to(torch.int32)
    return PagedBatch(q=batch.q, k_cache=k, v_cache=v, page_table=table,
                      seq_lens=batch.seq_lens, page_size=batch.page_size,
                      meta=dict(batch.meta, pool_perm_seed=seed))
