"""Pins for the fp64 oracle: facts fixed by mathematics or by a library routine.

Each ``check_*`` raises AssertionError when the oracle disagrees with the fact.
``test_oracle.py`` runs them against the oracle as it is; and
``test_oracle_mutations.py`` runs them against copies with planted mistakes
(a wrong causal offset, a dropped scale, swapped operands, a wrong page index)
to show that every such mistake fails at least one pin.

None of these re-types the oracle's own formula: the references are a
50-digit brute force, torch's ``scaled_dot_product_attention`` (the library
routine the definition reduces to), ``scipy.special.expit`` for two keys,
closed forms (V = 1, K = 0, causal row 0) and invariants of softmax.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads

F64 = torch.float64


def _rand(shape, seed, dtype=torch.float16, amp=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * amp).to(dtype)


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e}"


# --------------------------------------------------------------- brute force

def _mp_attention(q, k, v, causal, scale, dps=50):
    """50-digit brute force over one head: q [Sq,D], k/v [Skv,D] (python floats)."""
    import mpmath
    mpmath.mp.dps = dps
    Sq, Skv = len(q), len(k)
    D = len(v[0]) if Skv else len(q[0])
    out = []
    for i in range(Sq):
        keys = [j for j in range(Skv) if (not causal) or (j - i <= Skv - Sq)]
        if not keys:
            out.append([0.0] * D)
            continue
        logits = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i][d]) * mpmath.mpf(k[j][d])
                                                      for d in range(len(q[i]))) for j in keys}
        top = max(logits.values())
        w = {j: mpmath.exp(logits[j] - top) for j in keys}
        z = mpmath.fsum(w.values())
        out.append([float(mpmath.fsum(w[j] * mpmath.mpf(v[j][d]) for j in keys) / z)
                    for d in range(D)])
    return out


BRUTE_CASES = [
    # (B, H, Sq, Skv, D, causal)
    (1, 2, 3, 5, 4, False),
    (1, 1, 5, 3, 2, True),     # Sq > Skv: the first rows see no key
    (1, 2, 6, 6, 3, True),
    (1, 1, 4, 7, 4, True),     # Sq < Skv: bottom-right alignment
    (1, 1, 1, 7, 4, False),
    (2, 1, 2, 2, 1, True),
]


def check_bruteforce():
    for n, (B, H, Sq, Skv, D, causal) in enumerate(BRUTE_CASES):
        q = _rand((B, H, Sq, D), 100 + n)
        k = _rand((B, H, Skv, D), 200 + n)
        v = _rand((B, H, Skv, D), 300 + n)
        scale = 1.0 / math.sqrt(D)
        got = oracle.sdpa(q, k, v, causal=causal, scale=scale)
        for b in range(B):
            for h in range(H):
                ref = _mp_attention(q[b, h].double().tolist(), k[b, h].double().tolist(),
                                    v[b, h].double().tolist(), causal, scale)
                _close(got[b, h], ref, 1e-13, f"brute force case {n} b{b} h{h}")


# ------------------------------------------------------------ library routine

LIB_CASES = [
    # (B, H, Sq, Skv, D, causal, layout)
    (2, 3, 17, 17, 16, False, "BHSD"),
    (2, 3, 17, 17, 16, True, "BHSD"),
    (1, 2, 9, 23, 8, True, "BHSD"),      # bottom-right causal, Sq < Skv
    (1, 2, 23, 23, 8, True, "BSHD"),
    (2, 2, 11, 29, 32, False, "BSHD"),
    (1, 1, 40, 64, 64, True, "BSHD"),
]


def _torch_sdpa(q, k, v, causal, scale):
    """torch's routine on BHSD float64; bottom-right causal via a tril(diagonal) mask."""
    Sq, Skv = q.shape[2], k.shape[2]
    mask = None
    if causal:
        mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale).numpy()


def check_library_sdpa():
    for n, (B, H, Sq, Skv, D, causal, layout) in enumerate(LIB_CASES):
        q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "f16", layout, seed=400 + n)
        scale = 0.7 / math.sqrt(D)
        got = oracle.sdpa(q, k, v, causal=causal, scale=scale, layout=layout)
        if layout == "BSHD":
            qt, kt, vt = (t.transpose(1, 2).to(F64) for t in (q, k, v))
            ref = _torch_sdpa(qt, kt, vt, causal, scale).transpose(0, 2, 1, 3)
        else:
            ref = _torch_sdpa(q.to(F64), k.to(F64), v.to(F64), causal, scale)
        _close(got, ref, 1e-12, f"library case {n}")
        if causal and Sq == Skv and layout == "BHSD":
            ref2 = F.scaled_dot_product_attention(q.to(F64), k.to(F64), v.to(F64),
                                                  is_causal=True, scale=scale).numpy()
            _close(got, ref2, 1e-12, f"library is_causal case {n}")


def check_rows_match_full():
    B, H, Sq, Skv, D = 2, 3, 37, 45, 16
    for layout in ("BHSD", "BSHD"):
        for causal in (False, True):
            q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "bf16", layout, seed=7)
            full = oracle.sdpa(q, k, v, causal=causal, layout=layout)
            rows = [(1, 2, 0), (0, 0, 36), (1, 1, 17), (0, 2, 5)]
            part = oracle.sdpa_rows(q, k, v, rows, causal=causal, layout=layout)
            want = [full[b, h, i] if layout == "BHSD" else full[b, i, h] for b, h, i in rows]
            # sdpa_rows must agree with the library routine as well
            for (b, h, i), r in zip(rows, part):
                if layout == "BHSD":
                    qt, kt, vt = q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1]
                else:
                    qt, kt, vt = (t[b:b + 1, :, h:h + 1].transpose(1, 2) for t in (q, k, v))
                lib = _torch_sdpa(qt.to(F64), kt.to(F64), vt.to(F64), causal, 1 / math.sqrt(D))
                _close(r, lib[0, 0, i], 1e-12, f"sdpa_rows vs library {layout} {causal} {(b, h, i)}")
            _close(part, np.stack(want), 1e-14, f"sdpa_rows vs sdpa {layout} {causal}")


# -------------------------------------------------------------- closed forms

def check_ones_v():
    """V = 1 everywhere => O = 1 everywhere (softmax weights sum to one)."""
    for causal, (Sq, Skv) in ((False, (13, 21)), (True, (21, 21)), (True, (8, 30))):
        q = _rand((1, 2, Sq, 16), 11)
        k = _rand((1, 2, Skv, 16), 12)
        v = torch.ones((1, 2, Skv, 16), dtype=torch.float16)
        got = oracle.sdpa(q, k, v, causal=causal, scale=0.25)
        _close(got, np.ones_like(got), 1e-14, f"V=1 causal={causal}")


def check_causal_row0():
    """Causal, Sq = Skv: row 0 sees only key 0, so O[0] = V[0] exactly."""
    q, k, v = workloads.prefill_inputs(2, 2, 19, 19, 32, "bf16", "BHSD", seed=13)
    got = oracle.sdpa(q, k, v, causal=True)
    _close(got[:, :, 0], v[:, :, 0].double().numpy(), 0.0, "causal row 0")


def check_zero_keys():
    """K = 0 => uniform weights: O[i] = mean of the visible V rows."""
    B, H, S, D = 1, 2, 12, 8
    q = _rand((B, H, S, D), 21)
    k = torch.zeros((B, H, S, D), dtype=torch.float16)
    v = _rand((B, H, S, D), 22)
    vv = v.double().numpy()
    got = oracle.sdpa(q, k, v, causal=False)
    _close(got, np.broadcast_to(vv.mean(axis=2, keepdims=True), got.shape), 1e-14, "K=0 mean")
    got_c = oracle.sdpa(q, k, v, causal=True)
    prefix = np.cumsum(vv, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    _close(got_c, prefix, 1e-14, "K=0 causal prefix mean")


def check_two_keys():
    """Two keys: O = expit(d) v1 + (1 - expit(d)) v0, d = scale (q.k1 - q.k0)."""
    from scipy.special import expit
    q = _rand((1, 1, 5, 8), 31)
    k = _rand((1, 1, 2, 8), 32)
    v = _rand((1, 1, 2, 8), 33)
    scale = 0.6
    got = oracle.sdpa(q, k, v, causal=False, scale=scale)
    qd, kd, vd = (t.double().numpy()[0, 0] for t in (q, k, v))
    d = scale * (qd @ kd[1] - qd @ kd[0])
    w1 = expit(d)[:, None]
    _close(got[0, 0], w1 * vd[1] + (1 - w1) * vd[0], 1e-14, "two keys")


def check_dominant_key():
    """One key far more aligned with the query than the rest => O ~ that key's V."""
    D = 16
    q = torch.ones((1, 1, 1, D), dtype=torch.float16)
    k = _rand((1, 1, 9, D), 41, amp=0.1)
    k[0, 0, 4] = 8.0
    v = _rand((1, 1, 9, D), 42)
    got = oracle.sdpa(q, k, v, causal=False, scale=1.0)
    _close(got[0, 0, 0], v[0, 0, 4].double().numpy(), 1e-12, "dominant key")


def check_zero_scale():
    """scale = 0 => uniform weights over the visible keys."""
    q, k, v = workloads.prefill_inputs(1, 1, 6, 10, 4, "f16", "BHSD", seed=17)
    got = oracle.sdpa(q, k, v, causal=False, scale=0.0)
    _close(got[0, 0], np.broadcast_to(v[0, 0].double().numpy().mean(0), (6, 4)), 1e-14, "scale 0")


# ---------------------------------------------------------------- invariants

def check_probs_rows_sum_to_one():
    q = _rand((7, 16), 51).double().numpy()
    k = _rand((12, 16), 52).double().numpy()
    vis = oracle.n_visible(7, 12, True)
    p = oracle.attention_probs(q, k, 0.25, vis)
    _close(p.sum(axis=1), np.ones(7), 1e-14, "P row sums")
    assert np.all(p >= 0)
    for r in range(7):
        assert np.all(p[r, vis[r]:] == 0), "P nonzero past the visible keys"


def check_logit_shift():
    """k_j += u for every j adds <q_i, u> to row i's logits: softmax unchanged."""
    for causal in (False, True):
        q = _rand((1, 2, 10, 8), 61).double()
        k = _rand((1, 2, 14, 8), 62).double()
        v = _rand((1, 2, 14, 8), 63).double()
        u = _rand((8,), 64).double() * 3
        a = oracle.sdpa(q, k, v, causal=causal)
        b = oracle.sdpa(q, k + u, v, causal=causal)
        _close(a, b, 1e-12, f"logit shift causal={causal}")


def check_permutations():
    """Non-causal: O is invariant to a key permutation and equivariant to a query permutation."""
    q, k, v = workloads.prefill_inputs(1, 2, 9, 13, 8, "f16", "BHSD", seed=71)
    base = oracle.sdpa(q, k, v, causal=False)
    pk = torch.randperm(13, generator=torch.Generator().manual_seed(1))
    pq = torch.randperm(9, generator=torch.Generator().manual_seed(2))
    _close(oracle.sdpa(q, k[:, :, pk], v[:, :, pk], causal=False), base, 1e-13, "key permutation")
    _close(oracle.sdpa(q[:, :, pq], k, v, causal=False), base[:, :, pq.numpy()], 1e-14,
           "query permutation")


def check_layouts_agree():
    """BSHD input = BHSD input transposed => BSHD output = BHSD output transposed."""
    q, k, v = workloads.prefill_inputs(2, 3, 11, 11, 8, "bf16", "BHSD", seed=81)
    a = oracle.sdpa(q, k, v, causal=True, layout="BHSD")
    b = oracle.sdpa(*(t.transpose(1, 2).contiguous() for t in (q, k, v)), causal=True, layout="BSHD")
    _close(b.transpose(0, 2, 1, 3), a, 0.0, "BHSD vs BSHD")


# --------------------------------------------------------------- paged decode

def _decode_library(batch, b, scale):
    """torch's routine on sequence b's tokens, read from the cache by explicit (page, slot)."""
    n = int(batch.seq_lens[b])
    ps = batch.page_size
    tok = torch.arange(n)
    pages = batch.page_table[b].long()[tok // ps]
    kk = batch.k_cache[pages, tok % ps].to(F64).transpose(0, 1)   # [H, n, D]
    vv = batch.v_cache[pages, tok % ps].to(F64).transpose(0, 1)
    qq = batch.q[b].to(F64)[:, None, :]                            # [H, 1, D]
    return F.scaled_dot_product_attention(qq[None], kk[None], vv[None], scale=scale)[0, :, 0].numpy()


def check_decode_library():
    batch = workloads.paged_decode_inputs(B=6, H=3, D=16, dtype="f16", page_size=4, num_pages=64,
                                          seed=91, seq_lens=[1, 3, 4, 5, 16, 23])
    scale = 1 / 4
    got = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, scale=scale)
    for b in range(6):
        _close(got[b], _decode_library(batch, b, scale), 1e-12, f"decode vs library b{b}")


def check_decode_matches_prefill_row():
    """Paged decode of a sequence equals ordinary Sq=1 attention over its tokens."""
    batch = workloads.paged_decode_inputs(B=3, H=2, D=8, dtype="bf16", page_size=16, num_pages=32,
                                          seed=92, seq_lens=[15, 16, 17])
    got = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens)
    for b in range(3):
        n = int(batch.seq_lens[b])
        tok = torch.arange(n)
        pages = batch.page_table[b].long()[tok // 16]
        kk = batch.k_cache[pages, tok % 16].transpose(0, 1)[None]      # [1, H, n, D]
        vv = batch.v_cache[pages, tok % 16].transpose(0, 1)[None]
        qq = batch.q[b][None, :, None, :]
        ref = F.scaled_dot_product_attention(qq.to(F64), kk.to(F64), vv.to(F64)).numpy()
        _close(got[b], ref[0, :, 0], 1e-12, f"decode vs Sq=1 library b{b}")


def check_decode_pool_permutation():
    batch = workloads.paged_decode_inputs(B=4, H=2, D=8, page_size=16, num_pages=40, seed=93,
                                          max_seq=100)
    moved = workloads.permute_pool(batch, seed=5)
    a = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table, batch.seq_lens)
    b = oracle.paged_decode(moved.q, moved.k_cache, moved.v_cache, moved.page_table, moved.seq_lens)
    _close(a, b, 0.0, "pool permutation")


def check_decode_nan_poison():
    """Slots that hold no live token must not influence O (NaN there stays out)."""
    kw = dict(B=5, H=2, D=8, page_size=16, num_pages=48, seed=94, seq_lens=[1, 15, 16, 17, 40])
    clean = workloads.paged_decode_inputs(fill=0.0, **kw)
    dirty = workloads.paged_decode_inputs(fill=float("nan"), **kw)
    a = oracle.paged_decode(clean.q, clean.k_cache, clean.v_cache, clean.page_table, clean.seq_lens)
    b = oracle.paged_decode(dirty.q, dirty.k_cache, dirty.v_cache, dirty.page_table, dirty.seq_lens)
    assert np.all(np.isfinite(b))
    _close(a, b, 0.0, "NaN poison")


# ------------------------------------------------- grouped-query attention

GQA_CASES = [  # (B, H, H_kv, Sq, Skv, D, causal, layout)
    (2, 8, 2, 9, 13, 16, False, "BHSD"),
    (1, 8, 2, 12, 12, 8, True, "BSHD"),
    (1, 6, 1, 7, 10, 8, True, "BHSD"),     # multi-query
    (2, 4, 4, 5, 9, 8, False, "BSHD"),     # H_kv = H: ordinary multi-head
]


def check_gqa_library():
    """torch's routine with enable_gqa (consecutive query heads share a KV head)."""
    for n, (B, H, Hk, Sq, Skv, D, causal, layout) in enumerate(GQA_CASES):
        q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "bf16", layout, seed=500 + n, h_kv=Hk)
        got = oracle.sdpa(q, k, v, causal=causal, layout=layout)
        qt, kt, vt = ((t.transpose(1, 2) if layout == "BSHD" else t).to(F64) for t in (q, k, v))
        mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq) if causal else None
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True).numpy()
        if layout == "BSHD":
            ref = ref.transpose(0, 2, 1, 3)
        _close(got, ref, 1e-12, f"gqa library case {n}")


def check_gqa_group_locality():
    """Changing KV head g changes exactly the outputs of query heads in group g."""
    B, H, Hk, S, D = 1, 8, 4, 6, 8
    q, k, v = workloads.prefill_inputs(B, H, S, S, D, "f16", "BHSD", seed=510, h_kv=Hk)
    base = oracle.sdpa(q, k, v, causal=False)
    for g in range(Hk):
        k2, v2 = k.clone(), v.clone()
        k2[:, g] = -k2[:, g]
        v2[:, g] = v2[:, g] + 1
        moved = oracle.sdpa(q, k2, v2, causal=False)
        changed = [h for h in range(H) if not np.allclose(moved[0, h], base[0, h], atol=0)]
        assert changed == list(range(g * H // Hk, (g + 1) * H // Hk)), (g, changed)


def check_gqa_rows_and_decode():
    """Sampled rows and paged decode follow the same head mapping as the full output."""
    B, H, Hk, Sq, Skv, D = 2, 6, 3, 11, 20, 8
    for layout in ("BHSD", "BSHD"):
        q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "f16", layout, seed=520, h_kv=Hk)
        full = oracle.sdpa(q, k, v, causal=True, layout=layout)
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in (0, 5, Sq - 1)]
        got = oracle.sdpa_rows(q, k, v, rows, causal=True, layout=layout)
        ref = [full[b, h, i] if layout == "BHSD" else full[b, i, h] for b, h, i in rows]
        _close(got, np.array(ref), 1e-13, f"gqa rows {layout}")
    batch = workloads.paged_decode_inputs(B=4, H=8, D=16, page_size=4, num_pages=64, seed=521,
                                          seq_lens=[1, 4, 9, 30], h_kv=2)
    got = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens)
    for b in range(4):
        n = int(batch.seq_lens[b])
        tok = torch.arange(n)
        pages = batch.page_table[b].long()[tok // 4]
        kk = batch.k_cache[pages, tok % 4].to(F64).transpose(0, 1)[None]   # [1, H_kv, n, D]
        vv = batch.v_cache[pages, tok % 4].to(F64).transpose(0, 1)[None]
        qq = batch.q[b].to(F64)[None, :, None, :]                          # [1, H, 1, D]
        ref = F.scaled_dot_product_attention(qq, kk, vv, enable_gqa=True)[0, :, 0].numpy()
        _close(got[b], ref, 1e-12, f"gqa decode b{b}")


# ----------------------------------------------------------- extend attention

def _extend_library(batch, b, scale=None):
    """torch's routine for sequence b: prefix K/V read by explicit (page, slot),
    then the new tokens, with the bottom-right causal mask."""
    P = int(batch.prefix_lens[b])
    r0, r1 = int(batch.qo_start[b]), int(batch.qo_start[b + 1])
    E = r1 - r0
    tok = torch.arange(P)
    pages = batch.page_table[b].long()[tok // batch.page_size]
    kk = torch.cat([batch.k_cache[pages, tok % batch.page_size], batch.k[r0:r1]]).to(F64)
    vv = torch.cat([batch.v_cache[pages, tok % batch.page_size], batch.v[r0:r1]]).to(F64)
    qq = batch.q[r0:r1].to(F64)
    mask = torch.ones(E, P + E, dtype=torch.bool).tril(diagonal=P)
    out = F.scaled_dot_product_attention(qq.transpose(0, 1)[None], kk.transpose(0, 1)[None],
                                         vv.transpose(0, 1)[None], attn_mask=mask, scale=scale,
                                         enable_gqa=True)
    return out[0].transpose(0, 1).numpy()            # [E, H, D]


EXTEND_CASES = [  # (B, H, H_kv, D, prefix_lens, extend_lens)
    (3, 4, 2, 8, [0, 17, 40], [5, 1, 9]),
    (2, 3, 3, 16, [16, 3], [16, 20]),
    (2, 6, 1, 8, [31, 0], [2, 7]),
]


def check_extend_library():
    for n, (B, H, Hk, D, pl, el) in enumerate(EXTEND_CASES):
        batch = workloads.extend_inputs(B, H, D, pl, el, "bf16", page_size=16, seed=600 + n,
                                        h_kv=Hk)
        got = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                            batch.page_table, batch.prefix_lens, batch.qo_start, scale=0.3)
        for b in range(B):
            r0, r1 = int(batch.qo_start[b]), int(batch.qo_start[b + 1])
            _close(got[r0:r1], _extend_library(batch, b, 0.3), 1e-12, f"extend case {n} b{b}")


def check_extend_without_prefix_is_causal_prefill():
    batch = workloads.extend_inputs(2, 4, 16, [0, 0], [13, 30], "f16", seed=610, h_kv=2)
    got = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start)
    for b in range(2):
        r0, r1 = int(batch.qo_start[b]), int(batch.qo_start[b + 1])
        ref = oracle.sdpa(batch.q[None, r0:r1], batch.k[None, r0:r1], batch.v[None, r0:r1],
                          causal=True, layout="BSHD")[0]
        _close(got[r0:r1], ref, 1e-13, f"extend without prefix b{b}")


def check_extend_one_token_is_decode():
    """One new token: paged decode over the cache with that token appended."""
    B, H, Hk, D = 3, 4, 2, 8
    pl = [5, 16, 33]
    batch = workloads.extend_inputs(B, H, D, pl, [1, 1, 1], "f16", seed=620, h_kv=Hk)
    got = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start)
    kc, vc = batch.k_cache.clone(), batch.v_cache.clone()
    used = set(int(x) for b in range(B) for x in batch.page_table[b, :-(-pl[b] // 16)])
    free = [p for p in range(kc.shape[0]) if p not in used]
    table = torch.cat([batch.page_table, torch.zeros(B, 1, dtype=torch.int32)], dim=1)
    for b in range(B):
        P = pl[b]
        if P % 16 == 0:                       # the new token starts a fresh page
            table[b, P // 16] = free.pop()
        page = int(table[b, P // 16])
        kc[page, P % 16] = batch.k[b]
        vc[page, P % 16] = batch.v[b]
    ref = oracle.paged_decode(batch.q, kc, vc, table, torch.tensor(pl) + 1)
    _close(got, ref, 1e-13, "extend of one token vs decode")


def check_extend_chunking():
    """Extending by E1 then E2 tokens (the first chunk written to the cache in
    between) gives the same outputs as one extend by E1 + E2."""
    B, H, Hk, D = 2, 2, 1, 8
    pl, e1, e2 = [7, 32], [9, 16], [6, 3]
    full = workloads.extend_inputs(B, H, D, pl, [a + b for a, b in zip(e1, e2)], "f16",
                                   page_size=16, num_pages=64, seed=630, h_kv=Hk)
    one = oracle.extend(full.q, full.k, full.v, full.k_cache, full.v_cache, full.page_table,
                        full.prefix_lens, full.qo_start)
    kc, vc = full.k_cache.clone(), full.v_cache.clone()
    used = set(int(x) for b in range(B) for x in full.page_table[b, :-(-pl[b] // 16)])
    free = [p for p in range(kc.shape[0]) if p not in used]
    table = torch.zeros(B, 8, dtype=torch.int32)
    table[:, :full.page_table.shape[1]] = full.page_table
    rows1, rows2 = [], []
    for b in range(B):
        r0 = int(full.qo_start[b])
        for t in range(e1[b]):                # write the first chunk behind the prefix
            pos = pl[b] + t
            if pos % 16 == 0 and pos // 16 >= -(-pl[b] // 16):
                table[b, pos // 16] = free.pop()
            kc[int(table[b, pos // 16]), pos % 16] = full.k[r0 + t]
            vc[int(table[b, pos // 16]), pos % 16] = full.v[r0 + t]
        rows1 += list(range(r0, r0 + e1[b]))
        rows2 += list(range(r0 + e1[b], r0 + e1[b] + e2[b]))
    starts1 = torch.tensor([0] + list(np.cumsum(e1)), dtype=torch.int32)
    part1 = oracle.extend(full.q[rows1], full.k[rows1], full.v[rows1], full.k_cache,
                          full.v_cache, full.page_table, full.prefix_lens, starts1)
    starts2 = torch.tensor([0] + list(np.cumsum(e2)), dtype=torch.int32)
    part2 = oracle.extend(full.q[rows2], full.k[rows2], full.v[rows2], kc, vc, table,
                          torch.tensor([p + a for p, a in zip(pl, e1)], dtype=torch.int32),
                          starts2)
    _close(np.concatenate([part1, part2]), one[rows1 + rows2], 1e-13, "chunked extend")


# ----------------------------------------------------------------- fp8 inputs

def _e4m3fn_by_formula(code: int) -> float:
    """OCP e4m3fn from its bit fields: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 is subnormal; S.1111.111 is NaN; no infinities."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def check_fp8_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    got = oracle.dequantize_fp8(codes, 1.0)
    ref = np.array([_e4m3fn_by_formula(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    assert np.nanmax(np.abs(ref)) == 448.0


def check_fp8_quantize_round_trip():
    """Codes times descale reproduce the drawn values to e4m3fn precision, and
    attention of the dequantised inputs matches the library routine."""
    q8, k8, v8, (qs, ks, vs) = workloads.prefill_inputs_fp8(1, 2, 9, 12, 16, seed=700, h_kv=1)
    q = oracle.dequantize_fp8(q8, qs)
    assert np.abs(q).max() <= 448.0 * qs * (1 + 1e-12)
    got = oracle.sdpa(torch.from_numpy(q), torch.from_numpy(oracle.dequantize_fp8(k8, ks)),
                      torch.from_numpy(oracle.dequantize_fp8(v8, vs)), causal=True)
    mask = torch.ones(9, 12, dtype=torch.bool).tril(diagonal=12 - 9)  # bottom-right
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(oracle.dequantize_fp8(k8, ks)),
        torch.from_numpy(oracle.dequantize_fp8(v8, vs)), attn_mask=mask, enable_gqa=True).numpy()
    _close(got, ref, 1e-12, "fp8 dequantised attention")


# ------------------------------------------------------------------ backward

BWD_CASES = [  # (B, H, H_kv, Sq, Skv, D, causal, layout)
    (1, 2, 2, 7, 9, 8, False, "BHSD"),
    (2, 4, 2, 10, 10, 8, True, "BSHD"),
    (1, 3, 1, 6, 11, 4, True, "BHSD"),
]


def _autograd(q, k, v, do, causal, scale, layout):
    qt, kt, vt = ((t.transpose(1, 2) if layout == "BSHD" else t).to(F64).clone().requires_grad_()
                  for t in (q, k, v))
    Sq, Skv = qt.shape[2], kt.shape[2]
    mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq) if causal else None
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    dot = (do.transpose(1, 2) if layout == "BSHD" else do).to(F64)
    out.backward(dot)
    grads = [t.grad for t in (qt, kt, vt)]
    return [(g.transpose(1, 2) if layout == "BSHD" else g).numpy() for g in grads]


def check_backward_autograd():
    for n, (B, H, Hk, Sq, Skv, D, causal, layout) in enumerate(BWD_CASES):
        q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "bf16", layout, seed=800 + n, h_kv=Hk)
        do = workloads.prefill_inputs(B, H, Sq, Sq, D, "bf16", layout, seed=850 + n)[0]
        got = oracle.sdpa_backward(q, k, v, do, causal=causal, scale=0.4, layout=layout)
        ref = _autograd(q, k, v, do, causal, 0.4, layout)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            _close(a, b, 1e-11, f"backward case {n} {name}")


def check_backward_finite_differences():
    """Central differences of sum(sdpa(q, k, v) * dO) on a tiny case."""
    q, k, v = (t.double() for t in workloads.prefill_inputs(1, 2, 3, 4, 3, "f16", seed=860, h_kv=1))
    do = workloads.prefill_inputs(1, 2, 3, 3, 3, "f16", seed=861)[0].double()
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, causal=True, scale=0.7)
    L = lambda q_, k_, v_: float((oracle.sdpa(q_, k_, v_, causal=True, scale=0.7) * do.numpy()).sum())
    h = 1e-6
    for name, t, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*t.shape):
            tp, tm = t.clone(), t.clone()
            tp[idx] += h
            tm[idx] -= h
            args_p = {"q": (tp, k, v), "k": (q, tp, v), "v": (q, k, tp)}[name]
            args_m = {"q": (tm, k, v), "k": (q, tm, v), "v": (q, k, tm)}[name]
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def check_backward_closed_forms():
    """Softmax is invariant to a shift shared by all keys, so sum_j dK_j = 0 per
    KV head; and rows of P sum to 1, so sum_j dV_j = the sum of dO over the
    group's query rows."""
    B, H, Hk, Sq, Skv, D = 2, 4, 2, 9, 13, 8
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "f16", seed=870, h_kv=Hk)
    do = workloads.prefill_inputs(B, H, Sq, Sq, D, "f16", seed=871)[0]
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, causal=False)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    dos = do.double().numpy().reshape(B, Hk, H // Hk, Sq, D).sum(axis=(2, 3))
    _close(dv.sum(axis=2), dos, 1e-13, "sum of dV")


def check_backward_sampled_rows_autograd():
    """dQ at selected query rows and dK, dV at selected keys match autograd's
    full gradients (grouped heads, both layouts, causal with Sq != Skv)."""
    for n, (B, H, Hk, Sq, Skv, D, causal, layout) in enumerate(BWD_CASES):
        q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "bf16", layout, seed=890 + n, h_kv=Hk)
        do = workloads.prefill_inputs(B, H, Sq, Sq, D, "bf16", layout, seed=895 + n)[0]
        rdq, rdk, rdv = _autograd(q, k, v, do, causal, 0.4, layout)
        if layout == "BSHD":
            rdq, rdk, rdv = (x.transpose(0, 2, 1, 3) for x in (rdq, rdk, rdv))
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in (0, Sq // 2, Sq - 1)]
        keys = [(b, g, j) for b in range(B) for g in range(Hk) for j in (0, Skv // 3, Skv - 1)]
        got = oracle.sdpa_backward_dq_rows(q, k, v, do, rows, causal=causal, scale=0.4,
                                           layout=layout)
        _close(got, np.stack([rdq[b, h, i] for b, h, i in rows]), 1e-11, f"dq rows case {n}")
        gk, gv = oracle.sdpa_backward_kv_rows(q, k, v, do, keys, causal=causal, scale=0.4,
                                              layout=layout)
        _close(gk, np.stack([rdk[b, g, j] for b, g, j in keys]), 1e-11, f"dk rows case {n}")
        _close(gv, np.stack([rdv[b, g, j] for b, g, j in keys]), 1e-11, f"dv rows case {n}")


def check_lse_rows():
    B, H, Hk, Sq, Skv, D = 1, 2, 1, 6, 9, 8
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "f16", seed=880, h_kv=Hk)
    got = oracle.lse_rows(q, k, causal=True, scale=0.5)
    logits = 0.5 * (q.double() @ k.double().transpose(-1, -2))               # [1, 2, Sq, Skv]
    mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq)
    ref = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
    _close(got, ref, 1e-13, "lse rows")


ALL_CHECKS = [
    check_bruteforce, check_library_sdpa, check_rows_match_full, check_ones_v, check_causal_row0,
    check_zero_keys, check_two_keys, check_dominant_key, check_zero_scale,
    check_probs_rows_sum_to_one, check_logit_shift, check_permutations, check_layouts_agree,
    check_decode_library, check_decode_matches_prefill_row, check_decode_pool_permutation,
    check_decode_nan_poison, check_gqa_library, check_gqa_group_locality,
    check_gqa_rows_and_decode, check_extend_library, check_extend_without_prefix_is_causal_prefill,
    check_extend_one_token_is_decode, check_extend_chunking, check_fp8_decode,
    check_fp8_quantize_round_trip, check_backward_autograd, check_backward_finite_differences,
    check_backward_closed_forms, check_backward_sampled_rows_autograd, check_lse_rows,
]
