"""fp64 reference attention (test infrastructure only; see the package docstring).

Every function here is the textbook definition written out, with no tiling,
no online softmax and no reordering: a row's logits are formed in full, the
row maximum is subtracted (which leaves softmax unchanged), exponentiated,
normalised and multiplied by V.  Query rows are processed in chunks only to
bound memory; rows are independent, so chunking changes nothing.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def to_f64(x) -> np.ndarray:
    """Exact upcast of an fp16/bf16/fp32/fp64 tensor or array to float64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    return x.detach().to("cpu").to(torch.float64).numpy()


def n_visible(Sq: int, Skv: int, causal: bool) -> np.ndarray:
    """Number of leading keys each query row may attend to.

    Non-causal: all Skv keys.  Causal, bottom-right aligned: query i sees keys
    j <= i + (Skv - Sq), i.e. ``i + Skv - Sq + 1`` keys, clipped to [0, Skv].
    When Sq == Skv this is the usual lower-triangular mask.
    """
    i = np.arange(Sq, dtype=np.int64)
    if not causal:
        return np.full(Sq, Skv, dtype=np.int64)
    return np.clip(i + (Skv - Sq) + 1, 0, Skv)


def attention_probs(q_rows: np.ndarray, keys: np.ndarray, scale: float,
                    visible: np.ndarray) -> np.ndarray:
    """Softmax weights P [n, Skv] of query rows [n, D] against keys [Skv, D].

    Row r attends to keys 0 .. visible[r]-1.  A row with no visible key gets
    all-zero weights (its output is defined as 0).
    """
    skv = keys.shape[0]
    logits = scale * (q_rows @ keys.T)
    mask = np.arange(skv)[None, :] < np.asarray(visible)[:, None]
    logits = np.where(mask, logits, -np.inf)
    row_max = logits.max(axis=1, keepdims=True) if skv else np.full((len(q_rows), 1), -np.inf)
    row_max = np.where(np.isfinite(row_max), row_max, 0.0)
    w = np.exp(logits - row_max)
    denom = w.sum(axis=1, keepdims=True)
    return np.divide(w, denom, out=np.zeros_like(w), where=denom > 0)


def attend_rows(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                visible: np.ndarray) -> np.ndarray:
    """O rows [n, D] = P @ V for query rows [n, D] (all float64)."""
    p = attention_probs(q_rows, keys, scale, visible)
    return p @ values


def kv_head(h: int, H: int, H_kv: int) -> int:
    """KV head read by query head h when H query heads share H_kv KV heads.

    The pages do not define grouped-query attention; this is its plain
    reading: consecutive query heads form groups of H / H_kv that share one KV
    head (H_kv = H is ordinary multi-head attention, H_kv = 1 multi-query).
    """
    if H_kv <= 0 or H % H_kv:
        raise ValueError(f"{H} query heads cannot share {H_kv} KV heads evenly")
    return h // (H // H_kv)


def _bhsd(x: np.ndarray, layout: str) -> np.ndarray:
    if layout == "BHSD":
        return x
    if layout == "BSHD":
        return x.transpose(0, 2, 1, 3)
    raise ValueError(f"unknown layout {layout!r}")


def sdpa(q, k, v, *, causal: bool, scale: float | None = None, layout: str = "BHSD",
         chunk: int = 2048) -> np.ndarray:
    """Full attention output in float64, in the inputs' layout.

    q: [B,H,Sq,D] (BHSD) or [B,Sq,H,D] (BSHD); k, v likewise with Skv keys
    and H_kv heads (H_kv divides H; see ``kv_head``).
    """
    qf, kf, vf = (_bhsd(to_f64(t), layout) for t in (q, k, v))
    B, H, Sq, D = qf.shape
    H_kv, Skv = kf.shape[1], kf.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    out = np.zeros((B, H, Sq, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, chunk):
                r1 = min(Sq, r0 + chunk)
                g = kv_head(h, H, H_kv)
                out[b, h, r0:r1] = attend_rows(qf[b, h, r0:r1], kf[b, g], vf[b, g], scale, vis[r0:r1])
    return _bhsd(out, layout)


def sdpa_rows(q, k, v, rows, *, causal: bool, scale: float | None = None,
              layout: str = "BHSD") -> np.ndarray:
    """Attention output [len(rows), D] for selected query rows ``(b, h, i)``.

    Used at full problem size, where the whole output is too costly for the
    CPU: each selected row is computed exactly as ``sdpa`` would.
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        H_kv, Skv = k.shape[1], k.shape[2]

        def head(t, b, h):
            return t[b, h]
    elif layout == "BSHD":
        B, Sq, H, D = q.shape
        Skv, H_kv = k.shape[1], k.shape[2]

        def head(t, b, h):
            return t[b, :, h]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    out = np.zeros((len(rows), D), dtype=np.float64)
    groups: dict = {}
    for n, (b, h, i) in enumerate(rows):
        groups.setdefault((b, h), []).append((n, i))
    for (b, h), items in groups.items():
        kf = to_f64(head(k, b, kv_head(h, H, H_kv)))
        vf = to_f64(head(v, b, kv_head(h, H, H_kv)))
        qh = head(q, b, h)
        idx = np.array([i for _, i in items])
        qf = to_f64(qh[torch.as_tensor(idx)] if isinstance(qh, torch.Tensor) else qh[idx])
        res = attend_rows(qf, kf, vf, scale, vis[idx])
        for (n, _), r in zip(items, res):
            out[n] = r
    return out


def gather_sequence(cache, page_row, n_tokens: int, page_size: int):
    """Token-major [n_tokens, H, D] view of one sequence in a paged cache.

    Token t lives in page ``page_row[t // page_size]`` at slot ``t % page_size``;
    only the first ceil(n_tokens / page_size) page-table entries are read.
    """
    n_pages = -(-n_tokens // page_size)
    pages = torch.as_tensor(np.asarray(page_row[:n_pages], dtype=np.int64))
    sel = cache[pages]                       # [n_pages, page_size, H, D]
    return sel.reshape(n_pages * page_size, *sel.shape[2:])[:n_tokens]


def paged_decode(q, k_cache, v_cache, page_table, seq_lens, *, scale: float | None = None,
                 batch_indices=None) -> np.ndarray:
    """Decode attention (one query per sequence) through a page table, float64.

    q: [B, H, D]; k_cache, v_cache: [num_pages, page_size, H_kv, D] (H_kv
    divides H; see ``kv_head``); page_table: [B, max_pages] int; seq_lens: [B]
    int.  Returns [B, H, D] (or [len(batch_indices), H, D]).
    """
    B, H, D = q.shape
    page_size, H_kv = int(k_cache.shape[1]), int(k_cache.shape[2])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    table = np.asarray(page_table.cpu() if isinstance(page_table, torch.Tensor) else page_table)
    lens = np.asarray(seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens)
    bs = range(B) if batch_indices is None else list(batch_indices)
    out = np.zeros((len(bs), H, D), dtype=np.float64)
    for n_out, b in enumerate(bs):
        n = int(lens[b])
        kf = to_f64(gather_sequence(k_cache, table[b], n, page_size))   # [n, H, D]
        vf = to_f64(gather_sequence(v_cache, table[b], n, page_size))
        qf = to_f64(q[b])                                                # [H, D]
        for h in range(H):
            g = kv_head(h, H, H_kv)
            out[n_out, h] = attend_rows(qf[h:h + 1], kf[:, g], vf[:, g], scale,
                                        np.array([n]))[0]
    return out


def extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, *,
           scale: float | None = None, seqs=None) -> np.ndarray:
    """Extend attention (prefill of new tokens after a cached prefix), float64.

    Sequence b has prefix_lens[b] tokens in the paged cache (read through
    page_table[b] like paged decode) and E_b = qo_start[b+1] - qo_start[b] new
    tokens, packed token-major in q [T, H, D] and k, v [T, H_kv, D] at rows
    qo_start[b] .. qo_start[b+1]-1.  New token i attends to every prefix token
    and to new tokens 0..i: causal attention over the concatenated sequence
    (prefix, then new), bottom-right aligned.  Returns o [T, H, D] (rows of
    sequences not in ``seqs`` stay zero).
    """
    T, H, D = q.shape
    page_size, H_kv = int(k_cache.shape[1]), int(k_cache.shape[2])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    as_np = lambda t: np.asarray(t.cpu() if isinstance(t, torch.Tensor) else t)
    table, plen, starts = as_np(page_table), as_np(prefix_lens), as_np(qo_start)
    out = np.zeros((T, H, D), dtype=np.float64)
    for b in (range(len(plen)) if seqs is None else seqs):
        P, r0, r1 = int(plen[b]), int(starts[b]), int(starts[b + 1])
        E = r1 - r0
        keys = np.concatenate([to_f64(gather_sequence(k_cache, table[b], P, page_size)),
                               to_f64(k[r0:r1])])                       # [P + E, H_kv, D]
        vals = np.concatenate([to_f64(gather_sequence(v_cache, table[b], P, page_size)),
                               to_f64(v[r0:r1])])
        qf = to_f64(q[r0:r1])                                            # [E, H, D]
        vis = n_visible(E, P + E, causal=True)
        for h in range(H):
            g = kv_head(h, H, H_kv)
            out[r0:r1, h] = attend_rows(qf[:, h], keys[:, g], vals[:, g], scale, vis)
    return out


def dequantize_fp8(codes, descale: float) -> np.ndarray:
    """float64 values of e4m3fn codes (a torch.float8_e4m3fn tensor) times the
    per-tensor descale: the inputs an fp8 attention computes with."""
    return codes.detach().to("cpu").to(torch.float64).numpy() * float(descale)


def lse_rows(q, k, *, causal: bool, scale: float | None = None, layout: str = "BHSD") -> np.ndarray:
    """Natural log-sum-exp of each query row's scaled, masked logits [B, H, Sq]
    (-inf for a row with no visible key): log sum_j exp(scale <q_i, k_j> + M_ij)."""
    qf, kf = (_bhsd(to_f64(t), layout) for t in (q, k))
    B, H, Sq, D = qf.shape
    H_kv, Skv = kf.shape[1], kf.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    mask = np.arange(Skv)[None, :] < vis[:, None]
    out = np.full((B, H, Sq), -np.inf)
    for b in range(B):
        for h in range(H):
            logits = np.where(mask, scale * (qf[b, h] @ kf[b, kv_head(h, H, H_kv)].T), -np.inf)
            m = logits.max(axis=1) if Skv else np.full(Sq, -np.inf)
            ok = np.isfinite(m)
            out[b, h, ok] = m[ok] + np.log(np.exp(logits[ok] - m[ok, None]).sum(axis=1))
    return out


def sdpa_backward(q, k, v, do, *, causal: bool, scale: float | None = None,
                  layout: str = "BHSD"):
    """Gradients (dq, dk, dv) of L = sum(O * dO) for O = sdpa(q, k, v), float64,
    in the inputs' layout, from the chain rule written out:
        P = softmax rows,   dV_j = sum_i P_ij dO_i,   dP_ij = <dO_i, V_j>,
        dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
        dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i.
    Grouped heads: dK and dV of a KV head sum over the query heads sharing it."""
    qf, kf, vf, gf = (_bhsd(to_f64(t), layout) for t in (q, k, v, do))
    B, H, Sq, D = qf.shape
    H_kv, Skv = kf.shape[1], kf.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            P = attention_probs(qf[b, h], kf[b, g], scale, vis)       # [Sq, Skv]
            dv[b, g] += P.T @ gf[b, h]
            dP = gf[b, h] @ vf[b, g].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ kf[b, g])
            dk[b, g] += scale * (dS.T @ qf[b, h])
    return _bhsd(dq, layout), _bhsd(dk, layout), _bhsd(dv, layout)


def _head_getter(layout: str):
    if layout == "BHSD":
        return lambda t, b, h: t[b, h]
    if layout == "BSHD":
        return lambda t, b, h: t[b, :, h]
    raise ValueError(f"unknown layout {layout!r}")


def sdpa_backward_dq_rows(q, k, v, do, rows, *, causal: bool, scale: float | None = None,
                          layout: str = "BHSD") -> np.ndarray:
    """dQ [len(rows), D] at selected query rows ``(b, h, i)``, each exactly as
    ``sdpa_backward`` forms it: the row's P and dP_ij = <dO_i, V_j> over all
    keys, dS_ij = P_ij (dP_ij - sum_l P_il dP_il), dQ_i = scale sum_j dS_ij K_j.
    For full problem sizes, where the whole gradient is too costly here."""
    head = _head_getter(layout)
    B, H, Sq, D = _bhsd_shape(q, layout)
    H_kv, Skv = _bhsd_shape(k, layout)[1:3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    out = np.zeros((len(rows), D), dtype=np.float64)
    groups: dict = {}
    for n, (b, h, i) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append((n, int(i)))
    for (b, h), items in groups.items():
        g = kv_head(h, H, H_kv)
        kf, vf = to_f64(head(k, b, g)), to_f64(head(v, b, g))
        idx = torch.as_tensor([i for _, i in items])
        qr = to_f64(head(q, b, h)[idx])
        dor = to_f64(head(do, b, h)[idx])
        P = attention_probs(qr, kf, scale, vis[idx.numpy()])
        dP = dor @ vf.T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        for (n, _), r in zip(items, scale * (dS @ kf)):
            out[n] = r
    return out


def sdpa_backward_kv_rows(q, k, v, do, keys, *, causal: bool, scale: float | None = None,
                          layout: str = "BHSD"):
    """(dK, dV), each [len(keys), D], at selected keys ``(b, g, j)`` of KV head
    g, exactly as ``sdpa_backward`` forms them: sums over every query row of
    every query head sharing KV head g of dV_j = P_ij dO_i and
    dK_j = scale dS_ij Q_i.  For full problem sizes."""
    head = _head_getter(layout)
    B, H, Sq, D = _bhsd_shape(q, layout)
    H_kv, Skv = _bhsd_shape(k, layout)[1:3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    vis = n_visible(Sq, Skv, causal)
    dk = np.zeros((len(keys), D), dtype=np.float64)
    dv = np.zeros((len(keys), D), dtype=np.float64)
    groups: dict = {}
    for n, (b, g, j) in enumerate(keys):
        groups.setdefault((int(b), int(g)), []).append((n, int(j)))
    for (b, g), items in groups.items():
        kf, vf = to_f64(head(k, b, g)), to_f64(head(v, b, g))
        js = np.array([j for _, j in items])
        for h in range(H):
            if kv_head(h, H, H_kv) != g:
                continue
            qf, dof = to_f64(head(q, b, h)), to_f64(head(do, b, h))
            P = attention_probs(qf, kf, scale, vis)                   # [Sq, Skv]
            dP = dof @ vf.T
            delta = (P * dP).sum(axis=1, keepdims=True)
            dS = P[:, js] * (dP[:, js] - delta)
            del dP
            for t, (n, _) in enumerate(items):
                dv[n] += P[:, js[t]] @ dof
                dk[n] += scale * (dS[:, t] @ qf)
    return dk, dv


def _bhsd_shape(t, layout: str) -> tuple:
    """(B, heads, S, D) of a BHSD or BSHD tensor."""
    if layout == "BHSD":
        return tuple(t.shape)
    if layout == "BSHD":
        B, S, H, D = t.shape
        return (B, H, S, D)
    raise ValueError(f"unknown layout {layout!r}")
