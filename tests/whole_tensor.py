"""Whole-tensor comparison of full-size GPU results with the fp64 oracle.

Attention is independent per (batch, query head) and per query row, so the
oracle is called on slices of the inputs -- one (batch, head) and a block of
query rows, one decode or extend sequence, one (batch, KV head) group for the
backward -- and every slice's result is compared with the matching slice of
the GPU output.  Together the slices cover every element of the output.

For causal prefill a block of query rows [r0, r1) is passed with the keys
[0, r1 + Skv - Sq) only.  Under the bottom-right alignment the slice's row
i' sees keys j <= i' + (r1 + Skv - Sq) - (r1 - r0) = (r0 + i') + Skv - Sq,
exactly the keys row r0 + i' sees in the whole problem, and the keys left
out are invisible to every row of the block.

The slices run on a pool of threads (numpy releases the interpreter lock in
its array loops and matrix products; each thread's BLAS is held to one
thread).  Errors are accumulated over the whole output: max-abs, relative
Frobenius sqrt(sum diff^2 / sum ref^2), the largest |ref| (the gradients'
bars are relative to it) and the count of non-finite GPU values.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle


class Stats:
    def __init__(self):
        self.max_abs = 0.0
        self.sum_d2 = 0.0
        self.sum_r2 = 0.0
        self.max_ref = 0.0
        self.nonfinite = 0
        self.count = 0

    def add(self, got, ref):
        g = np.asarray(got, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        assert g.shape == r.shape, (g.shape, r.shape)
        bad = ~np.isfinite(g)
        self.nonfinite += int(bad.sum())
        d = np.where(bad, 0.0, g - r)
        if d.size:
            self.max_abs = max(self.max_abs, float(np.abs(d).max()))
            self.max_ref = max(self.max_ref, float(np.abs(r).max()))
        self.sum_d2 += float((d * d).sum())
        self.sum_r2 += float((r * r).sum())
        self.count += g.size

    @property
    def rel_fro(self):
        return math.sqrt(self.sum_d2 / self.sum_r2) if self.sum_r2 > 0 else math.sqrt(self.sum_d2)

    def __repr__(self):
        return (f"max_abs={self.max_abs:.3e} rel_fro={self.rel_fro:.3e} "
                f"max|ref|={self.max_ref:.3e} nonfinite={self.nonfinite} of {self.count}")


def default_workers():
    return max(1, min(16, os.cpu_count() or 1))


def compare(units, outputs, workers=None, progress=None, every_s=20.0):
    """Run every unit (a callable returning [(name, index, ref), ...]) and
    compare ``outputs[name][index]`` (CPU tensors) with ``ref``.  Returns
    {name: Stats}.  ``progress`` (if given) receives a line about every
    ``every_s`` seconds with the units compared so far."""
    import time
    from threadpoolctl import threadpool_limits
    stats = {name: Stats() for name in outputs}
    t0 = last = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers or default_workers()) as ex:
        # map yields in order and drops each result once yielded, so at most
        # the results that finished ahead of the one awaited are held at once
        for n, res in enumerate(ex.map(lambda u: u(), units), 1):
            for name, index, ref in res:
                stats[name].add(outputs[name][index].double().numpy(), ref)
            now = time.perf_counter()
            if progress is not None and now - last >= every_s:
                progress(f"[whole] {n}/{len(units)} oracle slices compared, {now - t0:.0f} s")
                last = now
    covered = {name: s.count for name, s in stats.items()}
    for name, out in outputs.items():
        assert covered[name] == out.numel(), f"{name}: compared {covered[name]} of {out.numel()}"
    return stats


def prefill_units(q, k, v, names, *, causal, scale, layout, row_block=1024):
    """Units over (batch, query head, block of query rows) for oracle.sdpa.
    q, k, v: CPU tensors (or float64 arrays) in ``layout``."""
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        H_kv, Skv = k.shape[1], k.shape[2]
    else:
        B, Sq, H, D = q.shape
        Skv, H_kv = k.shape[1], k.shape[2]
    units = []
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head(h, H, H_kv)
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                kend = min(Skv, max(0, r1 + Skv - Sq)) if causal else Skv

                def unit(b=b, h=h, g=g, r0=r0, r1=r1, kend=kend):
                    if layout == "BHSD":
                        qs, ks, vs = q[b:b + 1, h:h + 1, r0:r1], k[b:b + 1, g:g + 1, :kend], \
                            v[b:b + 1, g:g + 1, :kend]
                        index = (b, h, slice(r0, r1))
                    else:
                        qs, ks, vs = q[b:b + 1, r0:r1, h:h + 1], k[b:b + 1, :kend, g:g + 1], \
                            v[b:b + 1, :kend, g:g + 1]
                        index = (b, slice(r0, r1), h)
                    ref = oracle.sdpa(qs, ks, vs, causal=causal, scale=scale, layout=layout)
                    ref = ref.reshape(r1 - r0, D)
                    return [(n, index, ref) for n in names]
                units.append(unit)
    return units


def decode_units(batch, names, *, scale):
    """Units over the sequences of a paged-decode batch (oracle.paged_decode)."""
    units = []
    for b in range(batch.q.shape[0]):
        def unit(b=b):
            ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                                      batch.seq_lens, scale=scale, batch_indices=[b])[0]
            return [(n, b, ref) for n in names]
        units.append(unit)
    return units


def extend_units(batch, names, *, scale):
    """Units over the sequences of an extend batch (oracle.extend, one
    sequence at a time); each covers the sequence's new-token rows."""
    starts = batch.qo_start.tolist()
    units = []
    for b in range(len(starts) - 1):
        def unit(b=b):
            r0, r1 = starts[b], starts[b + 1]
            ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                                batch.page_table, batch.prefix_lens, batch.qo_start, scale=scale,
                                seqs=[b])[r0:r1]
            return [(n, slice(r0, r1), ref) for n in names]
        units.append(unit)
    return units


def backward_units(q, k, v, do, *, causal, scale, layout):
    """Units over (batch, KV head) for oracle.sdpa_backward: the KV head's
    query heads (consecutive, see oracle.kv_head) with their q and dO rows.
    Outputs are named "dq", "dk", "dv"."""
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        H_kv = k.shape[1]
    else:
        B, Sq, H, D = q.shape
        H_kv = k.shape[2]
    group = H // H_kv
    units = []
    for b in range(B):
        for g in range(H_kv):
            h0, h1 = g * group, (g + 1) * group
            assert all(oracle.kv_head(h, H, H_kv) == g for h in range(h0, h1))

            def unit(b=b, g=g, h0=h0, h1=h1):
                if layout == "BHSD":
                    sl_q, sl_k = (slice(b, b + 1), slice(h0, h1)), (slice(b, b + 1), slice(g, g + 1))
                    iq, ik = (b, slice(h0, h1)), (b, g)
                else:
                    sl_q = (slice(b, b + 1), slice(None), slice(h0, h1))
                    sl_k = (slice(b, b + 1), slice(None), slice(g, g + 1))
                    iq, ik = (b, slice(None), slice(h0, h1)), (b, slice(None), g)
                dq, dk, dv = oracle.sdpa_backward(q[sl_q], k[sl_k], v[sl_k], do[sl_q],
                                                  causal=causal, scale=scale, layout=layout)
                kv_shape = (dk.shape[2], D) if layout == "BHSD" else (dk.shape[1], D)
                return [("dq", iq, dq[0]), ("dk", ik, dk.reshape(kv_shape)),
                        ("dv", ik, dv.reshape(kv_shape))]
            units.append(unit)
    return units


def nan_like(t, dtype=None, device="cuda"):
    """A NaN-filled GPU tensor shaped like t (an output buffer: rows the
    kernel fails to write stay NaN and are counted as non-finite)."""
    return torch.full(tuple(t.shape), float("nan"), dtype=dtype or t.dtype, device=device)
