"""scale = 0 through every entry point: softmax(0) is uniform over each row's
visible keys, so O is the plain mean of the visible V rows (0 for a row with
none), the LSE is ln(number of visible keys), and dQ = dK = 0.  Masked scores
(causal, ragged tails, past a sequence's end) must stay out of the mean --
they enter the exponent as -inf times a zero multiplier, which would be NaN.
Checked against the fp64 oracle at scale 0."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.double().cpu().numpy()


@pytest.mark.parametrize("Sq,Skv,causal", [(200, 333, True), (333, 200, True), (129, 77, False)])
def test_prefill_scale_zero(gpu_lib, Sq, Skv, causal):
    q, k, v = workloads.prefill_inputs(1, 4, Sq, Skv, 128, "bf16", "BSHD", seed=Sq + Skv)
    print(f"[case] prefill scale 0 Sq{Sq} Skv{Skv} causal={causal}", flush=True)
    o, lse = gpu_lib.prefill_with_lse(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=0.0,
                                      layout="BSHD")
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, causal=causal, scale=0.0, layout="BSHD")
    assert_parity(_f64(o), ref, f"prefill scale 0 {Sq}x{Skv} causal={causal}")
    # visible keys per row: Skv, or min(Skv, i + 1 + Skv - Sq) under the bottom-right mask
    i = np.arange(Sq)
    n = np.clip(i + 1 + Skv - Sq, 0, Skv) if causal else np.full(Sq, Skv)
    want = np.where(n > 0, np.log(np.maximum(n, 1)), -np.inf)
    got = lse.cpu().double().numpy()  # [B, H, Sq]
    assert np.array_equal(np.isinf(got[0]), np.broadcast_to(np.isinf(want), got[0].shape))
    fin = np.isfinite(want)
    assert np.allclose(got[0][:, fin], want[fin], rtol=1e-5, atol=1e-5)


def test_backward_scale_zero(gpu_lib):
    q, k, v, do = workloads.backward_inputs(1, 4, 150, 260, 128, "f16", "BHSD", amp=0.5,
                                            seed=97, h_kv=2)
    print("[case] backward scale 0", flush=True)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, causal=True, scale=0.0)
    dq, dk, dv = gpu_lib.prefill_backward(qg, kg, vg, o, dog, lse, causal=True, scale=0.0)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.sdpa_backward(q, k, v, do, causal=True, scale=0.0)
    assert np.abs(rq).max() == 0 and np.abs(rk).max() == 0
    assert torch.count_nonzero(dq) == 0 and torch.count_nonzero(dk) == 0
    big = float(np.abs(rv).max())
    assert_parity(_f64(dv), rv, "dv scale 0", max_abs_tol=2e-3 * big, rel_fro_tol=1e-3)


@pytest.mark.parametrize("H,H_kv", [(8, 8), (8, 2), (32, 1)])
def test_decode_scale_zero(gpu_lib, H, H_kv):
    lens = [1, 17, 0, 700, 64, 1000]
    batch = workloads.paged_decode_inputs(B=len(lens), H=H, D=128, page_size=16, num_pages=256,
                                          seq_lens=lens, seed=98 + H_kv, h_kv=H_kv)
    print(f"[case] decode scale 0 H{H}/{H_kv}", flush=True)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    o = gpu_lib.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                             scale=0.0)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, scale=0.0)
    assert_parity(_f64(o), ref, f"decode scale 0 H{H}/{H_kv}")
    assert torch.count_nonzero(o[2]) == 0


def test_extend_scale_zero(gpu_lib):
    batch = workloads.extend_inputs(3, 8, 128, [40, 0, 130], [30, 17, 70], "f16", seed=99,
                                    h_kv=2)
    print("[case] extend scale 0", flush=True)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache",
                                              "page_table", "prefix_lens", "qo_start")}
    o = gpu_lib.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                       g["prefix_lens"], g["qo_start"], scale=0.0)
    torch.cuda.synchronize()
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, scale=0.0)
    assert_parity(_f64(o), ref, "extend scale 0")
