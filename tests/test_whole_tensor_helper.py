"""CPU checks of the whole-tensor comparison used by the full-size GPU tests:
slicing the oracle by (batch, head, row block) -- with the causal key cut --
by sequence and by KV-head group reproduces the oracle's whole result, every
element is compared exactly once, and a wrong or unwritten element is seen."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("Sq,Skv", [(70, 70), (50, 90), (90, 50), (33, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_slices_reproduce_whole_oracle(layout, Sq, Skv, causal):
    q, k, v = workloads.prefill_inputs(2, 4, Sq, Skv, 16, "f16", layout, seed=Sq + Skv, h_kv=2)
    full = torch.from_numpy(oracle.sdpa(q, k, v, causal=causal, scale=0.3, layout=layout))
    st = whole.compare(whole.prefill_units(q, k, v, ["o"], causal=causal, scale=0.3,
                                           layout=layout, row_block=16),
                       {"o": full}, workers=4)["o"]
    assert st.count == full.numel() and st.nonfinite == 0
    assert st.max_abs <= 1e-13 and st.rel_fro <= 1e-14, st


def test_compare_sees_a_wrong_and_an_unwritten_element():
    q, k, v = workloads.prefill_inputs(1, 2, 40, 40, 16, "f16", "BHSD", seed=3)
    full = torch.from_numpy(oracle.sdpa(q, k, v, causal=True, scale=0.25))
    bad = full.clone()
    bad[0, 1, 37, 5] += 0.02
    bad[0, 0, 39, 0] = float("nan")
    st = whole.compare(whole.prefill_units(q, k, v, ["o"], causal=True, scale=0.25,
                                           layout="BHSD", row_block=8), {"o": bad})["o"]
    assert st.nonfinite == 1
    assert abs(st.max_abs - 0.02) < 1e-12


def test_decode_and_extend_units_reproduce_whole_oracle():
    b = workloads.paged_decode_inputs(B=5, H=4, D=16, page_size=16, num_pages=64, seed=4,
                                      seq_lens=[1, 17, 40, 0, 100], h_kv=2)
    full = torch.from_numpy(oracle.paged_decode(b.q, b.k_cache, b.v_cache, b.page_table,
                                                b.seq_lens, scale=0.2))
    st = whole.compare(whole.decode_units(b, ["o"], scale=0.2), {"o": full})["o"]
    assert st.count == full.numel() and st.max_abs == 0.0
    e = workloads.extend_inputs(3, 4, 16, [20, 0, 33], [5, 9, 0], "f16", seed=5, h_kv=2)
    full = torch.from_numpy(oracle.extend(e.q, e.k, e.v, e.k_cache, e.v_cache, e.page_table,
                                          e.prefix_lens, e.qo_start, scale=0.2))
    st = whole.compare(whole.extend_units(e, ["o"], scale=0.2), {"o": full})["o"]
    assert st.count == full.numel() and st.max_abs == 0.0


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_backward_units_reproduce_whole_oracle(layout):
    q, k, v, do = workloads.backward_inputs(2, 4, 30, 45, 16, "f16", layout, seed=6, h_kv=2)
    dq, dk, dv = (torch.from_numpy(t) for t in
                  oracle.sdpa_backward(q, k, v, do, causal=True, scale=1 / math.sqrt(16),
                                       layout=layout))
    stats = whole.compare(whole.backward_units(q, k, v, do, causal=True,
                                               scale=1 / math.sqrt(16), layout=layout),
                          {"dq": dq, "dk": dk, "dv": dv})
    for name, st in stats.items():
        assert st.nonfinite == 0 and st.max_abs <= 1e-13 * max(st.max_ref, 1.0), (name, st)
    assert np.isclose(stats["dk"].max_ref, float(dk.abs().max()))
