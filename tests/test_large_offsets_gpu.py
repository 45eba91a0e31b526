"""Tensors past 2^31 elements (byte offsets past 4 GiB): prefill in both
layouts, causal and not, the backward, and extend, checked against the oracle
on the heads (or sequences) whose data lies around the 2^30- and
2^31-element marks and at the very end.  Inputs are drawn on the device by a
seeded generator (see workloads.device_normal); the oracle takes the checked
slices copied back.  Paged decode reaches byte offsets past 4 GiB in its
full-size workload (an 8 GiB page pool) already."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu

B, H, S, D = 1040, 128, 128, 128  # 2.18e9 elements per tensor (4.36 GB in 16-bit types)


def _picks():
    """(b, h) pairs around element offsets 2^30 and 2^31 (the int32 byte and
    element boundaries) and the last head."""
    per_head = S * D
    marks = [(1 << 30) // per_head, (1 << 31) // per_head]
    heads = sorted({m + d for m in marks for d in (-1, 0)} | {B * H - 1})
    return [(x // H, x % H) for x in heads]


# The backward's bar for bf16 gradients, relative to the largest reference
# value (derived from a CPU model of the kernels' rounding; see the docstring
# of test_backward_gpu.py): max-abs <= 1e-2 * max|ref|, rel_fro <= 6e-3.
BWD_BF16_TOL = (1e-2, 6e-3)


def _slice(t, b, h, layout):
    return (t[b:b + 1, h:h + 1] if layout == "BHSD" else t[b:b + 1, :, h:h + 1]).cpu()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_past_2g_elements(gpu_lib, layout, causal):
    shape = workloads.layout_shape(B, H, S, D, layout)
    print(f"[case] large prefill {shape} {layout} causal={causal}", flush=True)
    q = workloads.device_normal(shape, "f16", seed=401)
    k = workloads.device_normal(shape, "f16", seed=402)
    v = workloads.device_normal(shape, "f16", seed=403)
    o = torch.full_like(q, float("nan"))
    gpu_lib.prefill(q, k, v, causal=causal, layout=layout, out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "output not fully written"
    for b, h in _picks():
        ref = oracle.sdpa(_slice(q, b, h, layout), _slice(k, b, h, layout), _slice(v, b, h, layout),
                          causal=causal, layout=layout)
        assert_parity(_slice(o, b, h, layout).double().numpy(), ref,
                      f"prefill {layout} causal={causal} head ({b}, {h})")
    del q, k, v, o
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_backward_past_2g_elements(gpu_lib):
    layout = "BSHD"
    shape = workloads.layout_shape(B, H, S, D, layout)
    print(f"[case] large backward {shape} {layout} causal", flush=True)
    q = workloads.device_normal(shape, "bf16", seed=411, amp=0.5)
    k = workloads.device_normal(shape, "bf16", seed=412, amp=0.5)
    v = workloads.device_normal(shape, "bf16", seed=413, amp=0.5)
    do = workloads.device_normal(shape, "bf16", seed=414)
    o, lse = gpu_lib.prefill_with_lse(q, k, v, causal=True, layout=layout)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    gpu_lib.prefill_backward(q, k, v, o, do, lse, causal=True, layout=layout, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} not fully written"
    for b, h in _picks():
        refs = oracle.sdpa_backward(_slice(q, b, h, layout), _slice(k, b, h, layout),
                                    _slice(v, b, h, layout), _slice(do, b, h, layout),
                                    causal=True, layout=layout)
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            big = max(float(np.abs(ref).max()), 1e-3)
            assert_parity(_slice(got, b, h, layout).double().numpy(), ref,
                          f"backward {name} head ({b}, {h})",
                          max_abs_tol=BWD_BF16_TOL[0] * big, rel_fro_tol=BWD_BF16_TOL[1])
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_extend_past_2g_elements(gpu_lib):
    """4200 sequences of 128 new tokens and no prefix, 32 query heads: q and o
    hold 2.2e9 elements.  Each sequence's rows equal causal attention over its
    own tokens."""
    nseq, E, Hq, Hkv = 4200, 128, 32, 8
    T = nseq * E
    print(f"[case] large extend T{T} H{Hq}/{Hkv}", flush=True)
    q = workloads.device_normal((T, Hq, D), "bf16", seed=421)
    k = workloads.device_normal((T, Hkv, D), "bf16", seed=422)
    v = workloads.device_normal((T, Hkv, D), "bf16", seed=423)
    cache = torch.zeros((1, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((nseq, 1), dtype=torch.int32, device="cuda")
    plen = torch.zeros(nseq, dtype=torch.int32, device="cuda")
    starts = torch.arange(0, T + 1, E, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, float("nan"))
    gpu_lib.extend(q, k, v, cache, cache, table, plen, starts, max_extend_len=E, out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "output not fully written"
    per_seq = E * Hq * D
    seqs = sorted({(1 << 30) // per_seq, (1 << 31) // per_seq - 1, (1 << 31) // per_seq,
                   nseq - 1})
    for s in seqs:
        r = slice(s * E, (s + 1) * E)
        # [T, H, D] rows of one sequence are its BSHD tensor with B = 1
        ref = oracle.sdpa(q[r].unsqueeze(0).cpu(), k[r].unsqueeze(0).cpu(), v[r].unsqueeze(0).cpu(),
                          causal=True, layout="BSHD")[0]
        assert_parity(o[r].cpu().double().numpy(), ref, f"extend sequence {s}")
    del q, k, v, o
    torch.cuda.empty_cache()
