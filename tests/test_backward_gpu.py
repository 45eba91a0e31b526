"""GPU parity of the attention backward (attn_prefill_bwd, fed the LSE that
attn_prefill_lse writes) through the C ABI against the fp64 oracle's
gradients (oracle.sdpa_backward, and its sampled rows at full size).

Tolerances.  The gradients' scale differs from O's, so the bar is relative
to the largest reference value.  A CPU model of the kernels' rounding
(inputs and O in the storage type, P and dS rounded to it as MFMA operands,
fp32 sums, gradients rounded to the storage type) was compared with the
oracle at S = 1k..8k, D = 64 and 128, causal and not.  Its worst errors were
rel_fro 3.0e-4 and max-abs 6e-4 * max|ref| in fp16, and 2.45e-3 and
3.9e-3 * max|ref| in bf16.  The bars are about 2.5x those:
    fp16: rel_fro <= 1e-3,  max_abs <= 2e-3 * max|ref|
    bf16: rel_fro <= 6e-3,  max_abs <= 1e-2 * max|ref|
The LSE is compared to oracle.lse_rows with -inf at exactly the rows that see
no key, and within 1e-3 + 1e-6 |lse| elsewhere: the forward's row sum adds
the fp16-rounded probabilities (the values its O numerator uses), each within
2^-11 relative, so the sum, and the log of it, is off by at most 2^-11 =
4.9e-4, plus fp32 rounding of the logits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import assert_parity

pytestmark = pytest.mark.gpu

TOL = {"f16": (2e-3, 1e-3), "bf16": (1e-2, 6e-3)}  # (max_abs / max|ref|, rel_fro)


def _f64(t):
    return t.double().cpu().numpy()


def _check_grad(got, ref, dtype, what):
    ref = np.asarray(ref, dtype=np.float64)
    big = max(float(np.abs(ref).max()) if ref.size else 0.0, 1e-3)
    assert_parity(got, ref, what, max_abs_tol=TOL[dtype][0] * big, rel_fro_tol=TOL[dtype][1])


def _run(attn, q, k, v, do, causal, layout, grad_dtype=None, scale=None):
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.prefill_with_lse(qg, kg, vg, causal=causal, layout=layout, scale=scale)
    grads = attn.prefill_backward(qg, kg, vg, o, dog, lse, causal=causal, layout=layout,
                                  grad_dtype=grad_dtype, scale=scale)
    torch.cuda.synchronize()
    return o, lse, grads


SHAPES = [(200, 333), (333, 200), (64, 64), (1, 1), (129, 77), (300, 300)]
HEADS = [(2, 2), (8, 2), (4, 1)]
COMBOS = [("f16", "BHSD", False), ("bf16", "BSHD", True), ("f16", "BSHD", True),
          ("bf16", "BHSD", False)]


@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: f"{c[0]}-{c[1]}-{'causal' if c[2] else 'full'}")
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape_i", range(len(SHAPES)))
def test_backward_parity(gpu_lib, combo, D, shape_i):
    dtype, layout, causal = combo
    Sq, Skv = SHAPES[shape_i]
    H, H_kv = HEADS[shape_i % len(HEADS)]
    print(f"[case] backward B2 H{H}/{H_kv} Sq{Sq} Skv{Skv} D{D} {dtype} {layout} "
          f"causal={causal}", flush=True)
    q, k, v, do = workloads.backward_inputs(2, H, Sq, Skv, D, dtype, layout, amp=0.5,
                                            seed=100 + shape_i * 7 + D, h_kv=H_kv)
    _, lse, (dq, dk, dv) = _run(gpu_lib, q, k, v, do, causal, layout)
    ref = oracle.sdpa_backward(q, k, v, do, causal=causal, layout=layout)
    tag = f"H{H}/{H_kv} {Sq}x{Skv} D{D} {dtype} {layout} causal={causal}"
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check_grad(_f64(g), r, dtype, f"{name} {tag}")


@pytest.mark.parametrize("causal,Sq,Skv", [(False, 200, 333), (True, 333, 200), (True, 300, 300),
                                           (False, 1, 1), (True, 70, 64)])
@pytest.mark.parametrize("dtype,layout", [("f16", "BHSD"), ("bf16", "BSHD")])
def test_prefill_lse(gpu_lib, causal, Sq, Skv, dtype, layout):
    print(f"[case] lse {Sq}x{Skv} {dtype} {layout} causal={causal}", flush=True)
    q, k, v = workloads.prefill_inputs(2, 8, Sq, Skv, 128, dtype, layout, seed=Sq + Skv, h_kv=2)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, causal=causal, layout=layout)
    o_plain = gpu_lib.prefill(qg, kg, vg, causal=causal, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)  # the LSE output changes nothing else
    got = lse.double().cpu().numpy()
    ref = oracle.lse_rows(q, k, causal=causal, layout=layout)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all()
    err = np.abs(got[fin] - ref[fin])
    print(f"[parity] lse max_abs={err.max() if err.size else 0:.3e}", flush=True)
    assert (err <= 1e-3 + 1e-6 * np.abs(ref[fin])).all()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_fp32_gradients_round_to_the_storage_type(gpu_lib, dtype):
    """The fp32 gradients, rounded to the input type, are bitwise the gradients
    in the input type (same accumulators, only the store differs), and they
    meet the same bar."""
    q, k, v, do = workloads.backward_inputs(2, 8, 250, 190, 128, dtype, "BSHD", amp=0.5,
                                            seed=41, h_kv=2)
    print(f"[case] backward fp32 gradients {dtype}", flush=True)
    _, _, g16 = _run(gpu_lib, q, k, v, do, True, "BSHD")
    _, _, g32 = _run(gpu_lib, q, k, v, do, True, "BSHD", grad_dtype=torch.float32)
    ref = oracle.sdpa_backward(q, k, v, do, causal=True, layout="BSHD")
    for name, a, b, r in zip(("dq", "dk", "dv"), g16, g32, ref):
        assert b.dtype == torch.float32
        assert torch.equal(a, b.to(a.dtype)), name
        _check_grad(_f64(b), r, dtype, f"{name} fp32")


def test_backward_is_deterministic(gpu_lib):
    q, k, v, do = workloads.backward_inputs(1, 8, 700, 700, 128, "bf16", "BHSD", amp=0.5,
                                            seed=43, h_kv=2)
    print("[case] backward determinism", flush=True)
    _, _, a = _run(gpu_lib, q, k, v, do, True, "BHSD")
    _, _, b = _run(gpu_lib, q, k, v, do, True, "BHSD")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("Sq,Skv", [(0, 100), (100, 0), (0, 0)])
def test_backward_empty_sides(gpu_lib, Sq, Skv):
    """No queries: dk, dv are written as zeros; no keys: dq is zeros."""
    q, k, v, do = workloads.backward_inputs(2, 4, Sq, Skv, 64, "f16", "BHSD", seed=45, h_kv=2)
    print(f"[case] backward empty Sq={Sq} Skv={Skv}", flush=True)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, causal=False)
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = gpu_lib.prefill_backward(qg, kg, vg, o, dog, lse, dq=nan(qg), dk=nan(kg),
                                          dv=nan(vg))
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t) == 0


def test_backward_writes_every_row(gpu_lib):
    """Gradients pre-filled with NaN come back finite (causal, Sq > Skv: the
    first rows see no key and get dq = 0)."""
    q, k, v, do = workloads.backward_inputs(2, 4, 300, 130, 128, "bf16", "BSHD", amp=0.5,
                                            seed=47, h_kv=1)
    print("[case] backward writes every row", flush=True)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, causal=True, layout="BSHD")
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = gpu_lib.prefill_backward(qg, kg, vg, o, dog, lse, causal=True, layout="BSHD",
                                          dq=nan(qg), dk=nan(kg), dv=nan(vg))
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    assert torch.count_nonzero(dq[:, :170]) == 0   # rows 0..169 see no key


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [11, 12])
def test_backward_full_size_whole(gpu_lib, cfg, progress):
    """The 8k causal BSHD backward at full size (32 query heads; and with
    four query heads per KV head), in the bench's launch configuration:
    gradients written into NaN-prefilled buffers and compared with the
    oracle over the whole of dq, dk and dv."""
    attn = gpu_lib
    q, k, v, do, m = workloads.backward_config(cfg)
    print(f"[case] backward {m['name']} whole tensors", flush=True)
    kw = dict(causal=m["causal"], layout=m["layout"], scale=m["scale"])
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.prefill_with_lse(qg, kg, vg, **kw)
    dq, dk, dv = attn.prefill_backward(qg, kg, vg, o, dog, lse, dq=whole.nan_like(qg),
                                       dk=whole.nan_like(kg), dv=whole.nan_like(vg), **kw)
    torch.cuda.synchronize()
    outs = {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    del qg, kg, vg, dog, o, lse, dq, dk, dv
    stats = whole.compare(whole.backward_units(q, k, v, do, **kw), outs, workers=8,
                          progress=progress)
    for name, st in stats.items():
        print(f"[parity] config {cfg} {name} (whole tensor): {st}", flush=True)
        assert st.nonfinite == 0, f"{name}: {st.nonfinite} elements not written (or not finite)"
        big = max(st.max_ref, 1e-3)
        tol_abs, tol_rel = TOL[m["dtype"]]
        assert st.max_abs <= tol_abs * big and st.rel_fro <= tol_rel, f"config {cfg} {name}: {st}"