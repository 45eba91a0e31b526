"""GPU parity of FP8 prefill (attn_prefill_fp8: e4m3fn q, k, v with per-tensor
descales) through the C ABI against the fp64 oracle on the dequantised
inputs.  Same bar as the fp16/bf16 prefill; with an fp32 output 3e-3 / 5e-4."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import MAX_ABS_TOL, REL_FRO_TOL, assert_parity

pytestmark = pytest.mark.gpu


def _deq(q8, k8, v8, sc):
    return tuple(torch.from_numpy(oracle.dequantize_fp8(t, d)) for t, d in zip((q8, k8, v8), sc))


def _run(attn, q8, k8, v8, sc, **kw):
    print(f"[case] prefill_fp8 q{tuple(q8.shape)} k{tuple(k8.shape)} {kw}", flush=True)
    o = attn.prefill_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sc, **kw)
    torch.cuda.synchronize()
    return o.cpu()


@pytest.mark.parametrize("shape", [(1, 2, 77, 333), (2, 3, 300, 300), (1, 4, 513, 129)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("layout,causal", [("BHSD", False), ("BSHD", True), ("BHSD", True)])
def test_prefill_fp8_parity(gpu_lib, shape, D, layout, causal):
    B, H, Sq, Skv = shape
    q8, k8, v8, sc = workloads.prefill_inputs_fp8(B, H, Sq, Skv, D, layout, seed=Sq + D)
    o = _run(gpu_lib, q8, k8, v8, sc, causal=causal, layout=layout)
    ref = oracle.sdpa(*_deq(q8, k8, v8, sc), causal=causal, layout=layout)
    assert_parity(o.double().numpy(), ref, f"fp8 {shape} D{D} {layout} causal={causal}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_prefill_fp8_gqa_outputs(gpu_lib, out):
    q8, k8, v8, sc = workloads.prefill_inputs_fp8(2, 8, 200, 450, 128, "BSHD", seed=5, h_kv=2)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    o = _run(gpu_lib, q8, k8, v8, sc, causal=True, layout="BSHD", out_dtype=odt)
    assert o.dtype == odt
    ref = oracle.sdpa(*_deq(q8, k8, v8, sc), causal=True, layout="BSHD")
    tol = dict(max_abs_tol=3e-3, rel_fro_tol=5e-4) if out == "f32" else {}
    assert_parity(o.double().numpy(), ref, f"fp8 gqa out {out}", **tol)


def test_prefill_fp8_exact_identities(gpu_lib):
    """fp32 O rounds to the fp16 O; doubling the v descale doubles O; moving a
    factor 2 from the q descale to the k descale changes nothing."""
    q8, k8, v8, (qs, ks, vs) = workloads.prefill_inputs_fp8(1, 4, 260, 390, 128, seed=6)
    o16 = _run(gpu_lib, q8, k8, v8, (qs, ks, vs), causal=True)
    o32 = _run(gpu_lib, q8, k8, v8, (qs, ks, vs), causal=True, out_dtype=torch.float32)
    assert torch.equal(o32.to(torch.float16), o16)
    o32x2 = _run(gpu_lib, q8, k8, v8, (qs, ks, 2 * vs), causal=True, out_dtype=torch.float32)
    assert torch.equal(o32x2, 2 * o32)
    o_moved = _run(gpu_lib, q8, k8, v8, (2 * qs, ks / 2, vs), causal=True, out_dtype=torch.float32)
    assert torch.equal(o_moved, o32)


@pytest.mark.timeout(900)
def test_prefill_fp8_llama2_13b_whole(gpu_lib, progress):
    """fp8 prefill of the Llama-2-13B shape at full size: NaN-prefilled
    output, the whole tensor against the oracle on the dequantised inputs."""
    q8, k8, v8, m = workloads.prefill_config(10)
    print(f"[case] prefill_fp8 {m['name']} whole tensor", flush=True)
    out = torch.full(tuple(q8.shape), float("nan"), dtype=torch.float16, device="cuda")
    o = gpu_lib.prefill_fp8(q8.cuda(), k8.cuda(), v8.cuda(), m["descales"], causal=m["causal"],
                            scale=m["scale"], layout=m["layout"], out=out)
    torch.cuda.synchronize()
    q, k, v = _deq(q8, k8, v8, m["descales"])
    st = whole.compare(whole.prefill_units(q, k, v, ["o"], causal=m["causal"], scale=m["scale"],
                                           layout=m["layout"]), {"o": o.cpu()},
                       progress=progress)["o"]
    print(f"[parity] {m['name']} (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0, f"{st.nonfinite} elements not written (or not finite)"
    assert st.max_abs <= MAX_ABS_TOL and st.rel_fro <= REL_FRO_TOL, f"{m['name']}: {st}"
