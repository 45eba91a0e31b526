"""GPU parity of attn_prefill_splitkv (prefill with the keys of each query
tile split over workgroups and the partials merged by log-sum-exp) against
the fp64 oracle, on shapes whose grids are too small to fill the GPU: one
or a few heads, short query blocks against long key ranges, causal
(bottom-right, including rows that see no key) and not, grouped KV heads,
both layouts, fp16/bf16, D = 64 and 128, fp32 output.  Also: every element
written (NaN-prefilled output, NaN-filled workspace), run-to-run
determinism, and bitwise equality with attn_prefill_gqa when the plan does
not split."""
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu

CASES = [  # B, H, H_kv, Sq, Skv, D, dtype, layout, causal
    (1, 8, 8, 128, 9000, 128, "f16", "BHSD", False),
    (1, 8, 2, 200, 5000, 128, "bf16", "BSHD", True),
    (2, 4, 4, 1, 3000, 64, "f16", "BSHD", False),
    (1, 2, 1, 300, 20000, 64, "bf16", "BHSD", True),
    (1, 4, 4, 77, 1100, 128, "f16", "BHSD", True),
    (1, 2, 2, 1500, 1100, 128, "f16", "BSHD", True),   # rows 0..399 see no key
    (3, 3, 1, 513, 4097, 128, "bf16", "BHSD", False),
]


def _ids(c):
    B, H, H_kv, Sq, Skv, D, dtype, layout, causal = c
    return f"B{B}H{H}-{H_kv}S{Sq}x{Skv}D{D}{dtype}{layout}{'c' if causal else ''}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_splitkv_parity(gpu_lib, case):
    attn = gpu_lib
    B, H, H_kv, Sq, Skv, D, dtype, layout, causal = case
    n = attn.attn_prefill_splitkv_num_splits(B, H, Sq, Skv, D)
    assert n > 1, n  # every case here splits
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, dtype, layout, seed=Sq + Skv,
                                       h_kv=H_kv)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    print(f"[case] splitkv {_ids(case)} splits {n}", flush=True)
    out = torch.full(tuple(q.shape), float("nan"), dtype=q.dtype, device="cuda")
    need = attn.attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    o = attn.prefill_splitkv(qg, kg, vg, causal=causal, layout=layout, out=out, workspace=ws)
    o2 = attn.prefill_splitkv(qg, kg, vg, causal=causal, layout=layout)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o, o2)
    ref = oracle.sdpa(q, k, v, causal=causal, layout=layout)
    assert_parity(o.double().cpu().numpy(), ref, f"splitkv {_ids(case)}")
    o32 = attn.prefill_splitkv(qg, kg, vg, causal=causal, layout=layout,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the fp32 output: only the kernels' own error (fp16 P, fp32 sums)
    assert_parity(o32.double().cpu().numpy(), ref, f"splitkv fp32 {_ids(case)}",
                  max_abs_tol=3e-3, rel_fro_tol=5e-4)
    assert torch.equal(o32.to(q.dtype), o)


@pytest.mark.parametrize("layout,causal", [("BHSD", False), ("BSHD", True)])
def test_splitkv_without_split_is_prefill(gpu_lib, layout, causal):
    """Fewer than 16 key tiles: no split, no workspace, bitwise the plain
    prefill."""
    attn = gpu_lib
    B, H, Sq, Skv, D = 2, 4, 200, 960, 128
    assert attn.attn_prefill_splitkv_num_splits(B, H, Sq, Skv, D) == 1
    assert attn.attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D) == 0
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, "f16", layout, seed=5)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    print(f"[case] splitkv no split {layout} causal={causal}", flush=True)
    a = attn.prefill_splitkv(qg, kg, vg, causal=causal, layout=layout)
    b = attn.prefill(qg, kg, vg, causal=causal, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.timeout(900)
def test_splitkv_chunk_workload_whole(gpu_lib, progress):
    """The benchmark's chunked-prefill workload (B1 H32/8, a 512-token chunk
    against 32k keys, bottom-right causal, bf16 BSHD) in its launch
    configuration, compared with the oracle over the whole output
    (NaN-prefilled)."""
    import whole_tensor as whole
    attn = gpu_lib
    q, k, v, m = workloads.prefill_config(13)
    assert attn.attn_prefill_splitkv_num_splits(m["B"], m["H"], m["Sq"], m["Skv"], m["D"]) > 1
    print(f"[case] split-kv prefill {m['name']} whole tensor", flush=True)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    kw = dict(causal=m["causal"], scale=m["scale"], layout=m["layout"])
    o = attn.prefill_splitkv(qg, kg, vg, out=whole.nan_like(qg), **kw)
    torch.cuda.synchronize()
    outs = {"o": o.cpu()}
    del qg, kg, vg
    stats = whole.compare(whole.prefill_units(q, k, v, list(outs), **kw), outs,
                          progress=progress)
    st = stats["o"]
    print(f"[parity] {m['name']} (whole tensor): {st}", flush=True)
    assert st.nonfinite == 0, f"{st.nonfinite} elements not written (or not finite)"
    assert st.max_abs <= 1e-2 and st.rel_fro <= 2e-3, st
