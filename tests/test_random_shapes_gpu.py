"""A seeded sweep of random shapes through prefill (with and without the LSE
output), split-KV prefill, grouped-query decode, extend and split-KV
extend, the backward and fp8 prefill (with
the output in the input type or, in some draws, in fp32), each
against the fp64 oracle at its bar.  The draws mix batch, head counts and
grouping, lengths on and off tile boundaries (including Sq > Skv under the
bottom-right causal mask), head size, dtype, layout and scale, so that
combinations the hand-picked cases do not name are still exercised.  Sizes
stay small enough for the oracle to finish in seconds."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu


def _draw_prefill(i):
    r = np.random.default_rng(1000 + i)
    H_kv = int(r.choice([1, 2, 4]))
    H = H_kv * int(r.choice([1, 2, 3, 4]))
    return dict(B=int(r.integers(1, 3)), H=H, H_kv=H_kv, Sq=int(r.integers(1, 600)),
                Skv=int(r.integers(1, 700)), D=int(r.choice([64, 128])),
                dtype=str(r.choice(["f16", "bf16"])), layout=str(r.choice(["BHSD", "BSHD"])),
                causal=bool(r.integers(0, 2)), scale=float(r.uniform(0.02, 0.3)),
                lse=bool(r.integers(0, 2)), out32=bool(r.integers(0, 4) == 0))


@pytest.mark.parametrize("i", range(36))
def test_prefill_random(gpu_lib, i):
    c = _draw_prefill(i)
    print(f"[case] prefill random {i}: {c}", flush=True)
    q, k, v = workloads.prefill_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                       c["layout"], seed=2000 + i, h_kv=c["H_kv"])
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    odt = torch.float32 if c["out32"] else None
    if c["lse"]:
        o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, causal=c["causal"], scale=c["scale"],
                                          layout=c["layout"], out_dtype=odt)
    else:
        o = gpu_lib.prefill(qg, kg, vg, causal=c["causal"], scale=c["scale"], layout=c["layout"],
                            out_dtype=odt)
    assert o.dtype == (torch.float32 if c["out32"] else q.dtype)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, causal=c["causal"], scale=c["scale"], layout=c["layout"])
    assert_parity(o.double().cpu().numpy(), ref, f"prefill random {i}")
    if c["lse"]:
        want = oracle.lse_rows(q, k, causal=c["causal"], scale=c["scale"], layout=c["layout"])
        got = lse.double().cpu().numpy()
        fin = np.isfinite(want)
        assert np.array_equal(fin, np.isfinite(got))
        assert np.all(np.abs(got[fin] - want[fin]) <= 1e-3 + 1e-6 * np.abs(want[fin]))


@pytest.mark.parametrize("i", range(16))
def test_prefill_splitkv_random(gpu_lib, i):
    """Split-KV prefill on random small grids over 1k-9k keys (so that the
    plan splits), written into NaN-filled output and workspace."""
    r = np.random.default_rng(5000 + i)
    H_kv = int(r.choice([1, 2]))
    c = dict(B=int(r.integers(1, 3)), H=H_kv * int(r.integers(1, 5)), H_kv=H_kv,
             Sq=int(r.integers(1, 400)), Skv=int(r.integers(1024, 9000)),
             D=int(r.choice([64, 128])), dtype=str(r.choice(["f16", "bf16"])),
             layout=str(r.choice(["BHSD", "BSHD"])), causal=bool(r.integers(0, 2)),
             scale=float(r.uniform(0.02, 0.3)), out32=bool(r.integers(0, 4) == 0))
    n = gpu_lib.attn_prefill_splitkv_num_splits(c["B"], c["H"], c["Sq"], c["Skv"], c["D"])
    print(f"[case] splitkv random {i}: {c} splits {n}", flush=True)
    assert n > 1
    q, k, v = workloads.prefill_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                       c["layout"], seed=6000 + i, h_kv=c["H_kv"])
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    odt = torch.float32 if c["out32"] else q.dtype
    out = torch.full(tuple(q.shape), float("nan"), dtype=odt, device="cuda")
    need = gpu_lib.attn_prefill_splitkv_workspace_size(c["B"], c["H"], c["Sq"], c["Skv"], c["D"])
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    o = gpu_lib.prefill_splitkv(qg, kg, vg, causal=c["causal"], scale=c["scale"],
                                layout=c["layout"], out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    ref = oracle.sdpa(q, k, v, causal=c["causal"], scale=c["scale"], layout=c["layout"])
    assert_parity(o.double().cpu().numpy(), ref, f"splitkv random {i}")


@pytest.mark.parametrize("i", range(10))
def test_extend_splitkv_random(gpu_lib, i):
    """Split-KV extend on random small batches (1-3 sequences, prefixes up
    to 6k tokens, so that the plan splits), NaN in the cache's free slots,
    the output and the workspace."""
    r = np.random.default_rng(7000 + i)
    H_kv = int(r.choice([1, 2]))
    H = H_kv * int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 4))
    pl = r.integers(0, 6000, B).tolist()
    pl[0] = int(r.integers(1500, 6000))
    el = r.integers(1, 300, B).tolist()
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f16", "bf16"]))
    scale = float(r.uniform(0.02, 0.3))
    batch = workloads.extend_inputs(B, H, D, pl, el, dtype, seed=7500 + i, h_kv=H_kv,
                                    fill=float("nan"))
    T = batch.q.shape[0]
    sizes = (B, H, H_kv, D, T, max(el), batch.page_table.shape[1])
    n = gpu_lib.attn_extend_splitkv_num_splits(*sizes)
    print(f"[case] extend splitkv random {i}: B{B} H{H}/{H_kv} D{D} {dtype} prefix {pl} "
          f"new {el} splits {n}", flush=True)
    assert n > 1
    g = {m: getattr(batch, m).cuda() for m in ("q", "k", "v", "k_cache", "v_cache", "page_table",
                                              "prefix_lens", "qo_start")}
    out = torch.full(batch.q.shape, float("nan"), dtype=batch.q.dtype, device="cuda")
    ws = torch.full((gpu_lib.attn_extend_splitkv_workspace_size(*sizes),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    o = gpu_lib.extend_splitkv(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"],
                               g["page_table"], g["prefix_lens"], g["qo_start"], scale=scale,
                               out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, scale=scale)
    assert_parity(o.double().cpu().numpy(), ref, f"extend splitkv random {i}")


@pytest.mark.parametrize("i", range(18))
def test_decode_random(gpu_lib, i):
    r = np.random.default_rng(3000 + i)
    H_kv = int(r.choice([1, 2, 4, 8]))
    H = H_kv * int(r.choice([1, 2, 4, 8, 16]))
    B = int(r.integers(1, 40))
    lens = r.integers(0, 3000, B).tolist()
    lens[int(r.integers(0, B))] = int(r.integers(1, 5000))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f16", "bf16"]))
    scale = float(r.uniform(0.02, 0.3))
    out32 = bool(r.integers(0, 4) == 0)
    pages = sum(-(-n // 16) for n in lens)
    print(f"[case] decode random {i}: B{B} H{H}/{H_kv} D{D} {dtype} max_len {max(lens)} "
          f"out32={out32}", flush=True)
    batch = workloads.paged_decode_inputs(B=B, H=H, D=D, dtype=dtype, page_size=16,
                                          num_pages=pages + 32, seq_lens=lens, seed=4000 + i,
                                          h_kv=H_kv)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    o = gpu_lib.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                             scale=scale, out_dtype=torch.float32 if out32 else None)
    torch.cuda.synchronize()
    assert o.dtype == (torch.float32 if out32 else batch.q.dtype)
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, scale=scale)
    assert_parity(o.double().cpu().numpy(), ref, f"decode random {i}")


@pytest.mark.parametrize("i", range(8))
def test_decode_random_wide_groups(gpu_lib, i):
    """Groups wider than one 32-head query chunk and not a multiple of it
    (a last chunk of 4-16 heads), multi-query and two KV heads."""
    r = np.random.default_rng(3500 + i)
    group = int(r.choice([24, 40, 48, 80, 100]))
    H_kv = int(r.choice([1, 2]))
    H = H_kv * group
    B = int(r.integers(1, 12))
    lens = r.integers(0, 2500, B).tolist()
    lens[int(r.integers(0, B))] = int(r.integers(1, 4000))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f16", "bf16"]))
    scale = float(r.uniform(0.02, 0.3))
    pages = sum(-(-n // 16) for n in lens)
    print(f"[case] decode wide group {i}: B{B} H{H}/{H_kv} D{D} {dtype} lens {lens}", flush=True)
    batch = workloads.paged_decode_inputs(B=B, H=H, D=D, dtype=dtype, page_size=16,
                                          num_pages=pages + 8, seq_lens=lens, seed=4500 + i,
                                          h_kv=H_kv)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k_cache", "v_cache", "page_table",
                                              "seq_lens")}
    o = gpu_lib.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                             scale=scale)
    torch.cuda.synchronize()
    ref = oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache, batch.page_table,
                              batch.seq_lens, scale=scale)
    assert_parity(o.double().cpu().numpy(), ref, f"decode wide group {i}")


@pytest.mark.parametrize("i", range(14))
def test_extend_random(gpu_lib, i):
    r = np.random.default_rng(5000 + i)
    H_kv = int(r.choice([1, 2, 4]))
    H = H_kv * int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 6))
    pl = r.integers(0, 900, B).tolist()
    el = r.integers(0, 300, B).tolist()
    el[int(r.integers(0, B))] = int(r.integers(1, 300))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["f16", "bf16"]))
    scale = float(r.uniform(0.02, 0.3))
    out32 = bool(r.integers(0, 2) == 0)
    print(f"[case] extend random {i}: B{B} H{H}/{H_kv} D{D} {dtype} prefix {pl} new {el} "
          f"out32={out32}", flush=True)
    batch = workloads.extend_inputs(B, H, D, pl, el, dtype, seed=6000 + i, h_kv=H_kv)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache",
                                              "page_table", "prefix_lens", "qo_start")}
    o = gpu_lib.extend(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"],
                       g["prefix_lens"], g["qo_start"], scale=scale,
                       out_dtype=torch.float32 if out32 else None)
    torch.cuda.synchronize()
    assert o.dtype == (torch.float32 if out32 else batch.q.dtype)
    ref = oracle.extend(batch.q, batch.k, batch.v, batch.k_cache, batch.v_cache,
                        batch.page_table, batch.prefix_lens, batch.qo_start, scale=scale)
    assert_parity(o.double().cpu().numpy(), ref, f"extend random {i}")


# The backward's bar for gradients (relative to max|ref|; derived from a CPU
# model of the kernels' rounding, see the docstring of test_backward_gpu.py).
BWD_TOL = {"f16": (2e-3, 1e-3), "bf16": (1e-2, 6e-3)}


@pytest.mark.parametrize("i", range(16))
def test_backward_random(gpu_lib, i):
    c = _draw_prefill(100 + i)
    c["Sq"], c["Skv"] = min(c["Sq"], 400), min(c["Skv"], 400)
    print(f"[case] backward random {i}: {c}", flush=True)
    q, k, v, do = workloads.backward_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                            c["layout"], amp=0.5, seed=7000 + i, h_kv=c["H_kv"])
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kw = dict(causal=c["causal"], scale=c["scale"], layout=c["layout"])
    o, lse = gpu_lib.prefill_with_lse(qg, kg, vg, **kw)
    grads = gpu_lib.prefill_backward(qg, kg, vg, o, dog, lse, **kw)
    torch.cuda.synchronize()
    refs = oracle.sdpa_backward(q, k, v, do, **kw)
    ma, rf = BWD_TOL[c["dtype"]]
    for name, g, ref in zip(("dq", "dk", "dv"), grads, refs):
        big = max(float(np.abs(ref).max()) if ref.size else 0.0, 1e-3)
        assert_parity(g.double().cpu().numpy(), ref, f"backward random {i} {name}",
                      max_abs_tol=ma * big, rel_fro_tol=rf)


@pytest.mark.parametrize("i", range(14))
def test_prefill_fp8_random(gpu_lib, i):
    c = _draw_prefill(200 + i)
    print(f"[case] fp8 prefill random {i}: {c}", flush=True)
    q8, k8, v8, sc = workloads.prefill_inputs_fp8(c["B"], c["H"], c["Sq"], c["Skv"], c["D"],
                                                  c["layout"], seed=8000 + i, h_kv=c["H_kv"])
    o = gpu_lib.prefill_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sc, causal=c["causal"],
                            scale=c["scale"], layout=c["layout"],
                            out_dtype=torch.float32 if c["out32"] else None)
    torch.cuda.synchronize()
    deq = [torch.from_numpy(oracle.dequantize_fp8(t, d)) for t, d in zip((q8, k8, v8), sc)]
    ref = oracle.sdpa(*deq, causal=c["causal"], scale=c["scale"], layout=c["layout"])
    assert_parity(o.double().cpu().numpy(), ref, f"fp8 prefill random {i}")
