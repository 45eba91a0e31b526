"""GPU parity of attn_prefill (through the C ABI) against the fp64 oracle.

Bar: max-abs error <= 1e-2 and relative Frobenius error <= 2e-3, over the
whole output: for shapes the oracle finishes in seconds, and at the full
workload sizes in the launch configuration the bench times (written into
NaN-prefilled buffers; the oracle runs per head and row block on a thread
pool, see whole_tensor.py).
"""
import math
import zlib

import pytest
import torch

import oracle
import workloads
import whole_tensor as whole
from parity import MAX_ABS_TOL, REL_FRO_TOL, assert_parity

pytestmark = pytest.mark.gpu


def _run(attn, q, k, v, causal, scale, layout):
    print(f"[case] prefill q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} {layout} "
          f"causal={causal}", flush=True)
    o = attn.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, layout=layout)
    torch.cuda.synchronize()
    return o.cpu()


def _f64(t):
    return t.double().numpy()


# --------------------------------------------------------------- small shapes

ODD = [
    # (B, H, Sq, Skv)
    (2, 3, 300, 300),     # ragged query and key tiles
    (1, 2, 67, 1500),     # small odd query block, long ragged KV
    (1, 2, 257, 513),     # causal bottom-right with Sq < Skv
    (1, 2, 513, 257),     # Sq > Skv: causal rows that see no key give 0
]


@pytest.mark.parametrize("shape", ODD, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_odd_shapes(gpu_lib, shape, D, dtype, layout, causal):
    B, H, Sq, Skv = shape
    seed = zlib.crc32(repr((shape, D, dtype, layout, causal)).encode()) % 10000
    q, k, v = workloads.prefill_inputs(B, H, Sq, Skv, D, dtype, layout, seed=seed)
    scale = 1 / math.sqrt(D)
    o = _run(gpu_lib, q, k, v, causal, scale, layout)
    ref = oracle.sdpa(q, k, v, causal=causal, scale=scale, layout=layout)
    assert_parity(_f64(o), ref, f"{shape} D{D} {dtype} {layout} causal={causal}")


def test_prefill_tiny_mha_d64_full(gpu_lib):
    q, k, v, m = workloads.prefill_config(1)
    o = _run(gpu_lib, q, k, v, m["causal"], m["scale"], m["layout"])
    ref = oracle.sdpa(q, k, v, causal=m["causal"], scale=m["scale"], layout=m["layout"])
    assert_parity(_f64(o), ref, f"{m['name']} (full tensor)")


@pytest.mark.parametrize("Sq,Skv,causal", [(1, 1, False), (1, 1000, True), (1000, 1, True),
                                          (1, 64, False), (64, 1, False), (128, 128, True)])
def test_prefill_degenerate_lengths(gpu_lib, Sq, Skv, causal):
    q, k, v = workloads.prefill_inputs(1, 2, Sq, Skv, 128, "f16", "BHSD", seed=Sq * 7 + Skv)
    o = _run(gpu_lib, q, k, v, causal, 1 / math.sqrt(128), "BHSD")
    ref = oracle.sdpa(q, k, v, causal=causal, layout="BHSD")
    assert_parity(_f64(o), ref, f"Sq{Sq} Skv{Skv} causal={causal}")


def test_prefill_empty_and_no_keys(gpu_lib):
    attn = gpu_lib
    dev = torch.device("cuda")
    # B*H*Sq = 0: nothing to do, no launch
    z = torch.empty((0, 2, 16, 64), dtype=torch.float16, device=dev)
    assert attn.prefill(z, z, z).shape == z.shape
    # Skv = 0: every row sees no key, O = 0
    q = torch.randn((1, 2, 40, 64), device=dev).half()
    kv = torch.empty((1, 2, 0, 64), dtype=torch.float16, device=dev)
    o = attn.prefill(q, kv, kv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0


def test_prefill_scale_zero_is_uniform(gpu_lib):
    q, k, v = workloads.prefill_inputs(1, 2, 100, 300, 64, "f16", "BHSD", seed=5)
    o = _run(gpu_lib, q, k, v, False, 0.0, "BHSD")
    ref = oracle.sdpa(q, k, v, causal=False, scale=0.0)
    assert_parity(_f64(o), ref, "scale 0")


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_ones_v_gives_ones(gpu_lib, dtype):
    q, k, _ = workloads.prefill_inputs(1, 2, 200, 333, 128, dtype, "BHSD", seed=3)
    v = torch.ones_like(k)
    o = _run(gpu_lib, q, k, v, True, 1 / math.sqrt(128), "BHSD")
    assert float((o.double() - 1).abs().max()) <= 1e-3


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_causal_row0_is_v0_exactly(gpu_lib, dtype):
    q, k, v = workloads.prefill_inputs(2, 3, 150, 150, 128, dtype, "BSHD", seed=4)
    o = _run(gpu_lib, q, k, v, True, 1 / math.sqrt(128), "BSHD")
    assert torch.equal(o[:, 0], v[:, 0])


def test_prefill_layouts_bitwise_equal(gpu_lib):
    q, k, v = workloads.prefill_inputs(2, 3, 190, 270, 128, "bf16", "BHSD", seed=6)
    a = _run(gpu_lib, q, k, v, True, 0.1, "BHSD")
    b = _run(gpu_lib, *(t.transpose(1, 2).contiguous() for t in (q, k, v)), True, 0.1, "BSHD")
    assert torch.equal(a, b.transpose(1, 2))


def test_prefill_deterministic(gpu_lib):
    q, k, v = workloads.prefill_inputs(1, 4, 256, 512, 128, "f16", "BHSD", seed=8)
    a = _run(gpu_lib, q, k, v, False, 0.09, "BHSD")
    b = _run(gpu_lib, q, k, v, False, 0.09, "BHSD")
    assert torch.equal(a, b)


# ------------------------------------------------------ full workload sizes

# Output buffers start as NaN, so a row the kernel never writes is caught, and
# the whole output is compared with the oracle (tests/whole_tensor.py).  For
# the long-context workload the fp32 output is graded too, against the
# four-times tighter fp32 bar, so the pass does not rest on how the bf16
# rounding of O (up to 2^-8 |O|, and |O| reaches ~4 in its early causal rows)
# happens to fall.
F32_MAX_ABS_FULL, F32_REL_FRO_FULL = 3e-3, 5e-4


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_prefill_full_size_whole(gpu_lib, cfg, progress):
    attn = gpu_lib
    q, k, v, m = workloads.prefill_config(cfg)
    print(f"[case] prefill {m['name']} whole tensor", flush=True)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    kw = dict(causal=m["causal"], scale=m["scale"], layout=m["layout"])
    outs = {"o": attn.prefill(qg, kg, vg, out=whole.nan_like(qg), **kw)}
    if cfg == 5:
        outs["o_f32"] = attn.prefill(qg, kg, vg, out=whole.nan_like(qg, torch.float32), **kw)
    torch.cuda.synchronize()
    outs = {n: t.cpu() for n, t in outs.items()}
    del qg, kg, vg
    stats = whole.compare(whole.prefill_units(q, k, v, list(outs), **kw), outs,
                          progress=progress)
    for n, st in stats.items():
        print(f"[parity] {m['name']} {n} (whole tensor): {st}", flush=True)
        assert st.nonfinite == 0, f"{n}: {st.nonfinite} elements not written (or not finite)"
    st = stats["o"]
    assert st.max_abs <= MAX_ABS_TOL and st.rel_fro <= REL_FRO_TOL, f"{m['name']}: {st}"
    if "o_f32" in stats:
        st = stats["o_f32"]
        assert st.max_abs <= F32_MAX_ABS_FULL and st.rel_fro <= F32_REL_FRO_FULL, \
            f"{m['name']} fp32 output: {st}"
        assert torch.equal(outs["o_f32"].to(outs["o"].dtype), outs["o"])


# ------------------------------------------------------------ stress cases

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_prefill_mostly_idle_waves(gpu_lib, causal, layout):
    """Sq far below one 256-row workgroup: most waves have no query rows."""
    q, k, v = workloads.prefill_inputs(3, 5, 33, 2000, 128, "bf16", layout, seed=21)
    o = _run(gpu_lib, q, k, v, causal, 1 / math.sqrt(128), layout)
    ref = oracle.sdpa(q, k, v, causal=causal, layout=layout)
    assert_parity(_f64(o), ref, f"Sq33 Skv2000 {layout} causal={causal}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_long_kv_tiny_q_causal(gpu_lib, dtype):
    """Bottom-right causal with Sq << Skv: every row sees almost all keys."""
    q, k, v = workloads.prefill_inputs(2, 3, 7, 5000, 128, dtype, "BHSD", seed=22)
    o = _run(gpu_lib, q, k, v, True, 1 / math.sqrt(128), "BHSD")
    assert_parity(_f64(o), oracle.sdpa(q, k, v, causal=True), f"Sq7 Skv5000 {dtype}")


@pytest.mark.parametrize("dtype,amp", [("f16", 6.0), ("bf16", 8.0)])
def test_prefill_large_logits_force_rescales(gpu_lib, dtype, amp):
    """Large inputs make the running max jump often (the lazy rescale path)."""
    q, k, v = workloads.prefill_inputs(1, 4, 700, 1900, 128, dtype, "BHSD", amp=amp, seed=23)
    # Only the logits grow: V is brought to std 1/3, so |O| < 2.  Near one-hot
    # rows copy single V values, and rounding O to bf16 alone costs up to
    # 2^-9 |O|, which must stay well inside the 1e-2 bar.
    v = (v.float() / (3 * amp)).to(v.dtype)
    for causal in (False, True):
        o = _run(gpu_lib, q, k, v, causal, 1 / math.sqrt(128), "BHSD")
        assert_parity(_f64(o), oracle.sdpa(q, k, v, causal=causal),
                      f"amp {amp} {dtype} causal={causal}")


def test_prefill_near_argmax_scale(gpu_lib):
    """A large scale concentrates each row on its top keys."""
    q, k, v = workloads.prefill_inputs(1, 2, 300, 800, 64, "f16", "BSHD", seed=24)
    o = _run(gpu_lib, q, k, v, False, 2.0, "BSHD")
    assert_parity(_f64(o), oracle.sdpa(q, k, v, causal=False, scale=2.0, layout="BSHD"),
                  "scale 2.0")


def test_prefill_rejects_bad_tensors(gpu_lib):
    attn = gpu_lib
    q = torch.randn((1, 2, 64, 128), device="cuda").half()
    with pytest.raises(ValueError):
        attn.prefill(q, q.transpose(2, 3).contiguous().transpose(2, 3), q)   # non-contiguous k
    with pytest.raises(TypeError):
        attn.prefill(q, q.float(), q)
    with pytest.raises(attn.AttnError) as e:
        attn.prefill(q[..., :96].contiguous(), q[..., :96].contiguous(), q[..., :96].contiguous())
    assert e.value.status == attn.ATTN_E_UNSUPPORTED


# ------------------------------------------------------------ fp32 output

# With O stored in fp32 the only rounding left is the kernel's own (fp16 P,
# fp32 accumulation), so the bar is four times tighter than the default.
F32_MAX_ABS, F32_REL_FRO = 3e-3, 5e-4


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_out_f32(gpu_lib, dtype, D, causal):
    attn = gpu_lib
    q, k, v = workloads.prefill_inputs(2, 3, 200, 333, D, dtype, "BSHD", seed=51 + D)
    print(f"[case] prefill out_f32 {dtype} D{D} causal={causal}", flush=True)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o32 = attn.prefill(qg, kg, vg, causal=causal, layout="BSHD", out_dtype=torch.float32)
    o16 = attn.prefill(qg, kg, vg, causal=causal, layout="BSHD")
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    ref = oracle.sdpa(q, k, v, causal=causal, layout="BSHD")
    assert_parity(_f64(o32.cpu()), ref, f"out_f32 {dtype} D{D} causal={causal}",
                  max_abs_tol=F32_MAX_ABS, rel_fro_tol=F32_REL_FRO)
    # The default output is the fp32 result rounded to nearest even.
    assert torch.equal(o32.to(o16.dtype), o16)


# ---------------------------------------------------- causal query-tile pairs

@pytest.mark.parametrize("Sq", [1, 63, 64, 65, 255, 256, 257, 511, 767, 1024, 1280])
@pytest.mark.parametrize("D,H,H_kv", [(128, 2, 2), (64, 2, 2), (128, 8, 2)])
def test_prefill_causal_tile_pairs(gpu_lib, Sq, D, H, H_kv):
    """Causal prefill over a grid that fills the CUs at least twice gives each
    workgroup a pair of query tiles (the heaviest left, then the lightest; the
    middle one alone when the count is odd); a smaller grid keeps one tile per
    workgroup.  1 to 10 tiles of 256 (D = 128), 128 (D = 64) or, with four
    query heads per workgroup, 64 rows, with Skv = Sq + 37 so the diagonal is
    offset.  A batch of 256 (paired: at least 512 tiles) into a NaN-filled
    output; three of its sequences alone (unpaired) must give bitwise the
    same rows, and those match the oracle."""
    Skv = Sq + 37
    Bb = 256
    seed = Sq + D + H_kv
    print(f"[case] causal pairs B{Bb} Sq{Sq} Skv{Skv} D{D} H{H}/{H_kv}", flush=True)
    q = workloads.device_normal((Bb, H, Sq, D), "bf16", seed=3 * seed)
    k = workloads.device_normal((Bb, H_kv, Skv, D), "bf16", seed=3 * seed + 1)
    v = workloads.device_normal((Bb, H_kv, Skv, D), "bf16", seed=3 * seed + 2)
    o = gpu_lib.prefill(q, k, v, causal=True, out=whole.nan_like(q))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "paired grid left rows unwritten"
    for b in (0, 137, Bb - 1):
        qs, ks, vs = q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous()
        o1 = gpu_lib.prefill(qs, ks, vs, causal=True, out=whole.nan_like(qs))
        torch.cuda.synchronize()
        assert torch.equal(o1, o[b:b + 1]), f"sequence {b}: paired and unpaired rows differ"
        assert_parity(_f64(o1.cpu()), oracle.sdpa(qs.cpu(), ks.cpu(), vs.cpu(), causal=True),
                      f"causal pairs Sq{Sq} D{D} H{H}/{H_kv} sequence {b}")
