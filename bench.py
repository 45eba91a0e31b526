#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--configs 2,1,3,4,5,6,7,8,9,10,11,12,13,14]

One step is one pass of the prefill hot path (grid order, Q/K/V staging,
Q.K^T on MFMA, masking, online softmax, P.V on MFMA, epilogue: one
attn_prefill launch) over the Llama-2-13B-shaped workload B=4 H=40
Sq=Skv=4096 D=128 fp16 BHSD non-causal, with inputs resident in HBM.  The
headline `value` is its throughput in TFLOP/s (4*B*H*Sq*Skv*D flops per
step).  The other workloads (tiny 128x128, causal BSHD bf16 8k, paged
decode, long causal 32k, grouped-query causal 8k, grouped-query and
multi-query paged decode, extend after a paged prefix, fp8 prefill, the
backward of the causal 8k workload with and without grouped KV heads, and a
512-token chunk against 32k keys through the split-KV prefill and through
the split-KV extend after a 32k-token paged prefix) are measured the same way
and reported under "extra", decode in GB/s of algorithmic K/V bytes, the backward in
TFLOP/s of its five products (2.5x the forward's flops).

Timing: W untimed warmup steps, then K timed steps on the stream the kernels
run on, bracketed by torch.cuda.synchronize(); HIP events around every step
give the per-launch durations (mean is used for `value`, median and min are
reported too).  Alongside, per workload: a cold-cache pass (a 512 MiB write,
twice the 256 MiB last-level cache, before every timed step and outside its
events), the GFX clock sampled over a ~1.5 s sustained window of the same
step, and for the tiny 128x128 workload the median over 20 replays of a HIP
graph of 50 launches (launch overhead removed).  Also sampled over that
window: socket power, the power cap, the share of the window the firmware
spent limiting for package power or temperature, and the throttle status.
Every workload also carries a CPU baseline: the fp64 oracle timed on a
bounded sample of the same inputs (whole heads, sequences or KV-head groups
in order; ~15 s for the headline, ~3 s for the others), after the GPU timing,
with the host described (CPU model, CPU count, BLAS threads).  Prints ONE
JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2516.6   # TFLOP/s, MI355X dense fp16/bf16
PEAK_MFMA_FP8 = 5033.2   # TFLOP/s, MI355X dense fp8
PEAK_HBM = 8000.0        # GB/s, MI355X HBM3E
PREFILL_SRC = os.path.join(ROOT, "attention_flash_attn_prefill_amd", "csrc", "prefill.hip")
DECODE_GQA_SRC = os.path.join(ROOT, "attention_flash_attn_prefill_amd", "csrc", "decode_gqa.hip")
BACKWARD_SRC = os.path.join(ROOT, "attention_flash_attn_prefill_amd", "csrc", "backward.hip")


def prefill_flops(m):
    """4 B H D per visible (query, key) pair: all Sq x Skv pairs, or for causal
    attention half of them when Sq = Skv (the diagonal overcount ignored), and
    the exact count under the bottom-right mask when Sq != Skv."""
    full = 4.0 * m["B"] * m["H"] * m["Sq"] * m["Skv"] * m["D"]
    if not m["causal"]:
        return full
    if m["Sq"] == m["Skv"]:
        return full / 2
    Sq, Skv = m["Sq"], m["Skv"]
    off = Skv - Sq
    visible = sum(min(Skv, max(0, i + 1 + off)) for i in range(Sq))
    return 4.0 * m["B"] * m["H"] * m["D"] * visible


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(name, src):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (profiles/<kernel>__<workload>__traffic.json), if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}__traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_steps(fn, steps, warmup, stream, before=None):
    """Per-step HIP-event durations of fn on `stream`; `before` (if given) runs
    ahead of every timed step, outside its events."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if before is not None:
            before()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return dict(mean_ms=sum(ms) / len(ms), median_ms=ms[len(ms) // 2], min_ms=ms[0],
                wall_ms_per_step=1e3 * wall / steps)


class ClockProbe:
    """GFX clock of the visible GPU through amd-smi's Python bindings (shipped
    with ROCm under share/amd_smi), matched to torch's device by PCI bus id.
    The sensor refreshes about once a second, so clocks are read over a
    sustained window of the step being measured, not from the timed steps."""

    def __init__(self):
        self.handle = None
        try:
            import torch
            sys.path.append("/opt/rocm/share/amd_smi")
            import amdsmi
            amdsmi.amdsmi_init()
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for h in amdsmi.amdsmi_get_processor_handles():
                if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                    self.handle = h
            self.amdsmi = amdsmi
        except Exception as e:  # no bindings or no permission: clocks are reported as null
            print(f"[bench] clock probe unavailable: {e!r}", file=sys.stderr, flush=True)

    def read_mhz(self):
        clks = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle).get("current_gfxclks")
        vals = [c for c in (clks or []) if isinstance(c, int) and 0 < c < 10000]
        if vals:
            return sum(vals) / len(vals)
        return float(self.amdsmi.amdsmi_get_clock_info(self.handle,
                                                       self.amdsmi.AmdSmiClkType.GFX)["clk"])

    def read_power_w(self):
        """Socket power now, in W (gpu metrics; the power-info call as a fallback)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        for key in ("current_socket_power", "average_socket_power"):
            val = m.get(key)
            if isinstance(val, (int, float)) and 0 < val < 100000:
                return float(val)
        info = self.amdsmi.amdsmi_get_power_info(self.handle)
        val = info.get("current_socket_power")
        return float(val) if isinstance(val, (int, float)) else None

    def power_cap_w(self):
        try:
            cap = self.amdsmi.amdsmi_get_power_cap_info(self.handle).get("power_cap")
            return round(cap / 1e6, 1) if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:
            return None

    def violations(self):
        """Accumulated throttle-violation counters (package power, socket
        thermal) and their sample counter; None if unavailable."""
        try:
            v = self.amdsmi.amdsmi_get_violation_status(self.handle)
            vals = {k: v.get(k) for k in ("acc_counter", "acc_ppt_pwr", "acc_socket_thrm",
                                          "acc_prochot_thrm", "acc_hbm_thrm")}
            if not all(isinstance(x, int) for x in vals.values()):
                return None
            vals["per_ppt_pwr"] = v.get("per_ppt_pwr")  # the library's own percentage
            return vals
        except Exception:
            return None

    def sustained(self, fn, seconds=1.5, settle=1.0):
        """GFX clock (mean over XCDs) and socket power, medians of the samples
        taken after `settle` seconds of back-to-back fn() calls, with the
        power cap, the fraction of that window the firmware spent limiting
        for package power or temperature (violation counters read before and
        after it), and the throttle status at its end."""
        if self.handle is None:
            return {}
        import threading
        import torch
        clocks, powers, stop = [], [], threading.Event()
        t0 = time.perf_counter()

        def sample():
            while not stop.is_set():
                if time.perf_counter() - t0 >= settle:
                    try:
                        clocks.append(self.read_mhz())
                    except Exception:
                        return
                    try:
                        p = self.read_power_w()
                        if p is not None:
                            powers.append(p)
                    except Exception:
                        pass
                time.sleep(0.02)

        v0 = self.violations()
        th = threading.Thread(target=sample)
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        v1 = self.violations()
        med = lambda xs: round(sorted(xs)[len(xs) // 2], 1) if xs else None
        out = {"clock_mhz": med(clocks), "power_w": med(powers), "power_cap_w": self.power_cap_w()}
        if v0 and v1 and v1["acc_counter"] > v0["acc_counter"]:
            n = v1["acc_counter"] - v0["acc_counter"]
            out["limit_frac"] = {
                "package_power": round((v1["acc_ppt_pwr"] - v0["acc_ppt_pwr"]) / n, 3),
                "socket_thermal": round((v1["acc_socket_thrm"] - v0["acc_socket_thrm"]) / n, 3),
                "hbm_thermal": round((v1["acc_hbm_thrm"] - v0["acc_hbm_thrm"]) / n, 3),
                "samples": n, "package_power_pct_reported": v1.get("per_ppt_pwr")}
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
            out["throttle_status"] = m.get("throttle_status")
            out["indep_throttle_status"] = m.get("indep_throttle_status")
        except Exception:
            pass
        return out


def cache_flusher(mib=512):
    """Writes mib MiB (twice the 256 MiB last-level cache) so the next step
    starts with its inputs out of L2 and the MALL."""
    import torch
    buf = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    counter = [0]

    def flush():
        counter[0] = (counter[0] + 1) & 0xFF
        buf.fill_(counter[0])
    return flush, buf


COLD = True  # cleared by --no-cold (profiling runs that should see warm steps only)


def measure(fn, steps, warmup, stream, clock):
    """Warm timing, cold-cache timing and the sustained clock of one step."""
    t = time_steps(fn, steps, warmup, stream)
    t["cold_mean_ms"] = t["cold_median_ms"] = None
    if COLD:
        flush, buf = cache_flusher()
        cold = time_steps(fn, min(steps, 30), 2, stream, before=flush)
        del buf
        t["cold_mean_ms"] = cold["mean_ms"]
        t["cold_median_ms"] = cold["median_ms"]
    t["sustained"] = clock.sustained(fn) if clock is not None else {}
    return t


def graph_replay_us(fn, stream, launches=50, samples=20):
    """Median over `samples` replays of a HIP graph holding `launches` calls
    of fn, per launch, in microseconds."""
    import torch
    g = torch.cuda.CUDAGraph()
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(launches):
            fn()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(1e3 * e0.elapsed_time(e1) / launches)
    per.sort()
    return per[len(per) // 2]


def bench_prefill(attn, cfg, steps, warmup, clock, cpu_budget=0.0):
    import torch
    import workloads
    qc, kc, vc, m = workloads.prefill_config(cfg)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    stream = torch.cuda.current_stream()
    if m["dtype"] == "fp8":
        o = torch.empty(q.shape, dtype=torch.float16, device="cuda")

        def step():
            attn.prefill_fp8(q, k, v, m["descales"], causal=m["causal"], scale=m["scale"],
                             layout=m["layout"], out=o, stream=stream)
    elif m.get("splitkv"):
        o = torch.empty_like(q)
        need = attn.attn_prefill_splitkv_workspace_size(m["B"], m["H"], m["Sq"], m["Skv"], m["D"])
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

        def step():
            attn.prefill_splitkv(q, k, v, causal=m["causal"], scale=m["scale"],
                                 layout=m["layout"], out=o, workspace=ws, stream=stream)
    else:
        o = torch.empty_like(q)

        def step():
            attn.prefill(q, k, v, causal=m["causal"], scale=m["scale"], layout=m["layout"],
                         out=o, stream=stream)

    t = measure(step, steps, warmup, stream, clock)
    if m["Sq"] * m["Skv"] <= 128 * 128:  # launch-bound: also time it from a HIP graph
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            t["graph_us_per_launch"] = graph_replay_us(
                lambda: attn.prefill(q, k, v, causal=m["causal"], scale=m["scale"],
                                     layout=m["layout"], out=o, stream=side), side)
        stream.wait_stream(side)
    flops = prefill_flops(m)
    tflops = flops / (t["mean_ms"] * 1e-3) / 1e12
    cfg_out = {"workload": m["name"], "B": m["B"], "H": m["H"], "H_kv": m["H_kv"],
               "Sq": m["Sq"], "Skv": m["Skv"],
               "D": m["D"], "layout": m["layout"], "causal": m["causal"], "dtype": m["dtype"]}
    if m.get("splitkv"):
        cfg_out["entry_point"] = "attn_prefill_splitkv"
        cfg_out["key_splits"] = attn.attn_prefill_splitkv_num_splits(m["B"], m["H"], m["Sq"],
                                                                     m["Skv"], m["D"])
    traffic = load_traffic(f"prefill_fwd__{m['name']}", PREFILL_SRC)
    # fp8: the Q.K^T half of the flops runs on the fp8 MFMA (5.0 PFLOP/s), the
    # P.V half on fp16 (2.5): the peak for the mix is their harmonic blend.
    peak = PEAK_MFMA_F16 if m["dtype"] != "fp8" else 2.0 / (1.0 / PEAK_MFMA_FP8 + 1.0 / PEAK_MFMA_F16)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(peak, 1),
            "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic}
    del q, k, v, o
    torch.cuda.empty_cache()
    cpu = cpu_baseline_prefill(qc, kc, vc, m, cpu_budget) if cpu_budget > 0 else None
    return dict(config=cfg_out, timing=t, flops_per_step=flops, tflops=tflops, roofline=roof,
                cpu_baseline=cpu)


def bench_decode(attn, cfg, steps, warmup, clock, cpu_budget=0.0):
    import torch
    import workloads
    batch = workloads.decode_config(cfg)
    g = {k: getattr(batch, k).cuda() for k in ("q", "k_cache", "v_cache", "page_table",
                                               "seq_lens")}
    B, H, D = batch.q.shape
    H_kv = batch.k_cache.shape[2]
    need = attn.attn_paged_decode_gqa_workspace_size(B, H, H_kv, D, batch.max_pages_per_seq,
                                                     batch.page_size)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(g["q"])
    stream = torch.cuda.current_stream()
    scale = batch.meta["scale"]

    def step():
        attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                          scale=scale, out=o, workspace=ws, stream=stream)

    t = measure(step, steps, warmup, stream, clock)
    n_tok = int(batch.seq_lens.sum())
    nbytes = n_tok * H_kv * D * 2 * 2  # K and V rows of the live tokens
    gbs = nbytes / (t["mean_ms"] * 1e-3) / 1e9
    n_splits, tps = attn.attn_paged_decode_gqa_num_splits(B, H, H_kv, batch.max_pages_per_seq,
                                                          batch.page_size)
    cfg_out = {"workload": batch.meta["name"], "B": B, "H": H, "H_kv": H_kv, "D": D,
               "dtype": batch.meta["dtype"],
               "page_size": batch.page_size, "num_pages": batch.num_pages,
               "live_tokens": n_tok}
    # tiles of the whole batch cut into equal ranges on the device
    cfg_out.update(max_work_ranges=n_splits, min_tokens_per_range=tps)
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM, 4),
            "traffic": load_traffic(f"decode_gqa_split__{batch.meta['name']}", DECODE_GQA_SRC)}
    del g, ws, o
    torch.cuda.empty_cache()
    cpu = cpu_baseline_decode(batch, cpu_budget) if cpu_budget > 0 else None
    return dict(config=cfg_out, timing=t, bytes_per_step=nbytes, gbs=gbs, roofline=roof,
                cpu_baseline=cpu)


def extend_flops(batch):
    """4 * H * D * (keys seen by each new token), summed: token i of sequence b
    sees prefix_lens[b] + i + 1 keys."""
    H, D = batch.q.shape[1], batch.q.shape[2]
    total = 0
    for b in range(len(batch.prefix_lens)):
        P = int(batch.prefix_lens[b])
        E = int(batch.qo_start[b + 1] - batch.qo_start[b])
        total += E * P + E * (E + 1) // 2
    return 4.0 * H * D * total


def bench_extend(attn, cfg, steps, warmup, clock, cpu_budget=0.0):
    import torch
    import workloads
    batch = workloads.extend_config(cfg)
    g = {n: getattr(batch, n).cuda() for n in ("q", "k", "v", "k_cache", "v_cache", "page_table",
                                              "prefix_lens", "qo_start")}
    o = torch.empty_like(g["q"])
    stream = torch.cuda.current_stream()
    mx = batch.max_extend_len
    split = workloads.EXTEND_CONFIGS[cfg].get("splitkv", False)
    sizes = (len(batch.prefix_lens), batch.q.shape[1], batch.k.shape[1], batch.q.shape[2],
             batch.q.shape[0], mx, batch.page_table.shape[1])
    ws = (torch.empty(max(attn.attn_extend_splitkv_workspace_size(*sizes), 1), dtype=torch.uint8,
                      device="cuda") if split else None)

    def step():
        f = attn.extend_splitkv if split else attn.extend
        kw = dict(workspace=ws) if split else {}
        f(g["q"], g["k"], g["v"], g["k_cache"], g["v_cache"], g["page_table"], g["prefix_lens"],
          g["qo_start"], max_extend_len=mx, scale=batch.meta["scale"], out=o, stream=stream, **kw)

    t = measure(step, steps, warmup, stream, clock)
    flops = extend_flops(batch)
    tflops = flops / (t["mean_ms"] * 1e-3) / 1e12
    cfg_out = {"workload": batch.meta["name"], "B": len(batch.prefix_lens),
               "H": batch.q.shape[1], "H_kv": batch.k.shape[1], "D": batch.q.shape[2],
               "dtype": batch.meta["dtype"], "new_tokens": int(batch.q.shape[0]),
               "prefix_tokens": int(batch.prefix_lens.sum()), "max_extend_len": mx}
    if split:
        cfg_out["entry_point"] = "attn_extend_splitkv"
        cfg_out["key_splits"] = attn.attn_extend_splitkv_num_splits(*sizes)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16, 4),
            "traffic": load_traffic(f"prefill_fwd__{batch.meta['name']}", PREFILL_SRC)}
    del g, o, ws
    torch.cuda.empty_cache()
    cpu = cpu_baseline_extend(batch, cpu_budget) if cpu_budget > 0 else None
    return dict(config=cfg_out, timing=t, flops_per_step=flops, tflops=tflops, roofline=roof,
                cpu_baseline=cpu)


def backward_flops(m):
    """The backward's five products (S, dP, dV, dK, dQ, each 2*Sq*Skv*D per
    head; half under the causal mask): 2.5x the forward's two."""
    return 2.5 * prefill_flops(m)


def bench_backward(attn, cfg, steps, warmup, clock, cpu_budget=0.0):
    """One step: one attn_prefill_bwd call (delta, dK/dV and dQ kernels) on
    the forward's O and LSE, which are computed once before timing."""
    import torch
    import workloads
    qc, kc, vc, doc, m = workloads.backward_config(cfg)
    q, k, v, do = qc.cuda(), kc.cuda(), vc.cuda(), doc.cuda()
    stream = torch.cuda.current_stream()
    o, lse = attn.prefill_with_lse(q, k, v, causal=m["causal"], scale=m["scale"],
                                   layout=m["layout"], stream=stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(attn.attn_prefill_bwd_workspace_size(m["B"], m["H"], m["Sq"]), 1),
                     dtype=torch.uint8, device="cuda")

    def step():
        attn.prefill_backward(q, k, v, o, do, lse, causal=m["causal"], scale=m["scale"],
                              layout=m["layout"], dq=dq, dk=dk, dv=dv, workspace=ws,
                              stream=stream)

    t = measure(step, steps, warmup, stream, clock)
    flops = backward_flops(m)
    tflops = flops / (t["mean_ms"] * 1e-3) / 1e12
    cfg_out = {"workload": m["name"], "B": m["B"], "H": m["H"], "H_kv": m["H_kv"],
               "Sq": m["Sq"], "Skv": m["Skv"], "D": m["D"], "layout": m["layout"],
               "causal": m["causal"], "dtype": m["dtype"], "pass": "backward"}
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16, 4),
            "scope": "the whole backward call (3 kernels)",
            "traffic": load_traffic(f"prefill_bwd__{m['name']}", BACKWARD_SRC)}
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    cpu = cpu_baseline_backward(qc, kc, vc, doc, m, cpu_budget) if cpu_budget > 0 else None
    return dict(config=cfg_out, timing=t, flops_per_step=flops, tflops=tflops, roofline=roof,
                cpu_baseline=cpu)


def copy_calibration(mib):
    """A plain elementwise copy of known size (reads and writes mib MiB each),
    run so HBM byte counters can be scaled against it."""
    import torch
    n = mib * (1 << 20) // 2
    a = torch.ones(n, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 x neg over {mib} MiB (read {mib} MiB, write {mib} MiB)",
          file=sys.stderr, flush=True)
    del a, b
    torch.cuda.empty_cache()


def vendor_gemm_reference(n=16384, dtype_name="f16", clock=None):
    """Throughput of the vendor's tuned dense GEMM (torch.matmul -> hipBLASLt)
    on this GPU, as context for the MFMA roofline: sustained matrix-core load
    runs the chip below its 2.4 GHz peak clock.  With a clock probe, also the
    clock, socket power and limiter share over a sustained window of the
    same product, and the energy per flop they imply."""
    import torch
    dt = torch.float16 if dtype_name == "f16" else torch.bfloat16
    a = torch.randn(n, n, device="cuda", dtype=dt)
    b = torch.randn(n, n, device="cuda", dtype=dt)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    sus = clock.sustained(lambda: a @ b, seconds=2.5, settle=1.5) if clock is not None else {}
    del a, b
    torch.cuda.empty_cache()
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    out = {"what": f"torch.matmul {dtype_name} {n}x{n}x{n} (hipBLASLt)",
           "tflops": round(tflops, 1), "ms": round(ms, 3)}
    if sus:
        out["clock_mhz"] = sus.get("clock_mhz")
        out["power"] = {k: sus[k] for k in ("power_w", "power_cap_w", "limit_frac") if k in sus}
        if sus.get("power_w"):
            out["pj_per_flop"] = round(sus["power_w"] / (tflops * 1e12) * 1e12, 3)
    return out


def host_info():
    """The host the CPU baseline runs on: logical CPUs, the CPUs this process
    may run on, the CPU model, and the BLAS threads numpy's matrix products use
    (its elementwise loops run on one thread)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model,
            "blas_threads": blas, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _timed_units(units, budget_s):
    """Run (work, callable) units in order until about budget_s seconds have
    passed (at least one); returns (work done, seconds, units run)."""
    done, n = 0.0, 0
    t0 = time.perf_counter()
    for work, fn in units:
        fn()
        done += work
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0, n


def _cpu_record(value, unit, sample):
    h = host_info()
    return {"value": value, "unit": unit, "cores": h["blas_threads"] or h["affinity_cpus"],
            "kind": "oracle", "sample": sample}


def cpu_baseline_prefill(q, k, v, m, budget_s):
    """The fp64 oracle as it stands (oracle.sdpa; for fp8 inputs
    oracle.dequantize_fp8 first), on whole heads of the same workload in
    order, until about budget_s seconds of CPU work; scaled to TFLOP/s."""
    import oracle
    B, H, H_kv = m["B"], m["H"], m["H_kv"]
    bhsd = m["layout"] == "BHSD"
    per_head = prefill_flops(m) / (B * H)

    def head(b, h):
        g = oracle.kv_head(h, H, H_kv)
        if bhsd:
            qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1]
        else:
            qs, ks, vs = q[b:b + 1, :, h:h + 1], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1]
        if m["dtype"] == "fp8":
            qd, kd, vd = m["descales"]
            qs, ks, vs = (oracle.dequantize_fp8(qs, qd), oracle.dequantize_fp8(ks, kd),
                          oracle.dequantize_fp8(vs, vd))
        oracle.sdpa(qs, ks, vs, causal=m["causal"], scale=m["scale"], layout=m["layout"])

    units = [(per_head, lambda b=b, h=h: head(b, h)) for b in range(B) for h in range(H)]
    flops, dt, n = _timed_units(units, budget_s)
    return _cpu_record(round(flops / dt / 1e12, 6), "TFLOP/s",
                       f"{n} of {B * H} heads of the same workload, fp64 oracle, {dt:.1f} s")


def cpu_baseline_decode(batch, budget_s):
    """oracle.paged_decode on the batch's sequences in order until about
    budget_s seconds; GB/s of the algorithmic K/V bytes of those sequences."""
    import oracle
    B, H, D = batch.q.shape
    H_kv = batch.k_cache.shape[2]
    lens = batch.seq_lens.tolist()
    units = [(lens[b] * H_kv * D * 2 * 2,
              lambda b=b: oracle.paged_decode(batch.q, batch.k_cache, batch.v_cache,
                                              batch.page_table, batch.seq_lens,
                                              scale=batch.meta["scale"], batch_indices=[b]))
             for b in range(B)]
    nbytes, dt, n = _timed_units(units, budget_s)
    return _cpu_record(round(nbytes / dt / 1e9, 4), "GB/s",
                       f"{n} of {B} sequences of the same batch (page-table gather included), "
                       f"fp64 oracle, {dt:.1f} s")


def cpu_baseline_extend(batch, budget_s):
    """oracle.extend one sequence at a time, in order, until about budget_s
    seconds; TFLOP/s of those sequences' flops."""
    import oracle
    H, D = batch.q.shape[1], batch.q.shape[2]
    starts = batch.qo_start.tolist()
    plen = batch.prefix_lens.tolist()
    B = len(plen)

    def flops(b):
        E = starts[b + 1] - starts[b]
        return 4.0 * H * D * (E * plen[b] + E * (E + 1) // 2)

    units = [(flops(b), lambda b=b: oracle.extend(batch.q, batch.k, batch.v, batch.k_cache,
                                                  batch.v_cache, batch.page_table,
                                                  batch.prefix_lens, batch.qo_start,
                                                  scale=batch.meta["scale"], seqs=[b]))
             for b in range(B)]
    fl, dt, n = _timed_units(units, budget_s)
    return _cpu_record(round(fl / dt / 1e12, 6), "TFLOP/s",
                       f"{n} of {B} sequences of the same batch, fp64 oracle, {dt:.1f} s")


def cpu_baseline_backward(q, k, v, do, m, budget_s):
    """oracle.sdpa_backward on one (batch, KV head) -- its query heads -- at a
    time, in order, until about budget_s seconds; TFLOP/s of the backward's
    five products for those heads."""
    import oracle
    B, H, H_kv = m["B"], m["H"], m["H_kv"]
    group = H // H_kv
    per_head = backward_flops(m) / (B * H)
    bhsd = m["layout"] == "BHSD"

    def unit(b, g):
        hs = slice(g * group, (g + 1) * group)
        if bhsd:
            sq, sk = (slice(b, b + 1), hs), (slice(b, b + 1), slice(g, g + 1))
        else:
            sq = (slice(b, b + 1), slice(None), hs)
            sk = (slice(b, b + 1), slice(None), slice(g, g + 1))
        oracle.sdpa_backward(q[sq], k[sk], v[sk], do[sq], causal=m["causal"], scale=m["scale"],
                             layout=m["layout"])

    units = [(per_head * group, lambda b=b, g=g: unit(b, g)) for b in range(B)
             for g in range(H_kv)]
    fl, dt, n = _timed_units(units, budget_s)
    return _cpu_record(round(fl / dt / 1e12, 6), "TFLOP/s",
                       f"{n * group} of {B * H} heads ({n} KV-head groups) of the same workload, "
                       f"fp64 oracle, {dt:.1f} s")


def side_measurements(t, work=None, unit=None):
    """Cold-cache time, clock, power (and, for a flop count, the energy per
    flop at the sustained power and the warm time) of one workload."""
    r4 = lambda x: None if x is None else round(x, 4)
    sus = t.get("sustained") or {}
    out = {"cold_cache_ms": r4(t["cold_mean_ms"]), "cold_cache_median_ms": r4(t["cold_median_ms"]),
           "clock_mhz": sus.get("clock_mhz")}
    power = {k: sus[k] for k in ("power_w", "power_cap_w", "limit_frac", "throttle_status",
                                 "indep_throttle_status") if k in sus}
    if power:
        if work and unit == "flop" and power.get("power_w"):
            power["pj_per_flop"] = round(power["power_w"] * t["mean_ms"] * 1e-3 / work * 1e12, 3)
        out["power"] = power
    if "graph_us_per_launch" in t:
        out["graph_replay_us_per_launch"] = round(t["graph_us_per_launch"], 2)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--configs", default="2,1,3,4,5,6,7,8,9,10,11,12,13,14",
                    help="workloads to measure; the first prefill one is the headline")
    ap.add_argument("--no-clock", action="store_true", help="skip the GFX clock windows")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache passes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of fp64-oracle CPU work for the headline workload's baseline")
    ap.add_argument("--cpu-budget-extra", type=float, default=3.0,
                    help="seconds of oracle CPU work for each other workload's baseline")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip timing the vendor GEMM reference")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(prefill shards by (batch, head) with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_flash_attn_prefill_amd as attn
    import workloads
    attn.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)

    cfgs = [int(c) for c in args.configs.split(",") if c.strip()]
    head_cfg = next((c for c in cfgs if c in workloads.PREFILL_CONFIGS), 2)
    if head_cfg not in cfgs:
        cfgs.insert(0, head_cfg)

    global COLD
    COLD = not args.no_cold
    clock = None if args.no_clock else ClockProbe()
    results = {}
    for c in cfgs:
        print(f"[bench] config {c} ...", file=sys.stderr, flush=True)
        # The oracle's CPU baseline runs after the GPU timing of the same
        # inputs, never alongside it.
        budget = 0.0 if args.no_cpu_baseline else (
            args.cpu_budget if c == head_cfg else args.cpu_budget_extra)
        if c in workloads.DECODE_CONFIGS:
            results[c] = bench_decode(attn, c, args.steps, args.warmup, clock, budget)
        elif c in workloads.EXTEND_CONFIGS:
            results[c] = bench_extend(attn, c, args.steps, args.warmup, clock, budget)
        elif c in workloads.BACKWARD_CONFIGS:
            results[c] = bench_backward(attn, c, args.steps, args.warmup, clock, budget)
        else:
            results[c] = bench_prefill(attn, c, args.steps, args.warmup, clock, budget)
        r = results[c]
        cpu_msg = ""
        if r.get("cpu_baseline"):
            cpu_msg = f"; cpu oracle {r['cpu_baseline']['value']} {r['cpu_baseline']['unit']}"
        print(f"[bench] config {c}: {r['timing']['mean_ms']:.4f} ms "
              f"{r['roofline']['achieved']} {r['roofline']['unit']} "
              f"({100 * r['roofline']['frac']:.1f}% of peak){cpu_msg}", file=sys.stderr,
              flush=True)

    head = results[head_cfg]
    gemm_ref = None
    if not args.no_gemm_reference:
        print("[bench] vendor GEMM reference ...", file=sys.stderr, flush=True)
        gemm_ref = vendor_gemm_reference(clock=clock)
        print(f"[bench] vendor GEMM reference: {gemm_ref['tflops']} TFLOP/s", file=sys.stderr,
              flush=True)
    cpu = head.get("cpu_baseline")

    extra = {}
    for c, r in results.items():
        if c == head_cfg:
            continue
        e = {"config": r["config"], "ms_per_step": round(r["timing"]["mean_ms"], 4),
             "median_ms": round(r["timing"]["median_ms"], 4), "roofline": r["roofline"]}
        e.update(side_measurements(r["timing"], r.get("flops_per_step"), "flop"))
        e["cpu_baseline"] = r.get("cpu_baseline")
        extra[f"config{c}"] = e

    line = {
        "metric": "attention TFLOP/s (prefill) and HBM GB/s (paged decode), % of MI355X peak",
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["timing"]["mean_ms"], 4),
        "median_ms": round(head["timing"]["median_ms"], 4),
        "min_ms": round(head["timing"]["min_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["config"]["dtype"],
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": head["config"],
        "roofline": head["roofline"],
        **side_measurements(head["timing"], head.get("flops_per_step"), "flop"),
        "cpu_baseline": cpu,
        "cpu_host": None if args.no_cpu_baseline else host_info(),
        "extra": extra,
        "mfma_context": gemm_ref,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
