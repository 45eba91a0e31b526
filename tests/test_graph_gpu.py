"""The entry points are safe inside HIP graph capture (no allocation, no sync,
no host reads of device memory): a captured prefill + paged decode replays to
the eager results, several times, with eager work in between."""
import math

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_graph_capture_and_replay(gpu_lib):
    attn = gpu_lib
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in workloads.prefill_inputs(2, 4, 300, 520, 128, "bf16", "BSHD",
                                                           seed=31))
    b = workloads.paged_decode_inputs(B=8, H=8, D=128, page_size=16, num_pages=512,
                                      max_seq=900, seed=32)
    g = {n: getattr(b, n).to(dev) for n in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    ws = torch.empty(attn.attn_paged_decode_workspace_size(8, 8, 128, b.max_pages_per_seq, 16),
                     dtype=torch.uint8, device=dev)
    o_pre = torch.empty_like(q)
    o_dec = torch.empty_like(g["q"])

    def work(stream=None):
        attn.prefill(q, k, v, causal=True, layout="BSHD", out=o_pre, stream=stream)
        attn.paged_decode(g["q"], g["k_cache"], g["v_cache"], g["page_table"], g["seq_lens"],
                          out=o_dec, workspace=ws, stream=stream)

    work()
    torch.cuda.synchronize()
    ref_pre, ref_dec = o_pre.clone(), o_dec.clone()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o_pre.zero_()
        o_dec.zero_()
        with torch.cuda.graph(graph, stream=s):
            work(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for i in range(3):
        o_pre.fill_(float("nan"))
        o_dec.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_pre, ref_pre), f"prefill replay {i}"
        assert torch.equal(o_dec, ref_dec), f"decode replay {i}"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays


def test_graph_capture_backward_extend_fp8(gpu_lib):
    """The other entry points in one captured graph: forward with LSE,
    backward, extend after a paged prefix, fp8 prefill, grouped-query decode
    and split-KV prefill and extend, replayed three times against the eager
    results."""
    attn = gpu_lib
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in workloads.backward_inputs(1, 8, 200, 260, 128, "bf16",
                                                                "BSHD", amp=0.5, seed=33,
                                                                h_kv=2))
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, 200), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(attn.attn_prefill_bwd_workspace_size(1, 8, 200), dtype=torch.uint8,
                      device=dev)
    e = workloads.extend_inputs(3, 8, 128, [5, 0, 40], [30, 17, 9], "f16", seed=34, h_kv=2)
    ge = {n: getattr(e, n).to(dev) for n in ("q", "k", "v", "k_cache", "v_cache", "page_table",
                                             "prefix_lens", "qo_start")}
    o_ext = torch.empty_like(ge["q"])
    q8, k8, v8, desc = workloads.prefill_inputs_fp8(1, 4, 130, 150, 128, seed=35, h_kv=1)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o8 = torch.empty(q8.shape, dtype=torch.float16, device=dev)
    b = workloads.paged_decode_inputs(B=4, H=16, D=128, page_size=16, num_pages=256,
                                      max_seq=700, seed=36, h_kv=4)
    gd = {n: getattr(b, n).to(dev) for n in ("q", "k_cache", "v_cache", "page_table", "seq_lens")}
    dws = torch.empty(attn.attn_paged_decode_gqa_workspace_size(4, 16, 4, 128, b.max_pages_per_seq,
                                                                16),
                      dtype=torch.uint8, device=dev)
    o_dec = torch.empty_like(gd["q"])
    qs, ks, vs = (t.to(dev) for t in workloads.prefill_inputs(1, 4, 100, 3000, 128, "f16",
                                                              "BHSD", seed=37, h_kv=2))
    assert attn.attn_prefill_splitkv_num_splits(1, 4, 100, 3000, 128) > 1
    sws = torch.empty(attn.attn_prefill_splitkv_workspace_size(1, 4, 100, 3000, 128),
                      dtype=torch.uint8, device=dev)
    o_split = torch.empty_like(qs)
    x = workloads.extend_inputs(2, 8, 128, [1700, 300], [90, 40], "bf16", seed=38, h_kv=2)
    gx = {n: getattr(x, n).to(dev) for n in ("q", "k", "v", "k_cache", "v_cache", "page_table",
                                             "prefix_lens", "qo_start")}
    xargs = (2, 8, 2, 128, x.q.shape[0], x.max_extend_len, x.page_table.shape[1])
    assert attn.attn_extend_splitkv_num_splits(*xargs) > 1
    xws = torch.empty(attn.attn_extend_splitkv_workspace_size(*xargs), dtype=torch.uint8,
                      device=dev)
    o_xsplit = torch.empty_like(gx["q"])
    outs = (o, lse, dq, dk, dv, o_ext, o8, o_dec, o_split, o_xsplit)

    def work(stream=None):
        attn.prefill_with_lse(q, k, v, causal=True, layout="BSHD", out=o, lse=lse, stream=stream)
        attn.prefill_backward(q, k, v, o, do, lse, causal=True, layout="BSHD", dq=dq, dk=dk,
                              dv=dv, workspace=bws, stream=stream)
        attn.extend(ge["q"], ge["k"], ge["v"], ge["k_cache"], ge["v_cache"], ge["page_table"],
                    ge["prefix_lens"], ge["qo_start"], max_extend_len=e.max_extend_len,
                    out=o_ext, stream=stream)
        attn.prefill_fp8(q8, k8, v8, desc, causal=True, out=o8, stream=stream)
        attn.paged_decode(gd["q"], gd["k_cache"], gd["v_cache"], gd["page_table"],
                          gd["seq_lens"], out=o_dec, workspace=dws, stream=stream)
        attn.prefill_splitkv(qs, ks, vs, causal=True, out=o_split, workspace=sws, stream=stream)
        attn.extend_splitkv(gx["q"], gx["k"], gx["v"], gx["k_cache"], gx["v_cache"],
                            gx["page_table"], gx["prefix_lens"], gx["qo_start"],
                            max_extend_len=x.max_extend_len, out=o_xsplit, workspace=xws,
                            stream=stream)

    print("[case] graph capture of lse/backward/extend/fp8/gqa decode/split-kv prefill and "
          "extend", flush=True)
    work()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in outs:
            t.zero_()
        with torch.cuda.graph(graph, stream=s):
            work(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, (t, r) in enumerate(zip(outs, refs)):
            assert torch.equal(t, r), f"output {n}, replay {i}"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays
