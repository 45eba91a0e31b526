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
