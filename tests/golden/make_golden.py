"""Writes tests/golden/oracle_tiny.json: fp64 oracle outputs on tiny seeded inputs.

Calls only ``oracle`` and ``workloads``.  The stored values guard the oracle
against silent drift: a later change to its arithmetic must change this file
in the same commit, with the reason.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle      # noqa: E402
import workloads   # noqa: E402

CASES = [
    dict(B=1, H=2, Sq=5, Skv=7, D=4, dtype="f16", layout="BHSD", causal=True, seed=1001),
    dict(B=1, H=1, Sq=6, Skv=6, D=8, dtype="bf16", layout="BSHD", causal=False, seed=1002),
    dict(B=1, H=4, h_kv=2, Sq=4, Skv=6, D=4, dtype="f16", layout="BSHD", causal=True, seed=1004),
]
EXTEND = dict(B=2, H=2, D=4, prefix_lens=[3, 17], extend_lens=[2, 4], dtype="f16", seed=1006,
              h_kv=1)
DECODE_GQA = dict(B=2, H=4, h_kv=1, D=4, dtype="bf16", page_size=16, num_pages=8, seed=1005,
                  seq_lens=[3, 18])
DECODE = dict(B=3, H=2, D=4, dtype="f16", page_size=16, num_pages=8, seed=1003,
              seq_lens=[1, 16, 21])
BACKWARD = dict(B=1, H=2, Sq=5, Skv=7, D=4, dtype="f16", layout="BSHD", causal=True, seed=1007,
                h_kv=1)
FP8 = dict(B=1, H=2, Sq=4, Skv=6, D=8, layout="BHSD", causal=True, seed=1008, h_kv=2)


def build():
    out = {"prefill": [], "decode": None}
    for c in CASES:
        q, k, v = workloads.prefill_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                           c["layout"], seed=c["seed"], h_kv=c.get("h_kv"))
        o = oracle.sdpa(q, k, v, causal=c["causal"], layout=c["layout"])
        out["prefill"].append(dict(case=c, out=o.round(15).tolist()))
    b = workloads.paged_decode_inputs(**DECODE)
    o = oracle.paged_decode(b.q, b.k_cache, b.v_cache, b.page_table, b.seq_lens)
    out["decode"] = dict(case=DECODE, out=o.round(15).tolist())
    b = workloads.paged_decode_inputs(**DECODE_GQA)
    o = oracle.paged_decode(b.q, b.k_cache, b.v_cache, b.page_table, b.seq_lens)
    out["decode_gqa"] = dict(case=DECODE_GQA, out=o.round(15).tolist())
    e = workloads.extend_inputs(**EXTEND)
    o = oracle.extend(e.q, e.k, e.v, e.k_cache, e.v_cache, e.page_table, e.prefix_lens,
                      e.qo_start)
    out["extend"] = dict(case=EXTEND, out=o.round(15).tolist())
    c = BACKWARD
    q, k, v, do = workloads.backward_inputs(c["B"], c["H"], c["Sq"], c["Skv"], c["D"], c["dtype"],
                                            c["layout"], seed=c["seed"], h_kv=c["h_kv"])
    grads = oracle.sdpa_backward(q, k, v, do, causal=c["causal"], layout=c["layout"])
    lse = oracle.lse_rows(q, k, causal=c["causal"], layout=c["layout"])
    out["backward"] = dict(case=BACKWARD, dq=grads[0].round(15).tolist(),
                           dk=grads[1].round(15).tolist(), dv=grads[2].round(15).tolist(),
                           lse=lse.round(15).tolist())
    c = FP8
    q8, k8, v8, (qd, kd, vd) = workloads.prefill_inputs_fp8(c["B"], c["H"], c["Sq"], c["Skv"],
                                                             c["D"], c["layout"], seed=c["seed"],
                                                             h_kv=c["h_kv"])
    qf, kf, vf = (oracle.dequantize_fp8(t, d) for t, d in ((q8, qd), (k8, kd), (v8, vd)))
    o = oracle.sdpa(qf, kf, vf, causal=c["causal"], layout=c["layout"])
    out["fp8"] = dict(case=FP8, out=o.round(15).tolist())
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
