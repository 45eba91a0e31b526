"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutation below is a plausible slip in an attention reference: a
top-left instead of bottom-right causal offset, an off-by-one in the visible
key count, a dropped or negated scale, K and V swapped, softmax over the wrong
axis, and two wrong page-table gathers.  The test patches the mutated
function into the oracle module, runs the pins named for it, and requires at
least one of them to raise.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import oracle_pins as pins

_orig_n_visible = oa.n_visible
_orig_probs = oa.attention_probs
_orig_attend = oa.attend_rows


def _top_left(Sq, Skv, causal):
    i = np.arange(Sq, dtype=np.int64)
    return np.full(Sq, Skv, dtype=np.int64) if not causal else np.clip(i + 1, 0, Skv)


def _off_by_one(Sq, Skv, causal):
    v = _orig_n_visible(Sq, Skv, causal)
    return np.clip(v - 1, 0, Skv) if causal else v


def _no_scale(q_rows, keys, scale, visible):
    return _orig_probs(q_rows, keys, 1.0, visible)


def _neg_scale(q_rows, keys, scale, visible):
    return _orig_probs(q_rows, keys, -scale, visible)


def _swap_kv(q_rows, keys, values, scale, visible):
    return _orig_probs(q_rows, values, scale, visible) @ keys


def _wrong_axis(q_rows, keys, scale, visible):
    skv = keys.shape[0]
    logits = scale * (q_rows @ keys.T)
    mask = np.arange(skv)[None, :] < np.asarray(visible)[:, None]
    w = np.where(mask, np.exp(logits - logits.max()), 0.0)
    return w / w.sum(axis=0, keepdims=True).clip(min=1e-300)


def _gather_slot_major(cache, page_row, n_tokens, page_size):
    n_pages = -(-n_tokens // page_size)
    pages = torch.as_tensor(np.asarray(page_row[:n_pages], dtype=np.int64))
    sel = cache[pages].transpose(0, 1)          # slot-major: wrong token order
    return sel.reshape(n_pages * page_size, *sel.shape[2:])[:n_tokens]


def _gather_from_end(cache, page_row, n_tokens, page_size):
    n_pages = -(-n_tokens // page_size)
    pages = torch.as_tensor(np.asarray(page_row[len(page_row) - n_pages:], dtype=np.int64))
    sel = cache[pages]
    return sel.reshape(n_pages * page_size, *sel.shape[2:])[:n_tokens]


def _kv_head_strided(h, H, H_kv):
    return h % H_kv


def _kv_head_reversed(h, H, H_kv):
    return H_kv - 1 - h // (H // H_kv)


def _extend_without_prefix(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, *,
                           scale=None, seqs=None):
    return _real_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens * 0, qo_start,
                        scale=scale, seqs=seqs)


def _extend_top_left(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, *,
                     scale=None, seqs=None):
    """New token i sees only i + 1 keys in all (causal mask not offset by the prefix)."""
    real = oa.n_visible
    try:
        oa.n_visible = lambda Sq, Skv, causal: np.clip(np.arange(Sq) + 1, 0, Skv)
        return _real_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start,
                            scale=scale, seqs=seqs)
    finally:
        oa.n_visible = real


_real_extend = oa.extend


def _bwd_without_delta(q, k, v, do, *, causal, scale=None, layout="BHSD"):
    """dS = P * dP (the row term sum_l P dP dropped)."""
    real = oa.attention_probs
    qf, kf, vf, gf = (oa._bhsd(oa.to_f64(t), layout) for t in (q, k, v, do))
    B, H, Sq, D = qf.shape
    H_kv, Skv = kf.shape[1], kf.shape[2]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    vis = oa.n_visible(Sq, Skv, causal)
    dq, dk, dv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    for b in range(B):
        for h in range(H):
            g = oa.kv_head(h, H, H_kv)
            P = real(qf[b, h], kf[b, g], scale, vis)
            dv[b, g] += P.T @ gf[b, h]
            dS = P * (gf[b, h] @ vf[b, g].T)
            dq[b, h] = scale * (dS @ kf[b, g])
            dk[b, g] += scale * (dS.T @ qf[b, h])
    return oa._bhsd(dq, layout), oa._bhsd(dk, layout), oa._bhsd(dv, layout)


def _bwd_unscaled(q, k, v, do, *, causal, scale=None, layout="BHSD"):
    """dQ and dK without the softmax scale."""
    dq, dk, dv = _real_bwd(q, k, v, do, causal=causal, scale=scale, layout=layout)
    D = dq.shape[-1]
    s = 1.0 / np.sqrt(D) if scale is None else scale
    return dq / s, dk / s, dv


_real_bwd = oa.sdpa_backward
_real_dq_rows = oa.sdpa_backward_dq_rows
_real_kv_rows = oa.sdpa_backward_kv_rows


def _dq_rows_unscaled(q, k, v, do, rows, *, causal, scale=None, layout="BHSD"):
    """Sampled dQ without the softmax scale."""
    D = q.shape[-1]
    s = 1.0 / np.sqrt(D) if scale is None else scale
    return _real_dq_rows(q, k, v, do, rows, causal=causal, scale=scale, layout=layout) / s


def _kv_rows_first_head_only(q, k, v, do, keys, *, causal, scale=None, layout="BHSD"):
    """Sampled dK, dV summed over the first query head of each group only (the
    other heads' dO zeroed, which removes exactly their terms)."""
    H_kv = k.shape[1] if layout == "BHSD" else k.shape[2]
    H = q.shape[1] if layout == "BHSD" else q.shape[2]
    do2 = do.clone()
    for h in range(H):
        if h % (H // H_kv):
            if layout == "BHSD":
                do2[:, h] = 0
            else:
                do2[:, :, h] = 0
    return _real_kv_rows(q, k, v, do2, keys, causal=causal, scale=scale, layout=layout)

MUTATIONS = [
    ("n_visible", _top_left, [pins.check_library_sdpa, pins.check_bruteforce]),
    ("n_visible", _off_by_one, [pins.check_causal_row0, pins.check_library_sdpa]),
    ("attention_probs", _no_scale, [pins.check_library_sdpa, pins.check_two_keys]),
    ("attention_probs", _neg_scale, [pins.check_library_sdpa, pins.check_dominant_key]),
    ("attend_rows", _swap_kv, [pins.check_ones_v, pins.check_library_sdpa]),
    ("attention_probs", _wrong_axis, [pins.check_ones_v, pins.check_probs_rows_sum_to_one]),
    ("gather_sequence", _gather_slot_major, [pins.check_decode_library]),
    ("gather_sequence", _gather_from_end, [pins.check_decode_library,
                                           pins.check_decode_matches_prefill_row]),
    ("kv_head", _kv_head_strided, [pins.check_gqa_library, pins.check_gqa_group_locality]),
    ("kv_head", _kv_head_reversed, [pins.check_gqa_library, pins.check_gqa_rows_and_decode]),
    ("extend", _extend_without_prefix, [pins.check_extend_library,
                                        pins.check_extend_one_token_is_decode]),
    ("extend", _extend_top_left, [pins.check_extend_library, pins.check_extend_chunking]),
    ("gather_sequence", _gather_slot_major, [pins.check_extend_library]),
    ("sdpa_backward", _bwd_without_delta, [pins.check_backward_autograd,
                                           pins.check_backward_closed_forms]),
    ("sdpa_backward", _bwd_unscaled, [pins.check_backward_autograd,
                                      pins.check_backward_finite_differences]),
    ("sdpa_backward_dq_rows", _dq_rows_unscaled, [pins.check_backward_sampled_rows_autograd]),
    ("sdpa_backward_kv_rows", _kv_rows_first_head_only,
     [pins.check_backward_sampled_rows_autograd]),
]


@pytest.mark.parametrize("name,bad,checks", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, bad, checks):
    monkeypatch.setattr(oa, name, bad)
    if hasattr(oracle, name):  # the package re-exports some functions by value
        monkeypatch.setattr(oracle, name, bad)
    caught = []
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError, RuntimeError) as e:
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"planted mistake {bad.__name__} in {name} passed every pin"


def test_unmutated_oracle_passes_the_same_checks():
    for _, _, checks in MUTATIONS:
        for check in checks:
            check()
