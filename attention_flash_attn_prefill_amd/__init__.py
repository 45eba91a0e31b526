"""Python binding of the MI355X attention library (libmi355attn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``.  PyTorch supplies
device memory and the current stream; nothing here computes attention, and
there is no CPU fallback: if the shared library is missing the calls raise.

Low-level functions carry the C names (``attn_prefill``,
``attn_prefill_gqa``, ``attn_prefill_lse``, ``attn_prefill_splitkv``,
``attn_prefill_bwd``, ``attn_paged_decode``, ``attn_paged_decode_gqa``, their
workspace-size and split-plan queries, ``attn_prefill_fp8``, ``attn_extend``,
``attn_extend_splitkv``, ``attn_status_string``) and take tensors or raw
integer pointers; ``prefill``, ``prefill_with_lse``, ``prefill_splitkv``,
``prefill_backward``, ``prefill_fp8``, ``paged_decode``, ``extend`` and
``extend_splitkv`` are conveniences that derive
the sizes (including the number of KV heads) from tensor shapes and allocate
the output.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmi355attn.so")

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = range(5)
ATTN_BHSD, ATTN_BSHD = 0, 1
ATTN_F16, ATTN_BF16 = 0, 1
ATTN_OUT_F32 = 0x100
ATTN_DECODE_SCRATCH_BYTES = 32 << 20  # the no-allocation decode's device array per GPU
LAYOUTS = {"BHSD": ATTN_BHSD, "BSHD": ATTN_BSHD}

# Every symbol include/attn.h declares, with its ctypes signature.
_VP, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_prefill": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _F, _VP]),
    "attn_paged_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "attn_paged_decode": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _F,
                               _VP, _SZ, _VP]),
    "attn_paged_decode_num_splits": (_I, [_I, _I, _I, _I, ctypes.POINTER(_I)]),
    "attn_prefill_gqa": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _VP]),
    "attn_paged_decode_gqa": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I,
                                   _F, _VP, _SZ, _VP]),
    "attn_paged_decode_gqa_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "attn_paged_decode_gqa_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I,
                                           _I, _I, _F, _VP]),
    "attn_paged_decode_gqa_num_splits": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "attn_prefill_fp8": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _F, _F,
                              _F, _VP]),
    "attn_extend": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I,
                         _I, _I, _I, _F, _VP]),
    "attn_prefill_lse": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                              _VP]),
    "attn_prefill_splitkv": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                  _VP, _SZ, _VP]),
    "attn_prefill_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "attn_prefill_splitkv_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "attn_extend_splitkv": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I,
                                 _I, _I, _I, _I, _I, _F, _VP, _SZ, _VP]),
    "attn_extend_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_extend_splitkv_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_prefill_bwd_workspace_size": (_SZ, [_I, _I, _I]),
    "attn_prefill_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I,
                              _I, _I, _I, _F, _VP, _SZ, _VP]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")


def load_library(path: str | None = None):
    """Load libmi355attn.so (built by ``build()``); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with "
                          "`python -m attention_flash_attn_prefill_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float16 or bfloat16)")


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_prefill(q, k, v, o, B, H, Sq, Skv, D, layout, dtype, causal, scale, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Sq, Skv, D,
                                       layout, dtype, int(bool(causal)), float(scale),
                                       _stream(stream))


def attn_prefill_gqa(q, k, v, o, B, H, H_kv, Sq, Skv, D, layout, dtype, causal, scale,
                     stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, H_kv, Sq,
                                           Skv, D, layout, dtype, int(bool(causal)),
                                           float(scale), _stream(stream))


def attn_prefill_lse(q, k, v, o, lse, B, H, H_kv, Sq, Skv, D, layout, dtype, causal, scale,
                     stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                           H_kv, Sq, Skv, D, layout, dtype, int(bool(causal)),
                                           float(scale), _stream(stream))


def attn_prefill_splitkv(q, k, v, o, B, H, H_kv, Sq, Skv, D, layout, dtype, causal, scale,
                         workspace, workspace_bytes, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, H_kv,
                                               Sq, Skv, D, layout, dtype, int(bool(causal)),
                                               float(scale), _ptr(workspace),
                                               int(workspace_bytes), _stream(stream))


def attn_prefill_splitkv_num_splits(B, H, Sq, Skv, D) -> int:
    return int(load_library().attn_prefill_splitkv_num_splits(B, H, Sq, Skv, D))


def attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D) -> int:
    return int(load_library().attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D))


def attn_prefill_bwd_workspace_size(B, H, Sq) -> int:
    return int(load_library().attn_prefill_bwd_workspace_size(B, H, Sq))


def attn_prefill_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, Sq, Skv, D, layout, dtype,
                     causal, scale, workspace, workspace_bytes, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B,
        H, H_kv, Sq, Skv, D, layout, dtype, int(bool(causal)), float(scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream))


def attn_paged_decode_gqa_workspace_size(B, H, H_kv, D, max_pages_per_seq, page_size) -> int:
    return int(load_library().attn_paged_decode_gqa_workspace_size(B, H, H_kv, D,
                                                                   max_pages_per_seq, page_size))


def attn_paged_decode_gqa_num_splits(B, H, H_kv, max_pages_per_seq, page_size):
    """Work plan of paged decode: (the largest number of equal work ranges a
    call cuts the batch's KV tiles into, the fewest tokens a range covers
    unless the batch holds fewer)."""
    tps = ctypes.c_int(0)
    n = load_library().attn_paged_decode_gqa_num_splits(B, H, H_kv, max_pages_per_seq,
                                                        page_size, ctypes.byref(tps))
    return int(n), int(tps.value)


def attn_paged_decode_gqa(q, k_cache, v_cache, page_table, seq_lens, o, B, H, H_kv, D,
                          page_size, num_pages, max_pages_per_seq, dtype, scale, workspace,
                          workspace_bytes, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_paged_decode_gqa(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), _ptr(o), B, H,
        H_kv, D, page_size, num_pages, max_pages_per_seq, dtype, float(scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream))


def attn_paged_decode_gqa_noalloc(q, k_cache, v_cache, page_table, seq_lens, o, B, H, H_kv, D,
                                  page_size, num_pages, max_pages_per_seq, dtype, scale,
                                  stream=None) -> int:
    """Direct call of the C entry point (no workspace: the library's own
    device array of ATTN_DECODE_SCRATCH_BYTES); returns its status code."""
    return load_library().attn_paged_decode_gqa_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), _ptr(o), B, H,
        H_kv, D, page_size, num_pages, max_pages_per_seq, dtype, float(scale), _stream(stream))


def attn_prefill_fp8(q, k, v, o, B, H, H_kv, Sq, Skv, D, layout, out_dtype, causal, scale,
                     q_descale, k_descale, v_descale, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_prefill_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, H_kv, Sq,
                                           Skv, D, layout, out_dtype, int(bool(causal)),
                                           float(scale), float(q_descale), float(k_descale),
                                           float(v_descale), _stream(stream))


def attn_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o, B, H, H_kv, D,
                total_tokens, max_extend_len, page_size, num_pages, max_pages_per_seq, dtype,
                scale, stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_extend(
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(prefix_lens), _ptr(qo_start), _ptr(o), B, H, H_kv, D, total_tokens, max_extend_len,
        page_size, num_pages, max_pages_per_seq, dtype, float(scale), _stream(stream))


def attn_extend_splitkv(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o, B, H,
                        H_kv, D, total_tokens, max_extend_len, page_size, num_pages,
                        max_pages_per_seq, dtype, scale, workspace, workspace_bytes,
                        stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_extend_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(prefix_lens), _ptr(qo_start), _ptr(o), B, H, H_kv, D, total_tokens, max_extend_len,
        page_size, num_pages, max_pages_per_seq, dtype, float(scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream))


def attn_extend_splitkv_num_splits(B, H, H_kv, D, total_tokens, max_extend_len,
                                   max_pages_per_seq) -> int:
    return int(load_library().attn_extend_splitkv_num_splits(B, H, H_kv, D, total_tokens,
                                                             max_extend_len, max_pages_per_seq))


def attn_extend_splitkv_workspace_size(B, H, H_kv, D, total_tokens, max_extend_len,
                                       max_pages_per_seq) -> int:
    return int(load_library().attn_extend_splitkv_workspace_size(
        B, H, H_kv, D, total_tokens, max_extend_len, max_pages_per_seq))


def attn_paged_decode_workspace_size(B, H, D, max_pages_per_seq, page_size) -> int:
    return int(load_library().attn_paged_decode_workspace_size(B, H, D, max_pages_per_seq,
                                                               page_size))


def attn_paged_decode_num_splits(B, H, max_pages_per_seq, page_size):
    """attn_paged_decode_gqa_num_splits with H_kv = H."""
    tps = ctypes.c_int(0)
    n = load_library().attn_paged_decode_num_splits(B, H, max_pages_per_seq, page_size,
                                                    ctypes.byref(tps))
    return int(n), int(tps.value)


def attn_paged_decode(q, k_cache, v_cache, page_table, seq_lens, o, B, H, D, page_size,
                      num_pages, max_pages_per_seq, dtype, scale, workspace, workspace_bytes,
                      stream=None) -> int:
    """Direct call of the C entry point; returns its status code."""
    return load_library().attn_paged_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(page_table), _ptr(seq_lens), _ptr(o), B, H, D,
                                            page_size, num_pages, max_pages_per_seq, dtype,
                                            float(scale), _ptr(workspace), int(workspace_bytes),
                                            _stream(stream))


def _check(status, where):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _out_code(q, out, out_dtype):
    """dtype code for the C call and the output dtype (q's, or fp32)."""
    import torch
    want = out.dtype if out is not None else (out_dtype or q.dtype)
    if out_dtype is not None and want != out_dtype:
        raise TypeError("out and out_dtype disagree")
    if want == q.dtype:
        return _dtype_code(q), want
    if want == torch.float32:
        return _dtype_code(q) | ATTN_OUT_F32, want
    raise TypeError(f"output dtype must be {q.dtype} or torch.float32, not {want}")


def _prefill_shapes(q, k, v, layout):
    """(B, H, H_kv, Sq, Skv, D) of contiguous 4-D GPU tensors in `layout`."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        H_kv, Skv = k.shape[1], k.shape[2]
        kv_shape = (B, H_kv, Skv, D)
    else:
        B, Sq, H, D = q.shape
        Skv, H_kv = k.shape[1], k.shape[2]
        kv_shape = (B, Skv, H_kv, D)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"k and v must have shape {kv_shape}")
    return B, H, H_kv, Sq, Skv, D


def _like(t, ref, dtype, name):
    """`t` checked to be a contiguous GPU tensor shaped like `ref`, or a new one."""
    import torch
    if t is None:
        return torch.empty(ref.shape, dtype=dtype, device=ref.device)
    if t.shape != ref.shape or not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor shaped like {tuple(ref.shape)}")
    return t


def prefill(q, k, v, *, causal=False, scale=None, layout="BHSD", out=None, out_dtype=None,
            stream=None):
    """O = softmax(Q K^T * scale [+ causal mask]) V on the GPU.

    q: [B,H,Sq,D] (layout "BHSD") or [B,Sq,H,D] ("BSHD"); k, v likewise with
    Skv keys and H_kv heads (H_kv divides H: grouped-query attention, query
    head h reads KV head h // (H // H_kv)); fp16 or bf16 GPU tensors,
    contiguous.  Returns o like q, or in fp32 (unrounded) with
    out_dtype=torch.float32 or an fp32 `out`.
    """
    B, H, H_kv, Sq, Skv, D = _prefill_shapes(q, k, v, layout)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code, odt = _out_code(q, out, out_dtype)
    o = _like(out, q, odt, "out")
    _check(attn_prefill_gqa(q, k, v, o, B, H, H_kv, Sq, Skv, D, LAYOUTS[layout], code,
                            causal, scale, stream), "attn_prefill_gqa")
    return o


def prefill_splitkv(q, k, v, *, causal=False, scale=None, layout="BHSD", out=None,
                    out_dtype=None, workspace=None, stream=None):
    """``prefill`` through attn_prefill_splitkv: for grids too small to fill
    the GPU (few query tiles against many keys) the keys are split over
    workgroups and the partial results merged.  `workspace` (a uint8 GPU
    tensor of at least attn_prefill_splitkv_workspace_size bytes) is
    allocated when not given."""
    import torch
    B, H, H_kv, Sq, Skv, D = _prefill_shapes(q, k, v, layout)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code, odt = _out_code(q, out, out_dtype)
    o = _like(out, q, odt, "out")
    need = attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(attn_prefill_splitkv(q, k, v, o, B, H, H_kv, Sq, Skv, D, LAYOUTS[layout], code,
                                causal, scale, workspace, nbytes, stream),
           "attn_prefill_splitkv")
    return o


def prefill_with_lse(q, k, v, *, causal=False, scale=None, layout="BHSD", out=None,
                     out_dtype=None, lse=None, stream=None):
    """``prefill`` that also returns the natural-log log-sum-exp of every
    query row's scaled scores: (o, lse) with lse [B, H, Sq] fp32 (-inf for a
    row with no visible key), the statistic ``prefill_backward`` needs."""
    import torch
    B, H, H_kv, Sq, Skv, D = _prefill_shapes(q, k, v, layout)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code, odt = _out_code(q, out, out_dtype)
    o = _like(out, q, odt, "out")
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_cuda
          or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 GPU tensor of shape {(B, H, Sq)}")
    _check(attn_prefill_lse(q, k, v, o, lse, B, H, H_kv, Sq, Skv, D, LAYOUTS[layout], code,
                            causal, scale, stream), "attn_prefill_lse")
    return o, lse


def prefill_backward(q, k, v, o, dO, lse, *, causal=False, scale=None, layout="BHSD",
                     grad_dtype=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(O * dO) for O = prefill(q, k, v) (same
    causal, scale and layout), given O and lse from ``prefill_with_lse``.

    dO is like q and in q's dtype.  The gradients are in q's dtype, or fp32
    with grad_dtype=torch.float32 (or fp32 dq/dk/dv).  With H_kv < H the
    query heads of a group sum into their KV head's dk, dv.  The workspace (a
    uint8 GPU tensor of ``attn_prefill_bwd_workspace_size`` bytes) is
    allocated here if not given.
    """
    import torch
    B, H, H_kv, Sq, Skv, D = _prefill_shapes(q, k, v, layout)
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dO.dtype):
        raise TypeError("q, k, v, o and dO must share a dtype")
    for t, name in ((o, "o"), (dO, "dO")):
        if t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor shaped like q")
    if (tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 GPU tensor of shape {(B, H, Sq)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    given = next((t for t in (dq, dk, dv) if t is not None), None)
    code, gdt = _out_code(q, given, grad_dtype)
    dq = _like(dq, q, gdt, "dq")
    dk = _like(dk, k, gdt, "dk")
    dv = _like(dv, v, gdt, "dv")
    need = attn_prefill_bwd_workspace_size(B, H, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(attn_prefill_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, Sq, Skv, D,
                            LAYOUTS[layout], code, causal, scale, workspace,
                            workspace.numel() * workspace.element_size(), stream),
           "attn_prefill_bwd")
    return dq, dk, dv


def paged_decode(q, k_cache, v_cache, page_table, seq_lens, *, scale=None, out=None,
                 out_dtype=None, workspace=None, stream=None):
    """Decode attention of q [B,H,D] against a paged cache [num_pages, 16, H_kv, D]
    (H_kv divides H; query head h reads KV head h // (H // H_kv)).

    page_table [B, max_pages] and seq_lens [B] are int32 GPU tensors.  The
    workspace (a uint8 GPU tensor) is allocated here if not given.  O is like
    q, or fp32 with out_dtype=torch.float32 or an fp32 `out`.  A page id
    outside the pool makes that sequence's output NaN (checked on the GPU).
    """
    import torch
    B, H, D = q.shape
    num_pages, page_size, H_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (num_pages, page_size, H_kv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, H_kv, D]")
    if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("page_table and seq_lens must be int32")
    for t in (q, k_cache, v_cache, page_table, seq_lens):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all inputs must be contiguous GPU tensors")
    max_pages = page_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = attn_paged_decode_gqa_workspace_size(B, H, H_kv, D, max_pages, page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    code, odt = _out_code(q, out, out_dtype)
    o = torch.empty(q.shape, dtype=odt, device=q.device) if out is None else out
    if o.shape != q.shape or not o.is_cuda or not o.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped like q")
    _check(attn_paged_decode_gqa(q, k_cache, v_cache, page_table, seq_lens, o, B, H, H_kv, D,
                                 page_size, num_pages, max_pages, code, scale, workspace,
                                 workspace.numel() * workspace.element_size(), stream),
           "attn_paged_decode_gqa")
    return o


def _extend_args(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, max_extend_len,
                 scale, out, out_dtype):
    """Checks of extend's tensors; returns (o, sizes...) for the C call."""
    import torch
    T, H, D = q.shape
    H_kv = k.shape[1]
    if tuple(k.shape) != (T, H_kv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [total_tokens, H_kv, D]")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape) != (num_pages, page_size, H_kv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, H_kv, D]")
    for t in (page_table, prefix_lens, qo_start):
        if t.dtype != torch.int32:
            raise TypeError("page_table, prefix_lens and qo_start must be int32")
    for t in (q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all inputs must be contiguous GPU tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype or q.dtype != k_cache.dtype:
        raise TypeError("q, k, v and the cache must share a dtype")
    B = prefix_lens.shape[0]
    if tuple(qo_start.shape) != (B + 1,) or page_table.shape[0] != B:
        raise ValueError("qo_start must be [B+1] and page_table [B, max_pages]")
    if max_extend_len is None:
        max_extend_len = int((qo_start[1:] - qo_start[:-1]).max().item()) if B else 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code, odt = _out_code(q, out, out_dtype)
    o = torch.empty(q.shape, dtype=odt, device=q.device) if out is None else out
    if o.shape != q.shape or not o.is_cuda or not o.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped like q")
    return o, (B, H, H_kv, D, T, max_extend_len, page_size, num_pages, page_table.shape[1],
               code, scale)


def extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, *, max_extend_len=None,
           scale=None, out=None, out_dtype=None, stream=None):
    """Extend attention: new tokens (q [T,H,D], k, v [T,H_kv,D], packed by
    qo_start [B+1]) after cached prefixes (k_cache, v_cache [P,16,H_kv,D],
    page_table [B,max_pages], prefix_lens [B]); see attn_extend in attn.h.

    max_extend_len bounds every sequence's new-token count; if omitted it is
    read from qo_start, which synchronises with the device.
    """
    o, a = _extend_args(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start,
                        max_extend_len, scale, out, out_dtype)
    _check(attn_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o, *a,
                       stream), "attn_extend")
    return o


def extend_splitkv(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, *,
                   max_extend_len=None, scale=None, out=None, out_dtype=None, workspace=None,
                   stream=None):
    """``extend`` with each unit's keys split over workgroups when the grid is
    too small to fill the GPU (see attn_extend_splitkv in attn.h).
    `workspace` (a uint8 GPU tensor of at least
    attn_extend_splitkv_workspace_size bytes) is allocated when not given."""
    import torch
    o, a = _extend_args(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start,
                        max_extend_len, scale, out, out_dtype)
    B, H, H_kv, D, T, mx, _, _, max_pages = a[:9]
    need = attn_extend_splitkv_workspace_size(B, H, H_kv, D, T, mx, max_pages)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(attn_extend_splitkv(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o,
                               *a, workspace, nbytes, stream), "attn_extend_splitkv")
    return o


def prefill_fp8(q, k, v, descales, *, causal=False, scale=None, layout="BHSD",
                out_dtype=None, out=None, stream=None):
    """FP8 prefill: q, k, v are torch.float8_e4m3fn GPU tensors (shapes as in
    ``prefill``), descales = (q_descale, k_descale, v_descale) per tensor.
    O is fp16 by default, or out_dtype / out's dtype (fp16, bf16, fp32)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors")
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError("q, k, v must be torch.float8_e4m3fn")
    if layout == "BHSD":
        B, H, Sq, D = q.shape
        H_kv, Skv = k.shape[1], k.shape[2]
        kv_shape = (B, H_kv, Skv, D)
    else:
        B, Sq, H, D = q.shape
        Skv, H_kv = k.shape[1], k.shape[2]
        kv_shape = (B, Skv, H_kv, D)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"k and v must have shape {kv_shape}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    odt = out.dtype if out is not None else (out_dtype or torch.float16)
    codes = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16,
             torch.float32: ATTN_F16 | ATTN_OUT_F32}
    if odt not in codes:
        raise TypeError("the output dtype must be float16, bfloat16 or float32")
    o = torch.empty(q.shape, dtype=odt, device=q.device) if out is None else out
    if o.shape != q.shape or not o.is_cuda or not o.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped like q")
    qd, kd, vd = descales
    _check(attn_prefill_fp8(q, k, v, o, B, H, H_kv, Sq, Skv, D, LAYOUTS[layout], codes[odt],
                            causal, scale, qd, kd, vd, stream), "attn_prefill_fp8")
    return o
