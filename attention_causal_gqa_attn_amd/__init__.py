"""Causal grouped-query flash attention for AMD Instinct MI355X (gfx950).

Thin Python binding of libfa.so, whose C ABI is include/fa.h. This module only marshals
arguments: torch tensors become device pointers and sizes, torch's current HIP stream becomes
the stream argument, and a non-zero status becomes an FAError. Every step of the attention
runs in the HIP kernels of libfa.so; there is no Python or CPU fallback, and if the library is
missing every call raises.

Raw entry points with the C names (pointers and ints): fa_prefill, fa_prefill_split,
fa_prefill_workspace_bytes, fa_decode, fa_decode_paged, fa_prefill_paged,
fa_decode_workspace_bytes, fa_decode_noalloc, fa_standard_attention,
fa_standard_workspace_bytes, fa_prefill_stats, fa_decode_stats, fa_dequant_q4_0,
fa_quantize_q4_0, fa_strerror, fa_version.
Tensor helpers: prefill, prefill_split, prefill_workspace_bytes, prefill_paged, decode,
decode_paged, decode_workspace_bytes, standard_attention, standard_workspace_bytes,
prefill_stats, decode_stats, dequant_q4_0, quantize_q4_0.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# the library built in this directory; FA_LIBRARY names another build of the same sources (the
# sanitizer test loads a host-instrumented one this way)
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libfa.so")

FA_KV_F16, FA_KV_BF16, FA_KV_Q4_0 = 0, 1, 2
FA_KV_F16_Q4_0, FA_KV_Q4_0_F16 = 3, 4          # mixed caches: (K type, V type)
FA_SRC_F32, FA_SRC_F16, FA_SRC_BF16 = 0, 1, 2
Q4_0_BYTES = 18

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_DTYPE = -3
FA_ERR_UNSUPPORTED = -4
FA_ERR_WORKSPACE = -5
FA_ERR_ALIGN = -6
FA_ERR_HIP = -7
FA_ERR_VALUE = -8
FA_ERR_TOO_LARGE = -9
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("fa_prefill", "fa_prefill_split", "fa_prefill_workspace_bytes", "fa_decode",
           "fa_decode_paged", "fa_prefill_paged", "fa_decode_workspace_bytes", "fa_decode_noalloc",
           "fa_standard_attention", "fa_standard_workspace_bytes", "fa_prefill_stats",
           "fa_decode_stats", "fa_dequant_q4_0", "fa_quantize_q4_0", "fa_measure_read",
           "fa_strerror", "fa_version")
PAGE_KEYS = 64


class FAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_strerror(code)} (status {code})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m attention_causal_gqa_attn_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                 ctypes.c_size_t)
        attn = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, f32, i32]
        lib.fa_prefill.argtypes = attn + [vp]
        lib.fa_prefill.restype = i32
        lib.fa_prefill_split.argtypes = attn + [vp, sz, vp]
        lib.fa_prefill_split.restype = i32
        lib.fa_prefill_workspace_bytes.argtypes = [i32] * 7 + [i64, i32]
        lib.fa_prefill_workspace_bytes.restype = sz
        lib.fa_decode.argtypes = attn + [vp, sz, vp]
        lib.fa_decode.restype = i32
        lib.fa_decode_noalloc.argtypes = attn + [vp]
        lib.fa_decode_noalloc.restype = i32
        lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        i32, i32, f32, i32, vp, sz, vp]
        lib.fa_decode_paged.restype = i32
        lib.fa_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, i32, i32, f32, i32, vp]
        lib.fa_prefill_paged.restype = i32
        lib.fa_decode_workspace_bytes.argtypes = [i32] * 6
        lib.fa_decode_workspace_bytes.restype = sz
        lib.fa_standard_attention.argtypes = attn + [vp, sz, vp]
        lib.fa_standard_attention.restype = i32
        lib.fa_standard_workspace_bytes.argtypes = [i32] * 8
        lib.fa_standard_workspace_bytes.restype = sz
        lib.fa_prefill_stats.argtypes = attn + [vp, vp]
        lib.fa_prefill_stats.restype = i32
        lib.fa_decode_stats.argtypes = attn + [vp, sz, vp, vp]
        lib.fa_decode_stats.restype = i32
        lib.fa_dequant_q4_0.argtypes = [vp, i64, vp, vp, vp]
        lib.fa_dequant_q4_0.restype = i32
        lib.fa_quantize_q4_0.argtypes = [vp, i32, vp, i64, i64, i32, i64, i64, vp]
        lib.fa_quantize_q4_0.restype = i32
        lib.fa_measure_read.argtypes = [vp, i64, vp, ctypes.c_uint32, i32, vp]
        lib.fa_measure_read.restype = i32
        lib.fa_strerror.argtypes = [i32]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = i32
        _lib = lib
    return _lib


# ---- raw C entry points ---------------------------------------------------------------------

def fa_prefill(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
               stream) -> int:
    return load().fa_prefill(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale,
                             kv_dtype, stream)


def fa_prefill_split(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
                     workspace, workspace_bytes, stream) -> int:
    return load().fa_prefill_split(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, workspace, workspace_bytes, stream)


def fa_prefill_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, kv_dtype) -> int:
    return load().fa_prefill_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                             kv_dtype)


def fa_decode(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
              workspace, workspace_bytes, stream) -> int:
    return load().fa_decode(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale,
                            kv_dtype, workspace, workspace_bytes, stream)


def fa_decode_noalloc(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
                      stream) -> int:
    return load().fa_decode_noalloc(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                    scale, kv_dtype, stream)


def fa_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) -> int:
    return load().fa_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)


def fa_standard_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale,
                          kv_dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_standard_attention(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                        scale, kv_dtype, workspace, workspace_bytes, stream)


def fa_standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv_dtype, units_per_pass) -> int:
    return load().fa_standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv_dtype, units_per_pass)


def fa_prefill_stats(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
                     counts, stream) -> int:
    return load().fa_prefill_stats(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                   scale, kv_dtype, counts, stream)


def fa_decode_stats(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset, scale, kv_dtype,
                    workspace, workspace_bytes, counts, stream) -> int:
    return load().fa_decode_stats(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, causal_offset,
                                  scale, kv_dtype, workspace, workspace_bytes, counts, stream)


def fa_dequant_q4_0(blocks, n_blocks, out_f32, out_f16, stream) -> int:
    return load().fa_dequant_q4_0(blocks, n_blocks, out_f32, out_f16, stream)


def fa_prefill_paged(q, k_pages, v_pages, o, block_table, seq_lens, q_lens, B, Hq, Hkv, Sq, D,
                     max_pages, n_pages, causal, scale, kv_dtype, stream) -> int:
    return load().fa_prefill_paged(q, k_pages, v_pages, o, block_table, seq_lens, q_lens, B, Hq,
                                   Hkv, Sq, D, max_pages, n_pages, causal, scale, kv_dtype,
                                   stream)


def fa_decode_paged(q, k_pages, v_pages, o, block_table, seq_lens, B, Hq, Hkv, Sq, D,
                    max_pages, n_pages, causal, scale, kv_dtype, workspace, workspace_bytes,
                    stream) -> int:
    return load().fa_decode_paged(q, k_pages, v_pages, o, block_table, seq_lens, B, Hq, Hkv, Sq,
                                  D, max_pages, n_pages, causal, scale, kv_dtype, workspace,
                                  workspace_bytes, stream)


def fa_quantize_q4_0(x, x_dtype, blocks, n_seq, rows_per_seq, D, x_seq_stride,
                     blocks_seq_stride, stream) -> int:
    return load().fa_quantize_q4_0(x, x_dtype, blocks, n_seq, rows_per_seq, D, x_seq_stride,
                                   blocks_seq_stride, stream)


def fa_measure_read(buf, nbytes, sink, magic, workgroups, stream) -> int:
    return load().fa_measure_read(buf, nbytes, sink, magic, workgroups, stream)


def fa_strerror(code: int) -> str:
    return load().fa_strerror(code).decode()


def fa_version() -> int:
    return load().fa_version()


# ---- tensor helpers -------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _one_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_KV_F16
    if t.dtype == torch.bfloat16:
        return FA_KV_BF16
    if t.dtype == torch.uint8:
        return FA_KV_Q4_0
    raise TypeError(f"unsupported K/V dtype {t.dtype}")


def _kv_code(k, v=None) -> int:
    """The cache code of K and V (float16, bfloat16, or uint8 q4_0 blocks); K and V of
    different types give a mixed code (f16 with q4_0 only)."""
    ck = _one_code(k)
    cv = ck if v is None else _one_code(v)
    if ck == cv:
        return ck
    pair = {(FA_KV_F16, FA_KV_Q4_0): FA_KV_F16_Q4_0, (FA_KV_Q4_0, FA_KV_F16): FA_KV_Q4_0_F16}
    if (ck, cv) not in pair:
        raise TypeError(f"unsupported K/V dtype pair {k.dtype}, {v.dtype}")
    return pair[(ck, cv)]


def _row_width(code, D) -> int:
    return D // 32 * Q4_0_BYTES if code == FA_KV_Q4_0 else D


def _kv_parts(kv):
    """(K type, V type) of a cache code."""
    return {FA_KV_F16_Q4_0: (FA_KV_F16, FA_KV_Q4_0),
            FA_KV_Q4_0_F16: (FA_KV_Q4_0, FA_KV_F16)}.get(kv, (kv, kv))


def _stream(t, stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return int(_torch().cuda.current_stream(t.device).cuda_stream)


def _q_dtype(kv):
    """Q and O element type of a cache code: bfloat16 for bf16 caches, float16 otherwise."""
    torch = _torch()
    return torch.bfloat16 if kv == FA_KV_BF16 else torch.float16


def _check_q(q, kv):
    if q.dtype != _q_dtype(kv):
        raise ValueError(f"q is {q.dtype}; this cache type takes {_q_dtype(kv)} queries")


def _check_device(q, **others):
    """Every tensor must live on q's GPU: a host tensor's address or another device's would
    reach the kernels as a wild pointer. Runs after the dtype and shape checks, so those are
    testable with host tensors."""
    if q.device.type != "cuda":
        raise ValueError(f"q is on {q.device}; the kernels need GPU tensors")
    for name, t in others.items():
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")


def _check_out(out, q):
    if out is None:
        return
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {q.dtype} tensor of q's shape "
                         f"{tuple(q.shape)} (got {out.dtype} {tuple(out.shape)})")


def _check_workspace(ws):
    if ws is not None and not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _sizes(q, k, v, kv):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-d: [B, S, H, D] (q4_0: [B, S, H, D/32*18] bytes)")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.shape[:3] != v.shape[:3]:
        raise ValueError("k and v shapes differ")
    _check_q(q, kv)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, _ = k.shape
    if Bk != B:
        raise ValueError("batch sizes differ")
    _check_widths(k, v, kv, D)
    return B, Hq, Hkv, Sq, Sk, D


def _check_widths(k, v, kv, D):
    for name, t, code in (("k", k, _kv_parts(kv)[0]), ("v", v, _kv_parts(kv)[1])):
        if t.shape[-1] != _row_width(code, D):
            raise ValueError(f"{name} last dim {t.shape[-1]}, expected {_row_width(code, D)}")


def prefill(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
            scale: Optional[float] = None, out=None, stream=None):
    """O = softmax(scale * Q K^T + causal mask) V via fa_prefill. K/V dtype selects the cache
    type (float16, bfloat16, or uint8 q4_0 blocks). offset defaults to Sk - Sq."""
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_out(out, q)
    _check_device(q, k=k, v=v, out=out)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = _torch().empty_like(q)
    rc = fa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq,
                    Sk, D, int(bool(causal)), offset, scale, kv, _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_prefill")
    return out


def prefill_workspace_bytes(q, k, v, *, causal: bool = True, offset: Optional[int] = None) -> int:
    """Workspace bytes fa_prefill_split needs for these tensors (0: nothing to split)."""
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    offset = Sk - Sq if offset is None else int(offset)
    return fa_prefill_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), offset, kv)


def prefill_split(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
                  scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """Causal prefill balanced across workgroups via fa_prefill_split. A zero-filled
    workspace of prefill_workspace_bytes(...) bytes is allocated when none is given; a
    workspace passed in must have had its first 4096 bytes zero before its first use (every
    call leaves them zero)."""
    torch = _torch()
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_out(out, q)
    _check_workspace(workspace)
    _check_device(q, k=k, v=v, out=out, workspace=workspace)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = fa_prefill_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), offset, kv)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = fa_prefill_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv,
                          Sq, Sk, D, int(bool(causal)), offset, scale, kv, workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_prefill_split")
    return out


def decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D) -> int:
    return fa_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)


def decode(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
           scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """Split-K decode via fa_decode (Sq * Hq / Hkv <= 16). A workspace tensor of
    decode_workspace_bytes(...) bytes is allocated when none is given."""
    torch = _torch()
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_out(out, q)
    _check_workspace(workspace)
    _check_device(q, k=k, v=v, out=out, workspace=workspace)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq, Sk,
                   D, int(bool(causal)), offset, scale, kv, workspace.data_ptr(),
                   workspace.numel() * workspace.element_size(), _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_decode")
    return out


def standard_workspace_bytes(q, k, v, units_per_pass: int = 0) -> int:
    """Workspace bytes of fa_standard_attention for these tensors, units_per_pass (b, KV head)
    units at a time (0: all of them, 1: the minimum)."""
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    return fa_standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv, int(units_per_pass))


def standard_attention(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
                       scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """Standard (non-flash) attention via fa_standard_attention: a q4_0 K / V dequantized to
    f16, S = scale Q K^T materialised, row softmax, P V. A workspace for every unit at once is
    allocated when none is given (256-byte aligned)."""
    torch = _torch()
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_out(out, q)
    _check_workspace(workspace)
    _check_device(q, k=k, v=v, out=out, workspace=workspace)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = fa_standard_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv, 0)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    rc = fa_standard_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq,
                               Hkv, Sq, Sk, D, int(bool(causal)), offset, scale, kv,
                               workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_standard_attention")
    return out


def prefill_stats(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
                  scale: Optional[float] = None, stream=None):
    """fa_prefill_stats: (out, counts) with counts int32 [B, Sq, Hq, 2] (frame moves per row,
    tiles in which the row's wave ran the O rescale)."""
    torch = _torch()
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_device(q, k=k, v=v)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q)
    counts = torch.zeros((B, Sq, Hq, 2), dtype=torch.int32, device=q.device)
    rc = fa_prefill_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv,
                          Sq, Sk, D, int(bool(causal)), offset, scale, kv, counts.data_ptr(),
                          _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_prefill_stats")
    return out, counts


def decode_stats(q, k, v, *, causal: bool = True, offset: Optional[int] = None,
                 scale: Optional[float] = None, stream=None):
    """fa_decode_stats: (out, counts) with counts int32 [B, Sq, Hq, 2] (frame moves summed over
    the splits, splits that held keys)."""
    torch = _torch()
    kv = _kv_code(k, v)
    B, Hq, Hkv, Sq, Sk, D = _sizes(q, k, v, kv)
    _check_device(q, k=k, v=v)
    offset = Sk - Sq if offset is None else int(offset)
    scale = D ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q)
    counts = torch.zeros((B, Sq, Hq, 2), dtype=torch.int32, device=q.device)
    nbytes = decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = fa_decode_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv,
                         Sq, Sk, D, int(bool(causal)), offset, scale, kv, ws.data_ptr(),
                         ws.numel(), counts.data_ptr(), _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_stats")
    return out, counts


def _paged_sizes(q, k_pages, v_pages, block_table, seq_lens, q_lens=None):
    torch = _torch()
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens), ("q_lens", q_lens)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages]")
    if k_pages.dim() != 4 or k_pages.shape[1] != PAGE_KEYS or q.dim() != 4:
        raise ValueError("pages must be [n_pages, 64, Hkv, row]; q [B, Sq, Hq, D]")
    if not (q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous()):
        raise ValueError("q and the pages must be contiguous")
    B, Sq, Hq, D = q.shape
    n_pages, _, Hkv, _ = k_pages.shape
    if (block_table.shape[0] != B or seq_lens.numel() != B
            or v_pages.shape[:3] != k_pages.shape[:3]
            or (q_lens is not None and q_lens.numel() != B)):
        raise ValueError("block_table, seq_lens, q_lens and pages disagree with q")
    kv = _kv_code(k_pages, v_pages)
    _check_q(q, kv)
    _check_widths(k_pages, v_pages, kv, D)
    return B, Hq, Hkv, Sq, D, block_table.shape[1], n_pages


def prefill_paged(q, k_pages, v_pages, block_table, seq_lens, q_lens=None, *,
                  causal: bool = True, scale: Optional[float] = None, out=None, stream=None):
    """Prefill over paged caches via fa_prefill_paged. Pages, block_table and seq_lens as
    decode_paged; q_lens: int32 [B] or None (Sq each). Sequence b's q_lens[b] queries are rows
    [0, q_lens[b]) of q[b], its last q_lens[b] positions; rows past them of out are not
    written (out defaults to zeros)."""
    torch = _torch()
    kv = _kv_code(k_pages, v_pages)
    B, Hq, Hkv, Sq, D, max_pages, n_pages = _paged_sizes(q, k_pages, v_pages, block_table,
                                                         seq_lens, q_lens)
    _check_out(out, q)
    _check_device(q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
                  seq_lens=seq_lens, q_lens=q_lens, out=out)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.zeros_like(q)
    rc = fa_prefill_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                          block_table.data_ptr(), seq_lens.data_ptr(),
                          0 if q_lens is None else q_lens.data_ptr(), B, Hq, Hkv, Sq, D,
                          max_pages, n_pages, int(bool(causal)), scale, kv, _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_prefill_paged")
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, *, causal: bool = True,
                 scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """Split-K decode over paged caches via fa_decode_paged. k_pages, v_pages: [n_pages, 64,
    Hkv, D] (q4_0: uint8 [n_pages, 64, Hkv, D/32*18]); block_table: int32 [B, max_pages];
    seq_lens: int32 [B]. Sequence b's Sq queries are its last Sq positions."""
    torch = _torch()
    kv = _kv_code(k_pages, v_pages)
    B, Hq, Hkv, Sq, D, max_pages, n_pages = _paged_sizes(q, k_pages, v_pages, block_table,
                                                         seq_lens)
    _check_out(out, q)
    _check_workspace(workspace)
    _check_device(q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
                  seq_lens=seq_lens, out=out, workspace=workspace)
    scale = D ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = decode_workspace_bytes(B, Hq, Hkv, Sq, max_pages * PAGE_KEYS, D)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                         block_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, Sq, D,
                         max_pages, n_pages, int(bool(causal)), scale, kv, workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), _stream(q, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_decode_paged")
    return out


def dequant_q4_0(blocks, stream=None):
    """q4_0 blocks (uint8 device tensor, 18 bytes each) -> (float32 values, float16 values)."""
    torch = _torch()
    if blocks.dtype != torch.uint8 or not blocks.is_contiguous() or blocks.numel() % 18:
        raise ValueError("blocks must be a contiguous uint8 tensor of whole 18-byte blocks")
    _check_device(blocks)
    n = blocks.numel() // 18
    f32 = torch.empty(n * 32, dtype=torch.float32, device=blocks.device)
    f16 = torch.empty(n * 32, dtype=torch.float16, device=blocks.device)
    rc = fa_dequant_q4_0(blocks.data_ptr(), n, f32.data_ptr(), f16.data_ptr(),
                         _stream(blocks, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_dequant_q4_0")
    return f32, f16


def quantize_q4_0(x, out=None, stream=None):
    """q4_0 cache writer via fa_quantize_q4_0: a contiguous float32 / float16 / bfloat16 tensor
    [..., D] (D a multiple of 32) -> uint8 q4_0 blocks [..., D/32*18]. With `out` (a uint8 view
    whose rows of D/32*18 bytes are contiguous within out's first dimension, e.g. the positions
    [pos, pos + S_new) of a [B, Smax, Hkv, D/32*18] cache with x of [B, S_new, Hkv, D]) the
    blocks are written there."""
    torch = _torch()
    codes = {torch.float32: FA_SRC_F32, torch.float16: FA_SRC_F16, torch.bfloat16: FA_SRC_BF16}
    if x.dtype not in codes or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous float32, float16 or bfloat16 tensor")
    D = x.shape[-1]
    rowb = D // 32 * Q4_0_BYTES
    if out is None:
        out = torch.empty(*x.shape[:-1], rowb, dtype=torch.uint8, device=x.device)
    if out.dtype != torch.uint8 or tuple(out.shape) != (*x.shape[:-1], rowb):
        raise ValueError("out must be uint8 of x's shape with D/32*18 bytes last")
    if not (out[0] if out.dim() > 1 else out).is_contiguous():
        raise ValueError("out's rows must be contiguous within its first dimension")
    _check_device(x, out=out)
    n_seq = x.shape[0] if x.dim() > 1 else 1
    rows = x.numel() // D // max(n_seq, 1) if x.numel() else 0
    x_stride = x.stride(0) if x.dim() > 1 else x.numel()
    o_stride = out.stride(0) if out.dim() > 1 else out.numel()
    rc = fa_quantize_q4_0(x.data_ptr(), codes[x.dtype], out.data_ptr(), n_seq, rows, D,
                          x_stride, o_stride, _stream(x, stream))
    if rc != FA_OK:
        raise FAError(rc, "fa_quantize_q4_0")
    return out
