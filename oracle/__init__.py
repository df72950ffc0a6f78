"""CPU oracle for causal grouped-query attention — test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
It wraps liboracle.so (plain C, fa_oracle.c), which computes the plain definition
O = softmax(scale * Q K^T + causal mask) V in f32: a product, a softmax, a second product
(mlxcel PR #2306, commit message 2; mi210-llm-stack build guide, Verification). It shares no
code with the HIP path and never calls it.

It also holds the q4_0 cache writer's reference (quantize_q4_0: d = f16(max|x| / 8), codes
clamp(round_half_away(x / d) + 8, 0, 15)), a reading of the q4_0 format the pages name.

Argument conventions: q is [B, Sq, Hq, D] as numpy float16 (f16) or uint16 bit patterns
(bf16); k and v are [B, Sk, Hkv, D] in the same way, or uint8 [B, Sk, Hkv, D/32*18] q4_0
blocks. Results are float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

F16, BF16, Q4_0 = 0, 1, 2
_CODES = {"f16": F16, "bf16": BF16, "q4_0": Q4_0}


def _code(dtype) -> int:
    return _CODES[dtype] if isinstance(dtype, str) else int(dtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _shapes(q, k, kv_dtype):
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv = k.shape[:3]
    if Bk != B:
        raise ValueError("q and k batch sizes disagree")
    _check_rows(k, kv_dtype, D)
    return B, Sq, Hq, Sk, Hkv, D


def _check_rows(x, dtype, D):
    if _code(dtype) == Q4_0:
        if D % 32 or x.shape[3] != D // 32 * 18:
            raise ValueError("q4_0 rows must hold D/32 blocks of 18 bytes")
    elif x.shape[3] != D:
        raise ValueError("cache head dim disagrees with q")


class Oracle:
    """The oracle functions bound to one build of fa_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        lib.orc_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                      i64, f32, vp, i64, vp, i32]
        lib.orc_attention_kv.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                         i32, i32, i64, f32, vp, i64, vp, i32]
        lib.orc_probs.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i64,
                                  f32, i64, vp]
        lib.orc_dequant_q4_0.argtypes = [vp, i64, vp, vp]
        lib.orc_half_to_float.argtypes = [vp, i64, vp]
        lib.orc_float_to_half.argtypes = [vp, i64, vp]
        lib.orc_quantize_q4_0.argtypes = [vp, i32, i64, vp]
        for fn in (lib.orc_attention, lib.orc_attention_kv, lib.orc_probs,
                   lib.orc_dequant_q4_0, lib.orc_half_to_float, lib.orc_float_to_half,
                   lib.orc_quantize_q4_0):
            fn.restype = i32
        self.path = path
        self.lib = lib

    def attention(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, *, q_dtype, kv_dtype,
                  causal: bool = True, offset: Optional[int] = None,
                  scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
                  threads: int = 0, v_dtype=None) -> np.ndarray:
        """Attention output in float32.

        Without `rows` the result has q's [B, Sq, Hq, D] shape. With `rows` (flattened indices
        (b * Sq + i) * Hq + h) the result is [len(rows), D]. offset defaults to Sk - Sq and
        scale to 1/sqrt(D). kv_dtype is K's cache type and, unless v_dtype is given, V's.
        """
        q, k, v = _c(q), _c(k), _c(v)
        B, Sq, Hq, Sk, Hkv, D = _shapes(q, k, kv_dtype)
        v_dtype = kv_dtype if v_dtype is None else v_dtype
        if v.shape[:3] != k.shape[:3]:
            raise ValueError("k and v shapes differ")
        _check_rows(v, v_dtype, D)
        offset = Sk - Sq if offset is None else int(offset)
        scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
        if rows is None:
            out = np.empty((B, Sq, Hq, D), np.float32)
            n_rows, rptr = B * Sq * Hq, None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
            n_rows = rows_arr.size
            out = np.empty((n_rows, D), np.float32)
            rptr = _ptr(rows_arr)
        rc = self.lib.orc_attention_kv(_ptr(q), _ptr(k), _ptr(v), _code(q_dtype),
                                       _code(kv_dtype), _code(v_dtype), B, Hq, Hkv, Sq, Sk, D,
                                       int(bool(causal)), offset, scale, rptr, n_rows,
                                       _ptr(out), int(threads))
        if rc:
            raise ValueError(f"oracle rejected the arguments (code {rc})")
        return out

    def probs(self, q: np.ndarray, k: np.ndarray, *, q_dtype, kv_dtype, row: int,
              causal: bool = True, offset: Optional[int] = None,
              scale: Optional[float] = None) -> np.ndarray:
        """Softmax probabilities of one flattened query row over all Sk keys (float32 [Sk])."""
        q, k = _c(q), _c(k)
        B, Sq, Hq, Sk, Hkv, D = _shapes(q, k, kv_dtype)
        offset = Sk - Sq if offset is None else int(offset)
        scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
        out = np.empty(Sk, np.float32)
        rc = self.lib.orc_probs(_ptr(q), _ptr(k), _code(q_dtype), _code(kv_dtype), B, Hq, Hkv,
                                Sq, Sk, D, int(bool(causal)), offset, scale, int(row), _ptr(out))
        if rc:
            raise ValueError(f"oracle rejected the arguments (code {rc})")
        return out

    def dequant_q4_0(self, blocks: np.ndarray):
        """q4_0 blocks (uint8, 18 bytes each) -> (float32 values, f16 bit patterns)."""
        blocks = _c(np.asarray(blocks, dtype=np.uint8))
        if blocks.size % 18:
            raise ValueError("q4_0 data must be whole 18-byte blocks")
        n = blocks.size // 18
        f32 = np.empty(n * 32, np.float32)
        f16 = np.empty(n * 32, np.uint16)
        if self.lib.orc_dequant_q4_0(_ptr(blocks), n, _ptr(f32), _ptr(f16)):
            raise ValueError("oracle rejected the arguments")
        return f32, f16

    def quantize_q4_0(self, x: np.ndarray, src: str = "f32") -> np.ndarray:
        """q4_0 cache writer: source elements (float32 values for src "f32", uint16 bit
        patterns for "f16" / "bf16"), a multiple of 32 of them, -> uint8 blocks [n, 18]."""
        code = {"f32": 0, "f16": 1, "bf16": 2}[src]
        x = _c(np.asarray(x, dtype=np.float32 if src == "f32" else np.uint16))
        if x.size % 32:
            raise ValueError("the source must hold whole 32-element blocks")
        n = x.size // 32
        out = np.empty((n, 18), np.uint8)
        if self.lib.orc_quantize_q4_0(_ptr(x), code, n, _ptr(out)):
            raise ValueError("oracle rejected the arguments")
        return out

    def half_to_float(self, bits: np.ndarray) -> np.ndarray:
        bits = _c(np.asarray(bits, dtype=np.uint16))
        out = np.empty(bits.shape, np.float32)
        if self.lib.orc_half_to_float(_ptr(bits), bits.size, _ptr(out)):
            raise ValueError("bad arguments")
        return out

    def float_to_half(self, x: np.ndarray) -> np.ndarray:
        x = _c(np.asarray(x, dtype=np.float32))
        out = np.empty(x.shape, np.uint16)
        if self.lib.orc_float_to_half(_ptr(x), x.size, _ptr(out)):
            raise ValueError("bad arguments")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from fa_oracle.c (built on first use if no build exists); FA_ORACLE_LIB
    names another build of it (the sanitizer test loads an instrumented one this way)."""
    global _default
    if _default is None:
        path = os.environ.get("FA_ORACLE_LIB")
        if not path:
            if not os.path.exists(_build.LIB):
                _build.build()
            path = _build.LIB
        _default = Oracle(path)
    return _default


def attention(*a, **kw):
    return default().attention(*a, **kw)


def probs(*a, **kw):
    return default().probs(*a, **kw)


def dequant_q4_0(*a, **kw):
    return default().dequant_q4_0(*a, **kw)


def quantize_q4_0(*a, **kw):
    return default().quantize_q4_0(*a, **kw)


def half_to_float(*a, **kw):
    return default().half_to_float(*a, **kw)


def float_to_half(*a, **kw):
    return default().float_to_half(*a, **kw)
