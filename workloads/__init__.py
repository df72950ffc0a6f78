"""Seeded synthetic inputs for causal grouped-query flash attention.

This module is the only code that both sides of the parity check share: it draws the
N(0,1) tensors, casts them to the storage types and packs the 4-bit block-quantized
(q4_0) K/V cache. It holds none of the attention arithmetic, no dequantization and
nothing the HIP path computes; it also carries the measurement conventions
(algorithmic FLOPs and bytes) that the benchmark reports against.

Sources (the pages these workloads stand in for):
  * mlxcel PR #2306 "defer SDPA accumulator rescale, stage Q once per block", commit
    message and Measurements: 2,048-token query chunks placed at the end of 2K / 8K /
    16K keys, GQA 32/8, head dim 128, f16 and bf16, plus inputs whose scores climb along
    the keys so that rows outrun the rescale margin.
  * mi210-llm-stack "Build FlashAttention (CK backend) on gfx90a", Verification:
    B=2, S=512, H=8, D=64, causal, max_diff < 0.01.
  * mi210-llm-stack "FlashAttention on gfx90a", "-ctk q4_0 -ctv q4_0": a q4_0 KV cache.
    The pages name the format but never define it; the recipe below (32-element blocks,
    one f16 scale d = max|x|/8, codes c with value (c-8)*d, offset 8) is the plainest
    reading, and the byte layout follows the common GGML arrangement (byte t holds
    element t in its low nibble and element t+16 in its high nibble).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# dtype tags, identical to the enum in include/fa.h
KV_F16 = 0
KV_BF16 = 1
KV_Q4_0 = 2
KV_CODES = {"f16": KV_F16, "bf16": KV_BF16, "q4_0": KV_Q4_0}

Q4_0_ELEMS = 32      # elements per block (along the head dimension)
Q4_0_BYTES = 18      # little-endian f16 scale + 16 bytes of packed 4-bit codes

# rescale margin of the deferred softmax frame, natural-log units of the scaled score
RESCALE_MARGIN = 10.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call: shapes, storage types and the seed of its inputs.

    Layout is [B, S, H, D] contiguous for Q, K, V and O. Query i sits at absolute
    position i + offset and, when causal, sees key j iff j <= i + offset (bottom-right
    alignment: a chunk of Sq queries is the last Sq of Sk positions when offset = Sk - Sq).
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    kv: str = "f16"            # storage type of K and V: f16, bf16 or q4_0
    causal: bool = True
    offset: Optional[int] = None   # None means Sk - Sq
    ramp: float = 0.0          # per-key score ramp added through the last head-dim column
    seed: int = 0

    @property
    def causal_offset(self) -> int:
        return self.Sk - self.Sq if self.offset is None else self.offset

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def q_dtype(self) -> str:
        """Q and O are bf16 when K/V are bf16, f16 otherwise (f16 and q4_0 caches)."""
        return "bf16" if self.kv == "bf16" else "f16"

    @property
    def kv_code(self) -> int:
        return KV_CODES[self.kv]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _prefill(name, Sk, kv, seed, ramp=0.0):
    return Workload(name, B=1, Hq=32, Hkv=8, Sq=2048, Sk=Sk, D=128, kv=kv, ramp=ramp, seed=seed)


WORKLOADS = {w.name: w for w in [
    # tiny causal self-attention, the case the oracle finishes in well under a second
    Workload("tiny", B=1, Hq=2, Hkv=2, Sq=128, Sk=128, D=64, seed=1),
    # the flash-attn verification shape
    Workload("p2check", B=2, Hq=8, Hkv=8, Sq=512, Sk=512, D=64, seed=2),
    # chunked prefill: 2048 queries at the end of Sk keys, GQA 32/8, D=128
    _prefill("prefill_2k_f16", 2048, "f16", 3),
    _prefill("prefill_8k_f16", 8192, "f16", 3),
    _prefill("prefill_16k_f16", 16384, "f16", 3),
    _prefill("prefill_2k_bf16", 2048, "bf16", 3),
    _prefill("prefill_8k_bf16", 8192, "bf16", 3),
    _prefill("prefill_16k_bf16", 16384, "bf16", 3),
    _prefill("prefill_2k_f16_ramp", 2048, "f16", 3, ramp=0.05),
    _prefill("prefill_16k_f16_ramp", 16384, "f16", 3, ramp=0.05),
    _prefill("prefill_2k_bf16_ramp", 2048, "bf16", 3, ramp=0.05),
    _prefill("prefill_16k_bf16_ramp", 16384, "bf16", 3, ramp=0.05),
    # decode against a q4_0 cache: 4 sequences x 1 token, 32768 cached keys each
    Workload("decode_q4_0", B=4, Hq=32, Hkv=8, Sq=1, Sk=32768, D=128, kv="q4_0", seed=4),
    # chunked prefill against a q4_0 cache
    _prefill("prefill_16k_q4_0", 16384, "q4_0", 5),
    # a short chunk (256 queries) at the end of 16384 keys: few (b, KV head, query block) units
    Workload("chunk256_16k_f16", B=1, Hq=32, Hkv=8, Sq=256, Sk=16384, D=128, seed=6),
    Workload("chunk256_16k_q4_0", B=1, Hq=32, Hkv=8, Sq=256, Sk=16384, D=128, kv="q4_0", seed=7),
]}


# ----------------------------------------------------------------------------------------
# casts and packing (input recipe)
# ----------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even cast of finite float32 values to bfloat16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> 16) & 1
    return ((bits + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def _round_half_away(r: np.ndarray) -> np.ndarray:
    return np.sign(r) * np.floor(np.abs(r) + np.float32(0.5))


def quantize_q4_0(x: np.ndarray) -> np.ndarray:
    """Pack float32 data [..., D] (D % 32 == 0) into q4_0 blocks [..., D/32*18] uint8.

    Per 32-element block: d = f16(max|x| / 8) rounded to nearest even; each element gets
    the code c = clamp(round_half_away(x / d) + 8, 0, 15) (all codes 8 when d == 0). The
    block is stored as the two bytes of d (little endian) followed by 16 bytes where
    byte t = c[t] | c[t+16] << 4.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape[-1] % Q4_0_ELEMS:
        raise ValueError("last dimension must be a multiple of 32")
    lead = x.shape[:-1]
    nb_row = x.shape[-1] // Q4_0_ELEMS
    blocks = x.reshape(-1, Q4_0_ELEMS)
    n = blocks.shape[0]
    amax = np.abs(blocks).max(axis=1)
    d16 = (amax / np.float32(8.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = blocks / d32[:, None]
    c = np.clip(_round_half_away(r) + 8, 0, 15)
    c = np.where(d32[:, None] == 0, 8, c).astype(np.uint8)
    out = np.empty((n, Q4_0_BYTES), dtype=np.uint8)
    out[:, 0:2] = d16.astype("<f2").view(np.uint8).reshape(n, 2)
    out[:, 2:] = c[:, :16] | (c[:, 16:] << 4)
    return out.reshape(*lead, nb_row * Q4_0_BYTES)


def pack_q4_0_blocks(d16_bits: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Build q4_0 blocks from explicit scale bit patterns [n] and codes [n, 32] (0..15)."""
    d16_bits = np.asarray(d16_bits, dtype=np.uint16).reshape(-1)
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, Q4_0_ELEMS)
    n = codes.shape[0]
    out = np.empty((n, Q4_0_BYTES), dtype=np.uint8)
    out[:, 0] = d16_bits & 0xFF
    out[:, 1] = d16_bits >> 8
    out[:, 2:] = (codes[:, :16] & 15) | ((codes[:, 16:] & 15) << 4)
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 data to the storage form of `dtype` (f16 array, bf16 bits, q4_0 bytes)."""
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "q4_0":
        return quantize_q4_0(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    w: Workload
    q: np.ndarray   # [B, Sq, Hq, D]   float16, or uint16 bf16 bits
    k: np.ndarray   # [B, Sk, Hkv, D]  float16 / uint16 bits, or uint8 [B, Sk, Hkv, D/32*18]
    v: np.ndarray


def draw_f32(w: Workload, seed: Optional[int] = None):
    """N(0,1) float32 Q, K, V from numpy's PCG64, drawn in that order.

    With w.ramp != 0 the last head-dim column carries a per-key ramp: q[..., D-1] = 1 and
    k[b, j, g, D-1] = ramp * j / scale, so every score gains ramp * j (up to input rounding).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal((w.B, w.Sq, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Sk, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Sk, w.Hkv, w.D), dtype=np.float32)
    if w.ramp:
        q[..., w.D - 1] = 1.0
        k[:, :, :, w.D - 1] = (w.ramp / w.scale) * np.arange(w.Sk, dtype=np.float32)[None, :, None]
    return q, k, v


def normal_f16(shape, seed: int, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) values rounded to float16, drawn in float32 chunks from numpy's PCG64 (for caches
    too large to hold in float32 at once)."""
    rng = np.random.default_rng(seed)
    out = np.empty(int(np.prod(shape)), np.float16)
    for s in range(0, out.size, chunk):
        n = min(chunk, out.size - s)
        out[s:s + n] = rng.standard_normal(n, dtype=np.float32)
    return out.reshape(shape)


def random_q4_0(n_blocks: int, seed: int) -> np.ndarray:
    """q4_0 blocks [n_blocks, 18] for caches too large to quantize: uniform random 4-bit codes
    and scales d = f16 of U(0.25, 0.4), the range max|x|/8 takes for 32 N(0,1) values."""
    rng = np.random.default_rng(seed)
    out = np.empty((n_blocks, Q4_0_BYTES), np.uint8)
    step = 1 << 24
    for s in range(0, n_blocks, step):
        n = min(step, n_blocks - s)
        d = rng.uniform(0.25, 0.4, n).astype(np.float16)
        out[s:s + n, :2] = d.view(np.uint8).reshape(n, 2)
        out[s:s + n, 2:] = rng.integers(0, 256, (n, 16), dtype=np.uint8)
    return out


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    q, k, v = draw_f32(w, seed)
    return Inputs(w, encode(q, w.q_dtype), encode(k, w.kv), encode(v, w.kv))


# ----------------------------------------------------------------------------------------
# measurement conventions
# ----------------------------------------------------------------------------------------

def visible_pairs(Sq: int, Sk: int, causal: bool, offset: int) -> int:
    """Number of (query, key) pairs the mask lets through, diagonal included."""
    if not causal:
        return Sq * Sk
    i = np.arange(Sq, dtype=np.int64)
    return int(np.clip(i + offset + 1, 0, Sk).sum())


def attention_flops(w: Workload) -> int:
    """Algorithmic FLOPs = 4 * D * Hq * B * visible pairs (QK^T and PV, 2 FLOP per MAC).

    This is the count behind the (ms, TFLOP/s) pairs of the mlxcel PR's Measurements;
    softmax work, masked pairs and padding are not counted.
    """
    return 4 * w.D * w.Hq * w.B * visible_pairs(w.Sq, w.Sk, w.causal, w.causal_offset)


def kv_bytes(w: Workload) -> int:
    """Bytes of K plus V as stored."""
    per = w.B * w.Sk * w.Hkv
    if w.kv == "q4_0":
        return 2 * per * (w.D // Q4_0_ELEMS) * Q4_0_BYTES
    return 2 * per * w.D * 2


def algorithmic_bytes(w: Workload) -> int:
    """HBM bytes one call must move at least: K + V as stored, Q read once, O written once."""
    qo = 2 * w.B * w.Sq * w.Hq * w.D * 2
    return kv_bytes(w) + qo
