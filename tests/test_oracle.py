"""Pins for the CPU oracle: everything here checks the oracle against something other than
itself — brute force in float64, torch's scaled_dot_product_attention on the CPU in float64,
closed forms, invariants of the definition, numpy's IEEE half conversions, the pages' printed
(ms, TFLOP/s) pairs and a hand-written q4_0 fixture. A final test plants plausible mistakes in
copies of the oracle source and requires each to fail at least one of these checks.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------------------
# independent decoders (numpy / torch library routines, not the oracle's C converters)
# ----------------------------------------------------------------------------------------

def decode64(x: np.ndarray, dtype: str, D: int) -> np.ndarray:
    if dtype == "f16":
        return x.astype(np.float64)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    # q4_0, read byte by byte in Python
    lead = x.shape[:-1]
    flat = x.reshape(-1, D // 32, 18)
    out = np.empty((flat.shape[0], D), np.float64)
    for r in range(flat.shape[0]):
        for b in range(D // 32):
            blk = bytes(flat[r, b])
            d = float(np.frombuffer(blk[:2], dtype="<f2")[0])
            for t in range(16):
                out[r, 32 * b + t] = ((blk[2 + t] & 15) - 8) * d
                out[r, 32 * b + 16 + t] = ((blk[2 + t] >> 4) - 8) * d
    return out.reshape(*lead, D)


def brute_force(q64, k64, v64, causal, offset, scale):
    """Attention by pure-Python loops in float64, for tiny shapes only."""
    B, Sq, Hq, D = q64.shape
    Sk, Hkv = k64.shape[1], k64.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Sq, Hq, D))
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = h // G
                keys = [j for j in range(Sk) if (not causal) or j <= i + offset]
                if not keys:
                    continue
                s = [scale * sum(q64[b, i, h, d] * k64[b, j, g, d] for d in range(D)) for j in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[t] * v64[b, keys[t], g, d] for t in range(len(keys))) / tot
    return out


def make(B, Hq, Hkv, Sq, Sk, D, kv="f16", causal=True, offset=None, seed=0):
    w = W.Workload("t", B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, kv=kv, causal=causal,
                   offset=offset, seed=seed)
    return w, W.generate(w)


def run(orc, w, x, **kw):
    return orc.attention(x.q, x.k, x.v, q_dtype=w.q_dtype, kv_dtype=w.kv, causal=w.causal,
                         offset=w.causal_offset, scale=w.scale, **kw)


# ----------------------------------------------------------------------------------------
# checks (each raises AssertionError on a mismatch; used directly and by the mutation test)
# ----------------------------------------------------------------------------------------

BRUTE_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, kv, causal, offset
    (1, 2, 2, 5, 5, 8, "f16", True, 0),
    (2, 4, 2, 6, 9, 8, "f16", True, 3),
    (1, 4, 1, 7, 7, 16, "bf16", True, -2),
    (1, 2, 1, 4, 6, 32, "q4_0", True, 2),
    (2, 2, 2, 5, 7, 32, "q4_0", False, 0),
    (1, 3, 3, 4, 4, 8, "f16", True, 10),
    (1, 6, 2, 3, 8, 8, "bf16", False, 0),
    # mixed caches: K and V of different types (a tenth entry is V's type); q4_0 K with f16 V
    # first, so the planted mistake below (V read as K's type) is caught by a case where that
    # reading stays inside V's buffer (an f16 row holds more bytes than a q4_0 row)
    (2, 2, 1, 4, 6, 32, "q4_0", False, 0, "f16"),
    (1, 4, 2, 5, 7, 32, "f16", True, 2, "q4_0"),
]


def check_brute_force(orc, case):
    B, Hq, Hkv, Sq, Sk, D, kv, causal, offset = case[:9]
    vkv = case[9] if len(case) > 9 else kv
    w, x = make(B, Hq, Hkv, Sq, Sk, D, kv, causal, offset, seed=sum(case[:6]))
    v = x.v
    if vkv != kv:                     # V from a workload of V's type (same shape and seed)
        v = make(B, Hq, Hkv, Sq, Sk, D, vkv, causal, offset, seed=sum(case[:6]) + 1)[1].v
    got = orc.attention(x.q, x.k, v, q_dtype=w.q_dtype, kv_dtype=kv, v_dtype=vkv, causal=causal,
                        offset=w.causal_offset, scale=w.scale)
    ref = brute_force(decode64(x.q, w.q_dtype, D), decode64(x.k, kv, D), decode64(v, vkv, D),
                      causal, w.causal_offset, w.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)


def check_large_score_range(orc):
    """A steep per-key score ramp (scores spread over hundreds of units, as in the pages'
    ramp test) must still give finite outputs equal to the shifted-exponent brute force."""
    w = W.Workload("ramp", B=1, Hq=4, Hkv=2, Sq=6, Sk=12, D=16, ramp=25.0, seed=14)
    x = W.generate(w)
    got = run(orc, w, x)
    assert np.all(np.isfinite(got))
    ref = brute_force(decode64(x.q, "f16", 16), decode64(x.k, "f16", 16),
                      decode64(x.v, "f16", 16), True, w.causal_offset, w.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)


def sdpa64(q64, k64, v64, mask):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q64), t(k64), t(v64), attn_mask=None if mask is None else torch.from_numpy(mask),
        enable_gqa=True)
    return o.transpose(1, 2).numpy()


def check_torch_square_causal(orc, name):
    """Square causal: torch's own is_causal definition, float64 on the CPU."""
    w = W.WORKLOADS[name]
    x = W.generate(w)
    got = run(orc, w, x)
    t = lambda a: torch.from_numpy(decode64(a, w.kv, w.D)).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(x.q), t(x.k), t(x.v), is_causal=True).transpose(1, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)


def check_torch_rectangular(orc, Sq, Sk, offset, kv="f16"):
    """Chunk of queries against more keys, GQA 4:1, mask built with torch.tril(diagonal=offset)."""
    w, x = make(1, 8, 2, Sq, Sk, 64, kv, True, offset, seed=7)
    got = run(orc, w, x)
    mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=offset).numpy()
    ref = sdpa64(decode64(x.q, w.q_dtype, 64), decode64(x.k, kv, 64), decode64(x.v, kv, 64), mask)
    seen = mask.any(axis=1)
    np.testing.assert_allclose(got[:, seen], ref[:, seen], rtol=0, atol=1e-5)
    assert np.all(got[:, ~seen] == 0)


def check_prefix_mean(orc, Sq, Sk, offset, G):
    """Q = 0 makes every visible key equally likely: row i is the mean of V[0 .. i+offset]."""
    w, x = make(2, 2 * G, 2, Sq, Sk, 32, "f16", True, offset, seed=3)
    q = np.zeros_like(x.q)
    got = orc.attention(q, x.k, x.v, q_dtype="f16", kv_dtype="f16", causal=True,
                        offset=offset, scale=w.scale)
    v64 = x.v.astype(np.float64)
    csum = np.cumsum(v64, axis=1)
    for i in range(Sq):
        n = min(max(i + offset + 1, 0), Sk)
        for h in range(2 * G):
            ref = np.zeros((2, 32)) if n == 0 else csum[:, n - 1, h // G] / n
            np.testing.assert_allclose(got[:, i, h], ref, rtol=0, atol=1e-6)


def check_probs(orc):
    w, x = make(1, 8, 2, 40, 100, 32, "f16", True, 60, seed=5)
    for row in [0, 7, 8 * 13 + 5, 8 * 39 + 7]:
        i = (row // 8) % 40
        p = orc.probs(x.q, x.k, q_dtype="f16", kv_dtype="f16", row=row, offset=60, scale=w.scale)
        n = min(i + 61, 100)
        assert abs(float(p.astype(np.float64).sum()) - 1.0) <= 1e-6
        assert np.all(p[:n] > 0) and np.all(p[n:] == 0)


def check_constant_v(orc):
    w, x = make(1, 4, 2, 30, 50, 32, "bf16", True, -5, seed=6)
    c = W.f32_to_bf16_bits(np.full(x.v.shape, 0.7421875, np.float32))
    got = orc.attention(x.q, x.k, c, q_dtype="bf16", kv_dtype="bf16", offset=-5, scale=w.scale)
    for i in range(30):
        ref = 0.7421875 if i - 5 >= 0 else 0.0
        np.testing.assert_allclose(got[0, i], ref, rtol=0, atol=1e-6)


def check_single_key(orc):
    """A row that sees exactly one key returns that key's V row, bit for bit."""
    w, x = make(2, 4, 2, 6, 6, 32, "q4_0", True, -3, seed=8)
    got = run(orc, w, x)
    v = decode64(x.v, "q4_0", 32).astype(np.float32)
    for h in range(4):
        assert np.array_equal(got[:, 3, h], v[:, 0, h // 2])
        assert np.all(got[:, :3, h] == 0)


def check_future_keys_ignored(orc):
    w, x = make(1, 4, 4, 16, 24, 16, "f16", True, 8, seed=9)
    base = run(orc, w, x)
    k2, v2 = x.k.copy(), x.v.copy()
    rng = np.random.default_rng(0)
    k2[:, 13:] = rng.standard_normal(k2[:, 13:].shape).astype(np.float16)
    v2[:, 13:] = rng.standard_normal(v2[:, 13:].shape).astype(np.float16)
    got = orc.attention(x.q, k2, v2, q_dtype="f16", kv_dtype="f16", offset=8, scale=w.scale)
    assert np.array_equal(got[:, :5], base[:, :5])      # rows 0..4 see keys up to 12
    assert not np.array_equal(got[:, 5:], base[:, 5:])


def check_gqa_is_repeated_mha(orc):
    w, x = make(2, 8, 2, 12, 20, 32, "f16", True, 8, seed=10)
    got = run(orc, w, x)
    k4 = np.repeat(x.k, 4, axis=2)
    v4 = np.repeat(x.v, 4, axis=2)
    ref = orc.attention(x.q, k4, v4, q_dtype="f16", kv_dtype="f16", offset=8, scale=w.scale)
    assert np.array_equal(got, ref)


def check_noncausal_permutation(orc):
    w, x = make(1, 2, 1, 9, 33, 32, "f16", False, 0, seed=11)
    got = run(orc, w, x)
    perm = np.random.default_rng(1).permutation(33)
    ref = orc.attention(x.q, x.k[:, perm], x.v[:, perm], q_dtype="f16", kv_dtype="f16",
                        causal=False, scale=w.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6)


def check_scale_exponent(orc):
    """Doubling q and halving scale leaves every score, and so the output, bit-identical;
    halving the scale alone must change the output."""
    w, x = make(1, 2, 2, 8, 8, 32, "f16", True, 0, seed=12)
    base = run(orc, w, x)
    q2 = (x.q.astype(np.float32) * 2).astype(np.float16)
    got = orc.attention(q2, x.k, x.v, q_dtype="f16", kv_dtype="f16", offset=0, scale=w.scale / 2)
    assert np.array_equal(got, base)
    other = orc.attention(x.q, x.k, x.v, q_dtype="f16", kv_dtype="f16", offset=0, scale=w.scale / 2)
    assert not np.allclose(other[:, 1:], base[:, 1:], atol=1e-3)


def check_dominant_key(orc):
    """A key aligned with the query at a large score takes almost all of the weight."""
    w, x = make(1, 1, 1, 1, 10, 32, "f16", False, 0, seed=13)
    k = x.k.copy()
    k[0, 6, 0] = (x.q[0, 0, 0].astype(np.float32) * 4).astype(np.float16)
    got = orc.attention(x.q, k, x.v, q_dtype="f16", kv_dtype="f16", causal=False, scale=w.scale)
    np.testing.assert_allclose(got[0, 0, 0], x.v[0, 6, 0].astype(np.float32), atol=1e-3)


def check_half_decode(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.half_to_float(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def check_half_encode(orc):
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    # spread over the whole f16 range too, and exact ties
    y = (rng.standard_normal(400_000) * np.exp2(rng.integers(-26, 17, 400_000))).astype(np.float32)
    ties = (np.arange(-2048, 2048, dtype=np.float32) + 0.5) * np.float32(2.0 ** -10)
    edges = np.array([65504, 65519.99, 65520, 65536, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08,
                      2.9802326e-08, 0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)
    for arr in (x, y, ties, edges):
        got = orc.float_to_half(arr)
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).view(np.uint16)
        nan = np.isnan(arr)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def check_dequant_exhaustive(orc):
    """All 65,536 f16 scale patterns x all 16 codes, in both nibble positions."""
    d_bits = np.arange(65536, dtype=np.uint16)
    lo = np.arange(16, dtype=np.uint8)
    codes = np.concatenate([lo, 15 - lo])                 # elements 0..15 and 16..31
    blocks = W.pack_q4_0_blocks(d_bits, np.tile(codes, (65536, 1)))
    f32, f16 = orc.dequant_q4_0(blocks)
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        exact = d[:, None] * (codes.astype(np.float64) - 8)[None, :]
        ref32 = exact.astype(np.float32).reshape(-1)
        ref16 = exact.astype(np.float16).view(np.uint16).reshape(-1)
    nan = np.isnan(ref32)
    assert np.array_equal(np.isnan(f32), nan)
    assert np.array_equal(f32[~nan].view(np.uint32), ref32[~nan].view(np.uint32))
    assert np.array_equal(f16[~nan], ref16[~nan])
    assert np.all((f16[nan] & 0x7C00) == 0x7C00) and np.all((f16[nan] & 0x3FF) != 0)


def check_dequant_fixture(orc):
    g = json.load(open(os.path.join(GOLDEN, "q4_0_layout.json")))
    for blk in g["blocks"]:
        raw = np.frombuffer(bytes.fromhex(blk["hex"]) + bytes.fromhex(blk["codes_hex"]), np.uint8)
        f32, _ = orc.dequant_q4_0(raw)
        assert f32.tolist() == [float(e) for e in blk["expected"]], blk["note"]


def check_round_trip(orc):
    """Blocks whose scale is a positive normal f16 and that hold code 0 (value -8d, so
    max|x| = 8d) survive dequantize -> quantize unchanged."""
    rng = np.random.default_rng(4)
    n = 20000
    d_bits = rng.integers(0x0400, 0x7800, size=n).astype(np.uint16)   # normal, 8d finite
    codes = rng.integers(0, 16, size=(n, 32)).astype(np.uint8)
    codes[np.arange(n), rng.integers(0, 32, size=n)] = 0
    blocks = W.pack_q4_0_blocks(d_bits, codes)
    f32, _ = orc.dequant_q4_0(blocks)
    again = W.quantize_q4_0(f32.reshape(n, 32))
    assert np.array_equal(again, blocks)


# ---- q4_0 cache writer (quantize) ------------------------------------------------------------

def check_quant_round_trip(orc):
    """Blocks whose values are exactly (c - 8) d with a normal d and one code 0 (so max|x| = 8d)
    quantize back to themselves: pins the scale rule, the code mapping and the packing."""
    rng = np.random.default_rng(21)
    n = 4000
    d_bits = rng.integers(0x0400, 0x7800, size=n).astype(np.uint16)
    codes = rng.integers(0, 16, size=(n, 32)).astype(np.uint8)
    codes[np.arange(n), rng.integers(0, 32, size=n)] = 0
    blocks = W.pack_q4_0_blocks(d_bits, codes)
    f32, _ = orc.dequant_q4_0(blocks)
    assert np.array_equal(orc.quantize_q4_0(f32, "f32"), blocks)


def check_quant_hand_block(orc):
    """A hand-built block with max|x| = 4 (so d = 0.5): ties (k + 1/2) d round away from zero,
    +8d clamps to code 15, -8d is code 0, values inside round to the nearest code."""
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2], x[3] = 1.25, -1.25, 0.25, -0.25       # +-2.5 d, +-0.5 d (ties)
    x[4], x[5], x[6], x[7] = 4.0, -4.0, 0.74, -0.76         # +8d, -8d, 1.48 d, -1.52 d
    x[16], x[17], x[18] = 3.75, -3.75, 2.0                   # +-7.5 d (ties), 4 d
    codes = [11, 5, 9, 7, 15, 0, 9, 6] + [8] * 8 + [15, 0, 12] + [8] * 13
    expect = np.zeros(18, np.uint8)
    expect[0], expect[1] = 0x00, 0x38                        # f16 0.5 = 0x3800
    for t in range(16):
        expect[2 + t] = codes[t] | (codes[t + 16] << 4)
    assert np.array_equal(orc.quantize_q4_0(x, "f32")[0], expect)


def check_quant_zero_and_sources(orc):
    """An all-zero block gives d = 0 and codes 8; the same values given as f32, f16 and bf16
    (all exactly representable) give the same bytes."""
    z = orc.quantize_q4_0(np.zeros(32, np.float32), "f32")[0]
    assert np.array_equal(z, np.array([0, 0] + [0x88] * 16, np.uint8))
    rng = np.random.default_rng(22)
    v = (rng.integers(-64, 65, size=(64, 32)) * 2.0 ** rng.integers(-8, 3, size=(64, 1)))
    v = v.astype(np.float32)
    a = orc.quantize_q4_0(v, "f32")
    b = orc.quantize_q4_0(v.astype(np.float16).view(np.uint16), "f16")
    c = orc.quantize_q4_0((v.view(np.uint32) >> 16).astype(np.uint16), "bf16")
    assert np.array_equal(a, b) and np.array_equal(a, c)


def check_quant_matches_recipe(orc):
    """The input recipe's numpy quantizer (an independent implementation of the same reading)
    and the oracle agree byte for byte on N(0,1) data at several magnitudes, including blocks
    whose scale is a binary16 subnormal."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((3000, 32), dtype=np.float32)
    x *= (10.0 ** rng.uniform(-7, 3, size=(3000, 1))).astype(np.float32)
    assert np.array_equal(orc.quantize_q4_0(x, "f32"), W.quantize_q4_0(x))


ALL_CHECKS = (
    [(f"brute_force[{i}]", (lambda c: lambda o: check_brute_force(o, c))(c))
     for i, c in enumerate(BRUTE_CASES)]
    + [("torch_square_tiny", lambda o: check_torch_square_causal(o, "tiny")),
       ("torch_rect", lambda o: check_torch_rectangular(o, 48, 150, 102)),
       ("torch_rect_neg", lambda o: check_torch_rectangular(o, 40, 64, -9, "bf16")),
       ("prefix_mean", lambda o: check_prefix_mean(o, 12, 20, 8, 4)),
       ("prefix_mean_neg", lambda o: check_prefix_mean(o, 12, 10, -3, 2)),
       ("large_scores", check_large_score_range),
       ("probs", check_probs), ("constant_v", check_constant_v),
       ("single_key", check_single_key), ("future_keys", check_future_keys_ignored),
       ("gqa", check_gqa_is_repeated_mha), ("noncausal_perm", check_noncausal_permutation),
       ("scale", check_scale_exponent), ("dominant_key", check_dominant_key),
       ("half_decode", check_half_decode), ("half_encode", check_half_encode),
       ("dequant_exhaustive", check_dequant_exhaustive), ("dequant_fixture", check_dequant_fixture),
       ("round_trip", check_round_trip),
       ("quant_round_trip", check_quant_round_trip), ("quant_hand_block", check_quant_hand_block),
       ("quant_zero_sources", check_quant_zero_and_sources),
       ("quant_recipe", check_quant_matches_recipe)])


# ----------------------------------------------------------------------------------------
# tests
# ----------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("name,check", ALL_CHECKS, ids=[n for n, _ in ALL_CHECKS])
def test_oracle_pin(orc, name, check):
    check(orc)


def test_torch_square_causal_p2check(orc):
    """The flash-attn verification shape (B=2, S=512, H=8, D=64, causal) against torch SDPA."""
    check_torch_square_causal(orc, "p2check")


def test_flop_convention_matches_printed_pairs():
    """4*D*Hq*B*(visible pairs, diagonal included) reproduces every printed (ms, TFLOP/s)
    pair of the mlxcel PR's Measurements; the dense count does not."""
    g = json.load(open(os.path.join(GOLDEN, "mlxcel_pr2306_measurements.json")))
    for r in g["rows"]:
        w = W.WORKLOADS["prefill_2k_f16"].with_(Sk=r["Sk"])
        tf = W.attention_flops(w) / (r["ms"] * 1e-3) / 1e12
        assert abs(tf - r["tflops"]) <= 0.0051, (r, tf)
        dense = 4 * w.D * w.Hq * w.B * w.Sq * w.Sk / (r["ms"] * 1e-3) / 1e12
        if r["Sk"] == 2048:
            assert abs(dense - r["tflops"]) > 0.5
    lo, hi = g["fallback_arm"]["tflops_range"]
    for r in g["fallback_arm"]["rows"]:
        w = W.WORKLOADS["prefill_2k_f16"].with_(Sk=r["Sk"])
        tf = W.attention_flops(w) / (r["ms"] * 1e-3) / 1e12
        assert lo - 0.005 <= tf <= hi + 0.005


def test_quantizer_error_bound():
    """Input recipe check: q4_0 of N(0,1) data is within d/2 of the data, except elements
    above 7.5 d, whose code clamps at 15 (value 7d) and so lie within d + rounding of d."""
    x = np.random.default_rng(0).standard_normal((4096, 32), dtype=np.float32)
    blocks = W.quantize_q4_0(x)
    f32, _ = oracle.dequant_q4_0(blocks)
    back = f32.reshape(4096, 32)
    d = blocks[:, :2].copy().view("<f2").astype(np.float32)
    err = np.abs(back - x)
    dd = d.repeat(32, 1)
    top = x > 7.5 * dd
    assert np.all(err[~top] <= dd[~top] * 0.5 * (1 + 2e-3))
    assert np.all(err[top] <= dd[top] * 1.01)


MUTANTS = [
    ("off-by-one visibility", "int64_t n = i + p->offset + 1;", "int64_t n = i + p->offset;"),
    ("modulo head grouping", "const int64_t g = h / (p->Hq / p->Hkv);\n    const float *q",
     "const int64_t g = h % p->Hkv;\n    const float *q"),
    ("dropped scale", "prob[j] = p->scale * acc;", "prob[j] = acc;"),
    ("flipped exponent sign", "expf(prob[j] - m)", "expf(m - prob[j])"),
    ("V read through K", "const float *v = p->V +", "const float *v = p->K +"),
    ("missing normalisation", "prob[j] = prob[j] / l;", "prob[j] = prob[j];"),
    ("nibbles swapped", "out[t] = (float)(lo - 8) * d;", "out[t] = (float)(hi - 8) * d;"),
    ("wrong code offset", "out[t + 16] = (float)(hi - 8) * d;", "out[t + 16] = (float)(hi - 7) * d;"),
    ("half exponent bias", "ldexpf((float)(1024 + f), e - 25)", "ldexpf((float)(1024 + f), e - 24)"),
    ("half subnormal scale", "ldexpf((float)f, -24)", "ldexpf((float)f, -25)"),
    ("bf16 shift", "(uint32_t)h << 16", "(uint32_t)h << 15"),
    ("round to half away", "nearbyintf(ldexpf(a, 10 - k))", "roundf(ldexpf(a, 10 - k))"),
    ("query index", "const int64_t i = (r / p->Hq) % p->Sq;", "const int64_t i = (r / p->Hq) % p->Sk;"),
    ("max not taken", "if (prob[j] > m)\n            m = prob[j];", "if (prob[j] < m)\n            m = prob[j];"),
    ("writer rounds half to even", "v = (int)roundf(x[t] / d) + 8;", "v = (int)nearbyintf(x[t] / d) + 8;"),
    ("writer scale max/7", "float_to_half_bits_rne(amax / 8.0f)", "float_to_half_bits_rne(amax / 7.0f)"),
    ("writer scale not rounded", "const float d = half_bits_to_float(dbits);", "const float d = amax / 8.0f;"),
    ("writer nibbles swapped", "blk[2 + t] = (uint8_t)(c[t] | (c[t + 16] << 4));",
     "blk[2 + t] = (uint8_t)(c[t + 16] | (c[t] << 4));"),
    ("writer clamp at 16", "v = v < 0 ? 0 : (v > 15 ? 15 : v);", "v = v < 0 ? 0 : (v > 16 ? 16 : v);"),
    # the mixed-cache entry ignoring V's own type (caught by the q4_0-K / f16-V brute-force
    # case, where V's bytes read as q4_0 stay inside its buffer)
    ("V widened by K's type", "p.V = upcast_rows(v, v_dtype,", "p.V = upcast_rows(v, k_dtype,"),
]


def test_pins_catch_planted_mistakes(tmp_path):
    """Each plausible mistake planted in a copy of the oracle fails at least one pin."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")).read()
    quick = [(n, c) for n, c in ALL_CHECKS]
    survivors = []
    for idx, (name, old, new) in enumerate(MUTANTS):
        assert src.count(old) == 1, f"mutation site for {name!r} not unique"
        path = tmp_path / f"m{idx}.c"
        path.write_text(src.replace(old, new))
        so = tmp_path / f"m{idx}.so"
        subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(so),
                        "-lm"], check=True)
        mutant = oracle.Oracle(str(so))
        caught = False
        for cname, check in quick:
            try:
                check(mutant)
            except (AssertionError, ValueError):
                caught = True
                break
        if not caught:
            survivors.append(name)
    assert not survivors, f"mutants not caught by any pin: {survivors}"
