"""Caches larger than 4 GiB (maximum-size edge cases): two sequences whose K and V caches total
more than 4 GiB each, so the second sequence starts past 2 GiB and its last tiles past 4 GiB.
Every batch, sequence, head and tile base in the kernels is a 64-bit offset and only offsets
inside a 64-key tile are 32-bit; a 32-bit base anywhere would read the wrong keys here. Inputs
are seeded N(0,1) f16 values, or q4_0 blocks with random codes and N(0,1)-range scales (a
cache of this size is too large to quantize from float32 in the test); the oracle runs on
each sequence's own slice. The scale is 0.35 rather than 1/sqrt(D): at 1/sqrt(D) a row of a
million N(0,1) keys averages to ~1e-3, so keys read from a wrong place would pass the
tolerance; at 0.35 each row rests on its few highest-scoring keys (an effective 2-170 of
them, wherever they lie), and one 64-key tile read from elsewhere moves the output by 0.1-2."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import oracle
import workloads as W
from gpu_cases import TOL, say, to_host

pytestmark = pytest.mark.gpu

SCALE = 0.35


def _check(label, got, ref, tol):
    err = float(np.max(np.abs(got - ref)))
    say(f"  {label}: max|err| = {err:.3e} (tol {tol:.0e}, {ref.size // ref.shape[-1]} rows)")
    assert err <= tol, (label, err)


def test_f16_cache_beyond_4gib():
    B, Hq, Hkv, D, Sk, Sq = 2, 32, 8, 128, 1_100_003, 64
    scale = SCALE
    say(f"f16 cache: B={B} Sk={Sk} Hkv={Hkv} D={D}: {2 * B * Sk * Hkv * D * 2 / 2**30:.2f} GiB")
    k = W.normal_f16((B, Sk, Hkv, D), seed=201)
    v = W.normal_f16((B, Sk, Hkv, D), seed=202)
    qd = W.normal_f16((B, 1, Hq, D), seed=203)
    qp = W.normal_f16((B, Sq, Hq, D), seed=204)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    dec = fa.decode(torch.from_numpy(qd).cuda(), kd, vd, causal=True, offset=Sk - 1, scale=scale)
    qpd = torch.from_numpy(qp).cuda()
    pre = fa.prefill(qpd, kd, vd, causal=True, offset=Sk - Sq, scale=scale)
    spl = fa.prefill_split(qpd, kd, vd, causal=True, offset=Sk - Sq, scale=scale)
    # the same bytes as a pool of 64-key pages, dealt to the two sequences in shuffled order
    # (the paged prefill takes 4096 of them per sequence, its documented limit, from anywhere
    # in the pool)
    n_pages = B * Sk // 64
    half = n_pages // 2
    table = np.random.default_rng(208).permutation(n_pages).astype(np.int32)
    table = np.ascontiguousarray(table[:2 * half].reshape(2, half))
    lens = np.array([64 * half - 5, 64 * half - 37], np.int32)
    tpre = np.ascontiguousarray(table[:, :4096])
    lpre = np.array([64 * 4096 - 5, 64 * 4096 - 37], np.int32)
    pk = kd.reshape(-1)[:n_pages * 64 * Hkv * D].view(n_pages, 64, Hkv, D)
    pv = vd.reshape(-1)[:n_pages * 64 * Hkv * D].view(n_pages, 64, Hkv, D)
    tab_d, lens_d = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    pdec = fa.decode_paged(torch.from_numpy(qd).cuda(), pk, pv, tab_d, lens_d, causal=True,
                           scale=scale)
    ppre = fa.prefill_paged(qpd, pk, pv, torch.from_numpy(tpre).cuda(),
                            torch.from_numpy(lpre).cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    dec, pre, spl = to_host(dec), to_host(pre), to_host(spl)
    pdec, ppre = to_host(pdec), to_host(ppre)
    del kd, vd, pk, pv
    rows = [i * Hq + h for i in (0, Sq - 1) for h in (0, 13, 31)]
    hk = k.reshape(-1)[:n_pages * 64 * Hkv * D].reshape(n_pages, 64, Hkv, D)
    hv = v.reshape(-1)[:n_pages * 64 * Hkv * D].reshape(n_pages, 64, Hkv, D)
    for b in range(B):
        n = int(lens[b])
        kb = hk[table[b]].reshape(-1, Hkv, D)[None, :n]
        vb = hv[table[b]].reshape(-1, Hkv, D)[None, :n]
        ref = oracle.attention(qd[b:b + 1], kb, vb, q_dtype="f16", kv_dtype="f16", causal=True,
                               offset=n - 1, scale=scale)
        _check(f"paged decode sequence {b}", pdec[b:b + 1], ref, TOL["f16"])
        n = int(lpre[b])
        kb = hk[tpre[b]].reshape(-1, Hkv, D)[None, :n]
        vb = hv[tpre[b]].reshape(-1, Hkv, D)[None, :n]
        ref = oracle.attention(qp[b:b + 1], kb, vb, q_dtype="f16", kv_dtype="f16", causal=True,
                               offset=n - Sq, scale=scale, rows=rows)
        _check(f"paged prefill sequence {b}", ppre[b].reshape(Sq * Hq, D)[rows], ref, TOL["f16"])
        del kb, vb
    for b in range(B):
        ref = oracle.attention(qd[b:b + 1], k[b:b + 1], v[b:b + 1], q_dtype="f16",
                               kv_dtype="f16", causal=True, offset=Sk - 1, scale=scale)
        _check(f"decode sequence {b}", dec[b:b + 1], ref, TOL["f16"])
        ref = oracle.attention(qp[b:b + 1], k[b:b + 1], v[b:b + 1], q_dtype="f16",
                               kv_dtype="f16", causal=True, offset=Sk - Sq, scale=scale,
                               rows=rows)
        got = pre[b].reshape(Sq * Hq, D)[rows]
        _check(f"prefill sequence {b}", got, ref, TOL["f16"])
        _check(f"prefill_split sequence {b}", spl[b].reshape(Sq * Hq, D)[rows], ref, TOL["f16"])


def test_q4_0_cache_beyond_4gib():
    B, Hq, Hkv, D, Sk = 2, 32, 8, 128, 3_800_003
    scale = SCALE
    nb = B * Sk * Hkv * (D // 32)
    say(f"q4_0 cache: B={B} Sk={Sk} Hkv={Hkv} D={D}: {2 * nb * 18 / 2**30:.2f} GiB")
    k = W.random_q4_0(nb, seed=205).reshape(B, Sk, Hkv, D // 32 * 18)
    v = W.random_q4_0(nb, seed=206).reshape(B, Sk, Hkv, D // 32 * 18)
    qd = W.normal_f16((B, 1, Hq, D), seed=207)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    dec = fa.decode(torch.from_numpy(qd).cuda(), kd, vd, causal=True, offset=Sk - 1, scale=scale)
    torch.cuda.synchronize()
    dec = to_host(dec)
    del kd, vd
    for b in range(B):
        ref = oracle.attention(qd[b:b + 1], k[b:b + 1], v[b:b + 1], q_dtype="f16",
                               kv_dtype="q4_0", causal=True, offset=Sk - 1, scale=scale)
        _check(f"q4_0 decode sequence {b}", dec[b:b + 1], ref, TOL["q4_0"])
