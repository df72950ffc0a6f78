"""A seeded sweep of small random shapes through fa_prefill, fa_prefill_split and fa_decode,
every output row against the oracle. It reaches combinations the named cases do not: query
heads per KV head of 5-7 (a second head chunk with idle waves), batches with several KV heads
and odd offsets, mixed cache types at both head dims, empty key ranges, and queries placed
before or past the keys. Each case prints its parameters before it runs."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import oracle
import workloads as W
from gpu_cases import TOL, say, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 60
KV_PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("q4_0", "q4_0"), ("f16", "q4_0"), ("q4_0", "f16")]


def _cases():
    rng = np.random.default_rng(4242)
    out = []
    for i in range(N_CASES):
        entry = ("prefill", "split", "decode")[i % 3]
        kt, vt = KV_PAIRS[int(rng.integers(len(KV_PAIRS)))]
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
        while Hkv * G > 24:
            G = max(1, G // 2)
        B = int(rng.integers(1, 3))
        if entry == "decode":
            Sq = int(rng.integers(1, max(2, 16 // G + 1)))
            Sq = max(1, min(Sq, 16 // G))
            if G > 16:
                G, Sq = 16, 1
        else:
            Sq = int(rng.integers(1, 260))
        Sk = int(rng.choice([0, 1, 63, 64, 65])) if rng.random() < 0.15 else \
            int(rng.integers(1, 1800))
        causal = bool(rng.random() < 0.8)
        r = rng.random()
        if r < 0.5:
            offset = Sk - Sq                                  # the chunk at the end of the keys
        elif r < 0.75:
            offset = int(rng.integers(-Sq - 2, Sk + 3))       # anywhere, including before / past
        else:
            offset = int(rng.integers(0, max(1, Sk)))
        out.append(dict(i=i, entry=entry, kt=kt, vt=vt, B=B, Hq=Hkv * G, Hkv=Hkv, Sq=Sq, Sk=Sk,
                        D=D, causal=causal, offset=offset, seed=1000 + i))
    return out


CASES = _cases()


def _kv_code(kt, vt):
    if kt == vt:
        return W.KV_CODES[kt]
    return fa.FA_KV_F16_Q4_0 if kt == "f16" else fa.FA_KV_Q4_0_F16


@pytest.mark.parametrize("c", CASES, ids=[f"{c['i']}-{c['entry']}" for c in CASES])
def test_random_shape_matches_oracle(c):
    say(f"sweep case {c}")
    base = W.Workload(f"sweep{c['i']}", B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Sq=c["Sq"],
                      Sk=c["Sk"], D=c["D"], kv=c["kt"], causal=c["causal"], offset=c["offset"],
                      seed=c["seed"])
    xk = W.generate(base)
    xv = W.generate(base.with_(kv=c["vt"], seed=c["seed"] + 500)) if c["vt"] != c["kt"] else xk
    q_dtype = "bf16" if c["kt"] == "bf16" else "f16"
    q = to_dev(xk.q, q_dtype)
    k = to_dev(xk.k, c["kt"])
    v = to_dev(xv.v, c["vt"])
    kw = dict(causal=c["causal"], offset=c["offset"], scale=base.scale)
    if c["entry"] == "prefill":
        got = fa.prefill(q, k, v, **kw)
    elif c["entry"] == "split":
        got = fa.prefill_split(q, k, v, **kw)
    else:
        got = fa.decode(q, k, v, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention(xk.q, xk.k, xv.v, q_dtype=q_dtype, kv_dtype=c["kt"],
                           v_dtype=c["vt"], causal=c["causal"], offset=c["offset"],
                           scale=base.scale)
    got = got.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    tol = TOL["bf16" if q_dtype == "bf16" else "f16"]
    say(f"  max|err| = {err:.3e} (tol {tol:.0e}, {got.size // c['D']} rows)")
    assert err <= tol
