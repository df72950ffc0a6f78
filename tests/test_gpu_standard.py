"""The standard (non-flash) attention arm, fa_standard_attention (mi210-llm-stack,
"FlashAttention on gfx90a", Approach C: dequantize K and V, then the plain path of scores,
softmax and P V), against the oracle on every output row."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import workloads as W
from gpu_cases import TOL, compare, device_inputs, inputs, oracle_full, say, to_dev

pytestmark = pytest.mark.gpu


def wl(name, B, Hq, Hkv, Sq, Sk, D, kv="f16", causal=True, offset=None, seed=0):
    return W.Workload(name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, kv=kv, causal=causal,
                      offset=offset, seed=seed)


CASES = [
    W.WORKLOADS["tiny"],
    W.WORKLOADS["p2check"],
    wl("std_gqa4_ragged_f16", 2, 8, 2, 100, 300, 128, "f16", True, 200, seed=131),
    wl("std_gqa4_ragged_bf16", 2, 8, 2, 100, 300, 128, "bf16", True, 200, seed=132),
    wl("std_gqa4_ragged_q4_0", 2, 8, 2, 100, 300, 128, "q4_0", True, 200, seed=133),
    wl("std_d64_q4_0", 1, 4, 1, 70, 200, 64, "q4_0", True, 130, seed=134),
    wl("std_noncausal_d64_bf16", 1, 8, 1, 33, 65, 64, "bf16", False, 0, seed=135),
    wl("std_negative_offset", 1, 4, 2, 64, 64, 128, "f16", True, -20, seed=136),
    wl("std_g8", 1, 16, 2, 40, 100, 128, "f16", True, 60, seed=137),
    wl("std_sk1", 1, 4, 1, 3, 1, 128, "f16", True, 0, seed=138),
    # decode shapes: one query row tile per unit, so the P.V keys are split and summed
    wl("std_decode_q4_0", 4, 32, 8, 1, 5000, 128, "q4_0", True, 4999, seed=139),
    wl("std_decode_f16_sq4", 1, 8, 2, 4, 3000, 64, "f16", True, 2996, seed=140),
    # a mid-size chunked prefill: 512 queries at the end of 3000 keys, GQA 32/8
    wl("std_chunk_q4_0", 1, 32, 8, 512, 3000, 128, "q4_0", True, None, seed=141),
    wl("std_chunk_f16", 1, 32, 8, 512, 3000, 128, "f16", True, None, seed=142),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_standard_matches_oracle(w):
    say(f"standard attention {w}")
    q, k, v = device_inputs(w, inputs(w))
    o = fa.standard_attention(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    torch.cuda.synchronize()
    compare(w, o.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name)


def test_standard_no_keys_gives_zeros():
    w = wl("std_sk0", 1, 4, 1, 3, 0, 128, "f16", True, 0, seed=143)
    q, k, v = device_inputs(w, inputs(w))
    o = fa.standard_attention(q, k, v, causal=True, offset=0, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0


def test_standard_small_workspace_runs_in_passes():
    """The minimum workspace (one (b, KV head) unit per pass) and the one-pass workspace both
    match the oracle (their P.V key splits differ with the units per pass, so the f32 partial
    sums are added in another order and the bits may differ)."""
    w = wl("std_passes", 2, 16, 4, 300, 700, 128, "q4_0", True, None, seed=144)
    q, k, v = device_inputs(w, inputs(w))
    small = fa.standard_workspace_bytes(q, k, v, 1)
    full = fa.standard_workspace_bytes(q, k, v, 0)
    assert small < full
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    a = fa.standard_attention(q, k, v, causal=True, offset=w.causal_offset, scale=w.scale,
                              workspace=ws)
    b = fa.standard_attention(q, k, v, causal=True, offset=w.causal_offset, scale=w.scale)
    torch.cuda.synchronize()
    compare(w, a.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name + "/passes")
    compare(w, b.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name + "/one pass")


def test_standard_mixed_caches():
    for kt, vt in (("f16", "q4_0"), ("q4_0", "f16")):
        w = wl(f"std_mixed_{kt}_{vt}", 2, 8, 2, 100, 300, 128, "f16", True, 200, seed=145)
        xk = W.generate(w.with_(kv=kt))
        xv = W.generate(w.with_(kv=vt, seed=w.seed + 1000))
        import oracle
        ref = oracle.attention(xk.q, xk.k, xv.v, q_dtype="f16", kv_dtype=kt, v_dtype=vt,
                               causal=True, offset=w.causal_offset, scale=w.scale)
        o = fa.standard_attention(to_dev(xk.q, "f16"), to_dev(xk.k, kt), to_dev(xv.v, vt),
                                  causal=True, offset=w.causal_offset, scale=w.scale)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(o.float().cpu().numpy() - ref)))
        say(f"  {kt}/{vt}: max|err| = {err:.3e}")
        assert err <= TOL["q4_0"], (kt, vt, err)


@pytest.mark.parametrize("name", ["prefill_16k_q4_0", "decode_q4_0"])
def test_standard_full_size(name):
    """The two q4_0 workloads the benchmark times this arm on, every output row."""
    w = W.WORKLOADS[name]
    say(f"standard attention {w}")
    q, k, v = device_inputs(w, inputs(w))
    o = fa.standard_attention(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    torch.cuda.synchronize()
    compare(w, o.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name)
