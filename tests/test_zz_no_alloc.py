"""fa_decode_noalloc (the decode for callers that cannot allocate: its split partials live in
a fixed scratch array inside the library) against fa_decode with a caller workspace: two calls
in a row on one GPU, the second with a smaller input, each bit-identical to fa_decode (the same
kernels on the same inputs) and within the parity tolerance of the oracle."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import workloads as W
from gpu_cases import compare, device_inputs, inputs, oracle_full, say

pytestmark = pytest.mark.gpu


def _noalloc(w, q, k, v):
    out = torch.full_like(q, float("nan"))
    rc = fa.fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), w.B,
                              w.Hq, w.Hkv, w.Sq, w.Sk, w.D, int(w.causal), w.causal_offset,
                              w.scale, w.kv_code, torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    return out


def test_decode_noalloc_matches_decode():
    cases = [W.WORKLOADS["decode_q4_0"],
             W.Workload("noalloc_small_f16", B=2, Hq=16, Hkv=4, Sq=2, Sk=3000, D=128, kv="f16",
                        seed=121)]
    for w in cases:
        need = fa.fa_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D)
        say(f"decode_noalloc {w} (fa_decode workspace {need} bytes)")
        assert 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
        q, k, v = device_inputs(w, inputs(w))
        got = _noalloc(w, q, k, v)
        ref = fa.decode(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), w.name
        compare(w, got.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name)


def test_decode_noalloc_refuses_beyond_scratch():
    """A call needing more than the fixed scratch is refused before anything is launched."""
    B, Hq, Hkv, Sq, Sk, D = 4096, 1, 1, 16, 64, 128          # one split of 16 rows per head
    need = fa.fa_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    rc = fa.fa_decode_noalloc(fake, fake, fake, fake, B, Hq, Hkv, Sq, Sk, D, 1, Sk - Sq,
                              D ** -0.5, fa.FA_KV_F16, None)
    assert rc == fa.FA_ERR_TOO_LARGE
