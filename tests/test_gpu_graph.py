"""The entry points inside a captured HIP graph. The library allocates nothing and issues no
memset or copy: a call is kernel launches on the caller's stream, so a serving loop can capture
it once and replay it. Every replay is checked bit for bit against the same call run eagerly,
with eager work of the program and synchronisations between the replays, and new inputs are
copied into the captured buffers between replays (so each replay reads them afresh)."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import workloads as W
from gpu_cases import device_inputs, say

pytestmark = pytest.mark.gpu


def wl(name, B, Hq, Hkv, Sq, Sk, D, kv, seed):
    return W.Workload(name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, kv=kv, causal=True,
                      seed=seed)


PRE = wl("graph_prefill", 1, 8, 2, 300, 1000, 128, "f16", 301)
SPLIT = wl("graph_split", 1, 8, 2, 1024, 1024, 128, "f16", 302)
DEC = wl("graph_decode_q4_0", 2, 32, 8, 1, 5000, 128, "q4_0", 303)


def _calls(bufs):
    """The captured calls, writing into preallocated outputs and workspaces."""
    (qp, kp, vp, op), (qs, ks, vs, os_, wss), (qd, kd, vd, od, wsd) = bufs
    fa.prefill(qp, kp, vp, causal=True, offset=PRE.causal_offset, scale=PRE.scale, out=op)
    fa.prefill_split(qs, ks, vs, causal=True, offset=SPLIT.causal_offset, scale=SPLIT.scale,
                     out=os_, workspace=wss)
    fa.decode(qd, kd, vd, causal=True, offset=DEC.causal_offset, scale=DEC.scale, out=od,
              workspace=wsd)


def _load(bufs, seed_shift):
    """Copy fresh seeded inputs into the buffers (the same arrays every time for a shift)."""
    for (w, b) in zip((PRE, SPLIT, DEC), bufs):
        x = W.generate(w, seed=w.seed + seed_shift)
        for dst, src in zip(b[:3], device_inputs(w, x)):
            dst.copy_(src)


def _outs(bufs):
    return [b[3].clone() for b in bufs]


def test_replays_match_eager():
    bufs = []
    for w in (PRE, SPLIT, DEC):
        q, k, v = device_inputs(w, W.generate(w))
        b = [q, k, v, torch.empty_like(q)]
        if w is SPLIT:
            b.append(torch.zeros(max(fa.prefill_workspace_bytes(q, k, v, causal=True), 16),
                                 dtype=torch.uint8, device="cuda"))
        if w is DEC:
            n = fa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D)
            b.append(torch.empty(max(n, 16), dtype=torch.uint8, device="cuda"))
        bufs.append(b)
    # eager references for two input sets
    ref = {}
    for shift in (0, 1):
        _load(bufs, shift)
        _calls(bufs)
        torch.cuda.synchronize()
        ref[shift] = _outs(bufs)
    # capture (after a warm-up on a side stream, as torch recommends)
    _load(bufs, 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _calls(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _calls(bufs)
    other = wl("graph_eager_other", 1, 4, 1, 100, 700, 64, "f16", 304)
    qo, ko, vo = device_inputs(other, W.generate(other))
    for rep, shift in enumerate((0, 1, 0, 1, 1)):
        _load(bufs, shift)
        for b in bufs:
            b[3].fill_(float("nan"))          # a replay that wrote nothing would show
        torch.cuda.synchronize()
        g.replay()
        fa.prefill(qo, ko, vo, causal=True)   # eager work of the program between replays
        torch.cuda.synchronize()
        for name, got, want in zip(("prefill", "prefill_split", "decode"), _outs(bufs),
                                   ref[shift]):
            same = torch.equal(got.view(torch.int16), want.view(torch.int16))
            say(f"  replay {rep} inputs {shift} {name}: {'bit-identical' if same else 'DIFFERENT'}")
            assert same, (rep, shift, name)
