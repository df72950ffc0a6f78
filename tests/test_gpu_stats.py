"""The deferred rescale, observed: counter instances of the prefill and q4_0 decode kernels
(fa_prefill_stats, fa_decode_stats) report per query row how often its softmax frame moved
and, for the prefill, in how many tiles its wave ran the O rescale.

mlxcel PR #2306 ("What changed", "Test plan"): O and l are rescaled only for a block whose
maximum passes the row's frame by more than the margin, which ordinary inputs do not meet once
a row has its first frame; inputs whose scores climb along the keys are what make it happen. So on N(0,1)
inputs every row's frame moves exactly once (from -inf to its first block maximum) and its
wave rescales O once, while under the +0.05-per-key ramp the frame moves about every 3-4
tiles (the ramp climbs 3.2 per 64-key tile against a margin of 10). The counter instances
run the same kernel source, so their outputs must equal the plain calls' bit for bit."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import workloads as W
from gpu_cases import compare, device_inputs, inputs, oracle_full, say

pytestmark = pytest.mark.gpu


def _prefill_counts(w):
    q, k, v = device_inputs(w, inputs(w))
    out, counts = fa.prefill_stats(q, k, v, causal=w.causal, offset=w.causal_offset,
                                   scale=w.scale)
    plain = fa.prefill(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the counter instance changed the output"
    return out, counts.cpu().numpy()


def _tiles_seen(w):
    """64-key tiles each query row sees, [Sq]."""
    i = np.arange(w.Sq, dtype=np.int64)
    return (np.clip(i + w.causal_offset + 1, 0, w.Sk) + 63) // 64


@pytest.mark.parametrize("name", ["prefill_16k_f16", "prefill_16k_bf16", "prefill_16k_q4_0",
                                  "prefill_2k_f16"])
def test_prefill_steady_state_never_rescales(name):
    w = W.WORKLOADS[name]
    say(f"prefill counters, N(0,1): {w}")
    out, c = _prefill_counts(w)
    moves, resc = c[..., 0], c[..., 1]
    say(f"  frame moves per row: min {moves.min()} max {moves.max()}; wave rescales: "
        f"min {resc.min()} max {resc.max()}")
    assert np.all(moves == 1), np.unique(moves, return_counts=True)
    assert np.all(resc == 1), np.unique(resc, return_counts=True)
    compare(w, out.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), name)


@pytest.mark.parametrize("name", ["prefill_16k_f16_ramp", "prefill_16k_bf16_ramp",
                                  "prefill_2k_f16_ramp"])
def test_prefill_ramp_fires_the_deferred_branch(name):
    w = W.WORKLOADS[name]
    say(f"prefill counters, score ramp: {w}")
    out, c = _prefill_counts(w)
    moves, resc = c[0, ..., 0], c[0, ..., 1]            # [Sq, Hq]
    t = _tiles_seen(w)[:, None].repeat(w.Hq, axis=1)
    say(f"  tiles per row {t.min()}..{t.max()}; frame moves per row {moves.min()}..{moves.max()}"
        f" (mean {moves.mean():.1f}); moves per tile {np.mean(moves / t):.3f}; wave rescales "
        f"{resc.min()}..{resc.max()}")
    long_rows = t >= 8
    assert np.all(moves[long_rows] >= 2)
    # a move every 2-6 tiles (3.2 per tile against a margin of 10, up to input rounding)
    assert np.all(moves[long_rows] >= t[long_rows] // 6)
    assert np.all(moves <= t // 2 + 2)
    # the wave rescales when any of its 32 rows moved: at least as often as each row
    blocks = resc.reshape(w.Sq // 32, 32, w.Hq)
    assert np.all(blocks == blocks[:, :1, :]), "a wave block's rescale count differs by row"
    assert np.all(resc >= moves)
    compare(w, out.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), name)


def _decode_counts(w):
    q, k, v = device_inputs(w, inputs(w))
    out, counts = fa.decode_stats(q, k, v, causal=w.causal, offset=w.causal_offset,
                                  scale=w.scale)
    plain = fa.decode(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the counter instance changed the output"
    return out, counts.cpu().numpy()


def test_decode_steady_state_never_rescales():
    """Every split starts its own frame: on N(0,1) inputs each split's frame moves exactly once
    per row."""
    w = W.WORKLOADS["decode_q4_0"]
    say(f"decode counters, N(0,1): {w}")
    out, c = _decode_counts(w)
    moves, splits = c[..., 0], c[..., 1]
    say(f"  splits per row {splits.min()}..{splits.max()}; frame moves {moves.min()}.."
        f"{moves.max()}")
    assert np.all(splits > 1)
    assert np.all(moves == splits)
    compare(w, out.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name)


def test_decode_ramp_fires_the_deferred_branch():
    """With the ramp, a split of 512 keys climbs about 22 in score (the q4_0 block scale takes
    7/8 of the ramp column), so each split's frame moves more than once."""
    w = W.WORKLOADS["decode_q4_0"].with_(ramp=0.05)
    say(f"decode counters, score ramp: {w}")
    out, c = _decode_counts(w)
    moves, splits = c[..., 0], c[..., 1]
    say(f"  splits per row {splits.min()}..{splits.max()}; frame moves {moves.min()}.."
        f"{moves.max()}")
    assert np.all(moves >= 2 * splits)
    compare(w, out.float().cpu().numpy().reshape(-1, w.D), oracle_full(w), w.name)
