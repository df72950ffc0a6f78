"""Guard bands around every buffer a call writes. Each output and workspace is carved out of a
larger device buffer whose bytes on both sides (and in the padding after it) hold a fill
pattern; after the call the pattern must be intact, so no kernel wrote outside the buffers it
was given. The carved call's output must also equal the same call's output in a buffer of its
own, bit for bit (the fill pattern in a workspace is never read as data).

Shapes are small and ragged (tails of the 64-key tiles and 64-row blocks), and cover every
kernel family: the prefill instances (16-bit, q4_0, D = 64), the balanced prefill's pairing,
key split and f16 copy, the four decode kernels, the paged forms, the standard arm, the cache
writer and the dequantizer."""
import numpy as np
import pytest
import torch

import attention_causal_gqa_attn_amd as fa
import workloads as W
from gpu_cases import device_inputs, say, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of fill on each side of a carved buffer
FILL = 0xA5


class Arena:
    """Device buffers with fill-pattern guard bands around the region each one hands out."""

    def __init__(self):
        self.parts = []

    def carve(self, nbytes: int, dtype, shape):
        padded = (nbytes + 255) // 256 * 256
        buf = torch.full((GUARD + padded + GUARD,), FILL, dtype=torch.uint8, device="cuda")
        self.parts.append((buf, nbytes))
        region = buf[GUARD:GUARD + nbytes]
        return region.view(dtype).view(shape) if dtype != torch.uint8 else region.view(shape)

    def like(self, t):
        return self.carve(t.numel() * t.element_size(), t.dtype, tuple(t.shape))

    def check(self, label: str):
        torch.cuda.synchronize()
        for k, (buf, n) in enumerate(self.parts):
            pre = buf[:GUARD]
            post = buf[GUARD + n:]
            bad_pre = int((pre != FILL).sum().item())
            bad_post = int((post != FILL).sum().item())
            assert bad_pre == 0 and bad_post == 0, \
                f"{label}: buffer {k} has {bad_pre} bytes changed before it, {bad_post} after"


def wl(name, B, Hq, Hkv, Sq, Sk, D, kv="f16", causal=True, offset=None, seed=0):
    return W.Workload(name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, kv=kv, causal=causal,
                      offset=offset, seed=seed)


PREFILL = [
    wl("g_prefill_f16", 2, 8, 2, 100, 300, 128, "f16", True, 200, seed=201),
    wl("g_prefill_bf16_d64", 1, 6, 2, 70, 130, 64, "bf16", True, None, seed=202),
    wl("g_prefill_q4_0", 2, 8, 2, 90, 333, 128, "q4_0", True, 243, seed=203),
    wl("g_prefill_q4_0_d64", 1, 4, 1, 65, 200, 64, "q4_0", False, 0, seed=204),
]


@pytest.mark.parametrize("w", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_writes_only_its_output(w):
    say(f"guard: prefill {w}")
    q, k, v = device_inputs(w, W.generate(w))
    ref = fa.prefill(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    ar = Arena()
    out = ar.like(ref)
    fa.prefill(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale, out=out)
    ar.check(w.name)
    assert torch.equal(out, ref)


SPLIT = [
    # pairing (192 units), key split (8 units), the q4_0 copy with a key split, D = 64 bf16
    wl("g_split_pair", 3, 16, 8, 1024, 1100, 128, "f16", True, 76, seed=211),
    wl("g_split_parts", 1, 16, 4, 77, 2333, 64, "bf16", True, None, seed=212),
    wl("g_split_copy", 1, 8, 2, 1030, 1200, 128, "q4_0", True, 170, seed=213),
]


@pytest.mark.parametrize("w", SPLIT, ids=[w.name for w in SPLIT])
def test_prefill_split_writes_only_its_output_and_workspace(w):
    say(f"guard: prefill_split {w}")
    q, k, v = device_inputs(w, W.generate(w))
    ref = fa.prefill_split(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    nbytes = fa.prefill_workspace_bytes(q, k, v, causal=w.causal, offset=w.causal_offset)
    assert nbytes > 4096
    ar = Arena()
    out = ar.like(ref)
    ws = ar.carve(nbytes, torch.uint8, (nbytes,))
    ws[:4096].zero_()                      # the arrival counters start at zero
    fa.prefill_split(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale, out=out,
                     workspace=ws)
    ar.check(w.name)
    assert int(torch.count_nonzero(ws[:4096]).item()) == 0
    assert torch.equal(out, ref)


DECODE = [
    # head groups (GQA 32/8, 4 rows), wave-owned tiles (Hkv = 2), 16 rows per KV head, f16
    wl("g_decode_q4g", 4, 32, 8, 1, 5000, 128, "q4_0", True, None, seed=221),
    wl("g_decode_q4w", 2, 8, 2, 1, 777, 128, "q4_0", True, None, seed=222),
    wl("g_decode_q4_rows16", 2, 16, 2, 2, 1000, 64, "q4_0", True, None, seed=223),
    wl("g_decode_f16", 2, 8, 2, 3, 900, 128, "f16", True, None, seed=224),
    wl("g_decode_bf16_d64", 1, 8, 8, 1, 300, 64, "bf16", False, 0, seed=225),
]


@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_writes_only_its_output_and_workspace(w):
    say(f"guard: decode {w}")
    q, k, v = device_inputs(w, W.generate(w))
    ref = fa.decode(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale)
    nbytes = fa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D)
    ar = Arena()
    out = ar.like(ref)
    ws = ar.carve(nbytes, torch.uint8, (nbytes,))
    fa.decode(q, k, v, causal=w.causal, offset=w.causal_offset, scale=w.scale, out=out,
              workspace=ws)
    ar.check(w.name)
    assert torch.equal(out, ref)


def _in_order_pages(w, k, v):
    per = w.Sk // 64
    kp = k.view(w.B * per, 64, w.Hkv, -1)
    vp = v.view(w.B * per, 64, w.Hkv, -1)
    table = torch.arange(w.B * per, dtype=torch.int32, device="cuda").view(w.B, per)
    return kp, vp, table


@pytest.mark.parametrize("kv", ["q4_0", "f16"])
def test_paged_calls_write_only_their_outputs(kv):
    w = wl(f"g_paged_{kv}", 3, 8, 2, 2, 640, 128, kv, True, None, seed=231)
    say(f"guard: paged decode and prefill {w}")
    q, k, v = device_inputs(w, W.generate(w))
    kp, vp, table = _in_order_pages(w, k, v)
    lens = torch.tensor([640, 65, 1], dtype=torch.int32, device="cuda")
    ref = fa.decode_paged(q, kp, vp, table, lens, causal=True, scale=w.scale)
    nbytes = fa.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D)
    ar = Arena()
    out = ar.like(ref)
    ws = ar.carve(nbytes, torch.uint8, (nbytes,))
    fa.decode_paged(q, kp, vp, table, lens, causal=True, scale=w.scale, out=out, workspace=ws)
    ar.check(w.name + " decode")
    assert torch.equal(out, ref)

    wp = wl(f"g_paged_prefill_{kv}", 3, 8, 2, 100, 640, 128, kv, True, None, seed=232)
    q, k, v = device_inputs(wp, W.generate(wp))
    kp, vp, table = _in_order_pages(wp, k, v)
    lens = torch.tensor([640, 130, 64], dtype=torch.int32, device="cuda")
    qlens = torch.tensor([100, 37, 64], dtype=torch.int32, device="cuda")
    ref = fa.prefill_paged(q, kp, vp, table, lens, qlens, causal=True, scale=wp.scale)
    ar = Arena()
    out = ar.like(ref)
    out.zero_()                             # rows past a sequence's query count stay as given
    fa.prefill_paged(q, kp, vp, table, lens, qlens, causal=True, scale=wp.scale, out=out)
    ar.check(wp.name)
    assert torch.equal(out, ref)


def test_standard_attention_writes_only_its_output_and_workspace():
    w = wl("g_standard", 2, 8, 2, 150, 400, 128, "q4_0", True, 250, seed=241)
    say(f"guard: standard attention {w}")
    q, k, v = device_inputs(w, W.generate(w))
    ref = fa.standard_attention(q, k, v, causal=True, offset=w.causal_offset, scale=w.scale)
    for upp in (0, 1):
        nbytes = fa.standard_workspace_bytes(q, k, v, upp)
        ar = Arena()
        out = ar.like(ref)
        ws = ar.carve(nbytes, torch.uint8, (nbytes,))
        fa.standard_attention(q, k, v, causal=True, offset=w.causal_offset, scale=w.scale,
                              out=out, workspace=ws)
        ar.check(f"{w.name} units_per_pass={upp}")
        assert torch.equal(out, ref)


def test_writer_and_dequantizer_write_only_their_outputs():
    say("guard: q4_0 writer and dequantizer")
    rng = np.random.default_rng(251)
    x = torch.from_numpy(rng.standard_normal((3, 70, 2, 128), dtype=np.float32)).half().cuda()
    ref = fa.quantize_q4_0(x)
    ar = Arena()
    out = ar.like(ref)
    fa.quantize_q4_0(x, out=out)
    ar.check("quantize_q4_0")
    assert torch.equal(out, ref)

    blocks = ref.reshape(-1)
    n = blocks.numel() // 18
    f32_ref, f16_ref = fa.dequant_q4_0(blocks)
    ar = Arena()
    f32 = ar.carve(n * 32 * 4, torch.float32, (n * 32,))
    f16 = ar.carve(n * 32 * 2, torch.float16, (n * 32,))
    rc = fa.fa_dequant_q4_0(blocks.data_ptr(), n, f32.data_ptr(), f16.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK
    ar.check("dequant_q4_0")
    assert torch.equal(f32, f32_ref) and torch.equal(f16, f16_ref)
