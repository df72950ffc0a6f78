"""CPU checks of the C ABI: libfa.so loads, exports every function include/fa.h declares, and
rejects invalid arguments with the documented status codes before any HIP call (so no GPU is
needed). No call here passes arguments that would reach a kernel launch."""
import os
import re

import pytest

import attention_causal_gqa_attn_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000          # a 64 KiB-aligned fake device address: never dereferenced here
ODD = P + 2          # 2-byte aligned only


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def header_enums():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(FA_\w+)\s*=\s*(-?\d+)", text)}


def test_library_exports_every_declared_function():
    lib = fa.load()
    declared = header_functions()
    assert set(declared) == set(fa.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    enums = header_enums()
    for name, value in enums.items():
        assert getattr(fa, name) == value, name


def test_version_and_strerror():
    assert fa.fa_version() == 10000
    codes = [v for k, v in header_enums().items() if k.startswith("FA_OK") or k.startswith("FA_ERR")]
    texts = {fa.fa_strerror(c) for c in codes}
    assert len(texts) == len(codes)
    assert fa.fa_strerror(12345) == "unknown status code"


def prefill(**kw):
    args = dict(q=P, k=P, v=P, o=P, B=1, Hq=32, Hkv=8, Sq=16, Sk=64, D=128, causal=1,
                causal_offset=48, scale=0.088, kv_dtype=0, stream=None)
    args.update(kw)
    return fa.fa_prefill(*args.values())


def decode(**kw):
    args = dict(q=P, k=P, v=P, o=P, B=4, Hq=32, Hkv=8, Sq=1, Sk=4096, D=128, causal=1,
                causal_offset=4095, scale=0.088, kv_dtype=2, workspace=P, workspace_bytes=0,
                stream=None)
    args.update(kw)
    return fa.fa_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(kv_dtype=5), fa.FA_ERR_DTYPE),
    (dict(kv_dtype=-1), fa.FA_ERR_DTYPE),
    (dict(Hq=30), fa.FA_ERR_SHAPE),
    (dict(Hkv=0), fa.FA_ERR_SHAPE),
    (dict(B=-1), fa.FA_ERR_SHAPE),
    (dict(Sq=-5), fa.FA_ERR_SHAPE),
    (dict(Sk=-1), fa.FA_ERR_SHAPE),
    (dict(D=0), fa.FA_ERR_SHAPE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(D=256), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa.FA_ERR_VALUE),
    (dict(scale=-0.1), fa.FA_ERR_VALUE),
    (dict(scale=float("nan")), fa.FA_ERR_VALUE),
    (dict(scale=float("inf")), fa.FA_ERR_VALUE),
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL),
    (dict(k=None), fa.FA_ERR_NULL),
    (dict(v=None), fa.FA_ERR_NULL),
    (dict(q=ODD), fa.FA_ERR_ALIGN),
    (dict(o=P + 8), fa.FA_ERR_ALIGN),
    (dict(k=P + 4), fa.FA_ERR_ALIGN),
    (dict(v=P + 4, kv_dtype=1), fa.FA_ERR_ALIGN),
    (dict(v=ODD, kv_dtype=2), fa.FA_ERR_ALIGN),
    # mixed caches: each tensor aligned by its own type (f16 16 bytes, q4_0 4)
    (dict(k=P + 4, kv_dtype=3), fa.FA_ERR_ALIGN),
    (dict(v=ODD, kv_dtype=3), fa.FA_ERR_ALIGN),
    (dict(k=ODD, kv_dtype=4), fa.FA_ERR_ALIGN),
    (dict(v=P + 4, kv_dtype=4), fa.FA_ERR_ALIGN),
    (dict(B=1 << 30, Sq=1 << 30, Hq=1 << 20, Hkv=1 << 20), fa.FA_ERR_SHAPE),
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


def prefill_split(**kw):
    args = dict(q=P, k=P, v=P, o=P, B=1, Hq=32, Hkv=8, Sq=2048, Sk=16384, D=128, causal=1,
                causal_offset=14336, scale=0.088, kv_dtype=0, workspace=P, workspace_bytes=0,
                stream=None)
    args.update(kw)
    return fa.fa_prefill_split(*args.values())


def test_prefill_workspace_bytes():
    # 2048 queries at the end of 16384 keys, GQA 32/8: query block q of 64 rows holds 225 + q
    # tiles, 240.5 on average; with the cap at 241 + 3 the 12 blocks above 244 (q = 20..31) of
    # each of the 8 KV heads split (their mirrors q = 0..11 run the rest): 96 units, 2 parts x
    # 4 waves x 64 rows x 132 floats each, after 4096 bytes of counters
    n = fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 0)
    assert n == 4096 + 96 * 2 * 4 * 64 * 132 * 4
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 1) == n   # bf16
    # q4_0 and mixed caches with 16 or more query blocks per KV head (32 here) are widened to
    # f16 after the split's bytes, one copy [1, 16384, 8, 128] per q4_0 tensor, and split as
    # f16 (the same plan), at D = 64 too
    copy = 16384 * 8 * 128 * 2
    assert n % 256 == 0
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 2) == n + 2 * copy
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 3) == n + copy
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 4) == n + copy
    n64 = fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 64, 1, 14336, 0)
    assert n64 > 0
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 64, 1, 14336, 2) == \
        (n64 + 255) // 256 * 256 + copy
    # the copy sits after the 4096 counter bytes even when nothing is split (non-causal)
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 0, 0, 2) == 4096 + 2 * copy
    # key split: 512 queries (8 blocks x 8 KV heads = 64 units) run 256 / 64 = 4 runs a unit,
    # 1024 queries (128 units) 2; a run holds 4 waves x 64 rows x 132 floats. The q4_0 cache
    # at 8 blocks stays fused (the f16 plan), at 16 it is copied first.
    run = 4 * 64 * 132 * 4
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 512, 16384, 128, 1, 15872, 0) == \
        4096 + 64 * 4 * run
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 512, 16384, 128, 1, 15872, 2) == \
        4096 + 64 * 4 * run
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 1024, 16384, 128, 1, 15360, 0) == \
        4096 + 128 * 2 * run
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 1024, 16384, 128, 1, 15360, 2) == \
        4096 + 128 * 2 * run + 2 * copy
    # 192 units (1536 queries) are more than half the CUs: pairing, no key split
    n1536 = fa.fa_prefill_workspace_bytes(1, 32, 8, 1536, 16384, 128, 1, 14848, 0)
    assert 4096 < n1536 < 4096 + 192 * run
    # nothing splits: non-causal, one small query block, empty calls
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 0, 0, 0) == 0
    assert fa.fa_prefill_workspace_bytes(1, 2, 2, 128, 128, 64, 1, 0, 0) == 0
    assert fa.fa_prefill_workspace_bytes(0, 32, 8, 2048, 16384, 128, 1, 14336, 0) == 0
    # more than 256 units (one workgroup per CU): the workgroups run in several rounds, whose
    # dispatch already evens the load, and nothing is paired (the call is fa_prefill); a q4_0
    # cache of 16+ query blocks per KV head is still copied first. 10 or 64 sequences of the
    # 2048-query chunk (2560, 16384 units), 4096 x 4096 keys (512 units)
    assert fa.fa_prefill_workspace_bytes(10, 32, 8, 2048, 16384, 128, 1, 14336, 0) == 0
    assert fa.fa_prefill_workspace_bytes(64, 32, 8, 2048, 16384, 128, 1, 14336, 0) == 0
    assert fa.fa_prefill_workspace_bytes(64, 32, 8, 2048, 16384, 128, 1, 14336, 2) == \
        4096 + 2 * 64 * copy
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 4096, 4096, 128, 1, 0, 0) == 0
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 4096, 4096, 128, 1, 0, 2) == \
        4096 + 2 * 4096 * 8 * 128 * 2
    # 256 units (2048 x 2048, one round) are still paired
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 2048, 128, 1, 0, 0) > 4096
    # invalid sizes give 0 too
    assert fa.fa_prefill_workspace_bytes(1, 30, 8, 2048, 16384, 128, 1, 14336, 0) == 0
    assert fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 96, 1, 14336, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=None, workspace_bytes=1 << 30), fa.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=4096), fa.FA_ERR_WORKSPACE),
    (dict(workspace=P + 8, workspace_bytes=1 << 30), fa.FA_ERR_ALIGN),
    (dict(kv_dtype=9), fa.FA_ERR_DTYPE),
    (dict(scale=0.0), fa.FA_ERR_VALUE),
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
])
def test_prefill_split_rejects(kw, code):
    assert prefill_split(**kw) == code


def test_prefill_split_short_workspace_refused():
    n = fa.fa_prefill_workspace_bytes(1, 32, 8, 2048, 16384, 128, 1, 14336, 0)
    assert prefill_split(workspace_bytes=n - 1) == fa.FA_ERR_WORKSPACE
    assert prefill_split(B=0, q=None, o=None, workspace=None) == fa.FA_OK   # empty: no-op


def test_prefill_empty_is_a_no_op():
    # nothing to compute: accepted without touching the device, even with NULL data
    assert prefill(B=0, q=None, o=None, k=None, v=None) == fa.FA_OK
    assert prefill(Sq=0, q=None, o=None) == fa.FA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(Sq=5), fa.FA_ERR_UNSUPPORTED),           # 5 * 4 rows > 16
    (dict(Hq=64, Hkv=2), fa.FA_ERR_UNSUPPORTED),   # 32 rows
    (dict(workspace=None, workspace_bytes=1 << 30), fa.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(workspace=P + 4, workspace_bytes=1 << 30), fa.FA_ERR_ALIGN),
    (dict(kv_dtype=7), fa.FA_ERR_DTYPE),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(k=P + 2), fa.FA_ERR_ALIGN),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def test_decode_workspace_bound():
    n = fa.fa_decode_workspace_bytes(4, 32, 8, 1, 32768, 128)
    # about 512 workgroups in all: for a q4_0 cache one per 4 KV heads and key range, so 64
    # splits per (b, KV head) here (16 for the 16-bit caches); each split a row of 4 query
    # heads x (128 outputs + frame + sum) f32, and the bound covers every cache type
    assert n == 4 * 8 * 64 * 4 * 130 * 4
    assert fa.fa_decode_workspace_bytes(4, 32, 4, 1, 32768, 128) == 4 * 4 * 32 * 8 * 130 * 4
    assert fa.fa_decode_workspace_bytes(4, 32, 8, 1, 0, 128) == 4 * 8 * 1 * 4 * 130 * 4
    assert fa.fa_decode_workspace_bytes(0, 32, 8, 1, 100, 128) == 0
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 100, 96) == 0
    # one sequence fills the 512 workgroups alone: 256 splits per (b, KV head) of 2 tiles each
    # (the 16-wave merge, 129-256 splits); two sequences 128 (the 8-wave merge); one KV head of
    # a 16-bit cache at 40000 keys 512 (the looped merge)
    assert fa.fa_decode_workspace_bytes(1, 32, 8, 1, 32768, 128) == 1 * 8 * 256 * 4 * 130 * 4
    assert fa.fa_decode_workspace_bytes(2, 32, 8, 1, 32768, 128) == 2 * 8 * 128 * 4 * 130 * 4
    assert fa.fa_decode_workspace_bytes(1, 4, 1, 1, 40000, 64) == 1 * 1 * 512 * 4 * 66 * 4
    # a workspace one byte short of the bound is refused for the largest causal offsets too
    for off in (4095, 100000):
        assert decode(workspace_bytes=fa.fa_decode_workspace_bytes(4, 32, 8, 1, 4096, 128) - 1,
                      causal_offset=off) == fa.FA_ERR_WORKSPACE


def test_dequant_rejects():
    assert fa.fa_dequant_q4_0(P, -1, P, P, None) == fa.FA_ERR_SHAPE
    assert fa.fa_dequant_q4_0(P, 0, None, None, None) == fa.FA_OK
    assert fa.fa_dequant_q4_0(None, 4, P, P, None) == fa.FA_ERR_NULL
    assert fa.fa_dequant_q4_0(P, 4, None, None, None) == fa.FA_ERR_NULL
    assert fa.fa_dequant_q4_0(P + 1, 4, P, P, None) == fa.FA_ERR_ALIGN
    assert fa.fa_dequant_q4_0(P, 4, P + 2, P, None) == fa.FA_ERR_ALIGN


def test_decode_paged_rejects():
    d = fa.fa_decode_paged
    # (q, k, v, o, table, lens, B, Hq, Hkv, Sq, D, max_pages, n_pages, causal, scale, kv,
    #  workspace, workspace_bytes, stream)
    base = [P, P, P, P, P, P, 4, 32, 8, 1, 128, 512, 4096, 1, 0.088, 2, P, 1 << 30, None]

    def call(**kw):
        names = ["q", "k", "v", "o", "table", "lens", "B", "Hq", "Hkv", "Sq", "D", "max_pages",
                 "n_pages", "causal", "scale", "kv", "ws", "ws_bytes", "stream"]
        args = list(base)
        for key, val in kw.items():
            args[names.index(key)] = val
        return d(*args)

    assert call(table=None) == fa.FA_ERR_NULL
    assert call(lens=None) == fa.FA_ERR_NULL
    assert call(table=P + 2) == fa.FA_ERR_ALIGN
    assert call(max_pages=-1) == fa.FA_ERR_SHAPE
    assert call(n_pages=-1) == fa.FA_ERR_SHAPE
    assert call(n_pages=0) == fa.FA_ERR_SHAPE              # table entries must name a page
    assert call(max_pages=1 << 26) == fa.FA_ERR_SHAPE
    assert call(kv=7) == fa.FA_ERR_DTYPE
    assert call(Hkv=2, Sq=2) == fa.FA_ERR_UNSUPPORTED       # 32 query rows per KV head
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(ws_bytes=100) == fa.FA_ERR_WORKSPACE
    assert call(ws=P + 4) == fa.FA_ERR_ALIGN
    assert call(B=0) == fa.FA_OK
    assert call(Sq=0) == fa.FA_OK


def test_prefill_paged_rejects():
    d = fa.fa_prefill_paged
    # (q, k, v, o, table, lens, q_lens, B, Hq, Hkv, Sq, D, max_pages, n_pages, causal, scale,
    #  kv, stream); every case below must be refused before a launch
    base = [P, P, P, P, P, P, P, 4, 32, 8, 128, 128, 512, 4096, 1, 0.088, 2, None]

    def call(**kw):
        names = ["q", "k", "v", "o", "table", "lens", "q_lens", "B", "Hq", "Hkv", "Sq", "D",
                 "max_pages", "n_pages", "causal", "scale", "kv", "stream"]
        args = list(base)
        for key, val in kw.items():
            args[names.index(key)] = val
        return d(*args)

    assert call(table=None) == fa.FA_ERR_NULL
    assert call(lens=None) == fa.FA_ERR_NULL
    assert call(table=P + 2) == fa.FA_ERR_ALIGN
    assert call(lens=P + 1) == fa.FA_ERR_ALIGN
    assert call(q_lens=P + 2) == fa.FA_ERR_ALIGN
    assert call(q=ODD) == fa.FA_ERR_ALIGN
    assert call(max_pages=-1) == fa.FA_ERR_SHAPE
    assert call(n_pages=-1) == fa.FA_ERR_SHAPE
    assert call(n_pages=0) == fa.FA_ERR_SHAPE              # table entries must name a page
    assert call(Hq=30) == fa.FA_ERR_SHAPE
    assert call(max_pages=4097) == fa.FA_ERR_UNSUPPORTED   # page numbers are held in LDS
    assert call(D=96) == fa.FA_ERR_UNSUPPORTED
    assert call(kv=7) == fa.FA_ERR_DTYPE
    assert call(scale=0.0) == fa.FA_ERR_VALUE
    assert call(B=0) == fa.FA_OK
    assert call(Sq=0, q_lens=None) == fa.FA_OK


def test_quantize_rejects():
    q = fa.fa_quantize_q4_0
    # (x, x_dtype, blocks, n_seq, rows_per_seq, D, x_seq_stride, blocks_seq_stride, stream)
    assert q(P, 3, P, 1, 1, 32, 0, 0, None) == fa.FA_ERR_DTYPE
    assert q(P, -1, P, 1, 1, 32, 0, 0, None) == fa.FA_ERR_DTYPE
    assert q(P, 1, P, 1, 1, 48, 0, 0, None) == fa.FA_ERR_SHAPE          # D % 32
    assert q(P, 1, P, 1, 1, 0, 0, 0, None) == fa.FA_ERR_SHAPE
    assert q(P, 1, P, -1, 1, 32, 0, 0, None) == fa.FA_ERR_SHAPE
    assert q(P, 1, P, 1, -1, 32, 0, 0, None) == fa.FA_ERR_SHAPE
    assert q(P, 1, P, 2, 4, 32, 64, 72, None) == fa.FA_ERR_SHAPE        # x stride < 4 rows
    assert q(P, 1, P, 2, 4, 32, 128, 70, None) == fa.FA_ERR_SHAPE       # block stride < 72
    assert q(P, 1, P, 2, 1 << 40, 1 << 20, 1 << 62, 1 << 60, None) == fa.FA_ERR_SHAPE
    assert q(None, 1, P, 1, 1, 32, 0, 0, None) == fa.FA_ERR_NULL
    assert q(P, 1, None, 1, 1, 32, 0, 0, None) == fa.FA_ERR_NULL
    assert q(ODD, 1, P, 1, 1, 32, 0, 0, None) == fa.FA_ERR_ALIGN        # x not 16-byte aligned
    assert q(P, 1, P + 1, 1, 1, 32, 0, 0, None) == fa.FA_ERR_ALIGN     # blocks odd
    assert q(P, 1, P, 2, 1, 32, 36, 18, None) == fa.FA_ERR_ALIGN       # 72-byte x stride
    assert q(P, 1, P, 2, 1, 32, 44, 18, None) == fa.FA_ERR_ALIGN       # 88-byte x stride
    assert q(P, 1, P, 2, 1, 32, 32, 19, None) == fa.FA_ERR_ALIGN       # odd block stride
    assert q(None, 1, None, 0, 5, 32, 0, 0, None) == fa.FA_OK          # nothing to do
    assert q(None, 1, None, 3, 0, 32, 0, 0, None) == fa.FA_OK


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    """The product path fails loudly when the HIP library is missing: no fallback."""
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fa.load()


# ---- tensor helpers: type, shape and device checks that run before any pointer is taken ----
# Host tensors are enough here: every rejection below is raised before the C ABI is called,
# and a host tensor with the right types is itself rejected (its address would reach the
# kernels as a wild pointer).

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _qkv(q_dtype, kv_dtype, D=128, Sq=4, Sk=8):
    import torch
    width = D // 32 * 18 if kv_dtype == torch.uint8 else D
    return (_t((1, Sq, 8, D), q_dtype), _t((1, Sk, 2, width), kv_dtype),
            _t((1, Sk, 2, width), kv_dtype))


@pytest.mark.parametrize("call", ["prefill", "prefill_split", "decode"])
def test_helpers_reject_wrong_q_type(call):
    import torch
    fn = getattr(fa, call)
    for qd, kvd in [(torch.float32, torch.float16), (torch.bfloat16, torch.float16),
                    (torch.float16, torch.bfloat16), (torch.float32, torch.uint8),
                    (torch.bfloat16, torch.uint8)]:
        q, k, v = _qkv(qd, kvd)
        with pytest.raises(ValueError, match="queries"):
            fn(q, k, v)


@pytest.mark.parametrize("call", ["prefill", "prefill_split", "decode"])
def test_helpers_reject_bad_out(call):
    import torch
    fn = getattr(fa, call)
    q, k, v = _qkv(torch.float16, torch.float16)
    for out in (_t((1, 4, 8, 64), torch.float16),            # too small
                _t((1, 4, 8, 128), torch.float32),           # wrong type
                _t((1, 8, 4, 128), torch.float16).transpose(1, 2)):   # not contiguous
        with pytest.raises(ValueError, match="out must be"):
            fn(q, k, v, out=out)


@pytest.mark.parametrize("call", ["prefill", "prefill_split", "decode"])
def test_helpers_reject_host_tensors(call):
    import torch
    fn = getattr(fa, call)
    for kvd in (torch.float16, torch.uint8):
        q, k, v = _qkv(torch.float16, kvd)
        with pytest.raises(ValueError, match="GPU tensors"):
            fn(q, k, v)
    q, k, v = _qkv(torch.bfloat16, torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        fn(q, k, v, out=torch.empty_like(q))


def test_paged_helpers_reject_wrong_types_and_host_tensors():
    import torch
    q = _t((2, 4, 8, 128), torch.float32)
    pages = _t((3, 64, 2, 128), torch.float16)
    table = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="queries"):
        fa.decode_paged(q, pages, pages, table, lens)
    with pytest.raises(ValueError, match="queries"):
        fa.prefill_paged(q, pages, pages, table, lens)
    q = q.half()
    with pytest.raises(ValueError, match="out must be"):
        fa.decode_paged(q, pages, pages, table, lens, out=_t((2, 4, 8, 64), torch.float16))
    with pytest.raises(ValueError, match="GPU tensors"):
        fa.decode_paged(q, pages, pages, table, lens)
    with pytest.raises(ValueError, match="GPU tensors"):
        fa.prefill_paged(q, pages, pages, table, lens)


def test_dequant_and_writer_reject_host_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU tensors"):
        fa.dequant_q4_0(_t((36,), torch.uint8))
    with pytest.raises(ValueError, match="GPU tensors"):
        fa.quantize_q4_0(_t((4, 32), torch.float16))


def test_stats_entry_points_reject():
    """The counter instances take the documented subset and check their counts buffer."""
    st = fa.fa_prefill_stats
    args = [P, P, P, P, 1, 32, 8, 16, 64, 128, 1, 48, 0.088]
    assert st(*args, 0, None, None) == fa.FA_ERR_NULL                   # counts missing
    assert st(*args, 0, ODD, None) == fa.FA_ERR_ALIGN                   # counts misaligned
    assert st(*args, 3, P, None) == fa.FA_ERR_UNSUPPORTED               # mixed cache
    assert st(*args[:9], 64, 1, 48, 0.125, 0, P, None) == fa.FA_ERR_UNSUPPORTED   # D = 64
    assert st(*args, 7, P, None) == fa.FA_ERR_DTYPE
    assert st(P, P, P, P, 1, 32, 8, 0, 64, 128, 1, 48, 0.088, 0, None, None) == fa.FA_OK
    dt = fa.fa_decode_stats
    dargs = [P, P, P, P, 4, 32, 8, 1, 4096, 128, 1, 4095, 0.088]
    nbytes = fa.fa_decode_workspace_bytes(4, 32, 8, 1, 4096, 128)
    assert dt(*dargs, 2, P, nbytes, None, None) == fa.FA_ERR_NULL
    assert dt(*dargs, 2, P, nbytes, ODD, None) == fa.FA_ERR_ALIGN
    assert dt(*dargs, 2, P, 16, P, None) == fa.FA_ERR_WORKSPACE
    assert dt(*dargs, 0, P, nbytes, P, None) == fa.FA_ERR_UNSUPPORTED    # f16: other kernel
    assert dt(P, P, P, P, 4, 32, 8, 2, 4096, 128, 1, 4094, 0.088, 2, P, nbytes, P,
              None) == fa.FA_ERR_UNSUPPORTED                             # 8 rows per KV head
    assert dt(P, P, P, P, 4, 8, 2, 1, 4096, 128, 1, 4095, 0.088, 2, P, nbytes, P,
              None) == fa.FA_ERR_UNSUPPORTED                             # Hkv not 4k


def test_standard_attention_rejects():
    sa = fa.fa_standard_attention
    args = [P, P, P, P, 1, 32, 8, 16, 64, 128, 1, 48, 0.088, 2]
    need = fa.fa_standard_workspace_bytes(1, 32, 8, 16, 64, 128, 2, 1)
    allu = fa.fa_standard_workspace_bytes(1, 32, 8, 16, 64, 128, 2, 0)
    assert 0 < need < allu
    assert sa(*args, None, need, None) == fa.FA_ERR_WORKSPACE
    assert sa(*args, P, need - 1, None) == fa.FA_ERR_WORKSPACE
    assert sa(*args, P + 16, need, None) == fa.FA_ERR_ALIGN             # 256-byte alignment
    assert sa(P, P, P, P, 1, 30, 8, 16, 64, 128, 1, 48, 0.088, 2, P, need,
              None) == fa.FA_ERR_SHAPE
    assert sa(P, P, P, P, 1, 32, 8, 16, 64, 96, 1, 48, 0.088, 2, P, need,
              None) == fa.FA_ERR_UNSUPPORTED
    assert sa(P, P, P, P, 1, 32, 8, 0, 64, 128, 1, 48, 0.088, 2, None, 0, None) == fa.FA_OK
    assert fa.fa_standard_workspace_bytes(1, 32, 8, 0, 64, 128, 2, 0) == 0
    # f16 caches need no dequantized copies: less workspace than q4_0 at the same shape
    assert fa.fa_standard_workspace_bytes(1, 32, 8, 16, 64, 128, 0, 1) < need
