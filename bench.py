"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

One step = one pass of the whole path over resident inputs:
  * prefill: 2048 f16 queries as the last positions of 16384 keys, GQA 32/8, D=128, causal
    (fa_prefill, one MFMA kernel) — `value`;
  * decode:  4 sequences x 1 query against 32768 q4_0-cached keys, GQA 32/8, D=128
    (fa_decode, split kernel + merge kernel) — `decode`;
  * the same prefill against a q4_0 cache (fa_prefill, dequantization in the kernel) and its
    two comparison arms: fa_dequant_q4_0 of K and V into f16 buffers then the f16 fa_prefill
    ("unfused"), and the standard non-flash path fa_standard_attention (dequantize, S =
    scale Q K^T materialised, softmax, P V); the decode workload the same three ways; and the
    standard path on the f16 caches beside the f16 flash kernels (the pages' FA-off arm);
  * a plain streaming read of as many bytes as the decode moves (fa_measure_read): the HBM
    read rate the decode is compared with on this GPU (`read_ceiling`);
  * the q4_0 cache writer: fa_quantize_q4_0 of the prefill workload's f16 K and V;
  * the decode over a paged cache (2048 shuffled 64-key pages) and the prefill over one (256);
  * mixed caches (f16 K, q4_0 V); head dim 64 (the prefill at D = 64, and the B=2, S=512,
    8-head D=64 causal check shape); the decode shape with an f16 cache;
  * `prefill_sweep`: 2048 queries at the end of 2048 and 8192 keys (f16, bf16), bf16 at 16384,
    the score ramp at 16384 (f16, bf16), and the balanced causal prefill (fa_prefill_split) at
    2048, 8192 and 16384 keys (f16) and at 16384 over the q4_0 cache.
Before each call a 1 GiB buffer is read so that no call finds its inputs in the 256 MB
last-level cache (the decode working set, 151 MB, would otherwise stay resident). The flush
reads rather than writes: a written flush leaves up to 256 MB of dirty lines in that cache,
and their write-back then runs inside the timed call.

Warm-up: untimed steps for 0.25 s of wall time (the GPU's clocks settle under load), then the
W warm-up steps; then K timed steps. Each call is bracketed by HIP events on its launch stream;
every leg reports the mean (its `value` figure) and the median, min and p90.

Idle check: before the warm-up and after the timed steps, the processes other than this one
that hold the GPU and the GPU use figure, from rocm-smi.

Prints one JSON line. `roofline` is for the prefill kernel, `roofline_decode` for the decode
pair. `cpu_baseline` times the CPU oracle on a bounded sample of the prefill workload's rows,
and on the whole decode workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-sweep]
                    [--gate]
    python bench.py --calibrate-copy     # a plain 256 MiB device copy, for HBM counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s at 2K-query×16K-key GQA32/8 D=128 f16; q4_0 decode HBM GB/s"
PEAK_MFMA_F16_TFLOPS = 2500.0      # MI355X dense f16/bf16 MFMA, published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E, published
PAGES_PREFILL_16K_TFLOPS = 1.20    # the pages' fixed kernel at 16K keys (Radeon 8060S, gfx1151)
FLUSH_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_16k_f16_traffic.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_q4_0_traffic.txt")
MFMA_UTIL_FILE = os.path.join(ROOT, "profiles", "prefill_16k_mfma_util.txt")
CLOCK_WARMUP_S = 0.25
# the chunked-prefill configuration's other key counts, dtypes and the score ramp, and a short
# chunk of 256 queries against 16384 keys
SWEEP = ["prefill_2k_f16", "prefill_8k_f16", "prefill_2k_bf16", "prefill_8k_bf16",
         "prefill_16k_bf16", "prefill_16k_f16_ramp", "prefill_16k_bf16_ramp",
         "chunk256_16k_f16", "chunk256_16k_q4_0"]
# the balanced causal prefill (fa_prefill_split) beside fa_prefill at these shapes (the 256-query
# chunks take its key split)
SWEEP_SPLIT = ["prefill_16k_f16", "prefill_2k_f16", "prefill_8k_f16", "prefill_16k_q4_0",
               "chunk256_16k_f16", "chunk256_16k_q4_0"]


def source_hash() -> str:
    """Hash of the kernel sources, to tell whether stored counter readings still apply."""
    csrc = os.path.join(ROOT, "attention_causal_gqa_attn_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch from a committed counter summary, if it was taken on the current
    kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(torch):
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n}), flush=True)


def stored_mfma_util():
    """(MFMA busy %, clock MHz) of the f16 prefill kernel from the committed counter summary, if
    it was taken on the current kernel sources."""
    if not os.path.exists(MFMA_UTIL_FILE):
        return None
    text = open(MFMA_UTIL_FILE).read()
    if f"source_hash {source_hash()}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("prefill16_kernel<128/0/0/false>,"):
            f = [x.strip() for x in line.split(",")]
            return float(f[3]), float(f[2])
    return None


class ClockSampler:
    """Samples the GPU's current shader-clock DPM level (the marked line of the amdgpu driver's
    pp_dpm_sclk) every 10 ms on a host thread; None where the file is not readable. This is the
    level the driver set, not the average clock under load, which the counter summary gives."""

    def __init__(self):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.mhz = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self.run, daemon=True)

    def read(self):
        for path in self.paths:
            try:
                for line in open(path):
                    if "*" in line:
                        return float(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def run(self):
        while not self.stop.wait(0.01):
            v = self.read()
            if v is not None:
                self.mhz.append(v)

    def __enter__(self):
        if self.paths:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.thread.is_alive():
            self.thread.join()

    def summary(self):
        if not self.mhz:
            return None
        import numpy as np
        a = np.array(self.mhz)
        return {"samples": int(a.size), "median_mhz": float(np.median(a)),
                "min_mhz": float(a.min()), "max_mhz": float(a.max()),
                "source": "pp_dpm_sclk (the DPM level set), every 10 ms during the timed steps"}


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, seconds: float):
    """The oracle, as it stands, on a random sample of the prefill workload's rows."""
    import numpy as np
    import oracle
    import workloads as W

    threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    total = w.B * w.Sq * w.Hq

    def run(n):
        rows = np.sort(rng.choice(total, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.attention(x.q, x.k, x.v, q_dtype=w.q_dtype, kv_dtype=w.kv, causal=w.causal,
                         offset=w.causal_offset, scale=w.scale, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        i = (rows // w.Hq) % w.Sq
        keys = np.clip(i + w.causal_offset + 1, 0, w.Sk)
        return dt, int(4 * w.D * keys.sum()), n

    # the oracle widens all of K and V once per call, a fixed cost: grow the sample until the
    # per-row work dominates, then size the timed sample to about `seconds`
    n = max(threads, 16)
    dt, _, _ = run(n)
    while dt < seconds / 8 and n < total:
        n = min(total, 4 * n)
        dt, _, _ = run(n)
    n_big = int(min(total, max(n, n * seconds / max(dt, 1e-3))))
    dt, flops, n = run(n_big)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": host_cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{n} of {total} query rows of the 2Kx16K f16 prefill (uniform random), "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s, {threads} OpenMP threads",
            "seconds": dt}


# Throughput floors of --gate (exit status 1 below either). The mlxcel PR gates its 16K-key
# call at a floor between the throughputs before and after its change; these sit 5 % under
# the figures this kernel set measured (bench.py on an MI355X: prefill_16k_f16 TFLOP/s, decode
# GB/s).
GATE_PREFILL_TFLOPS = 990.0
GATE_DECODE_GBS = 3380.0


def idle_check():
    """Processes other than this one that hold a GPU (the KFD's per-process directory) and
    the GPU busy figures the driver reports, read from sysfs."""
    import glob
    me = os.getpid()
    out = {"source": "/sys/class/kfd/kfd/proc and /sys/class/drm/card*/device/gpu_busy_percent"}
    try:
        out["other_gpu_pids"] = sorted(int(d) for d in os.listdir("/sys/class/kfd/kfd/proc")
                                       if d.isdigit() and int(d) != me)
    except OSError:
        out["other_gpu_pids"] = None
    busy = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/gpu_busy_percent")):
        try:
            busy.append(int(open(path).read().strip()))
        except (OSError, ValueError):
            continue
    out["gpu_busy_percent"] = busy or None
    return out


def toolchain():
    from attention_causal_gqa_attn_amd import build as fb
    info = fb.build_info()
    return {"hipcc_at_build": info.get("hipcc_version"),
            "tested_compiler": info.get("tested_compiler")}


def cpu_baseline_decode(w, x):
    """The oracle, as it stands, on every row of the decode workload (it widens all of K and V
    first, as for any call)."""
    import oracle
    import workloads as W

    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.attention(x.q, x.k, x.v, q_dtype=w.q_dtype, kv_dtype=w.kv, causal=w.causal,
                     offset=w.causal_offset, scale=w.scale, threads=threads)
    dt = time.perf_counter() - t0
    nbytes = W.algorithmic_bytes(w)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.B * w.Sq * w.Hq} rows of the 4 x 32768-key q4_0 decode, "
                      f"{nbytes / 1e6:.1f} MB in {dt:.2f} s, {threads} OpenMP threads",
            "seconds": dt}


def stats(ms):
    import numpy as np
    return {"ms_mean": round(float(ms.mean()), 5), "ms_median": round(float(np.median(ms)), 5),
            "ms_min": round(float(ms.min()), 5),
            "ms_p90": round(float(np.percentile(ms, 90)), 5)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    # leave out the prefill sweep and the batch-1 decode, which run the headline kernels at
    # other sizes: a kernel-trace profile of the run then averages only the headline launches
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--gate", action="store_true",
                    help="exit with status 1 if the prefill or decode falls below its floor")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

    idle_before = idle_check()

    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return

    import attention_causal_gqa_attn_amd as fa
    import workloads as W

    fa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    wp = W.WORKLOADS["prefill_16k_f16"]
    wd = W.WORKLOADS["decode_q4_0"]
    wq = W.WORKLOADS["prefill_16k_q4_0"]
    xp = W.generate(wp)
    xd = W.generate(wd)
    xq = W.generate(wq)
    pq, pk, pv = to_dev(xp.q, "f16"), to_dev(xp.k, "f16"), to_dev(xp.v, "f16")
    dq, dk, dv = to_dev(xd.q, "f16"), to_dev(xd.k, "q4_0"), to_dev(xd.v, "q4_0")
    qq, qk, qv = to_dev(xq.q, "f16"), to_dev(xq.k, "q4_0"), to_dev(xq.v, "q4_0")
    del xq
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    ws = torch.empty(max(16, fa.decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.Sq, wd.Sk, wd.D)),
                     dtype=torch.uint8, device=dev)

    def dequant(src, dst):
        rc = fa.fa_dequant_q4_0(src.data_ptr(), src.numel() // 18, None, dst.data_ptr(), sid)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_dequant_q4_0")

    legs = []          # (name, call)

    def leg(name):
        def add(fn):
            legs.append((name, fn))
            return fn
        return add

    # ---- headline legs and the q4_0 arms ------------------------------------------------
    po, do_, qo = torch.empty_like(pq), torch.empty_like(dq), torch.empty_like(qq)
    leg("prefill")(lambda: fa.prefill(pq, pk, pv, causal=True, offset=wp.causal_offset,
                                      scale=wp.scale, out=po, stream=stream))
    leg("decode")(lambda: fa.decode(dq, dk, dv, causal=True, offset=wd.causal_offset,
                                    scale=wd.scale, out=do_, workspace=ws, stream=stream))
    leg("prefill_q4_0")(lambda: fa.prefill(qq, qk, qv, causal=True, offset=wq.causal_offset,
                                           scale=wq.scale, out=qo, stream=stream))
    kf = torch.empty(wq.B, wq.Sk, wq.Hkv, wq.D, dtype=torch.float16, device=dev)
    vf = torch.empty_like(kf)
    qo2 = torch.empty_like(qq)

    @leg("prefill_q4_0_unfused")
    def _():
        dequant(qk, kf)
        dequant(qv, vf)
        fa.prefill(qq, kf, vf, causal=True, offset=wq.causal_offset, scale=wq.scale, out=qo2,
                   stream=stream)

    dkf_ = torch.empty(wd.B, wd.Sk, wd.Hkv, wd.D, dtype=torch.float16, device=dev)
    dvf_ = torch.empty_like(dkf_)
    do5 = torch.empty_like(dq)

    @leg("decode_q4_0_unfused")
    def _():
        dequant(dk, dkf_)
        dequant(dv, dvf_)
        fa.decode(dq, dkf_, dvf_, causal=True, offset=wd.causal_offset, scale=wd.scale,
                  out=do5, workspace=ws, stream=stream)

    # the standard (non-flash) arm: one workspace for the largest of its calls
    std_bytes = max(fa.standard_workspace_bytes(qq, qk, qv, 0),
                    fa.standard_workspace_bytes(pq, pk, pv, 0),
                    fa.standard_workspace_bytes(dq, dk, dv, 0))
    std_ws = torch.empty(std_bytes, dtype=torch.uint8, device=dev)
    qo3, po4, do6 = torch.empty_like(qq), torch.empty_like(pq), torch.empty_like(dq)
    leg("prefill_q4_0_standard")(lambda: fa.standard_attention(
        qq, qk, qv, causal=True, offset=wq.causal_offset, scale=wq.scale, out=qo3,
        workspace=std_ws, stream=stream))
    leg("decode_q4_0_standard")(lambda: fa.standard_attention(
        dq, dk, dv, causal=True, offset=wd.causal_offset, scale=wd.scale, out=do6,
        workspace=std_ws, stream=stream))
    leg("prefill_f16_standard")(lambda: fa.standard_attention(
        pq, pk, pv, causal=True, offset=wp.causal_offset, scale=wp.scale, out=po4,
        workspace=std_ws, stream=stream))

    # the read ceiling: a plain read of as many bytes as the decode moves
    dbytes = W.algorithmic_bytes(wd)
    rbuf = torch.ones((dbytes + 15) // 16 * 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    @leg("read_ceiling")
    def _():
        rc = fa.fa_measure_read(rbuf.data_ptr(), rbuf.numel() * 4, sink.data_ptr(), 0x9E3779B9,
                                0, sid)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_measure_read")

    # ---- the cache writer, paged, mixed, D = 64, f16 decode ---------------------------------
    wk = torch.empty(pk.numel() // 32 * 18, dtype=torch.uint8, device=dev)
    wv = torch.empty_like(wk)
    wbytes = (pk.numel() + pv.numel()) * 2 + wk.numel() + wv.numel()

    @leg("quantize_q4_0")
    def _():
        fa.quantize_q4_0(pk.view(-1, wp.D), out=wk.view(-1, wp.D // 32 * 18), stream=stream)
        fa.quantize_q4_0(pv.view(-1, wp.D), out=wv.view(-1, wp.D // 32 * 18), stream=stream)

    per = wd.Sk // 64
    order = torch.from_numpy(np.random.default_rng(7).permutation(wd.B * per)).to(dev)
    dkp = dk.view(wd.B * per, 64, wd.Hkv, -1)[order].contiguous()
    dvp = dv.view(wd.B * per, 64, wd.Hkv, -1)[order].contiguous()
    table = torch.empty(wd.B * per, dtype=torch.int32, device=dev)
    table[order] = torch.arange(wd.B * per, dtype=torch.int32, device=dev)
    table = table.view(wd.B, per)
    lens = torch.full((wd.B,), wd.Sk, dtype=torch.int32, device=dev)
    do2 = torch.empty_like(dq)
    leg("decode_paged")(lambda: fa.decode_paged(dq, dkp, dvp, table, lens, causal=True,
                                                scale=wd.scale, out=do2, workspace=ws,
                                                stream=stream))
    pper = wp.Sk // 64
    porder = torch.from_numpy(np.random.default_rng(8).permutation(wp.B * pper)).to(dev)
    pkp = pk.view(wp.B * pper, 64, wp.Hkv, -1)[porder].contiguous()
    pvp = pv.view(wp.B * pper, 64, wp.Hkv, -1)[porder].contiguous()
    ptable = torch.empty(wp.B * pper, dtype=torch.int32, device=dev)
    ptable[porder] = torch.arange(wp.B * pper, dtype=torch.int32, device=dev)
    ptable = ptable.view(wp.B, pper)
    plens = torch.full((wp.B,), wp.Sk, dtype=torch.int32, device=dev)
    pqlens = torch.full((wp.B,), wp.Sq, dtype=torch.int32, device=dev)
    po2 = torch.empty_like(pq)
    leg("prefill_paged")(lambda: fa.prefill_paged(pq, pkp, pvp, ptable, plens, pqlens,
                                                  causal=True, scale=wp.scale, out=po2,
                                                  stream=stream))
    po3 = torch.empty_like(pq)
    leg("prefill_mixed")(lambda: fa.prefill(pq, pk, qv, causal=True, offset=wp.causal_offset,
                                            scale=wp.scale, out=po3, stream=stream))
    dkf = to_dev(W.generate(wd.with_(kv="f16")).k, "f16")
    do3 = torch.empty_like(dq)
    mbytes = dkf.numel() * 2 + dv.numel() + 2 * dq.numel() * 2
    leg("decode_mixed")(lambda: fa.decode(dq, dkf, dv, causal=True, offset=wd.causal_offset,
                                          scale=wd.scale, out=do3, workspace=ws, stream=stream))
    dvf = to_dev(W.generate(wd.with_(kv="f16", seed=wd.seed + 1)).v, "f16")
    do4 = torch.empty_like(dq)
    fbytes = (dkf.numel() + dvf.numel()) * 2 + 2 * dq.numel() * 2
    leg("decode_f16")(lambda: fa.decode(dq, dkf, dvf, causal=True, offset=wd.causal_offset,
                                        scale=wd.scale, out=do4, workspace=ws, stream=stream))
    do7 = torch.empty_like(dq)
    leg("decode_f16_standard")(lambda: fa.standard_attention(
        dq, dkf, dvf, causal=True, offset=wd.causal_offset, scale=wd.scale, out=do7,
        workspace=std_ws, stream=stream))
    # one sequence of the decode cache (a batch-1 step): its key ranges fill the chip by
    # themselves, 256 per head group, so the merge combines more than 64 splits per row. A
    # sweep leg (the same kernels at another grid, kept out of the --no-sweep runs that the
    # per-kernel profiles average)
    dq1, dk1, dv1 = dq[:1], dk[:1], dv[:1]
    b1bytes = dk1.numel() + dv1.numel() + 2 * dq1.numel() * 2
    if not args.no_sweep:
        ws1 = torch.empty(max(fa.decode_workspace_bytes(1, wd.Hq, wd.Hkv, wd.Sq, wd.Sk, wd.D),
                              16), dtype=torch.uint8, device=dev)
        do8 = torch.empty_like(dq1)
        leg("decode_q4_0_b1")(lambda: fa.decode(dq1, dk1, dv1, causal=True,
                                                offset=wd.causal_offset, scale=wd.scale,
                                                out=do8, workspace=ws1, stream=stream))
    w64 = wp.with_(D=64)
    x64 = W.generate(w64)
    q64, k64, v64 = to_dev(x64.q, "f16"), to_dev(x64.k, "f16"), to_dev(x64.v, "f16")
    del x64
    o64 = torch.empty_like(q64)
    leg("prefill_d64")(lambda: fa.prefill(q64, k64, v64, causal=True, offset=w64.causal_offset,
                                          scale=w64.scale, out=o64, stream=stream))
    wsm = W.WORKLOADS["p2check"]
    xsm = W.generate(wsm)
    qsm, ksm, vsm = to_dev(xsm.q, "f16"), to_dev(xsm.k, "f16"), to_dev(xsm.v, "f16")
    osm = torch.empty_like(qsm)
    leg("check_d64")(lambda: fa.prefill(qsm, ksm, vsm, causal=True, offset=wsm.causal_offset,
                                        scale=wsm.scale, out=osm, stream=stream))

    # ---- the chunked-prefill sweep and the balanced prefill -------------------------------
    sweep = []
    for name in ([] if args.no_sweep else SWEEP):
        w = W.WORKLOADS[name]
        x = W.generate(w)
        sq_ = to_dev(x.q, w.q_dtype)
        sweep.append((w, sq_, to_dev(x.k, w.kv), to_dev(x.v, w.kv), torch.empty_like(sq_)))
        del x
    for w, q_, k_, v_, o_ in sweep:
        leg("sweep:" + w.name)((lambda w, q_, k_, v_, o_: lambda: fa.prefill(
            q_, k_, v_, causal=True, offset=w.causal_offset, scale=w.scale, out=o_,
            stream=stream))(w, q_, k_, v_, o_))
    split_legs = []
    if not args.no_sweep:
        have = {w.name: (w, q_, k_, v_) for w, q_, k_, v_, _o in sweep}
        have[wp.name] = (wp, pq, pk, pv)
        have[wq.name] = (wq, qq, qk, qv)
        for name in SWEEP_SPLIT:
            w, q_, k_, v_ = have[name]
            nb_ = fa.prefill_workspace_bytes(q_, k_, v_, offset=w.causal_offset)
            # zero-filled once: every call leaves its arrival counters at zero again
            ws_ = torch.zeros(max(16, nb_), dtype=torch.uint8, device=dev)
            split_legs.append((w, q_, k_, v_, torch.empty_like(q_), ws_))
    for w, q_, k_, v_, o_, ws_ in split_legs:
        leg("split:" + w.name)((lambda w, q_, k_, v_, o_, ws_: lambda: fa.prefill_split(
            q_, k_, v_, causal=True, offset=w.causal_offset, scale=w.scale, out=o_,
            workspace=ws_, stream=stream))(w, q_, k_, v_, o_, ws_))

    # float32, so sum() is one reduction kernel that only reads (an int32 sum would first
    # write an int64 copy)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(legs))]
          for _ in range(args.steps)]

    def step(i=None):
        for c, (_name, call) in enumerate(legs):
            flush.sum()
            if i is not None:
                ev[i][2 * c].record(stream)
            call()
            if i is not None:
                ev[i][2 * c + 1].record(stream)

    # Warm-up: the GPU's clocks take tens of milliseconds of load to settle, so before the W
    # counted warm-up steps run untimed steps until CLOCK_WARMUP_S of wall time has passed.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < CLOCK_WARMUP_S:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    time.sleep(0.2)
    idle_after = idle_check()

    ms = {name: np.array([e[2 * c].elapsed_time(e[2 * c + 1]) for e in ev])
          for c, (name, _call) in enumerate(legs)}

    def tflops_of(flops, name):
        return flops / (float(ms[name].mean()) * 1e-3) / 1e12

    def gbs_of(nbytes, name):
        return nbytes / (float(ms[name].mean()) * 1e-3) / 1e9

    def mfma_leg(flops, name, **extra):
        tf = tflops_of(flops, name)
        return {**extra, "tflops": round(tf, 3), **stats(ms[name]),
                "frac_of_mfma_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4)}

    def hbm_leg(nbytes, name, **extra):
        g = gbs_of(nbytes, name)
        return {**extra, "value": round(g, 1), "unit": "GB/s", "bytes": int(nbytes),
                **stats(ms[name]), "frac_of_hbm_peak": round(g / PEAK_HBM_GBS, 4)}

    prefill_sweep = {}
    for w, *_rest in sweep:
        prefill_sweep[w.name] = mfma_leg(
            W.attention_flops(w), "sweep:" + w.name,
            shape=f"B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.kv}"
                  + (f", score ramp +{w.ramp} per key" if w.ramp else ""))
    for w, *_rest in split_legs:
        prefill_sweep[w.name + "_split"] = mfma_leg(
            W.attention_flops(w), "split:" + w.name,
            shape=f"B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.kv}, "
                  f"fa_prefill_split (balanced causal prefill)")
    flops = W.attention_flops(wp)
    qflops = W.attention_flops(wq)
    tflops = tflops_of(flops, "prefill")
    gbs = gbs_of(dbytes, "decode")
    read_gbs = gbs_of(rbuf.numel() * 4, "read_ceiling")

    traffic = stored_traffic()
    dtraffic = stored_traffic(DECODE_TRAFFIC_FILE)
    util = stored_mfma_util()
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGES_PREFILL_16K_TFLOPS, 2),
        "vs_baseline_note": "ratio to the pages' 1.20 TFLOP/s (429.2 ms) at 16K keys, measured on "
                            "a Radeon 8060S (gfx1151): context from other hardware, not a target",
        "dtype": "f16",
        "data": "synthetic: seeded N(0,1) Q/K/V; q4_0 K/V quantized from N(0,1)",
        "config": {"workload": "prefill_16k_f16 (B=1 Sq=2048 Sk=16384 Hq=32 Hkv=8 D=128 causal, "
                               "offset Sk-Sq) + decode_q4_0 (B=4 Sq=1 Sk=32768 Hq=32 Hkv=8 D=128)",
                   "global_batch": wp.B, "seq_len": wp.Sk, "parallelism": "none (1 GPU)",
                   "cache_flush_bytes_read_before_each_call": FLUSH_BYTES},
        "prefill": {"tflops": round(tflops, 3), **stats(ms["prefill"]),
                    "gflop": round(flops / 1e9, 3)},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", **stats(ms["decode"]),
                   "algorithmic_bytes": dbytes,
                   "kernels": "decode_q4g_kernel + decode_merge4_kernel",
                   "frac_of_read_ceiling": round(gbs / read_gbs, 4)},
        "read_ceiling": {"what": "fa_measure_read: a plain 16-byte-load read of as many bytes as "
                                 "the decode moves, after the same read flush",
                         "value": round(read_gbs, 1), "unit": "GB/s",
                         "bytes": int(rbuf.numel() * 4), **stats(ms["read_ceiling"]),
                         "frac_of_hbm_peak": round(read_gbs / PEAK_HBM_GBS, 4)},
        "gpu_clock": clocks.summary(),
        "idle_check": {"before": idle_before, "after": idle_after},
        "toolchain": toolchain(),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_MFMA_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill16_kernel<128, f16, f16, contiguous>",
                     "algorithmic_flops_per_launch": flops,
                     # from profiles/prefill_16k_mfma_util.txt (rocprofv3 counters), if current
                     "mfma_busy_pct_counters": util[0] if util else None,
                     "clock_mhz_counters": util[1] if util else None,
                     "frac_of_clock_corrected_peak": (
                         round(tflops / (PEAK_MFMA_F16_TFLOPS * util[1] / 2400.0), 4)
                         if util else None)},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                            "traffic": dtraffic,
                            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "algorithmic_bytes_per_call": dbytes},
        "prefill_q4_0": mfma_leg(qflops, "prefill_q4_0",
                                 workload="prefill_16k_q4_0 (the prefill workload against a q4_0 "
                                          "K/V cache, dequantized in the kernel)",
                                 kernel="prefill16_kernel<128, q4_0, q4_0, contiguous>"),
        "prefill_q4_0_unfused": mfma_leg(qflops, "prefill_q4_0_unfused",
                                         what="fa_dequant_q4_0 of K and V to f16 buffers (two "
                                              "launches), then the f16 fa_prefill",
                                         extra_bytes=int(kf.numel() * 2 * 2)),
        "prefill_q4_0_standard": mfma_leg(qflops, "prefill_q4_0_standard",
                                          what="fa_standard_attention: K and V dequantized to "
                                               "f16, S materialised in f32, softmax, P V (the "
                                               "non-flash path)",
                                          workspace_bytes=int(fa.standard_workspace_bytes(
                                              qq, qk, qv, 0))),
        "prefill_f16_standard": mfma_leg(flops, "prefill_f16_standard",
                                         what="fa_standard_attention on the f16 prefill "
                                              "workload (the non-flash path with f16 V)"),
        "decode_q4_0_unfused": hbm_leg(dbytes, "decode_q4_0_unfused",
                                       what="fa_dequant_q4_0 of the decode cache to f16, then "
                                            "the f16 fa_decode (GB/s of the q4_0 bytes)"),
        "decode_q4_0_standard": hbm_leg(dbytes, "decode_q4_0_standard",
                                        what="fa_standard_attention on the decode workload "
                                             "(GB/s of the q4_0 bytes)"),
        "decode_paged": hbm_leg(dbytes, "decode_paged",
                                what="the decode workload over its cache as 2048 shuffled pages "
                                     "of 64 keys (fa_decode_paged, split + merge)"),
        "prefill_paged": mfma_leg(flops, "prefill_paged",
                                  what="the prefill workload over its cache as 256 shuffled "
                                       "pages of 64 keys (fa_prefill_paged)"),
        "prefill_mixed": mfma_leg(flops, "prefill_mixed",
                                  what="the prefill workload with f16 K and q4_0 V "
                                       "(FA_KV_F16_Q4_0)"),
        "decode_mixed": hbm_leg(mbytes, "decode_mixed",
                                what="4 x 1 query against 32768 keys, f16 K and q4_0 V "
                                     "(FA_KV_F16_Q4_0, split + merge)"),
        "prefill_d64": mfma_leg(W.attention_flops(w64), "prefill_d64",
                                what="the prefill workload at head dim 64 (2048 x 16384, GQA "
                                     "32/8, f16)"),
        "check_d64": {"what": "causal self-attention B=2, S=512, Hq=Hkv=8, D=64, f16 (one call)",
                      "us_mean": round(float(ms["check_d64"].mean()) * 1e3, 2),
                      "tflops": round(tflops_of(W.attention_flops(wsm), "check_d64"), 3)},
        "decode_f16": hbm_leg(fbytes, "decode_f16",
                              what="4 x 1 query against 32768 keys, f16 K and V (split + merge)"),
        "decode_f16_standard": hbm_leg(fbytes, "decode_f16_standard",
                                       what="fa_standard_attention on the f16 decode shape"),
        "decode_q4_0_b1": None if args.no_sweep else hbm_leg(
            b1bytes, "decode_q4_0_b1",
            what="1 x 1 query against 32768 q4_0 keys (the decode workload's first sequence: "
                 "256 key ranges per head group, merged by the 16-wave merge)"),
        "quantize_q4_0": hbm_leg(wbytes, "quantize_q4_0",
                                 what="fa_quantize_q4_0 of f16 K and V [1, 16384, 8, 128] (two "
                                      "launches)"),
        "prefill_sweep": prefill_sweep,
        "source_hash": source_hash(),
    }
    gate_ok = tflops >= GATE_PREFILL_TFLOPS and gbs >= GATE_DECODE_GBS
    line["gate"] = {"prefill_floor_tflops": GATE_PREFILL_TFLOPS,
                    "decode_floor_gbs": GATE_DECODE_GBS, "pass": bool(gate_ok)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wp, xp, args.cpu_seconds)
        line["cpu_baseline_decode"] = cpu_baseline_decode(wd, xd)
    print(json.dumps(line), flush=True)
    if args.gate and not gate_ok:
        print(f"gate: prefill {tflops:.1f} TFLOP/s (floor {GATE_PREFILL_TFLOPS}), decode "
              f"{gbs:.1f} GB/s (floor {GATE_DECODE_GBS})", file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
