"""Benchmark of the causal GQA flash-attention hot path on one MI355X.

One step = one pass of the whole path over resident inputs:
  * prefill: 2048 f16 queries as the last positions of 16384 keys, GQA 32/8, D=128, causal
    (fa_prefill, one MFMA kernel);
  * decode:  4 sequences x 1 query against 32768 q4_0-cached keys, GQA 32/8, D=128
    (fa_decode, split kernel + merge kernel);
  * the same prefill against a q4_0 cache (fa_prefill, dequantization in the kernel), and
    the unfused arm beside it: fa_dequant_q4_0 of K and V into f16 buffers, then the f16
    fa_prefill (reported, not part of `value`);
  * the q4_0 cache writer: fa_quantize_q4_0 of the prefill workload's f16 K and V (16384
    keys x 8 heads x 128) into q4_0 blocks (reported, HBM-bound);
  * the decode over a paged cache: the same 4 x 32768 q4_0 keys as 2048 pages of 64 keys in
    a shuffled order (fa_decode_paged; reported, HBM-bound);
  * the prefill over a paged cache: the f16 prefill's 16384 keys as 256 shuffled pages
    (fa_prefill_paged; reported, MFMA-bound);
  * mixed caches (f16 K, q4_0 V): the prefill workload and the decode workload's shape with
    those types (reported);
  * head dim 64: the prefill workload at D = 64, and the B=2, S=512, 8-head D=64 causal
    self-attention check shape (reported; the latter is launch- and latency-bound);
  * the decode workload's shape with an f16 cache (537 MB; the 16-bit split kernel);
  * the rest of the chunked-prefill configuration: 2048 queries at the end of 2048 and 8192
    keys (f16 and bf16), bf16 at 16384 keys, and the score-ramp variant at 16384 keys (f16 and
    bf16), and the balanced causal prefill (fa_prefill_split) at 2048, 8192 and 16384 keys
    (f16) and at 16384 keys over the q4_0 cache, under `prefill_sweep` (reported).
Before each call a 1 GiB buffer is read so that neither call finds its inputs in the 256 MB
last-level cache (the decode working set, 151 MB, would otherwise stay resident). The flush
reads rather than writes: a written flush leaves up to 256 MB of dirty lines in that cache,
and their write-back then runs inside the timed call (a plain 151 MB read kernel takes 61.7 us
after a 1 GiB fill, 33.1 us after a 1 GiB read, 27 us with its data cached).

Warm-up: untimed steps for 0.25 s of wall time (the GPU's clocks settle under load), then the
W warm-up steps; then K timed steps.

Prints one JSON line. `value` is prefill TFLOP/s (algorithmic FLOPs / mean kernel time from
HIP events on the launch stream); the decode HBM GB/s figure sits in `decode`. `roofline` is
for the prefill kernel, `roofline_decode` for the decode pair. `cpu_baseline` times the CPU
oracle on a bounded sample of the prefill workload's rows.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-sweep]
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
# the chunked-prefill configuration's other key counts, dtypes and the score ramp
SWEEP = ["prefill_2k_f16", "prefill_8k_f16", "prefill_2k_bf16", "prefill_8k_bf16",
         "prefill_16k_bf16", "prefill_16k_f16_ramp", "prefill_16k_bf16_ramp"]
# the balanced causal prefill (fa_prefill_split) beside fa_prefill at these shapes
SWEEP_SPLIT = ["prefill_16k_f16", "prefill_2k_f16", "prefill_8k_f16", "prefill_16k_q4_0"]


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    # leave out the prefill sweep, whose f16 legs run the headline prefill's kernel at other
    # sizes: a kernel-trace profile of the run then averages only the headline launches
    ap.add_argument("--no-sweep", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

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
    po = torch.empty_like(pq)
    do = torch.empty_like(dq)
    qo = torch.empty_like(qq)
    qo2 = torch.empty_like(qq)
    kf = torch.empty(wq.B, wq.Sk, wq.Hkv, wq.D, dtype=torch.float16, device=dev)
    vf = torch.empty_like(kf)
    q_blocks = qk.numel() // 18
    # the decode cache as 64-key pages in a seeded random order, and the block table
    per = wd.Sk // 64
    order = torch.from_numpy(np.random.default_rng(7).permutation(wd.B * per)).to(dev)
    dkp = dk.view(wd.B * per, 64, wd.Hkv, -1)[order].contiguous()
    dvp = dv.view(wd.B * per, 64, wd.Hkv, -1)[order].contiguous()
    table = torch.empty(wd.B * per, dtype=torch.int32, device=dev)
    table[order] = torch.arange(wd.B * per, dtype=torch.int32, device=dev)
    table = table.view(wd.B, per)
    lens = torch.full((wd.B,), wd.Sk, dtype=torch.int32, device=dev)
    do2 = torch.empty_like(dq)
    # the prefill cache the same way
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
    # mixed caches: f16 K with q4_0 V (the q4_0 prefill's V; a decode-shaped f16 K)
    po3 = torch.empty_like(pq)
    dkf = to_dev(W.generate(wd.with_(kv="f16")).k, "f16")
    do3 = torch.empty_like(dq)
    mbytes = dkf.numel() * 2 + dv.numel() + 2 * dq.numel() * 2
    # the decode shape with an f16 cache (K from the mixed leg's f16 draw, V its own)
    dvf = to_dev(W.generate(wd.with_(kv="f16", seed=wd.seed + 1)).v, "f16")
    do4 = torch.empty_like(dq)
    fbytes = (dkf.numel() + dvf.numel()) * 2 + 2 * dq.numel() * 2
    # head dim 64
    w64 = wp.with_(D=64)
    x64 = W.generate(w64)
    q64, k64, v64 = to_dev(x64.q, "f16"), to_dev(x64.k, "f16"), to_dev(x64.v, "f16")
    o64 = torch.empty_like(q64)
    wsm = W.WORKLOADS["p2check"]
    xsm = W.generate(wsm)
    qsm, ksm, vsm = to_dev(xsm.q, "f16"), to_dev(xsm.k, "f16"), to_dev(xsm.v, "f16")
    osm = torch.empty_like(qsm)
    wk = torch.empty(pk.numel() // 32 * 18, dtype=torch.uint8, device=dev)
    wv = torch.empty_like(wk)
    wbytes = (pk.numel() + pv.numel()) * 2 + wk.numel() + wv.numel()
    ws = torch.empty(max(16, fa.decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.Sq, wd.Sk, wd.D)),
                     dtype=torch.uint8, device=dev)
    sweep = []
    for name in ([] if args.no_sweep else SWEEP):
        w = W.WORKLOADS[name]
        x = W.generate(w)
        sq_ = to_dev(x.q, w.q_dtype)
        sweep.append((w, sq_, to_dev(x.k, w.kv), to_dev(x.v, w.kv), torch.empty_like(sq_)))
        del x
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
    # float32, so sum() is one reduction kernel that only reads (an int32 sum would first
    # write an int64 copy)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def prefill():
        fa.prefill(pq, pk, pv, causal=True, offset=wp.causal_offset, scale=wp.scale, out=po,
                   stream=stream)

    def decode():
        fa.decode(dq, dk, dv, causal=True, offset=wd.causal_offset, scale=wd.scale, out=do,
                  workspace=ws, stream=stream)

    def prefill_q4():
        fa.prefill(qq, qk, qv, causal=True, offset=wq.causal_offset, scale=wq.scale, out=qo,
                   stream=stream)

    def prefill_q4_unfused():
        for src, dst in ((qk, kf), (qv, vf)):
            rc = fa.fa_dequant_q4_0(src.data_ptr(), q_blocks, None, dst.data_ptr(),
                                    stream.cuda_stream)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, "fa_dequant_q4_0")
        fa.prefill(qq, kf, vf, causal=True, offset=wq.causal_offset, scale=wq.scale, out=qo2,
                   stream=stream)

    def quantize():
        fa.quantize_q4_0(pk.view(-1, wp.D), out=wk.view(-1, wp.D // 32 * 18), stream=stream)
        fa.quantize_q4_0(pv.view(-1, wp.D), out=wv.view(-1, wp.D // 32 * 18), stream=stream)

    def decode_paged():
        fa.decode_paged(dq, dkp, dvp, table, lens, causal=True, scale=wd.scale, out=do2,
                        workspace=ws, stream=stream)

    def prefill_paged():
        fa.prefill_paged(pq, pkp, pvp, ptable, plens, pqlens, causal=True, scale=wp.scale,
                         out=po2, stream=stream)

    def prefill_mixed():
        fa.prefill(pq, pk, qv, causal=True, offset=wp.causal_offset, scale=wp.scale, out=po3,
                   stream=stream)

    def decode_mixed():
        fa.decode(dq, dkf, dv, causal=True, offset=wd.causal_offset, scale=wd.scale, out=do3,
                  workspace=ws, stream=stream)

    def prefill_d64():
        fa.prefill(q64, k64, v64, causal=True, offset=w64.causal_offset, scale=w64.scale,
                   out=o64, stream=stream)

    def check_d64():
        fa.prefill(qsm, ksm, vsm, causal=True, offset=wsm.causal_offset, scale=wsm.scale,
                   out=osm, stream=stream)

    def decode_f16():
        fa.decode(dq, dkf, dvf, causal=True, offset=wd.causal_offset, scale=wd.scale, out=do4,
                  workspace=ws, stream=stream)

    def sweep_call(w, q_, k_, v_, o_):
        def call():
            fa.prefill(q_, k_, v_, causal=True, offset=w.causal_offset, scale=w.scale, out=o_,
                       stream=stream)
        return call

    calls = [prefill, decode, prefill_q4, prefill_q4_unfused, quantize, decode_paged,
             prefill_paged, prefill_mixed, decode_mixed, prefill_d64, check_d64, decode_f16]
    def split_call(w, q_, k_, v_, o_, ws_):
        def call():
            fa.prefill_split(q_, k_, v_, causal=True, offset=w.causal_offset, scale=w.scale,
                             out=o_, workspace=ws_, stream=stream)
        return call

    n_fixed = len(calls)
    calls += [sweep_call(*c) for c in sweep]
    calls += [split_call(*c) for c in split_legs]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(calls))]
          for _ in range(args.steps)]

    def step(i=None, k=0):
        for c, call in enumerate(calls):
            flush.sum()
            if i is not None:
                ev[i][2 * c].record(stream)
            call()
            if i is not None:
                ev[i][2 * c + 1].record(stream)

    # Warm-up: the GPU's clocks take tens of milliseconds of load to settle, so before the W
    # counted warm-up steps run untimed steps until CLOCK_WARMUP_S of wall time has passed.
    t_warm = time.perf_counter()
    k = 0
    while time.perf_counter() - t_warm < CLOCK_WARMUP_S:
        step(None, k)
        torch.cuda.synchronize()
        k += 1
    for k in range(args.warmup):
        step(None, k)
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    p_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    d_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    q_ms = np.array([e[4].elapsed_time(e[5]) for e in ev])
    u_ms = np.array([e[6].elapsed_time(e[7]) for e in ev])
    w_ms = np.array([e[8].elapsed_time(e[9]) for e in ev])
    g_ms = np.array([e[10].elapsed_time(e[11]) for e in ev])
    pp_ms = np.array([e[12].elapsed_time(e[13]) for e in ev])
    pm_ms = np.array([e[14].elapsed_time(e[15]) for e in ev])
    dm_ms = np.array([e[16].elapsed_time(e[17]) for e in ev])
    d64_ms = np.array([e[18].elapsed_time(e[19]) for e in ev])
    sm_ms = np.array([e[20].elapsed_time(e[21]) for e in ev])
    df_ms = np.array([e[22].elapsed_time(e[23]) for e in ev])
    prefill_sweep = {}
    for j, (w, *_rest) in enumerate(sweep):
        c = n_fixed + j
        ms = np.array([e[2 * c].elapsed_time(e[2 * c + 1]) for e in ev])
        tf = W.attention_flops(w) / (float(ms.mean()) * 1e-3) / 1e12
        prefill_sweep[w.name] = {
            "shape": f"B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.kv}"
                     + (f", score ramp +{w.ramp} per key" if w.ramp else ""),
            "tflops": round(tf, 3), "ms_mean": round(float(ms.mean()), 5),
            "ms_median": round(float(np.median(ms)), 5),
            "frac_of_mfma_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4)}
    for j, (w, *_rest) in enumerate(split_legs):
        c = n_fixed + len(sweep) + j
        ms = np.array([e[2 * c].elapsed_time(e[2 * c + 1]) for e in ev])
        tf = W.attention_flops(w) / (float(ms.mean()) * 1e-3) / 1e12
        prefill_sweep[w.name + "_split"] = {
            "shape": f"B={w.B} Sq={w.Sq} Sk={w.Sk} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.kv}, "
                     f"fa_prefill_split (balanced causal prefill)",
            "tflops": round(tf, 3), "ms_mean": round(float(ms.mean()), 5),
            "ms_median": round(float(np.median(ms)), 5),
            "frac_of_mfma_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4)}
    f64 = W.attention_flops(w64)
    fsm = W.attention_flops(wsm)
    qflops = W.attention_flops(wq)
    flops = W.attention_flops(wp)
    dbytes = W.algorithmic_bytes(wd)
    p_s = float(p_ms.mean()) * 1e-3
    d_s = float(d_ms.mean()) * 1e-3
    tflops = flops / p_s / 1e12
    gbs = dbytes / d_s / 1e9

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
        "prefill": {"tflops": round(tflops, 3), "ms_mean": round(float(p_ms.mean()), 5),
                    "ms_median": round(float(np.median(p_ms)), 5),
                    "ms_min": round(float(p_ms.min()), 5),
                    "ms_p90": round(float(np.percentile(p_ms, 90)), 5),
                    "gflop": round(flops / 1e9, 3)},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", "ms_mean": round(float(d_ms.mean()), 5),
                   "ms_median": round(float(np.median(d_ms)), 5),
                   "ms_min": round(float(d_ms.min()), 5),
                   "ms_p90": round(float(np.percentile(d_ms, 90)), 5),
                   "algorithmic_bytes": dbytes,
                   "kernels": "decode_q4g_kernel + decode_merge4_kernel"},
        "gpu_clock": clocks.summary(),
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
        "prefill_q4_0": {"workload": "prefill_16k_q4_0 (the prefill workload against a q4_0 "
                                     "K/V cache, dequantized in the kernel)",
                         "tflops": round(qflops / (float(q_ms.mean()) * 1e-3) / 1e12, 3),
                         "ms_mean": round(float(q_ms.mean()), 5),
                         "ms_median": round(float(np.median(q_ms)), 5),
                         "frac_of_mfma_peak": round(qflops / (float(q_ms.mean()) * 1e-3) / 1e12
                                                    / PEAK_MFMA_F16_TFLOPS, 4),
                         "kernel": "prefill16_kernel<128, q4_0, q4_0, contiguous>"},
        "prefill_q4_0_unfused": {"tflops": round(qflops / (float(u_ms.mean()) * 1e-3) / 1e12, 3),
                                 "ms_mean": round(float(u_ms.mean()), 5),
                                 "ms_median": round(float(np.median(u_ms)), 5),
                                 "what": "fa_dequant_q4_0 of K and V to f16 buffers (two "
                                         "launches), then the f16 fa_prefill",
                                 "extra_bytes": int(kf.numel() * 2 * 2)},
        "decode_paged": {"what": "the decode workload over its cache as 2048 shuffled pages of "
                                 "64 keys (fa_decode_paged, split + merge)",
                         "value": round(dbytes / (float(g_ms.mean()) * 1e-3) / 1e9, 1),
                         "unit": "GB/s", "ms_mean": round(float(g_ms.mean()), 5),
                         "frac_of_hbm_peak": round(dbytes / (float(g_ms.mean()) * 1e-3) / 1e9
                                                   / PEAK_HBM_GBS, 4)},
        "prefill_paged": {"what": "the prefill workload over its cache as 256 shuffled pages of "
                                  "64 keys (fa_prefill_paged)",
                          "tflops": round(flops / (float(pp_ms.mean()) * 1e-3) / 1e12, 3),
                          "ms_mean": round(float(pp_ms.mean()), 5),
                          "frac_of_mfma_peak": round(flops / (float(pp_ms.mean()) * 1e-3) / 1e12
                                                     / PEAK_MFMA_F16_TFLOPS, 4)},
        "prefill_mixed": {"what": "the prefill workload with f16 K and q4_0 V "
                                  "(FA_KV_F16_Q4_0)",
                          "tflops": round(flops / (float(pm_ms.mean()) * 1e-3) / 1e12, 3),
                          "ms_mean": round(float(pm_ms.mean()), 5),
                          "frac_of_mfma_peak": round(flops / (float(pm_ms.mean()) * 1e-3) / 1e12
                                                     / PEAK_MFMA_F16_TFLOPS, 4)},
        "decode_mixed": {"what": "4 x 1 query against 32768 keys, f16 K and q4_0 V "
                                 "(FA_KV_F16_Q4_0, split + merge)",
                         "value": round(mbytes / (float(dm_ms.mean()) * 1e-3) / 1e9, 1),
                         "unit": "GB/s", "bytes": int(mbytes),
                         "ms_mean": round(float(dm_ms.mean()), 5),
                         "frac_of_hbm_peak": round(mbytes / (float(dm_ms.mean()) * 1e-3) / 1e9
                                                   / PEAK_HBM_GBS, 4)},
        "prefill_d64": {"what": "the prefill workload at head dim 64 (2048 x 16384, GQA 32/8, f16)",
                        "tflops": round(f64 / (float(d64_ms.mean()) * 1e-3) / 1e12, 3),
                        "ms_mean": round(float(d64_ms.mean()), 5),
                        "frac_of_mfma_peak": round(f64 / (float(d64_ms.mean()) * 1e-3) / 1e12
                                                   / PEAK_MFMA_F16_TFLOPS, 4)},
        "check_d64": {"what": "causal self-attention B=2, S=512, Hq=Hkv=8, D=64, f16 (one call)",
                      "us_mean": round(float(sm_ms.mean()) * 1e3, 2),
                      "tflops": round(fsm / (float(sm_ms.mean()) * 1e-3) / 1e12, 3)},
        "decode_f16": {"what": "4 x 1 query against 32768 keys, f16 K and V (split + merge)",
                       "value": round(fbytes / (float(df_ms.mean()) * 1e-3) / 1e9, 1),
                       "unit": "GB/s", "bytes": int(fbytes),
                       "ms_mean": round(float(df_ms.mean()), 5),
                       "frac_of_hbm_peak": round(fbytes / (float(df_ms.mean()) * 1e-3) / 1e9
                                                 / PEAK_HBM_GBS, 4)},
        "quantize_q4_0": {"what": "fa_quantize_q4_0 of f16 K and V [1, 16384, 8, 128] (two "
                                  "launches)",
                          "gbs": round(wbytes / (float(w_ms.mean()) * 1e-3) / 1e9, 1),
                          "ms_mean": round(float(w_ms.mean()), 5),
                          "bytes": int(wbytes),
                          "frac_of_hbm_peak": round(wbytes / (float(w_ms.mean()) * 1e-3) / 1e9
                                                    / PEAK_HBM_GBS, 4)},
        "prefill_sweep": prefill_sweep,
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wp, xp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
