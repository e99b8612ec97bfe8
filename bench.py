"""Benchmark of the fused attention forward pass on one MI355X.

A step is one call of the C ABI entry point ``attn_fwd`` over one batch of
synthetic inputs already resident in HBM: the causal B=8, H=32, N=2048,
d=128 bf16 workload by default (the throughput target).  The run prints one
JSON line with whole-job TFLOP/s, the MFMA roofline fraction of the kernel
(live, from HIP events on the launch stream), and the fp64 CPU oracle timed
on a bounded sample of the same workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--workload llama] [--no-cpu-baseline]
    python bench.py --kernel softmax [--softmax-workload scores]

FLOPs are algorithmic: 4*B*H*N^2*d, halved when causal (masked-tile waste and
padding are not counted).

Warm-up runs W untimed steps and continues until at least 0.5 s of GPU work
has passed: the GPU reaches its sustained clocks only after tens of
milliseconds of load, and timing before that under-reports a loaded GPU by
about 10 %.

``--kernel gemm`` times ``gemm_bf16`` with the bias + GELU epilogue on the
MLP up-projection workload (M=16384 tokens, K=4096, N=16384): 2*M*N*K FLOPs
against the dense bf16 MFMA peak.

``--kernel unfused`` times ``attn_fwd_unfused`` (scores in HBM, row softmax, P V)
on the same workload and reports its TFLOP/s (same FLOP count) and the HBM
roofline of its three-kernel step.

``--kernel softmax`` times the row-wise softmax entry point ``softmax_rows``
instead: a step is one softmax over a [rows, cols] matrix resident in HBM,
reported in GB/s of algorithmic traffic (each element read once and written
once) against the HBM roofline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FlashAttention fwd TFLOP/s (causal & non-causal) + % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = 2516.6          # MI355X dense bf16/fp16 MFMA
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "tiled_tensor_core_amd", "csrc", "attn_fwd_kernel.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_causal_b8h32n2048d128_traffic.txt")
SOFTMAX_METRIC = "row softmax GB/s (algorithmic bytes: one read and one write per element) + % of MI355X HBM peak"
SOFTMAX_SRC = os.path.join(ROOT, "tiled_tensor_core_amd", "csrc", "softmax_kernel.hip")
GEMM_METRIC = "GEMM + bias + GELU TFLOP/s (2*M*N*K) + % of MI355X bf16 MFMA peak"
GEMM_SRC = os.path.join(ROOT, "tiled_tensor_core_amd", "csrc", "gemm_kernel.hip")
UNFUSED_METRIC = ("un-fused attention fwd (scores in HBM, row softmax, P V) TFLOP/s + HBM roofline of the "
                  "three-kernel step")
UNFUSED_SRC = os.path.join(ROOT, "tiled_tensor_core_amd", "csrc", "unfused_kernel.hip")


def flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def kernel_source_hash(path=KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(path=TRAFFIC_FILE, src=KERNEL_SRC):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash(src):
        return None
    return float(t.group(1))


WARMUP_MIN_S = 0.5


class ClockSampler:
    """Samples the GPU's current shader clock every ``period`` seconds on a
    background thread while the timed loops run, as context beside the
    timings (the chip is power-bound, and boxes hold different clocks under
    load).  The clock is the starred level of the amdgpu driver's
    ``pp_dpm_sclk`` file (deep-sleep readings, marked ``S:``, are skipped); the
    summary is None where no such file is readable.  Only the host reads a
    file here; nothing is launched on the GPU."""

    def __init__(self, period=0.001):
        import glob

        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if "*" in line and not line.lstrip().startswith("S:"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading

        if self.path is not None:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        v = np.asarray(self.samples, dtype=np.float64)
        return {"median": float(np.median(v)), "min": float(v.min()), "max": float(v.max()),
                "samples": int(v.size), "source": self.path}


def warm_up(torch, launch, warmup, min_seconds=WARMUP_MIN_S):
    """Run ``warmup`` untimed launches, and more until ``min_seconds`` of
    wall time have passed with the GPU busy (synchronising every 8 launches,
    so the clock follows the GPU).  The GPU raises its clocks only after tens
    of milliseconds of sustained load: a timed loop that starts after a few
    milliseconds of warm-up runs about 10 % slower than every later one."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_seconds:
        launch()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_launches(torch, launch, stream, steps, warmup, warmup_s=WARMUP_MIN_S):
    """Time ``steps`` calls of ``launch()`` on ``stream`` after the warm-up.
    The whole-loop time per step comes from a loop bracketed by two events
    only; the per-launch times from a second loop of the same length with an
    event pair around each launch."""
    warm_up(torch, launch, warmup, warmup_s)
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    with ClockSampler() as clk:
        t_all0.record(stream)
        for _ in range(steps):
            launch()
        t_all1.record(stream)
        torch.cuda.synchronize()
        for i in range(steps):
            starts[i].record(stream)
            launch()
            ends[i].record(stream)
        torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    per = sorted(st.elapsed_time(e) for st, e in zip(starts, ends))
    return {
        "ms_per_step": total_ms / steps,
        "kernel_ms_mean": float(np.mean(per)),
        "kernel_ms_median": float(np.median(per)),
        "kernel_ms_min": float(per[0]),
        "kernel_ms_p90": float(np.percentile(per, 90)),
        "sclk_mhz": clk.summary(),
    }


def time_workload(attn, torch, w, causal, steps, warmup, inputs, warmup_s=WARMUP_MIN_S, cfg=None):
    q, k, v = inputs
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if cfg is None:
        launch = lambda: attn.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, w.scale, stream)
    else:
        launch = lambda: attn.attn_fwd_cfg(q, k, v, o, lse, B, H, N, d, causal, w.scale, stream, cfg=cfg)
    r = time_launches(torch, launch, stream, steps, warmup, warmup_s)
    r["flops"] = flops(B, H, N, d, causal)
    return r


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, causal, bits, budget_s):
    """The fp64 oracle on whole heads of the workload until ``budget_s`` of
    CPU time has passed; FLOPs credited with the same algorithmic count."""
    from oracle import attention_rows
    from tiled_tensor_core_amd import synth

    qb, kb, vb = bits
    cores = len(os.sched_getaffinity(0))
    from threadpoolctl import threadpool_info, threadpool_limits

    heads = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    rows = np.arange(w.N)
    with threadpool_limits(limits=cores):
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        for bh in range(w.B * w.H):
            b, h = divmod(bh, w.H)
            qh = synth.bits_to_f64(qb[b, h][None, None], w.dtype)
            kh = synth.bits_to_f64(kb[b, h][None, None], w.dtype)
            vh = synth.bits_to_f64(vb[b, h][None, None], w.dtype)
            ts = time.perf_counter()
            for r0 in range(0, w.N, 512):
                attention_rows(qh, kh, vh, causal, w.scale, 0, 0, rows[r0:r0 + 512])
            elapsed += time.perf_counter() - ts
            heads += 1
            if elapsed >= budget_s:
                break
    f = flops(1, heads, w.N, w.d, causal)
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                   if p.get("user_api") == "blas"})
    return {
        "value": f / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": host_cpu_model(),
        "blas": ", ".join(blas) or None,
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} heads (all {w.N} rows each), fp64 numpy, "
                  f"{elapsed:.1f} s; wall {time.perf_counter() - t0:.1f} s",
    }


def softmax_cpu_baseline(w, x, budget_s):
    """The fp64 softmax oracle on blocks of rows of the workload until
    ``budget_s`` of CPU time has passed (or every row is done); GB/s over the
    same algorithmic bytes.  numpy's element-wise max, exp and sum run on one
    thread, so one core is used."""
    from oracle import softmax_rows_ref
    from tiled_tensor_core_amd import synth

    block = max(1, (1 << 21) // w.cols)      # about 2M elements per call
    done = 0
    elapsed = 0.0
    t0 = time.perf_counter()
    for r0 in range(0, w.rows, block):
        xb = synth.softmax_to_f64(x[r0:r0 + block], w.dtype)
        ts = time.perf_counter()
        softmax_rows_ref(xb)
        elapsed += time.perf_counter() - ts
        done += xb.shape[0]
        if elapsed >= budget_s:
            break
    nbytes = 2.0 * done * w.cols * w.elem_bytes
    return {
        "value": nbytes / elapsed / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {w.rows} rows (all {w.cols} columns each), fp64 numpy, "
                  f"{elapsed:.1f} s; wall {time.perf_counter() - t0:.1f} s",
    }


def run_softmax(a, torch, attn, synth):
    w = synth.SOFTMAX_WORKLOADS[a.softmax_workload]
    print(f"[bench] generating softmax input {w.describe()}", file=sys.stderr, flush=True)
    x = synth.make_softmax_workload(w)
    xt = synth.softmax_to_torch(x, w.dtype, "cuda")
    yt = torch.empty_like(xt)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} softmax steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    r = time_launches(torch, lambda: attn.softmax_rows(xt, yt, w.rows, w.cols, stream=stream),
                      stream, a.steps, a.warmup, a.warmup_seconds)
    nbytes = 2.0 * w.rows * w.cols * w.elem_bytes
    value = nbytes / (r["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (r["kernel_ms_mean"] * 1e-3) / 1e9
    traffic = measured_traffic(os.path.join(ROOT, "profiles", f"softmax_{w.name}_r{w.rows}c{w.cols}_traffic.txt"),
                               SOFTMAX_SRC)
    out = {
        "metric": SOFTMAX_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"row softmax {w.name} {w.describe()}", "rows": w.rows, "cols": w.cols,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "sclk_mhz": r["sclk_mhz"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
            "kernel_ms_median": round(r["kernel_ms_median"], 5),
            "kernel_ms_min": round(r["kernel_ms_min"], 5),
            "kernel_ms_p90": round(r["kernel_ms_p90"], 5),
        },
    }
    if a.extra:
        per = {}
        for name, ow in synth.SOFTMAX_WORKLOADS.items():
            ox = synth.softmax_to_torch(synth.make_softmax_workload(ow), ow.dtype, "cuda")
            oy = torch.empty_like(ox)
            rr = time_launches(torch, lambda: attn.softmax_rows(ox, oy, ow.rows, ow.cols, stream=stream),
                               stream, 20, 5, a.warmup_seconds)
            per[f"{name} {ow.describe()}"] = round(
                2.0 * ow.rows * ow.cols * ow.elem_bytes / (rr["kernel_ms_median"] * 1e-3) / 1e9, 1)
            del ox, oy
            print(f"[bench] timed softmax {name}", file=sys.stderr, flush=True)
        out["per_workload_gbs"] = per
        # a plain device-to-device copy of the same bytes (torch's copy kernel),
        # as an empirical ceiling for a read-once, write-once kernel
        rc = time_launches(torch, lambda: yt.copy_(xt), stream, 20, 5, a.warmup_seconds)
        out["copy_same_bytes_gbs"] = round(nbytes / (rc["kernel_ms_median"] * 1e-3) / 1e9, 1)
    if not a.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{a.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = softmax_cpu_baseline(w, x, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def gemm_cpu_baseline(w, a_bits, w_bits, bias, budget_s):
    """The fp64 GEMM + bias + GELU oracle on blocks of 64 rows of A until
    ``budget_s`` of CPU time has passed; TFLOP/s over 2 * rows * N * K."""
    from oracle import EPI_BIAS_GELU, gemm_ref
    from tiled_tensor_core_amd import synth

    cores = len(os.sched_getaffinity(0))
    from threadpoolctl import threadpool_info, threadpool_limits

    w64 = synth.bits_to_f64(w_bits, "bf16")
    b64 = bias.astype(np.float64)
    done = 0
    elapsed = 0.0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        for r0 in range(0, w.M, 64):
            a64 = synth.bits_to_f64(a_bits[r0:r0 + 64], "bf16")
            ts = time.perf_counter()
            gemm_ref(a64, w64, b64, EPI_BIAS_GELU)
            elapsed += time.perf_counter() - ts
            done += a64.shape[0]
            if elapsed >= budget_s:
                break
    f = 2.0 * done * w.N * w.K
    return {
        "value": f / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {w.M} rows of A (all {w.N} outputs each), fp64 numpy, "
                  f"{elapsed:.1f} s; wall {time.perf_counter() - t0:.1f} s",
    }


def run_gemm(a, torch, attn, synth):
    wl = synth.GEMM_WORKLOADS[a.gemm_workload]
    print(f"[bench] generating GEMM inputs {wl.describe()}", file=sys.stderr, flush=True)
    a_bits, w_bits, bias = synth.make_gemm_workload(wl)
    at = synth.to_torch(a_bits, "bf16", "cuda")
    wt = synth.to_torch(w_bits, "bf16", "cuda")
    bt = torch.from_numpy(bias).cuda()
    ct = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} GEMM steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    r = time_launches(torch, lambda: attn.gemm_bf16(at, wt, bt, ct, wl.M, wl.N, wl.K, attn.GEMM_EPI_BIAS_GELU,
                                                    stream), stream, a.steps, a.warmup, a.warmup_seconds)
    f = wl.flops()
    value = f / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = f / (r["kernel_ms_mean"] * 1e-3) / 1e12
    traffic = measured_traffic(os.path.join(ROOT, "profiles", f"gemm_{wl.name}_m{wl.M}n{wl.N}k{wl.K}_traffic.txt"),
                               GEMM_SRC)
    out = {
        "metric": GEMM_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gemm + bias + gelu {wl.name} {wl.describe()}", "M": wl.M, "N": wl.N, "K": wl.K,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "sclk_mhz": r["sclk_mhz"],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
            "kernel_ms_median": round(r["kernel_ms_median"], 5),
            "kernel_ms_min": round(r["kernel_ms_min"], 5),
            "kernel_ms_p90": round(r["kernel_ms_p90"], 5),
        },
    }
    if a.extra:
        per = {}
        for name, ow in synth.GEMM_WORKLOADS.items():
            if name == wl.name:
                continue
            oa, ow_, ob = synth.make_gemm_workload(ow)
            oat, owt = synth.to_torch(oa, "bf16", "cuda"), synth.to_torch(ow_, "bf16", "cuda")
            obt = torch.from_numpy(ob).cuda()
            oct = torch.empty((ow.M, ow.N), dtype=torch.bfloat16, device="cuda")
            rr = time_launches(torch, lambda: attn.gemm_bf16(oat, owt, obt, oct, ow.M, ow.N, ow.K,
                                                             attn.GEMM_EPI_BIAS_GELU, stream),
                               stream, 20, 5, a.warmup_seconds)
            per[f"{name} {ow.describe()}"] = round(ow.flops() / (rr["kernel_ms_median"] * 1e-3) / 1e12, 1)
        out["per_workload_tflops"] = per
        # context: eager PyTorch on the same inputs (the library GEMM, then the bias and GELU
        # as separate elementwise kernels), whole-call time per step
        import torch.nn.functional as F

        rt = time_launches(torch, lambda: F.gelu(torch.addmm(bt.to(torch.bfloat16), at, wt.t())),
                           stream, 20, 5, a.warmup_seconds)
        out["eager_torch_tflops"] = round(f / (rt["kernel_ms_median"] * 1e-3) / 1e12, 1)
    if not a.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{a.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = gemm_cpu_baseline(wl, a_bits, w_bits, bias, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def unfused_bytes(B, H, N, d, causal):
    """Algorithmic HBM bytes of the un-fused path: the score matrix written
    (fp32), read and written by the row softmax, and read by P V (causal:
    only the N(N+1)/2 visible entries need reading); Q, K, V read once; O
    (fp32) and LSE written once."""
    bh = B * H
    vis = N * (N + 1) // 2 if causal else N * N
    return 4.0 * bh * (3 * N * N + vis) + bh * N * d * (3 * 2 + 4) + bh * N * 4


def run_unfused(a, torch, attn, synth):
    w = synth.WORKLOADS[a.workload]
    causal = w.causal[-1]
    print(f"[bench] generating {w.name} inputs {w.describe()}", file=sys.stderr, flush=True)
    bits = synth.make_workload(w)
    q, k, v = (synth.to_torch(x, w.dtype, "cuda") for x in bits)
    B, H, N, d = w.B, w.H, w.N, w.d
    need = attn.attn_unfused_workspace_bytes(B, H, N)
    ws = torch.empty((need // 4,), dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} un-fused steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    launch = lambda: attn.attn_fwd_unfused(q, k, v, o, lse, ws, need, B, H, N, d, causal, w.scale, stream)
    r = time_launches(torch, launch, stream, a.steps, a.warmup, a.warmup_seconds)
    f = flops(B, H, N, d, causal)
    nbytes = unfused_bytes(B, H, N, d, causal)
    value = f / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = nbytes / (r["kernel_ms_mean"] * 1e-3) / 1e9
    traffic = measured_traffic(os.path.join(ROOT, "profiles", f"unfused_{w.name}_traffic.txt"), UNFUSED_SRC)
    out = {
        "metric": UNFUSED_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"un-fused attention fwd {'causal' if causal else 'non-causal'} {w.describe()}",
            "B": B, "H": H, "N": N, "d": d, "causal": causal, "workspace_bytes": need,
            "parallelism": "none (1 GPU)",
        },
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "sclk_mhz": r["sclk_mhz"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": nbytes,
            "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
            "kernel_ms_median": round(r["kernel_ms_median"], 5),
            "kernel_ms_min": round(r["kernel_ms_min"], 5),
            "kernel_ms_p90": round(r["kernel_ms_p90"], 5),
            "note": "the three launches of one step (scores, row softmax, P V) between one event pair",
        },
    }
    if not a.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{a.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, causal, bits, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# Shapes of equal non-causal work (B*H*N^2 fixed, d = 128, bf16) whose items
# of 128 query rows hold 16, 32 and 64 key tiles of 64: the time split fit.
SPLIT_SHAPES = [(8, 128, 1024), (8, 32, 2048), (8, 8, 4096)]


def run_split(a, torch, attn, synth):
    """Where the attention kernel's time goes, from launch timings alone.

    Non-causal, a launch does items * tiles tile steps (tiles = N / 64 per
    128-row item) plus a fixed cost per item (loading Q, the first scores,
    the last P V, the epilogue).  The three shapes have the same number of
    tile steps and 2048, 4096 and 8192 items, so a straight-line fit of the
    kernel time against the item count gives the cost of the tile steps (the
    intercept) and of one item (the slope).  A causal item of query block qb
    does 2 (qb + 1) tile steps, the last two of them masked; the causal time
    minus the fit's prediction for those steps and items is the extra cost of
    the masked diagonal steps."""
    d = 128
    rows = []
    for B, H, N in SPLIT_SHAPES:
        w = synth.Workload(f"split{N}", B, H, N, d, "bf16", (False, True), synth.N01, synth.N01, synth.N01)
        print(f"[bench] split: generating {w.describe()}", file=sys.stderr, flush=True)
        inputs = tuple(synth.to_torch(x, w.dtype, "cuda") for x in synth.make_workload(w))
        nq = (N + 127) // 128
        for causal in (False, True):
            r = time_workload(attn, torch, w, causal, a.steps, a.warmup, inputs, a.warmup_seconds)
            steps = B * H * (nq * (nq + 1) if causal else nq * (N // 64))
            rows.append({"B": B, "H": H, "N": N, "causal": causal, "items": B * H * nq, "tile_steps": steps,
                         "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
                         "tflops": round(r["flops"] / (r["kernel_ms_mean"] * 1e-3) / 1e12, 2)})
            print(f"[bench] split: timed N={N} causal={causal}", file=sys.stderr, flush=True)
        del inputs
        torch.cuda.empty_cache()
    nc = [r for r in rows if not r["causal"]]
    x = [r["items"] for r in nc]
    y = [r["kernel_ms_mean"] for r in nc]
    n = len(x)
    mx, my = sum(x) / n, sum(y) / n
    slope = sum((xi - mx) * (yi - my) for xi, yi in zip(x, y)) / sum((xi - mx) ** 2 for xi in x)
    icpt = my - slope * mx
    t_step = icpt / nc[0]["tile_steps"]          # ms per tile step, device-wide
    split = {}
    for r in rows:
        if not r["causal"]:
            continue
        steps_ms = r["tile_steps"] * t_step
        item_ms = r["items"] * slope
        diag_ms = r["kernel_ms_mean"] - steps_ms - item_ms
        split[f"causal N={r['N']}"] = {
            "kernel_ms_mean": r["kernel_ms_mean"],
            "tile_steps_share": round(steps_ms / r["kernel_ms_mean"], 4),
            "per_item_share": round(item_ms / r["kernel_ms_mean"], 4),
            "masked_diagonal_extra_share": round(diag_ms / r["kernel_ms_mean"], 4),
        }
    for r in nc:
        split[f"non-causal N={r['N']}"] = {
            "kernel_ms_mean": r["kernel_ms_mean"],
            "tile_steps_share": round(r["tile_steps"] * t_step / r["kernel_ms_mean"], 4),
            "per_item_share": round(r["items"] * slope / r["kernel_ms_mean"], 4),
        }
    out = {
        "metric": "attention fwd time split (launch timings, straight-line fit over equal-work shapes)",
        "unit": "share of the kernel time",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"shapes": [f"B={B},H={H},N={N},d={d}" for B, H, N in SPLIT_SHAPES]},
        "fit": {"ms_per_tile_step_device": t_step, "ms_per_item_device": slope,
                "item_cost_in_tile_steps": round(slope / t_step, 3),
                "tile_step_tflops": round(2 * 2 * 128 * 64 * d / (t_step * 1e-3) / 1e12, 1)},
        "runs": rows,
        "split": split,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 700 steps: over 200 ms of timed launches on the default workload (about 0.3 ms each)
    ap.add_argument("--steps", type=int, default=700)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama")
    ap.add_argument("--kernel", choices=["attention", "softmax", "gemm", "unfused"], default="attention",
                    help="which entry point to time (default: the attention forward pass)")
    ap.add_argument("--softmax-workload", default="scores")
    ap.add_argument("--gemm-workload", default="mlp")
    ap.add_argument("--tuned", action="store_true",
                    help="run attention with the launch configuration cached by tiled_tensor_core_amd.tune "
                         "for this workload (attn_fwd_cfg) instead of the built-in one (attn_fwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-noncausal", action="store_true",
                    help="skip timing the causal workload's inputs without the mask")
    ap.add_argument("--warmup-seconds", type=float, default=WARMUP_MIN_S,
                    help="minimum warm-up time in seconds (0: exactly --warmup steps, as counter runs want)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--split", action="store_true",
                    help="time equal-work attention shapes and split the kernel time into tile steps, "
                         "per-item costs and the masked diagonal steps")
    ap.add_argument("--extra", action="store_true",
                    help="also time the other workloads (causal and non-causal) and report them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run three plain device-to-device copies of BYTES bytes (torch's copy "
                         "kernel), so HBM counters can be scaled by a transfer of known size")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the attention forward pass shards over "
              "(batch, head) with no exchange, so only the one-GPU figure is measured",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tiled_tensor_core_amd import attn, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.load_library()
    if a.copy_calibration > 0:
        n = a.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {n * 4} bytes three times", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()
    if a.kernel == "softmax":
        run_softmax(a, torch, attn, synth)
        return
    if a.kernel == "gemm":
        run_gemm(a, torch, attn, synth)
        return
    if a.kernel == "unfused":
        run_unfused(a, torch, attn, synth)
        return
    if a.split:
        run_split(a, torch, attn, synth)
        return
    w = synth.WORKLOADS[a.workload]
    causal = w.causal[-1]
    print(f"[bench] generating {w.name} inputs {w.describe()}", file=sys.stderr, flush=True)
    bits = synth.make_workload(w)
    inputs = tuple(synth.to_torch(x, w.dtype, "cuda") for x in bits)
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps after {a.warmup} warm-up", file=sys.stderr, flush=True)
    cfg = None
    if a.tuned:
        from tiled_tensor_core_amd import tune

        cfg = tune.lookup(w.dtype, w.d, causal, w.B * w.H, w.N)
        if cfg is None:
            print(f"[bench] no cached launch configuration for {w.name}; using the built-in one",
                  file=sys.stderr, flush=True)
    r = time_workload(attn, torch, w, causal, a.steps, a.warmup, inputs, a.warmup_seconds, cfg)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = r["flops"] / (r["kernel_ms_mean"] * 1e-3) / 1e12
    # the committed counter summary covers the causal B=8 H=32 N=2048 d=128 run
    traffic = measured_traffic() if (w.name == "llama" and causal) else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"attention fwd {'causal' if causal else 'non-causal'} {w.describe()}",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
            "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
            "launch": (f"tuned {list(cfg.as_tuple())}" if cfg is not None else "built-in"),
        },
        "pct_of_peak": round(100 * value / PEAK_TFLOPS, 2),
        "sclk_mhz": r["sclk_mhz"],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
            "kernel_ms_median": round(r["kernel_ms_median"], 5),
            "kernel_ms_min": round(r["kernel_ms_min"], 5),
            "kernel_ms_p90": round(r["kernel_ms_p90"], 5),
        },
    }
    if causal and not a.no_noncausal:
        # the same inputs without the causal mask, timed the same way (the
        # metric names both masks)
        rn = time_workload(attn, torch, w, False, a.steps, a.warmup, inputs, a.warmup_seconds, None)
        out["noncausal"] = {
            "value": round(rn["flops"] / (rn["ms_per_step"] * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(rn["ms_per_step"], 5),
            "kernel_ms_mean": round(rn["kernel_ms_mean"], 5),
            "frac": round(rn["flops"] / (rn["kernel_ms_mean"] * 1e-3) / 1e12 / PEAK_TFLOPS, 4),
            "sclk_mhz": rn["sclk_mhz"],
            "workload": f"attention fwd non-causal {w.describe()}",
        }
        print("[bench] timed the non-causal mask", file=sys.stderr, flush=True)
    if a.extra:
        per = {}
        for name, ow in synth.WORKLOADS.items():
            ob = bits if name == w.name else synth.make_workload(ow)
            oin = inputs if name == w.name else tuple(synth.to_torch(x, ow.dtype, "cuda") for x in ob)
            for c in (False, True):
                rr = time_workload(attn, torch, ow, c, 20, 5, oin, a.warmup_seconds)
                per[f"{name} {'causal' if c else 'non-causal'}"] = round(
                    rr["flops"] / (rr["kernel_ms_median"] * 1e-3) / 1e12, 2)
            del oin
            torch.cuda.empty_cache()
            print(f"[bench] timed {name}", file=sys.stderr, flush=True)
        out["per_workload_tflops"] = per
    if not a.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{a.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, causal, bits, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
