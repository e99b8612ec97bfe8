"""Tile-variant and launch-schedule search for the attention kernel, with a
per-workload cache.

The TileLang tutorial's sections on schedule exploration and on autotuning
define a search space of tile shapes, pipeline depths and thread counts,
drop the configurations whose shared memory does not fit, and then compile,
benchmark and check the rest, keeping the fastest per workload in a cache.
Here the search space has two levels (include/attn.h, ``attn_launch_cfg``):

* the kernel variant, ``(mode, tile)``: ``tile`` is 128 query rows per work
  item on 4 waves (two workgroups per compute unit) or 256 rows on 8 waves
  (one per compute unit, each K/V tile in LDS shared by twice the rows);
  ``mode`` is the online softmax's exponent reference, fixed per item (no
  per-tile maximum or rescale) or the running maximum -- each is a different
  per-step instruction schedule, compiled as its own kernel;
* the launch schedule around a variant: ``n_dom`` (8 head domains, one per
  XCD, or 1), ``n_work`` (persistent workgroups per domain), ``grp`` (heads
  per group in the item order), ``prio`` (progress-based wave priority).

Every variant is compiled into the library (``python -m tiled_tensor_core_amd.
tune --build`` rebuilds it first).  Before timing, the search drops variants
whose compiled resources, as the device reports them (``attn_tile_info``),
spill registers to scratch, do not fit the compute unit's 160 KiB of LDS, or
run no workgroup on a compute unit.  Then each surviving variant's launch
schedules are checked to give O and LSE bit-identical to that variant's
built-in schedule (a schedule only reassigns work items), and each variant's
output is checked against the built-in variant's within the accuracy they
share.  The GPU tests tie every variant to the CPU oracle.

Timing is on the launch stream with HIP events after the GPU has reached its
sustained clocks; the short list is re-timed in interleaved rounds so clock
drift favours no candidate.  A candidate replaces the built-in one only if
faster by more than ``min_gain`` (the run-to-run spread).

The cache is JSON keyed by dtype, d, causal, B*H and N; each search also
records the winning variant per (dtype, d, causal) with its schedule left to
the built-in choice, which ``lookup`` falls back to for shapes never tuned.
"""

from __future__ import annotations

import json
import os
import time

from . import attn

CACHE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuned_cfgs.json")
LDS_PER_CU = 160 * 1024

# (mode, tile) pairs the library is compiled with
VARIANTS = [
    (attn.ATTN_REF_FIXED, attn.ATTN_TILE_128),
    (attn.ATTN_REF_RUNNING, attn.ATTN_TILE_128),
    (attn.ATTN_REF_FIXED, attn.ATTN_TILE_256),
]


def cache_key(dtype: str, d: int, causal: bool, BH: int | None = None, N: int | None = None) -> str:
    base = f"{dtype}/d{int(d)}/{'causal' if causal else 'full'}"
    return base if BH is None else f"{base}/BH{int(BH)}/N{int(N)}"


def _dtype_name(t) -> str:
    import torch

    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "fp16"
    raise TypeError(f"q must be bfloat16 or float16, got {t.dtype}")


def variant_fits(info: dict) -> tuple[bool, str]:
    """The search's resource filter for one compiled variant."""
    if info["scratch_bytes"] > 0:
        return False, f"spills {info['scratch_bytes']} bytes per lane"
    if info["groups_per_cu"] < 1:
        return False, "no workgroup fits a compute unit"
    if info["lds_bytes"] * info["groups_per_cu"] > LDS_PER_CU:
        return False, f"{info['lds_bytes']} B of LDS x {info['groups_per_cu']} workgroups exceeds 160 KiB"
    return True, "fits"


def variants(d, causal, dtype_code, log=None):
    """The (mode, tile) pairs that pass the resource filter, with their resources."""
    out = []
    for mode, tile in VARIANTS:
        info = attn.attn_tile_info(tile, mode, dtype_code, d, int(causal))
        ok, why = variant_fits(info)
        if log:
            log(f"  variant mode={mode} tile={tile}: {info} -> {why}")
        if ok:
            out.append((mode, tile, info))
    return out


def candidates(B, H, N, d, causal, dtype_code, mode=0, tile=0, wide=True):
    """Resolved, distinct launch schedules of one variant (its built-in first)."""
    base = attn.attn_resolve_cfg(B, H, N, d, causal, dtype_code, attn.LaunchCfg(0, 0, 0, 0, mode, tile))
    BH = B * H
    doms = [1, 8] if BH % 8 == 0 else [1]
    # n_work in units of the built-in total grid, spread over the domains
    total = base.n_dom * base.n_work
    fracs = (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0) if wide else (0.5, 1.0, 1.5, 2.0)
    grps = (0, 1, 2, 4, 8, 16) if wide else (0, 4, 8)
    seen, out = set(), []

    def add(c):
        r = attn.attn_resolve_cfg(B, H, N, d, causal, dtype_code, c)
        t = r.as_tuple()
        if t not in seen:
            seen.add(t)
            out.append(r)

    add(attn.LaunchCfg(0, 0, 0, 0, mode, tile))
    for nd in doms:
        for f in fracs:
            nw = max(1, int(round(total * f / nd)))
            for g in grps:
                for pr in (attn.ATTN_PRIO_ON, attn.ATTN_PRIO_OFF):
                    add(attn.LaunchCfg(nd, nw, g, pr, mode, tile))
    return out


def _time(torch, launch, stream, reps):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        launch()
        e.record(stream)
    torch.cuda.synchronize()
    ts = sorted(s.elapsed_time(e) for s, e in ev)
    return ts[len(ts) // 2] * 1e3   # median, microseconds


def tune(q, k, v, causal: bool, scale: float, reps: int = 10, top: int = 6, rounds: int = 5,
         warm_s: float = 0.5, min_gain: float = 0.01, cache_path: str | None = CACHE_PATH, log=None):
    """Search kernel variants and launch schedules for q, k, v ([B, H, N, d] on the GPU).

    Returns a dict with the chosen configuration and its median time, the
    built-in configuration and its time, the variants the resource filter
    kept or dropped, and every candidate's first-pass time.  Writes the entry
    (and the per-(dtype, d, causal) variant) to ``cache_path`` unless None.
    """
    import torch

    B, H, N, d = q.shape
    dname = _dtype_name(q)
    code = attn.ATTN_BF16 if dname == "bf16" else attn.ATTN_FP16
    stream = torch.cuda.current_stream()
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)

    def launch_with(c):
        return lambda: attn.attn_fwd_cfg(q, k, v, o, lse, B, H, N, d, causal, scale, stream, code, c)

    kept = variants(d, causal, code, log)
    dropped = [(m, t) for m, t in VARIANTS if (m, t) not in [(a, b) for a, b, _ in kept]]
    default = attn.attn_resolve_cfg(B, H, N, d, causal, code)
    cands = []
    for mode, tile, _ in kept:
        cands += candidates(B, H, N, d, causal, code, mode, tile, wide=(mode, tile) == (default.mode, default.tile))
    # the built-in configuration first
    cands.sort(key=lambda c: c.as_tuple() != default.as_tuple())
    assert cands[0].as_tuple() == default.as_tuple()

    # reference outputs: each variant's built-in schedule
    refs = {}
    for mode, tile, _ in kept:
        launch_with(attn.LaunchCfg(0, 0, 0, 0, mode, tile))()
        torch.cuda.synchronize()
        refs[(mode, tile)] = (o.clone(), lse.clone())
    o_def, l_def = refs[(default.mode, default.tile)]
    for key, (ov, lv) in refs.items():
        # variants differ in rounding only: far inside twice the oracle tolerance
        if not (float((ov - o_def).abs().max()) <= 2e-2 and float((lv - l_def).abs().max()) <= 2e-3):
            raise AssertionError(f"variant {key} disagrees with the built-in variant")
    # reach sustained clocks
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < warm_s:
        launch_with(cands[0])()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    first = []
    for c in cands:
        o.zero_()
        lse.zero_()
        launch_with(c)()
        torch.cuda.synchronize()
        ro, rl = refs[(c.mode, c.tile)]
        if not (torch.equal(o, ro) and torch.equal(lse, rl)):
            raise AssertionError(f"configuration {c} changed its variant's output")
        first.append((_time(torch, launch_with(c), stream, reps), c))
        if log:
            log(f"  {c}: {first[-1][0]:.1f} us")
    first.sort(key=lambda x: x[0])
    short = [c for _, c in first[:top]]
    # every variant's best schedule and the built-in configuration are re-timed too
    for mode, tile, _ in kept:
        best_v = next(c for _, c in first if (c.mode, c.tile) == (mode, tile))
        if best_v.as_tuple() not in [c.as_tuple() for c in short]:
            short.append(best_v)
    if cands[0].as_tuple() not in [c.as_tuple() for c in short]:
        short.append(cands[0])
    times = {c.as_tuple(): [] for c in short}
    for _ in range(rounds):
        for c in short:
            times[c.as_tuple()].append(_time(torch, launch_with(c), stream, reps))
    med = {t: sorted(v)[len(v) // 2] for t, v in times.items()}
    best = min(med, key=med.get)
    dflt = cands[0].as_tuple()
    fastest = best
    if med[dflt] < med[best] * (1.0 + min_gain):
        best = dflt
    per_variant = {}
    for t, m in med.items():
        key = f"mode{t[4]}/tile{t[5]}"
        if key not in per_variant or m < per_variant[key][0]:
            per_variant[key] = (round(m, 2), list(t))
    entry = {
        "cfg": list(best),
        "us": round(med[best], 2),
        "default_cfg": list(dflt),
        "default_us": round(med[dflt], 2),
        "speedup": round(med[dflt] / med[best], 4),
        "fastest_cfg": list(fastest),
        "fastest_us": round(med[fastest], 2),
        "best_per_variant": per_variant,
        "variants_kept": [[m, t, info] for m, t, info in kept],
        "variants_dropped": [list(x) for x in dropped],
        "candidates": len(cands),
        "validated": "every schedule bit-identical to its variant's built-in; every variant within 2e-2 (O) "
                     "and 2e-3 (LSE) of the built-in variant",
        "device": torch.cuda.get_device_name(q.device),
    }
    if cache_path is not None:
        store(cache_key(dname, d, causal, B * H, N), entry, cache_path)
        # the winning variant for this (dtype, d, causal), schedule left to the built-in choice
        store(cache_key(dname, d, causal), {"cfg": [0, 0, 0, 0, best[4], best[5]], "from": cache_key(
            dname, d, causal, B * H, N), "work": B * H * N * N * d}, cache_path, keep_larger_work=True)
    entry["first_pass"] = [(round(t, 2), c.as_tuple()) for t, c in first]
    return entry


def load_cache(cache_path: str = CACHE_PATH) -> dict:
    if not os.path.exists(cache_path):
        return {}
    with open(cache_path) as f:
        return json.load(f)


def store(key: str, entry: dict, cache_path: str = CACHE_PATH, keep_larger_work: bool = False) -> None:
    """Write one cache entry.  With ``keep_larger_work`` (the per-(dtype, d,
    causal) entries) an existing entry taken on a larger workload is kept."""
    data = load_cache(cache_path)
    if keep_larger_work and key in data and data[key].get("work", 0) > entry.get("work", 0):
        return
    data[key] = {k: v for k, v in entry.items() if k != "first_pass"}
    tmp = cache_path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    os.replace(tmp, cache_path)


def lookup(dtype: str, d: int, causal: bool, BH: int, N: int, cache_path: str = CACHE_PATH):
    """The cached LaunchCfg for a workload (exact shape first, then the
    winning variant for its dtype, d and mask), or None."""
    data = load_cache(cache_path)
    e = data.get(cache_key(dtype, d, causal, BH, N)) or data.get(cache_key(dtype, d, causal))
    return attn.LaunchCfg(*e["cfg"]) if e else None


def fwd_tuned(q, k, v, causal: bool, scale: float, stream=None, cache_path: str = CACHE_PATH):
    """attn.fwd with the cached configuration for this workload (built-in if none)."""
    B, H, N, d = q.shape
    cfg = lookup(_dtype_name(q), d, causal, B * H, N, cache_path)
    return attn.fwd(q, k, v, causal, scale, stream, cfg=cfg)


def main(argv=None):
    import argparse

    import torch

    from . import synth

    ap = argparse.ArgumentParser(description="search attention kernel variants and launch schedules; cache the best")
    ap.add_argument("--workload", action="append", help="synthetic workload name (repeatable; default all)")
    ap.add_argument("--cache", default=CACHE_PATH)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--build", action="store_true", help="compile every variant into the library first")
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    if a.build:
        from . import build

        print(build.build(), flush=True)
    torch.cuda.init()
    attn.load_library()
    names = a.workload or list(synth.WORKLOADS)
    log = (lambda s: print(s, flush=True)) if a.verbose else None
    for name in names:
        w = synth.WORKLOADS[name]
        q, k, v = (synth.to_torch(x, w.dtype, "cuda") for x in synth.make_workload(w))
        for causal in (False, True):
            r = tune(q, k, v, causal, w.scale, reps=a.reps, cache_path=a.cache, log=log)
            print(json.dumps({"workload": name, "causal": causal, **{k_: r[k_] for k_ in r if k_ != "first_pass"}}),
                  flush=True)
        del q, k, v
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
