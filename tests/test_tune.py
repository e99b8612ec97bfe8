"""Tile-variant and launch-schedule search (tiled_tensor_core_amd/tune.py).

CPU: the cache helpers and the resource filter.  GPU: every kernel variant
the search can choose matches the fp64 oracle (ragged shapes, both dtypes and
head dims, both masks, and the mid and llama workloads whole); every variant
reports resources that pass the filter; every launch schedule gives its
variant's output bit for bit; and a search on a small workload writes a cache
entry that fwd_tuned then uses.
"""

import json

import pytest

from tiled_tensor_core_amd import attn, synth, tune
from parity import full_check, gpu_available, run_hip, whole_check


def test_cache_roundtrip(tmp_path):
    path = str(tmp_path / "cache.json")
    assert tune.lookup("bf16", 128, True, 256, 2048, path) is None
    key = tune.cache_key("bf16", 128, True, 256, 2048)
    assert key == "bf16/d128/causal/BH256/N2048"
    tune.store(key, {"cfg": [8, 64, 4, 1, 1, 2], "us": 1.0, "first_pass": [1, 2]}, path)
    tune.store(tune.cache_key("fp16", 64, False, 12, 100), {"cfg": [1, 5, 2, 2, 2, 1], "us": 2.0}, path)
    data = json.load(open(path))
    assert set(data) == {key, "fp16/d64/full/BH12/N100"}
    assert "first_pass" not in data[key]
    assert tune.lookup("bf16", 128, True, 256, 2048, path).as_tuple() == (8, 64, 4, 1, 1, 2)
    assert tune.lookup("fp16", 64, False, 12, 100, path).as_tuple() == (1, 5, 2, 2, 2, 1)
    assert tune.lookup("fp16", 64, True, 12, 100, path) is None
    # the per-(dtype, d, causal) variant is the fallback for untuned shapes,
    # and an entry from a larger workload is not replaced by a smaller one's
    tune.store(tune.cache_key("bf16", 128, True), {"cfg": [0, 0, 0, 0, 1, 2], "work": 100}, path,
               keep_larger_work=True)
    tune.store(tune.cache_key("bf16", 128, True), {"cfg": [0, 0, 0, 0, 2, 1], "work": 10}, path,
               keep_larger_work=True)
    assert tune.lookup("bf16", 128, True, 8, 77, path).as_tuple() == (0, 0, 0, 0, 1, 2)


def test_resource_filter():
    ok = dict(rows=128, waves=4, vgprs=250, lds_bytes=65552, scratch_bytes=0, groups_per_cu=2)
    assert tune.variant_fits(ok)[0]
    assert not tune.variant_fits(dict(ok, scratch_bytes=8))[0]
    assert not tune.variant_fits(dict(ok, groups_per_cu=0))[0]
    assert not tune.variant_fits(dict(ok, lds_bytes=96 * 1024))[0]     # 2 x 96 KiB > 160 KiB
    assert tune.variant_fits(dict(ok, lds_bytes=96 * 1024, groups_per_cu=1))[0]


def test_committed_cache_entries_are_well_formed():
    for key, e in tune.load_cache().items():
        parts = key.split("/")
        assert parts[0] in ("bf16", "fp16") and parts[1] in ("d64", "d128") and parts[2] in ("causal", "full")
        n_dom, n_work, grp, prio, mode, tile = e["cfg"]
        assert (mode, tile) in tune.VARIANTS
        if len(parts) == 5:
            assert n_dom in (1, 8) and n_work >= 1 and grp >= 1 and prio in (1, 2)
            assert e["us"] > 0 and e["default_us"] > 0
        else:
            assert (n_dom, n_work, grp, prio) == (0, 0, 0, 0)


def _inputs(B, H, N, d, dtype, seed):
    q, k, v = synth.make_qkv(B, H, N, d, dtype, seed=seed)
    return tuple(synth.to_torch(x, dtype, "cuda") for x in (q, k, v))


SHAPES = [  # B, H, N, d, dtype: 8 domains; 1 domain (B*H % 8 != 0); ragged N
    (2, 8, 1024, 64, "bf16"), (1, 6, 700, 128, "bf16"), (3, 5, 333, 64, "fp16"), (2, 4, 2048, 128, "fp16"),
]


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d,dtype", SHAPES)
def test_every_candidate_is_bit_identical(B, H, N, d, dtype, causal):
    """Every launch schedule the search tries gives its variant's built-in
    output bit for bit (schedules only reassign work items)."""
    import torch

    q, k, v = _inputs(B, H, N, d, dtype, seed=N)
    code = attn.ATTN_BF16 if dtype == "bf16" else attn.ATTN_FP16
    scale = d ** -0.5
    for mode, tile in tune.VARIANTS:
        o0, l0 = attn.fwd(q, k, v, causal, scale, cfg=(0, 0, 0, 0, mode, tile))
        cands = tune.candidates(B, H, N, d, causal, code, mode, tile)
        assert (cands[0].mode, cands[0].tile) == (mode, tile)
        print(f"[tune] {B},{H},{N},{d} {dtype} causal={causal} variant {mode},{tile}: {len(cands)} schedules",
              flush=True)
        for c in cands:
            o, lse = attn.fwd(q, k, v, causal, scale, cfg=c)
            torch.cuda.synchronize()
            assert torch.equal(o, o0) and torch.equal(lse, l0), f"{c} changed the output"


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_every_variant_fits_and_reports_its_resources(dtype, d, causal):
    code = attn.ATTN_BF16 if dtype == "bf16" else attn.ATTN_FP16
    for mode, tile in tune.VARIANTS:
        info = attn.attn_tile_info(tile, mode, code, d, int(causal))
        print(f"[tile] {dtype} d={d} causal={causal} mode={mode} tile={tile}: {info}", flush=True)
        assert info["rows"] == (256 if tile == attn.ATTN_TILE_256 else 128)
        assert info["waves"] * 32 == info["rows"]
        assert tune.variant_fits(info)[0], info
        assert 0 < info["vgprs"] <= 256
    with pytest.raises(attn.AttnError):
        attn.attn_tile_info(attn.ATTN_TILE_256, attn.ATTN_REF_RUNNING, code, d, int(causal))


VARIANT_SHAPES = [1, 33, 65, 200, 257, 383, 700]


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
@pytest.mark.parametrize("variant", tune.VARIANTS, ids=lambda v: f"mode{v[0]}-tile{v[1]}")
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_every_variant_matches_the_oracle(variant, dtype, d, causal):
    """Each kernel variant the search can choose, against the fp64 oracle, on
    ragged lengths that span one to several 256-row items."""
    mode, tile = variant
    for N in VARIANT_SHAPES:
        qb, kb, vb = synth.make_qkv(1, 3, N, d, dtype, seed=N + 17)
        full_check(qb, kb, vb, dtype, causal, d ** -0.5, cfg=(0, 0, 0, 0, mode, tile),
                   tag=f"variant {variant} {dtype} d={d} causal={causal} N={N}")


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
@pytest.mark.parametrize("variant", tune.VARIANTS, ids=lambda v: f"mode{v[0]}-tile{v[1]}")
@pytest.mark.parametrize("name", ["mid", "llama"])
def test_every_variant_on_the_workloads(variant, name):
    """Each variant on whole workloads (every row of every head) against the oracle."""
    w = synth.WORKLOADS[name]
    q, k, v = synth.make_workload(w)
    mode, tile = variant
    for causal in w.causal:
        o, lse = run_hip(q, k, v, w.dtype, causal, w.scale, cfg=(0, 0, 0, 0, mode, tile))
        whole_check(q, k, v, w.dtype, causal, w.scale, o.cpu().numpy(), lse.cpu().numpy(),
                    tag=f"variant {variant} {name} causal={causal}")


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
def test_resolved_builtin_configuration():
    # 4096 items, at least 4 per resident workgroup: one domain, twice the resident grid, groups of 8
    c = attn.attn_resolve_cfg(8, 32, 2048, 128, 1, attn.ATTN_BF16)
    assert c.n_dom == 1 and c.grp == 8 and c.prio == attn.ATTN_PRIO_ON and 2 <= c.n_work <= 8 * 32 * 16
    # 512 items, one per resident workgroup on this device: 8 domains, the resident grid
    cm = attn.attn_resolve_cfg(4, 16, 1024, 64, 1, attn.ATTN_BF16)
    assert cm.n_dom == 8 and 1 <= cm.n_work <= 4 * 16 * 8 // 8 and cm.grp >= 1
    assert c.n_work >= 2 * cm.n_work * cm.n_dom or c.n_work == 8 * 32 * 16
    c1 = attn.attn_resolve_cfg(1, 3, 500, 64, 0, attn.ATTN_FP16)
    assert c1.n_dom == 1 and c1.n_work <= 3 * 4 and c1.grp <= 3
    # explicit fields are kept, within what the shape allows
    c2 = attn.attn_resolve_cfg(8, 32, 2048, 128, 1, attn.ATTN_BF16, attn.LaunchCfg(1, 10 ** 6, 1000, 2))
    assert c2.as_tuple() == (1, 8 * 32 * 16, 8 * 32, 2, attn.ATTN_REF_FIXED, attn.ATTN_TILE_128)


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
def test_search_writes_a_validated_cache_entry(tmp_path):
    import torch

    path = str(tmp_path / "cache.json")
    q, k, v = _inputs(4, 16, 1024, 64, "bf16", seed=3)
    r = tune.tune(q, k, v, True, 0.125, reps=3, top=3, rounds=2, warm_s=0.1, cache_path=path)
    assert r["us"] <= r["default_us"] * 1.0001
    cfg = tune.lookup("bf16", 64, True, 64, 1024, path)
    assert cfg is not None and list(cfg.as_tuple()) == r["cfg"]
    o0, l0 = attn.fwd(q, k, v, True, 0.125)
    o1, l1 = tune.fwd_tuned(q, k, v, True, 0.125, cache_path=path)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
