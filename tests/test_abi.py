"""CPU tests of the C ABI: the library loads, exports what include/attn.h
declares, and rejects every invalid argument on the host with its status
code before any HIP call (so no GPU is needed)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

from tiled_tensor_core_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "softmax.h"), os.path.join(ROOT, "include", "gemm.h")]

# fake, 16-byte-aligned, well separated "device" addresses: validation never
# dereferences them, and every case below fails validation
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, causal=0, scale=0.125)


def _call(fn="attn_fwd", dtype=0, **over):
    a = dict(GOOD)
    a.update(over)
    lib = attn.load_library()
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
            a["causal"], a["scale"], None)
    if fn == "attn_fwd":
        return lib.attn_fwd(*args, dtype)
    if fn == "attn_fwd_cfg":
        cfg = over.get("cfg")
        return lib.attn_fwd_cfg(*args, dtype, ctypes.byref(cfg) if cfg is not None else None)
    return getattr(lib, fn)(*args)


def declared_functions():
    names = set()
    for header in HEADERS:
        text = open(header).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b((?:attn|softmax|gemm)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(attn.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = attn.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT ((?:attn|softmax|gemm)_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_library_is_built_for_gfx950():
    """The offload bundle of our own build names gfx950 and nothing else."""
    data = open(attn.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"hipv4-amdgcn-amd-amdhsa-[-a-z0-9:+]*", data))
    assert targets == {b"hipv4-amdgcn-amd-amdhsa--gfx950"}


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_bf16", "attn_fwd_fp16", "attn_fwd_cfg"])
@pytest.mark.parametrize("over,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(N=-5), 2), (dict(B=1 << 16, H=1 << 16), 2),
    # one head's fp32 O plus 128 rows must stay within 32-bit byte offsets
    (dict(B=1, H=1, N=(1 << 23) - 128, d=128), 2), (dict(B=1, H=1, N=(1 << 24) - 128, d=64), 2),
    (dict(d=96), 3), (dict(d=0), 3), (dict(d=256), 3),
    (dict(q=Q + 8), 4), (dict(o=O + 4), 4), (dict(lse=L + 2), 4),
    (dict(scale=math.nan), 7), (dict(scale=math.inf), 7), (dict(scale=-math.inf), 7),
    (dict(scale=3.0e38), 7),
    (dict(causal=2), 8), (dict(causal=-1), 8),
    (dict(o=Q), 9), (dict(lse=V + 16), 9), (dict(lse=O + 64), 9),
])
def test_rejects_invalid_arguments(fn, over, code):
    assert _call(fn, **over) == code


def test_rejects_unknown_dtype():
    assert _call("attn_fwd", dtype=2) == 5
    assert _call("attn_fwd", dtype=-1) == 5


def test_status_strings():
    lib = attn.load_library()
    seen = set()
    for code in attn.STATUS:
        s = attn.attn_status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == len(attn.STATUS)
    assert attn.attn_status_str(99) == "unknown status"
    assert lib.attn_last_error() == b""


def test_block_rows():
    assert attn.attn_block_rows(64) > 0 and attn.attn_block_rows(128) > 0
    assert attn.attn_block_rows(96) == 0


def test_binding_raises_named_error():
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd(Q, K, V, O, L, 2, 3, 100, 96, 0, 0.1, stream=0, dtype=0)
    assert e.value.code == 3 and e.value.name == "ATTN_ERR_UNSUPPORTED_D"
    with pytest.raises(TypeError):
        attn.attn_fwd(Q, K, V, O, L, 2, 3, 100, 64, 0, 0.1, stream=0)


def test_missing_library_fails_loudly(tmp_path):
    import importlib

    mod = importlib.reload(attn)
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        importlib.reload(attn)


# ---- row softmax entry point -------------------------------------------------

SM_GOOD = dict(x=Q, y=O, rows=4, cols=100, dtype=1)


@pytest.mark.parametrize("over,code", [
    (dict(x=0), 1), (dict(y=0), 1),
    (dict(rows=0), 2), (dict(cols=0), 2), (dict(rows=-1), 2), (dict(cols=1 << 30), 2),
    (dict(dtype=3), 5), (dict(dtype=-1), 5),
    (dict(x=Q + 2), 4), (dict(y=O + 8), 4),
    (dict(y=Q + 16), 9),
])
def test_softmax_rejects_invalid_arguments(over, code):
    a = dict(SM_GOOD)
    a.update(over)
    lib = attn.load_library()
    assert lib.softmax_rows(a["x"], a["y"], a["rows"], a["cols"], a["dtype"], None) == code


BAD_CFGS = [  # (n_dom, n_work, grp, prio)
    (2, 0, 0, 0), (-1, 0, 0, 0), (16, 0, 0, 0), (0, -1, 0, 0), (0, (1 << 20) + 1, 0, 0),
    (0, 0, -3, 0), (0, 0, 0, 3), (0, 0, 0, -1), (0, 0, 0, 0, 3), (0, 0, 0, 0, -1),
    (0, 0, 0, 0, 0, 3), (0, 0, 0, 0, 0, -1), (0, 0, 0, 0, 2, 2),
]


@pytest.mark.parametrize("fields", BAD_CFGS, ids=str)
def test_cfg_rejects_out_of_range_fields(fields):
    """Checked on the host before any HIP call (no GPU here)."""
    cfg = attn.LaunchCfg(*fields)
    assert _call("attn_fwd_cfg", cfg=cfg) == 10
    assert attn.load_library().attn_resolve_cfg(2, 4, 256, 64, 0, 0, ctypes.byref(cfg)) == 10


def test_cfg_eight_domains_need_heads_divisible_by_eight():
    cfg = attn.LaunchCfg(n_dom=8)
    assert _call("attn_fwd_cfg", B=1, H=3, cfg=cfg) == 10
    lib = attn.load_library()
    assert lib.attn_resolve_cfg(1, 3, 256, 64, 0, 0, ctypes.byref(cfg)) == 10


@pytest.mark.parametrize("args,code", [
    ((0, 4, 256, 64, 0, 0), 2), ((2, 0, 256, 64, 0, 0), 2), ((2, 4, 0, 64, 0, 0), 2),
    ((2, 4, 256, 96, 0, 0), 3), ((2, 4, 256, 64, 2, 0), 8), ((2, 4, 256, 64, 0, 7), 5),
])
def test_resolve_cfg_rejects_invalid_shapes(args, code):
    cfg = attn.LaunchCfg()
    assert attn.load_library().attn_resolve_cfg(*args, ctypes.byref(cfg)) == code


def test_resolve_cfg_rejects_null():
    assert attn.load_library().attn_resolve_cfg(2, 4, 256, 64, 0, 0, None) == 1


def test_cfg_forms():
    assert attn._cfg((8, 64, 4, 1)).as_tuple() == (8, 64, 4, 1, 0, 0)
    assert attn._cfg((8, 64, 4, 1, 2)).as_tuple() == (8, 64, 4, 1, 2, 0)
    assert attn._cfg({"n_work": 3}).as_tuple() == (0, 3, 0, 0, 0, 0)
    assert attn._cfg(None) is None


GA, GW, GB, GC = 0x10000000, 0x20000000, 0x30000000, 0x40000000
GEMM_GOOD = dict(a=GA, w=GW, bias=GB, c=GC, M=100, N=64, K=32, epi=2)


@pytest.mark.parametrize("over,code", [
    (dict(a=0), 1), (dict(w=0), 1), (dict(c=0), 1), (dict(bias=0), 1), (dict(bias=0, epi=1), 1),
    (dict(M=0), 2), (dict(M=-1), 2), (dict(N=0), 2), (dict(N=12), 2), (dict(K=4), 2), (dict(K=30), 2),
    (dict(N=4194304), 2), (dict(K=4194304), 2),
    (dict(a=GA + 8), 4), (dict(w=GW + 2), 4), (dict(c=GC + 4), 4), (dict(bias=GB + 4), 4),
    (dict(c=GA), 9), (dict(c=GW + 16), 9), (dict(bias=GC + 64), 9),
    (dict(epi=3), 10), (dict(epi=-1), 10),
])
def test_gemm_rejects_invalid_arguments(over, code):
    a = dict(GEMM_GOOD)
    a.update(over)
    lib = attn.load_library()
    assert lib.gemm_bf16(a["a"], a["w"], a["bias"], a["c"], a["M"], a["N"], a["K"], a["epi"], None) == code


def test_gemm_bias_may_be_null_without_a_bias_epilogue():
    """NULL bias passes validation with GEMM_EPI_NONE: the call then fails only
    at a later check (here: misaligned c), never on the bias."""
    lib = attn.load_library()
    assert lib.gemm_bf16(GA, GW, None, GC + 4, 100, 64, 32, 0, None) == 4


# ---- the size limit is the same for every entry point, and exact ---------------

@pytest.mark.parametrize("d,n_max", [(128, (1 << 23) - 129), (64, (1 << 24) - 129)])
def test_length_limit_is_exact(d, n_max):
    """The longest N whose fp32 O head plus 128 rows, (N + 128) * d * 4 bytes,
    fits unsigned 32-bit offsets passes the shape check (the call then stops
    at the misaligned q, before any HIP call); one more is rejected by both
    attn_fwd and attn_resolve_cfg."""
    assert (n_max + 128) * d * 4 <= 0xFFFFFFFF < (n_max + 129) * d * 4
    assert _call("attn_fwd", B=1, H=1, N=n_max, d=d, q=Q + 8) == 4
    assert _call("attn_fwd", B=1, H=1, N=n_max + 1, d=d, q=Q + 8) == 2
    lib = attn.load_library()
    cfg = attn.LaunchCfg()
    assert lib.attn_resolve_cfg(1, 1, n_max + 1, d, 0, 0, ctypes.byref(cfg)) == 2
    assert lib.attn_resolve_cfg(1, 1, n_max, d, 0, 0, ctypes.byref(cfg)) != 2


# ---- tensor arguments are checked before their addresses go to the C ABI --------

def _cpu_args(B=1, H=2, N=8, d=64, dtype=None):
    import torch

    dtype = dtype or torch.bfloat16
    q, k, v = (torch.zeros((B, H, N, d), dtype=dtype) for _ in range(3))
    o = torch.zeros((B, H, N, d), dtype=torch.float32)
    lse = torch.zeros((B, H, N), dtype=torch.float32)
    return dict(q=q, k=k, v=v, o=o, lse=lse)


def _bad_tensor_cases():
    import torch

    return [
        ("o", lambda a: a["o"].to(torch.bfloat16), TypeError, "o must be float32"),
        ("o", lambda a: a["o"].to(torch.float16), TypeError, "o must be float32"),
        ("lse", lambda a: a["lse"].to(torch.float64), TypeError, "lse must be float32"),
        ("k", lambda a: a["k"].to(torch.float16), TypeError, "share one dtype"),
        ("q", lambda a: a["q"].to(torch.float32), TypeError, "bfloat16 or float16"),
        ("o", lambda a: a["o"][..., :32], ValueError, "elements"),
        ("lse", lambda a: a["lse"][:, :, :4], ValueError, "elements"),
        ("v", lambda a: torch.zeros((1, 2, 9, 64), dtype=torch.bfloat16), ValueError, "elements"),
        ("q", lambda a: a["q"].transpose(2, 3).contiguous().transpose(2, 3), ValueError, "contiguous"),
        ("o", lambda a: a["o"].transpose(2, 3).contiguous().transpose(2, 3), ValueError, "contiguous"),
    ]


@pytest.mark.parametrize("case", range(10))
@pytest.mark.parametrize("entry", ["attn_fwd", "attn_fwd_cfg", "attn_fwd_bf16"])
def test_binding_checks_tensors(case, entry):
    name, mutate, exc, msg = _bad_tensor_cases()[case]
    a = _cpu_args()
    a[name] = mutate(a)
    with pytest.raises(exc, match=msg):
        getattr(attn, entry)(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 8, 64, 0, 0.125, stream=0)


def test_binding_checks_entry_point_dtype_and_device():
    import torch

    a = _cpu_args(dtype=torch.float16)
    with pytest.raises(TypeError, match="bfloat16 for this entry point"):
        attn.attn_fwd_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 8, 64, 0, 0.125, stream=0)
    # every property right but the device: CPU tensors are refused
    with pytest.raises(ValueError, match="on a GPU"):
        attn.attn_fwd_fp16(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 8, 64, 0, 0.125, stream=0)
    with pytest.raises(ValueError, match="on a GPU"):
        attn.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 8, 64, 0, 0.125, stream=0)


def test_binding_checks_softmax_and_gemm_tensors():
    import torch

    x = torch.zeros((4, 10), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="y must be"):
        attn.softmax_rows(x, torch.zeros((4, 10), dtype=torch.float32), 4, 10, stream=0)
    with pytest.raises(ValueError, match="elements"):
        attn.softmax_rows(x, torch.zeros((4, 9), dtype=torch.bfloat16), 4, 10, stream=0)
    with pytest.raises(ValueError, match="on a GPU"):
        attn.softmax_rows(x, torch.zeros((4, 10), dtype=torch.bfloat16), 4, 10, stream=0)
    a = torch.zeros((16, 32), dtype=torch.bfloat16)
    w = torch.zeros((24, 32), dtype=torch.bfloat16)
    b = torch.zeros((24,), dtype=torch.float32)
    with pytest.raises(TypeError, match="c must be"):
        attn.gemm_bf16(a, w, b, torch.zeros((16, 24), dtype=torch.float32), 16, 24, 32, stream=0)
    with pytest.raises(ValueError, match="elements"):
        attn.gemm_bf16(a, w, b[:8], torch.zeros((16, 24), dtype=torch.bfloat16), 16, 24, 32, stream=0)
    with pytest.raises(ValueError, match="on a GPU"):
        attn.gemm_bf16(a, w, b, torch.zeros((16, 24), dtype=torch.bfloat16), 16, 24, 32, stream=0)


# ---- un-fused attention entry point ---------------------------------------------

WS = 0x60000000


def _unf(dtype=0, **over):
    a = dict(GOOD, ws=WS, ws_bytes=1 << 30)
    a.update(over)
    lib = attn.load_library()
    return lib.attn_fwd_unfused(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["ws_bytes"], a["B"], a["H"],
                                a["N"], a["d"], a["causal"], a["scale"], None, dtype)


def test_unfused_workspace_bytes():
    lib = attn.load_library()
    assert lib.attn_unfused_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 100 * 4
    assert lib.attn_unfused_workspace_bytes(1, 65535, 1) == 65535 * 4
    assert lib.attn_unfused_workspace_bytes(1, 65536, 1) == 0          # B*H beyond one grid dimension
    assert lib.attn_unfused_workspace_bytes(1, 1 << 14, 1 << 17) == 0  # B*H*N rows beyond an int
    assert lib.attn_unfused_workspace_bytes(0, 3, 100) == 0


@pytest.mark.parametrize("over,code", [
    (dict(q=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(B=1, H=65536), 2), (dict(B=1 << 14, H=1, N=1 << 17), 2),
    (dict(d=96), 3), (dict(q=Q + 8), 4), (dict(scale=math.nan), 7), (dict(causal=3), 8),
    (dict(ws=0), 11), (dict(ws=WS + 4), 11), (dict(ws_bytes=2 * 3 * 100 * 100 * 4 - 1), 11),
    (dict(ws=O), 9), (dict(ws=V - 16), 9),
])
def test_unfused_rejects_invalid_arguments(over, code):
    assert _unf(**over) == code
    assert _unf(dtype=1, **over) == code


def test_unfused_rejects_unknown_dtype():
    assert _unf(dtype=2) == 5


def test_unfused_noalloc_rejects_oversize_before_any_hip_call():
    """B*H*N*N*4 above the 64 MiB scratch returns ATTN_ERR_SCRATCH; the host
    checks run first (no GPU here)."""
    lib = attn.load_library()
    args = (Q, K, V, O, L)
    # 1 x 16 x 1024: exactly 64 MiB of scores fits; one more row does not
    assert lib.attn_fwd_unfused_noalloc(*args, 1, 16, 1025, 64, 0, 0.125, None, 0) == 12
    assert lib.attn_fwd_unfused_noalloc(*args, 4, 16, 1024, 64, 1, 0.125, None, 1) == 12
    assert lib.attn_fwd_unfused_noalloc(*args, 1, 16, 1024, 96, 0, 0.125, None, 0) == 3
    assert lib.attn_fwd_unfused_noalloc(Q + 8, K, V, O, L, 1, 2, 64, 64, 0, 0.125, None, 0) == 4
    assert attn.attn_status_str(12) != "unknown status"
