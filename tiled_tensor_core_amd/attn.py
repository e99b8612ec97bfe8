"""Python binding of the C ABI in include/attn.h and include/softmax.h
(ctypes; marshalling only).

Every step of the attention forward pass runs in the HIP library
``libttc_attn.so``; this module only turns tensors into pointers, sizes and
a stream handle.  There is no fallback: if the library has not been built,
or a call is rejected, an exception says so.

Entry points (same names as the C functions):

* ``attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None, dtype=None)``
* ``attn_fwd_bf16(...)`` / ``attn_fwd_fp16(...)`` (same arguments, no dtype)
* ``attn_status_str(code)``, ``attn_last_error()``, ``attn_block_rows(d)``
* ``softmax_rows(x, y, rows, cols, dtype, stream=None)`` (row-wise softmax)

``q, k, v, o, lse`` are torch tensors on the GPU (or raw device addresses as
ints).  ``stream`` is a ``torch.cuda.Stream``, a raw ``hipStream_t`` int, or
None for torch's current stream on the tensors' device.

``fwd(q, k, v, causal, scale)`` allocates ``o`` (fp32) and ``lse`` (fp32)
with torch and calls ``attn_fwd``; ``softmax(x)`` allocates ``y`` like ``x``
(a 2-D fp32/bf16/fp16 tensor) and calls ``softmax_rows``.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttc_attn.so")

ATTN_BF16 = 0
ATTN_FP16 = 1

SOFTMAX_F32 = 0
SOFTMAX_BF16 = 1
SOFTMAX_FP16 = 2

STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED_D",
    4: "ATTN_ERR_ALIGN",
    5: "ATTN_ERR_DTYPE",
    6: "ATTN_ERR_HIP",
    7: "ATTN_ERR_SCALE",
    8: "ATTN_ERR_CAUSAL",
    9: "ATTN_ERR_ALIAS",
    10: "ATTN_ERR_CONFIG",
    11: "ATTN_ERR_WORKSPACE",
    12: "ATTN_ERR_SCRATCH",
}

ATTN_PRIO_DEFAULT = 0
ATTN_PRIO_ON = 1
ATTN_PRIO_OFF = 2
ATTN_REF_DEFAULT = 0
ATTN_REF_FIXED = 1
ATTN_REF_RUNNING = 2
ATTN_TILE_DEFAULT = 0
ATTN_TILE_128 = 1
ATTN_TILE_256 = 2
ATTN_MAX_WORKGROUPS = 1 << 20


class LaunchCfg(ctypes.Structure):
    """attn_launch_cfg of include/attn.h (a field of 0 takes the built-in choice)."""

    _fields_ = [("n_dom", ctypes.c_int), ("n_work", ctypes.c_int), ("grp", ctypes.c_int),
                ("prio", ctypes.c_int), ("mode", ctypes.c_int), ("tile", ctypes.c_int)]

    def as_tuple(self):
        return (self.n_dom, self.n_work, self.grp, self.prio, self.mode, self.tile)

    def __repr__(self):
        return (f"LaunchCfg(n_dom={self.n_dom}, n_work={self.n_work}, grp={self.grp}, prio={self.prio}, "
                f"mode={self.mode}, tile={self.tile})")


class TileResources(ctypes.Structure):
    """attn_tile_resources of include/attn.h."""

    _fields_ = [(n, ctypes.c_int) for n in ("rows", "waves", "vgprs", "lds_bytes", "scratch_bytes",
                                            "groups_per_cu")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

GEMM_EPI_NONE = 0
GEMM_EPI_BIAS = 1
GEMM_EPI_BIAS_GELU = 2

EXPORTS = ["attn_fwd", "attn_fwd_bf16", "attn_fwd_fp16", "attn_fwd_cfg", "attn_resolve_cfg",
           "attn_status_str", "attn_last_error", "attn_block_rows", "softmax_rows", "gemm_bf16",
           "attn_fwd_unfused", "attn_unfused_workspace_bytes", "attn_fwd_unfused_noalloc", "attn_tile_info"]

ATTN_UNFUSED_SCRATCH_BYTES = 64 << 20


class AttnError(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__(f"{self.name}: {detail}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m tiled_tensor_core_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    fwd_args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_void_p]
    for name in ("attn_fwd_bf16", "attn_fwd_fp16"):
        fn = getattr(lib, name)
        fn.argtypes = fwd_args
        fn.restype = ctypes.c_int
    lib.attn_fwd.argtypes = fwd_args + [ctypes.c_int]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_cfg.argtypes = fwd_args + [ctypes.c_int, ctypes.POINTER(LaunchCfg)]
    lib.attn_fwd_cfg.restype = ctypes.c_int
    lib.attn_resolve_cfg.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(LaunchCfg)]
    lib.attn_resolve_cfg.restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_block_rows.argtypes = [ctypes.c_int]
    lib.attn_block_rows.restype = ctypes.c_int
    lib.softmax_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.softmax_rows.restype = ctypes.c_int
    lib.gemm_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gemm_bf16.restype = ctypes.c_int
    lib.attn_fwd_unfused.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.c_ulonglong] + [ctypes.c_int] * 5 +
                                     [ctypes.c_float, ctypes.c_void_p, ctypes.c_int])
    lib.attn_fwd_unfused.restype = ctypes.c_int
    lib.attn_tile_info.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(TileResources)]
    lib.attn_tile_info.restype = ctypes.c_int
    lib.attn_fwd_unfused_noalloc.argtypes = fwd_args + [ctypes.c_int]
    lib.attn_fwd_unfused_noalloc.restype = ctypes.c_int
    lib.attn_unfused_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.attn_unfused_workspace_bytes.restype = ctypes.c_ulonglong
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream, like) -> int | None:
    if stream is None:
        import torch

        if like is not None and hasattr(like, "device") and like.device.type == "cuda":
            return torch.cuda.current_stream(like.device).cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(q, dtype):
    if dtype is not None:
        return int(dtype)
    import torch

    if q.dtype == torch.bfloat16:
        return ATTN_BF16
    if q.dtype == torch.float16:
        return ATTN_FP16
    raise TypeError(f"q must be bfloat16 or float16, got {q.dtype}")


def _check(code: int) -> None:
    if code != 0:
        lib = load_library()
        detail = lib.attn_status_str(code).decode()
        if code == 6:
            detail += ": " + lib.attn_last_error().decode()
        raise AttnError(code, detail)


def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "dtype")


def check_tensors(q, k, v, o, lse, B, H, N, d, dtype_code=None) -> None:
    """Host-side checks of tensor arguments before their pointers go to the C ABI.

    The C ABI sees only addresses and sizes, so it cannot tell a wrongly
    typed or sized buffer from a right one.  When the arguments are torch
    tensors this checks what it would otherwise trust: q, k, v are 16-bit
    floats of one dtype (the one ``dtype_code`` names, if given) with
    B*H*N*d elements each; o is fp32 with B*H*N*d elements and lse fp32 with
    B*H*N; every tensor is contiguous (the kernel reads and writes them as
    dense [B, H, N, d] / [B, H, N] arrays) and all sit on one GPU.  Raw int
    addresses are passed through unchecked (the caller's contract).
    """
    args = {"q": q, "k": k, "v": v, "o": o, "lse": lse}
    tensors = {n: x for n, x in args.items() if _is_tensor(x)}
    if not tensors:
        return
    import torch

    half = (torch.bfloat16, torch.float16)
    want = {ATTN_BF16: torch.bfloat16, ATTN_FP16: torch.float16}.get(dtype_code)
    in_dtypes = {tensors[n].dtype for n in ("q", "k", "v") if n in tensors}
    for n in ("q", "k", "v"):
        if n in tensors and tensors[n].dtype not in half:
            raise TypeError(f"{n} must be bfloat16 or float16, got {tensors[n].dtype}")
    if len(in_dtypes) > 1:
        raise TypeError(f"q, k, v must share one dtype, got {sorted(map(str, in_dtypes))}")
    if want is not None and in_dtypes and in_dtypes != {want}:
        raise TypeError(f"q, k, v must be {want} for this entry point, got {in_dtypes.pop()}")
    for n in ("o", "lse"):
        if n in tensors and tensors[n].dtype != torch.float32:
            raise TypeError(f"{n} must be float32, got {tensors[n].dtype}")
    n_qkv = int(B) * int(H) * int(N) * int(d)
    sizes = {"q": n_qkv, "k": n_qkv, "v": n_qkv, "o": n_qkv, "lse": int(B) * int(H) * int(N)}
    for n, x in tensors.items():
        if x.numel() != sizes[n]:
            raise ValueError(f"{n} has {x.numel()} elements; B={B}, H={H}, N={N}, d={d} needs {sizes[n]}")
        if not x.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    devices = {x.device for x in tensors.values()}
    if any(dv.type != "cuda" for dv in devices):
        raise ValueError(f"every tensor must be on a GPU, got {sorted(map(str, devices))}")
    if len(devices) > 1:
        raise ValueError(f"every tensor must be on one GPU, got {sorted(map(str, devices))}")


def _args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype_code=None):
    check_tensors(q, k, v, o, lse, B, H, N, d, dtype_code)
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d),
            int(causal), float(scale), _stream_handle(stream, q))


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None, dtype=None) -> None:
    """Enqueue the attention forward pass (see include/attn.h)."""
    lib = load_library()
    if dtype is None and isinstance(q, int):
        raise TypeError("dtype is required when q is a raw address")
    code = _dtype_code(q, dtype)
    _check(lib.attn_fwd(*_args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, code), code))


def attn_unfused_workspace_bytes(B, H, N) -> int:
    """Workspace bytes attn_fwd_unfused needs (0 if the shape is outside its limits)."""
    return int(load_library().attn_unfused_workspace_bytes(int(B), int(H), int(N)))


def attn_fwd_unfused(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, causal, scale, stream=None,
                     dtype=None) -> None:
    """Enqueue the un-fused attention forward (see include/attn.h): scores into
    ``workspace``, row softmax in place, then P V."""
    lib = load_library()
    if dtype is None and isinstance(q, int):
        raise TypeError("dtype is required when q is a raw address")
    code = _dtype_code(q, dtype)
    if _is_tensor(workspace):
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        have = workspace.numel() * workspace.element_size()
        if int(workspace_bytes) > have:
            raise ValueError(f"workspace_bytes {workspace_bytes} exceeds the tensor's {have} bytes")
    args = _args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, code)
    _check(lib.attn_fwd_unfused(*args[:5], _ptr(workspace), int(workspace_bytes), *args[5:], code))


def attn_fwd_unfused_noalloc(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None, dtype=None) -> None:
    """attn_fwd_unfused with the library's fixed scratch for the scores (see
    include/attn.h): allocates nothing; B*H*N*N*4 <= ATTN_UNFUSED_SCRATCH_BYTES."""
    lib = load_library()
    if dtype is None and isinstance(q, int):
        raise TypeError("dtype is required when q is a raw address")
    code = _dtype_code(q, dtype)
    _check(lib.attn_fwd_unfused_noalloc(*_args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, code), code))


def fwd_unfused(q, k, v, causal: bool, scale: float, stream=None):
    """O (fp32) and LSE (fp32) by the un-fused path, allocating its workspace with torch."""
    import torch

    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors of one shape")
    B, H, N, d = q.shape
    need = attn_unfused_workspace_bytes(B, H, N)
    if need == 0:
        raise ValueError(f"B={B}, H={H}, N={N} is outside the un-fused path's limits")
    ws = torch.empty((need // 4,), dtype=torch.float32, device=q.device)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    attn_fwd_unfused(q, k, v, o, lse, ws, need, B, H, N, d, bool(causal), scale, stream)
    return o, lse


def _cfg(cfg) -> LaunchCfg | None:
    if cfg is None or isinstance(cfg, LaunchCfg):
        return cfg
    if isinstance(cfg, dict):
        return LaunchCfg(**cfg)
    return LaunchCfg(*cfg)


def attn_fwd_cfg(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None, dtype=None, cfg=None) -> None:
    """attn_fwd with a launch configuration (LaunchCfg, a 4-tuple or a dict; None: built-in)."""
    lib = load_library()
    if dtype is None and isinstance(q, int):
        raise TypeError("dtype is required when q is a raw address")
    code = _dtype_code(q, dtype)
    c = _cfg(cfg)
    _check(lib.attn_fwd_cfg(*_args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, code), code,
                            ctypes.byref(c) if c is not None else None))


def attn_resolve_cfg(B, H, N, d, causal, dtype, cfg=None) -> LaunchCfg:
    """The configuration attn_fwd_cfg would run for this shape (fields of 0 resolved)."""
    lib = load_library()
    c = _cfg(cfg) or LaunchCfg()
    c = LaunchCfg(*c.as_tuple())
    _check(lib.attn_resolve_cfg(int(B), int(H), int(N), int(d), int(causal), int(dtype), ctypes.byref(c)))
    return c


def attn_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> None:
    lib = load_library()
    _check(lib.attn_fwd_bf16(*_args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, ATTN_BF16)))


def attn_fwd_fp16(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> None:
    lib = load_library()
    _check(lib.attn_fwd_fp16(*_args(q, k, v, o, lse, B, H, N, d, causal, scale, stream, ATTN_FP16)))


def attn_tile_info(tile, mode, dtype, d, causal) -> dict:
    """Compiled resources of a kernel variant on the current device (see include/attn.h)."""
    r = TileResources()
    _check(load_library().attn_tile_info(int(tile), int(mode), int(dtype), int(d), int(causal), ctypes.byref(r)))
    return r.as_dict()


def attn_status_str(code: int) -> str:
    return load_library().attn_status_str(int(code)).decode()


def attn_last_error() -> str:
    return load_library().attn_last_error().decode()


def attn_block_rows(d: int) -> int:
    return int(load_library().attn_block_rows(int(d)))


def fwd(q, k, v, causal: bool, scale: float, stream=None, cfg=None):
    """O (fp32) and LSE (fp32) for [B, H, N, d] tensors q, k, v on the GPU
    (cfg: an optional launch configuration, see attn_fwd_cfg)."""
    import torch

    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors of one shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if cfg is None:
        attn_fwd(q, k, v, o, lse, B, H, N, d, bool(causal), scale, stream)
    else:
        attn_fwd_cfg(q, k, v, o, lse, B, H, N, d, bool(causal), scale, stream, cfg=cfg)
    return o, lse


def _softmax_dtype(x):
    import torch

    codes = {torch.float32: SOFTMAX_F32, torch.bfloat16: SOFTMAX_BF16, torch.float16: SOFTMAX_FP16}
    if x.dtype not in codes:
        raise TypeError(f"x must be float32, bfloat16 or float16, got {x.dtype}")
    return codes[x.dtype]


def _check_plain(named, device_of=None):
    """Tensors among ``named`` ({name: (tensor or int, dtype or None, numel)})
    must have that dtype and element count, be contiguous and share one GPU."""
    tensors = {n: spec for n, spec in named.items() if _is_tensor(spec[0])}
    for n, (x, dt, numel) in tensors.items():
        if dt is not None and x.dtype != dt:
            raise TypeError(f"{n} must be {dt}, got {x.dtype}")
        if x.numel() != numel:
            raise ValueError(f"{n} has {x.numel()} elements, the sizes given need {numel}")
        if not x.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    devices = {spec[0].device for spec in tensors.values()}
    if any(dv.type != "cuda" for dv in devices):
        raise ValueError(f"every tensor must be on a GPU, got {sorted(map(str, devices))}")
    if len(devices) > 1:
        raise ValueError(f"every tensor must be on one GPU, got {sorted(map(str, devices))}")


def softmax_rows(x, y, rows, cols, dtype=None, stream=None) -> None:
    """Enqueue the row-wise softmax of [rows, cols] x into y (see include/softmax.h)."""
    lib = load_library()
    if dtype is None:
        if isinstance(x, int):
            raise TypeError("dtype is required when x is a raw address")
        dtype = _softmax_dtype(x)
    if _is_tensor(x) or _is_tensor(y):
        import torch

        want = {SOFTMAX_F32: torch.float32, SOFTMAX_BF16: torch.bfloat16, SOFTMAX_FP16: torch.float16}.get(int(dtype))
        n = int(rows) * int(cols)
        _check_plain({"x": (x, want, n), "y": (y, want, n)})
    _check(lib.softmax_rows(_ptr(x), _ptr(y), int(rows), int(cols), int(dtype), _stream_handle(stream, x)))


def softmax(x, stream=None):
    """Row-wise softmax of a contiguous 2-D GPU tensor; returns a new tensor like x."""
    import torch

    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D tensor")
    y = torch.empty_like(x)
    softmax_rows(x, y, x.shape[0], x.shape[1], _softmax_dtype(x), stream)
    return y


def gemm_bf16(a, w, bias, c, M, N, K, epilogue=GEMM_EPI_BIAS_GELU, stream=None) -> None:
    """Enqueue C = epilogue(A W^T + bias) (see include/gemm.h); bias may be None with GEMM_EPI_NONE."""
    lib = load_library()
    if any(_is_tensor(x) for x in (a, w, bias, c)):
        import torch

        M_, N_, K_ = int(M), int(N), int(K)
        _check_plain({"a": (a, torch.bfloat16, M_ * K_), "w": (w, torch.bfloat16, N_ * K_),
                      "bias": (bias, torch.float32, N_), "c": (c, torch.bfloat16, M_ * N_)})
    _check(lib.gemm_bf16(_ptr(a), _ptr(w), _ptr(bias) if bias is not None else None, _ptr(c), int(M), int(N),
                         int(K), int(epilogue), _stream_handle(stream, a)))


def gemm(a, w, bias=None, epilogue=None, stream=None):
    """GELU(a @ w.T + bias) (or the epilogue given) for contiguous bf16 a [M, K], w [N, K] and fp32
    bias [N] on the GPU; returns a new bf16 [M, N] tensor."""
    import torch

    if epilogue is None:
        epilogue = GEMM_EPI_NONE if bias is None else GEMM_EPI_BIAS_GELU
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError("a must be [M, K] and w [N, K]")
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("a and w must be bfloat16")
    if not (a.is_contiguous() and w.is_contiguous()):
        raise ValueError("a and w must be contiguous")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (w.shape[0],) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [N] tensor")
    M, K = a.shape
    N = w.shape[0]
    c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    gemm_bf16(a, w, bias, c, M, N, K, epilogue, stream)
    return c
