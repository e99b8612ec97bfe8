"""HIP-graph capture of the entry points that allocate nothing.

The fused attention forward, the un-fused attention (with a caller-supplied
workspace), the row softmax and the GEMM enqueue only their kernels on the
caller's stream, with no allocation, memset or synchronisation, so a caller
can record a call into a HIP graph and replay it.  Each test records one call,
then replays the graph several times with new contents copied into the
recorded input buffers, with the program's own eager work (fills, other
launches, synchronisations) between the replays, and checks every replay bit
for bit against an eager call on the same inputs; the attention replays are
also compared with the fp64 oracle.
"""

import numpy as np
import pytest

from oracle import attention_ref
from parity import assert_close, gpu_available, run_hip
from tiled_tensor_core_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

REPLAYS = 5


def _same(a, b):
    import torch

    return torch.equal(a.contiguous().view(torch.int32 if a.element_size() == 4 else torch.int16),
                       b.contiguous().view(torch.int32 if b.element_size() == 4 else torch.int16))


def _record(fn):
    """Warm fn up on a side stream (first-call set-up happens outside the
    graph), then record one call of it into a graph."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("fp16", 64, False), ("bf16", 64, True)])
def test_fused_attention_replays(dtype, d, causal):
    import torch

    from tiled_tensor_core_amd import attn

    B, H, N = 2, 4, 700
    scale = d ** -0.5
    seeds = [81 + r for r in range(REPLAYS)]
    bits = [synth.make_qkv(B, H, N, d, dtype, seed=s) for s in seeds]
    q, k, v = (synth.to_torch(x, dtype, "cuda") for x in bits[0])
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    g = _record(lambda: attn.attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale))
    for r, (qb, kb, vb) in enumerate(bits):
        print(f"[graph] fused {dtype} d={d} causal={causal} replay {r}", flush=True)
        for dst, src in zip((q, k, v), (qb, kb, vb)):
            dst.copy_(synth.to_torch(src, dtype, "cuda"))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = run_hip(qb, kb, vb, dtype, causal, scale)   # eager, between the replays
        assert _same(o, o_e) and _same(lse, lse_e), f"replay {r} differs from the eager call"
        if r < 2:
            o_ref, lse_ref = attention_ref(synth.bits_to_f64(qb, dtype), synth.bits_to_f64(kb, dtype),
                                           synth.bits_to_f64(vb, dtype), causal, scale)
            assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, tag=f"graph replay {r}")


def test_unfused_attention_replays():
    import torch

    from tiled_tensor_core_amd import attn

    B, H, N, d, dtype, causal = 1, 4, 520, 64, "bf16", True
    scale = d ** -0.5
    bits = [synth.make_qkv(B, H, N, d, dtype, seed=91 + r) for r in range(REPLAYS)]
    q, k, v = (synth.to_torch(x, dtype, "cuda") for x in bits[0])
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    nbytes = attn.attn_unfused_workspace_bytes(B, H, N)
    ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    g = _record(lambda: attn.attn_fwd_unfused(q, k, v, o, lse, ws, nbytes, B, H, N, d, int(causal), scale))
    for r, (qb, kb, vb) in enumerate(bits):
        print(f"[graph] unfused replay {r}", flush=True)
        for dst, src in zip((q, k, v), (qb, kb, vb)):
            dst.copy_(synth.to_torch(src, dtype, "cuda"))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = attn.fwd_unfused(*(synth.to_torch(x, dtype, "cuda") for x in (qb, kb, vb)), causal, scale)
        torch.cuda.synchronize()
        assert _same(o, o_e) and _same(lse, lse_e), f"replay {r} differs from the eager call"
        if r == 0:
            o_ref, lse_ref = attention_ref(synth.bits_to_f64(qb, dtype), synth.bits_to_f64(kb, dtype),
                                           synth.bits_to_f64(vb, dtype), causal, scale)
            assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, tag="unfused graph replay")


@pytest.mark.parametrize("dtype,cols", [("bf16", 1000), ("fp32", 4096), ("fp16", 1001)])
def test_softmax_replays(dtype, cols):
    import torch

    from tiled_tensor_core_amd import attn

    rows = 300
    xs = [synth.make_softmax_input(rows, cols, dtype, seed=101 + r) for r in range(REPLAYS)]
    x = synth.softmax_to_torch(xs[0], dtype, "cuda")
    y = torch.empty_like(x)
    g = _record(lambda: attn.softmax_rows(x, y, rows, cols))
    for r, xb in enumerate(xs):
        print(f"[graph] softmax {dtype} {rows}x{cols} replay {r}", flush=True)
        x.copy_(synth.softmax_to_torch(xb, dtype, "cuda"))
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        y_e = attn.softmax(synth.softmax_to_torch(xb, dtype, "cuda"))
        torch.cuda.synchronize()
        assert _same(y, y_e), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("M,N,K", [(1000, 776, 328), (4096, 4096, 1024)])
def test_gemm_replays(M, N, K):
    import torch

    from tiled_tensor_core_amd import attn

    ins = [synth.make_gemm_inputs(M, N, K, seed=111 + r) for r in range(REPLAYS)]
    a = synth.to_torch(ins[0][0], "bf16", "cuda")
    w = synth.to_torch(ins[0][1], "bf16", "cuda")
    b = torch.from_numpy(ins[0][2]).cuda()
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    g = _record(lambda: attn.gemm_bf16(a, w, b, c, M, N, K, attn.GEMM_EPI_BIAS_GELU))
    for r, (ab, wb, bias) in enumerate(ins):
        print(f"[graph] gemm {M}x{N}x{K} replay {r}", flush=True)
        a.copy_(synth.to_torch(ab, "bf16", "cuda"))
        w.copy_(synth.to_torch(wb, "bf16", "cuda"))
        b.copy_(torch.from_numpy(bias).cuda())
        c.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        c_e = attn.gemm(synth.to_torch(ab, "bf16", "cuda"), synth.to_torch(wb, "bf16", "cuda"),
                        torch.from_numpy(bias).cuda(), epilogue=attn.GEMM_EPI_BIAS_GELU)
        torch.cuda.synchronize()
        assert _same(c, c_e), f"replay {r} differs from the eager call"
        assert not torch.isnan(c).any()
