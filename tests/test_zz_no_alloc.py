"""GPU test of attn_fwd_unfused_noalloc, the entry point that allocates
nothing (its score matrix lives in the library's fixed scratch): two calls in
a row, the second on a smaller shape, each against attn_fwd_unfused with a
workspace (the same kernels, so bit for bit) and against the oracle."""

import numpy as np
import pytest

from oracle import attention_ref
from parity import assert_close, gpu_available
from tiled_tensor_core_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _outputs(q, k, v, noalloc, causal, scale):
    import torch

    from tiled_tensor_core_amd import attn

    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        attn.attn_fwd_unfused_noalloc(q, k, v, o, lse, B, H, N, d, int(causal), scale)
    else:
        need = attn.attn_unfused_workspace_bytes(B, H, N)
        ws = torch.empty((need // 4,), dtype=torch.float32, device="cuda")
        attn.attn_fwd_unfused(q, k, v, o, lse, ws, need, B, H, N, d, int(causal), scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("fp16", 64, False)])
def test_noalloc_matches_workspace_entry_point(dtype, d, causal):
    dist = synth.Dist("normal", 1.0)
    # the first call fills 2 x 8 x 1024^2 x 4 = 64 MiB, the whole scratch; the
    # second, smaller one must not see its leftovers
    for i, (B, H, N) in enumerate([(2, 8, 1024), (1, 3, 333)]):
        qb, kb, vb = synth.make_qkv(B, H, N, d, dtype, dist, dist, dist, seed=100 + i)
        q, k, v = (synth.to_torch(x, dtype, "cuda") for x in (qb, kb, vb))
        scale = 1 / np.sqrt(d)
        print(f"[case] noalloc {dtype} d={d} causal={causal} B={B} H={H} N={N}", flush=True)
        o1, l1 = _outputs(q, k, v, True, causal, scale)
        o2, l2 = _outputs(q, k, v, False, causal, scale)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        o_ref, l_ref = attention_ref(synth.bits_to_f64(qb, dtype), synth.bits_to_f64(kb, dtype),
                                     synth.bits_to_f64(vb, dtype), causal, scale)
        assert_close(o1, l1, o_ref, l_ref, f"noalloc {dtype} B={B} H={H} N={N}")
