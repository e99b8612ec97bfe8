"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare.

Tolerances (fp32 accumulation of bf16/fp16 products, probabilities rounded
to the input type before the second product):
  O:   max |O - O_ref| <= 1e-2  and  ||O - O_ref||_F / ||O_ref||_F <= 5e-3
  LSE: max |LSE - LSE_ref| <= 1e-3
"""

from __future__ import annotations

import numpy as np

from oracle import attention_ref, attention_rows
from tiled_tensor_core_amd import synth

O_MAX_ABS = 1e-2
O_REL_FRO = 5e-3
LSE_MAX_ABS = 1e-3


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def run_hip(qb, kb, vb, dtype, causal, scale, stream=None, entry="attn_fwd", cfg=None):
    """Run the HIP path on storage bits; returns (O, LSE) as torch tensors on the GPU.
    ``cfg``: a launch configuration for attn_fwd_cfg (a tuple, dict or LaunchCfg)."""
    import torch

    from tiled_tensor_core_amd import attn

    q = synth.to_torch(qb, dtype, "cuda")
    k = synth.to_torch(kb, dtype, "cuda")
    v = synth.to_torch(vb, dtype, "cuda")
    B, H, N, d = q.shape
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    if cfg is not None:
        attn.attn_fwd_cfg(q, k, v, o, lse, B, H, N, d, int(causal), scale, stream, cfg=cfg)
    else:
        fn = getattr(attn, entry)
        fn(q, k, v, o, lse, B, H, N, d, int(causal), scale, stream)
    torch.cuda.synchronize()
    return o, lse


def metrics(o, lse, o_ref, lse_ref):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    diff = o - o_ref
    return {
        "o_max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "o_rel_fro": float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-300)),
        "lse_max_abs": float(np.max(np.abs(lse - lse_ref))) if lse.size else 0.0,
        "finite": bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse))),
    }


def assert_close(o, lse, o_ref, lse_ref, tag=""):
    m = metrics(o, lse, o_ref, lse_ref)
    print(f"[parity] {tag} {m}", flush=True)
    assert m["finite"], f"{tag}: non-finite output {m}"
    assert m["o_max_abs"] <= O_MAX_ABS, f"{tag}: O max-abs {m}"
    assert m["o_rel_fro"] <= O_REL_FRO, f"{tag}: O rel-Frobenius {m}"
    assert m["lse_max_abs"] <= LSE_MAX_ABS, f"{tag}: LSE max-abs {m}"
    return m


def full_check(qb, kb, vb, dtype, causal, scale, tag="", cfg=None):
    """Whole-tensor comparison against the one-shot oracle."""
    o, lse = run_hip(qb, kb, vb, dtype, causal, scale, cfg=cfg)
    o_ref, lse_ref = attention_ref(synth.bits_to_f64(qb, dtype), synth.bits_to_f64(kb, dtype),
                                   synth.bits_to_f64(vb, dtype), causal, scale)
    return assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, tag)


def sampled_check(qb, kb, vb, dtype, causal, scale, o, lse, full_heads, rows_per_head, seed=0,
                  tag=""):
    """Compare GPU outputs (numpy) with the oracle on whole heads ``full_heads``
    (flat b*H+h indices) plus ``rows_per_head`` random rows (and the first and
    last row) of every head."""
    B, H, N, d = qb.shape
    rng = np.random.default_rng(seed)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for bh in range(B * H):
        b, h = divmod(bh, H)
        if bh in full_heads:
            rows = np.arange(N)
        else:
            rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, rows_per_head)]))
        qh = synth.bits_to_f64(qb[b, h][None, None], dtype)
        kh = synth.bits_to_f64(kb[b, h][None, None], dtype)
        vh = synth.bits_to_f64(vb[b, h][None, None], dtype)
        parts = [attention_rows(qh, kh, vh, causal, scale, 0, 0, rows[i:i + 512])
                 for i in range(0, len(rows), 512)]
        ro = np.concatenate([x[0] for x in parts])
        rl = np.concatenate([x[1] for x in parts])
        got_o.append(o[b, h, rows]); got_l.append(lse[b, h, rows])
        ref_o.append(ro); ref_l.append(rl)
    return assert_close(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o),
                        np.concatenate(ref_l), tag)


def whole_check(qb, kb, vb, dtype, causal, scale, o, lse, tag=""):
    """Compare whole GPU outputs (numpy) with the one-shot oracle, one head at
    a time (bounded memory); the metrics are taken over the whole tensor."""
    B, H, N, d = qb.shape
    sq_diff = 0.0
    sq_ref = 0.0
    o_max = 0.0
    l_max = 0.0
    finite = bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse)))
    for b in range(B):
        for h in range(H):
            ro, rl = attention_ref(synth.bits_to_f64(qb[b, h][None, None], dtype),
                                   synth.bits_to_f64(kb[b, h][None, None], dtype),
                                   synth.bits_to_f64(vb[b, h][None, None], dtype), causal, scale)
            diff = o[b, h].astype(np.float64) - ro[0, 0]
            sq_diff += float(np.sum(diff * diff))
            sq_ref += float(np.sum(ro * ro))
            o_max = max(o_max, float(np.max(np.abs(diff))))
            l_max = max(l_max, float(np.max(np.abs(lse[b, h].astype(np.float64) - rl[0, 0]))))
    m = {"o_max_abs": o_max, "o_rel_fro": float(np.sqrt(sq_diff / max(sq_ref, 1e-300))),
         "lse_max_abs": l_max, "finite": finite, "rows": B * H * N}
    print(f"[parity] {tag} {m}", flush=True)
    assert m["finite"], f"{tag}: non-finite output {m}"
    assert m["o_max_abs"] <= O_MAX_ABS, f"{tag}: O max-abs {m}"
    assert m["o_rel_fro"] <= O_REL_FRO, f"{tag}: O rel-Frobenius {m}"
    assert m["lse_max_abs"] <= LSE_MAX_ABS, f"{tag}: LSE max-abs {m}"
    return m
