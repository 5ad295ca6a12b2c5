"""Shared helpers of the GPU parity tests: device copies, the error metric and
oracle calls spread over threads (numpy releases the GIL inside its kernels)."""
import concurrent.futures
import os

import numpy as np
import torch

import oracle

# Error metric of the diffusers issue "Ring attention backward uses stale iteration-0 KV",
# section Reproduction: ||got - ref|| / ||ref|| over the whole tensor (Frobenius).
BF16_TOL = 2e-2
LSE_TOL_BF16 = 1e-3
F32_TOL = 1e-5

_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test needs a HIP device")
    return torch.device("cuda", 0)


def np64(t):
    """Exact fp64 copy of a (bf16 or fp32) tensor."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def max_abs(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max())


def oracle_by_head(q, k, v, dout, heads, scale=None, backward=True, row_block=512, kmask=None):
    """Oracle forward (and backward) restricted to query heads ``heads`` of a
    [B,S,H,D] problem, one thread per head.  Returns dict with out/lse/dq for
    those heads (head axis in the order given) and dk/dv summed per kv head
    over the given query heads (full kv-head axis)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv

    def one(h):
        g = h // G
        qs, ks, vs = q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1]
        o, l = oracle.attention_forward(qs, ks, vs, scale=scale, row_block=row_block, kmask=kmask)
        res = {"out": o[:, :, 0], "lse": l[:, 0]}
        if backward:
            dq, dk, dv = oracle.attention_backward(qs, ks, vs, dout[:, :, h:h + 1], scale=scale, row_block=row_block,
                                                   kmask=kmask)
            res.update(dq=dq[:, :, 0], dk=dk[:, :, 0], dv=dv[:, :, 0], g=g)
        return res

    parts = list(_POOL.map(one, heads))
    out = {"out": np.stack([p["out"] for p in parts], axis=2), "lse": np.stack([p["lse"] for p in parts], axis=1)}
    if backward:
        out["dq"] = np.stack([p["dq"] for p in parts], axis=2)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for p in parts:
            dk[:, :, p["g"]] += p["dk"]
            dv[:, :, p["g"]] += p["dv"]
        out["dk"], out["dv"] = dk, dv
    return out
