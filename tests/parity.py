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


def vec_rel_max(got, ref, floor=0.25):
    """Largest relative error of one D-vector (the last axis: one (batch, row, head) of an
    output or gradient), each against its own oracle vector.  A whole-tensor Frobenius
    ratio barely moves when a single row or tile is wrong (one bad row of 4096 adds about
    1/64 to it); this bound sees it.  The denominator is the vector's own norm, floored at
    ``floor`` times the RMS vector norm of the tensor, so that vectors whose true value is
    tiny are held to an absolute bound instead of a relative one."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got.shape[-1]
    e = np.linalg.norm((got - ref).reshape(-1, d), axis=1)
    n = np.linalg.norm(ref.reshape(-1, d), axis=1)
    if n.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(n * n)))
    den = np.maximum(n, floor * rms if rms > 0 else 1.0)
    return float((e / den).max())


def check_bf16(name, got, ref, tol=BF16_TOL, log=True):
    """The parity gate of a bf16 output or gradient: the whole-tensor metric of the
    diffusers issue "Ring attention backward uses stale iteration-0 KV" (section
    Reproduction) and, on top, every D-vector separately, both <= tol.  The element-wise
    max-abs error is printed as a diagnostic."""
    r, v = rel(got, ref), vec_rel_max(got, ref)
    if log:
        print(f"{name}: rel {r:.2e}  worst vector {v:.2e}  max-abs {max_abs(got, ref):.2e}")
    assert r <= tol, (name, "rel", r)
    assert v <= tol, (name, "worst vector", v)
    return r, v


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


def oracle_grads_by_head(q, k, v, dout, heads, scale=None, row_block=512):
    """Oracle gradients only (no separate forward) for query heads ``heads``, one thread
    per head: dq of those heads (head axis in the order given) and dk/dv summed per kv
    head over them (full kv-head axis)."""
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv

    def one(h):
        g = h // G
        dq, dk, dv = oracle.attention_backward(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1],
                                               dout[:, :, h:h + 1], scale=scale, row_block=row_block)
        return dq[:, :, 0], dk[:, :, 0], dv[:, :, 0], g

    parts = list(_POOL.map(one, heads))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for _, pk, pv, g in parts:
        dk[:, :, g] += pk
        dv[:, :, g] += pv
    return np.stack([p[0] for p in parts], axis=2), dk, dv
