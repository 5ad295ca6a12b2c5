"""The ring backward's plan under smaller workspaces, on the GPU.

ra_ring_bwd plans from the room the caller's workspace leaves above the minimum
(delta plus an fp32 accumulator per bf16 gradient): with less room the stored-dS
route groups fewer chunks per dQ pass, sweeps a chunk in query-row slices, or
falls back to the recompute route.  Every plan computes the same step ([P1] =
the diffusers issue "Ring attention backward uses stale iteration-0 KV", sections
Root cause and Expected behavior: each backward step against its own chunk), so
each is held to the oracle, and to the fastest plan's result.
"""
import numpy as np
import pytest
import torch

import context_attention_lse_kv_amd as ra
import oracle
import workloads as W
from parity import LSE_TOL_BF16, check_bf16, dev, max_abs, np64, oracle_by_head, rel

pytestmark = pytest.mark.gpu


def _bwd_with(q, k, v, out, do, lse, ch, nbytes):
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)[:nbytes] if nbytes else None
    grads = [torch.empty(t.shape, dtype=torch.bfloat16, device=q.device) for t in (q, k, v)]
    ra.ring_bwd(q, k, v, out, do, lse, ch, workspace=ws, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return grads


def test_small_workspace_plans_match_oracle():
    d = dev()
    B, Sq, Sk, Hq, Hkv, D = 2, 200, 600, 8, 2, 64
    q = W.randn((B, Sq, Hq, D), 70, "bf16"); k = W.randn((B, Sk, Hkv, D), 71, "bf16")
    v = W.randn((B, Sk, Hkv, D), 72, "bf16"); do = W.randn((B, Sq, Hq, D), 73, "bf16")
    gq, gk, gv, gdo = (t.to(d) for t in (q, k, v, do))
    lens, order = [200, 200, 200], [1, 0, 2]
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(gq, gk, gv, ch)
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do))
    lo = ra.ring_bwd_workspace_bytes(gq, gk, minimum=True)
    hi = ra.ring_bwd_workspace_bytes(gq, gk)
    one_chunk_ds = ra.bwd_ds_bytes(gq, gk[:, :200])
    assert lo < hi
    assert ra.ring_bwd_plan(gq, gk, ch, hi) == {"slice_rows": 0, "rows": [200] * 3, "accumulators": []}
    assert ra.ring_bwd_plan(gq, gk, ch, lo + one_chunk_ds + 4096) == \
        {"slice_rows": 0, "rows": [200] * 3, "accumulators": ["dq"]}
    results = {}
    # minimum: every chunk on the recompute route; + one chunk's dS: one chunk per dQ pass
    # (fp32 dQ accumulator, bf16 dK/dV direct); recommended: one dQ pass for all three
    for name, nbytes in (("minimum", lo), ("one chunk of dS", lo + one_chunk_ds + 4096), ("recommended", hi)):
        g = _bwd_with(gq, gk, gv, out, gdo, lse, ch, nbytes)
        for gname, a, r in zip(("dq", "dk", "dv"), g, ref):
            check_bf16(f"{name} {gname}", np64(a), r)
        results[name] = g
    for name in ("minimum", "one chunk of dS"):
        for a, b in zip(results[name], results["recommended"]):
            assert rel(np64(a), np64(b)) <= 5e-3


@pytest.mark.parametrize("masked,grad_dtype", [(False, torch.bfloat16), (True, torch.bfloat16), (False, torch.float32)],
                         ids=["dense", "masked", "f32_grads"])
def test_slice_major_plan_matches_oracle(masked, grad_dtype):
    """A workspace whose room holds the dS of every chunk only for part of the query rows (at
    least 4096): the sweep runs slice by slice, each slice running the chunk steps of every
    chunk and then one dQ pass over all of them.  Ragged chunks (not multiples of a tile) and
    a ragged last slice; with and without a key mask; bf16 gradients (dK/dV summed over the
    slices in fp32 accumulators, dq rows written by each slice's pass) and fp32 gradients
    (their own accumulators).  Against the oracle on every head and against the plan with
    room for all of the dS (one dQ pass over the whole query)."""
    d = dev()
    B, Sq, Hq, Hkv, D = 1, 8292, 2, 1, 128
    lens, order = [700, 1000, 300], [1, 0, 2]
    Sk = sum(lens)
    seed = 84 + (10 if masked else 0)
    q = W.randn((B, Sq, Hq, D), seed, "bf16"); k = W.randn((B, Sk, Hkv, D), seed + 1, "bf16")
    v = W.randn((B, Sk, Hkv, D), seed + 2, "bf16"); do = W.randn((B, Sq, Hq, D), seed + 3, "bf16")
    m = W.make_key_mask(B, Sk, seed + 4, p_keep=0.8, valid_len=(1900,), masked_ranges=[(0, 100, 400)]) \
        if masked else None
    gq, gk, gv, gdo = (t.to(d) for t in (q, k, v, do))
    gm = None if m is None else m.to(d)
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(gq, gk, gv, ch, kmask=gm)
    starts = [sum(lens[:i]) for i in range(len(lens))]
    room = sum(ra.bwd_ds_bytes(gq[:, :4096], gk[:, s0:s0 + n]) for s0, n in zip(starts, lens))
    lo = ra.ring_bwd_workspace_bytes(gq, gk, grad_dtype, grad_dtype, minimum=True)
    plan = ra.ring_bwd_plan(gq, gk, ch, lo + room, grad_dtype, grad_dtype)
    assert 4096 <= plan["slice_rows"] < Sq and Sq % plan["slice_rows"] != 0, plan
    assert plan["accumulators"] == (["dk", "dv"] if grad_dtype == torch.bfloat16 else []), plan
    # room for every chunk's dS at every row: one dQ pass over the whole query (the
    # recommended size, which sees no chunk table, counts the keys' tiles as one chunk's)
    hi = lo + sum(ra.bwd_ds_bytes(gq, gk[:, s0:s0 + n]) for s0, n in zip(starts, lens))
    assert ra.ring_bwd_plan(gq, gk, ch, hi, grad_dtype, grad_dtype) == \
        {"slice_rows": 0, "rows": [Sq] * 3, "accumulators": []}

    def run(nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=d)
        g = [torch.empty(t.shape, dtype=grad_dtype, device=d) for t in (q, k, v)]
        ra.ring_bwd(gq, gk, gv, out, gdo, lse, ch, workspace=ws, dq=g[0], dk=g[1], dv=g[2], kmask=gm)
        torch.cuda.synchronize()
        return g

    sliced, full = run(lo + room), run(hi)
    mn = None if m is None else m.numpy().astype(np.uint8)
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do), kmask=mn)
    for name, a, r in zip(("dq", "dk", "dv"), sliced, ref):
        check_bf16(f"slice-major {name}", np64(a), r)
    for a, b in zip(sliced, full):
        assert rel(np64(a), np64(b)) <= 5e-3


@pytest.mark.slow
def test_video_shard_with_2gib_ds_budget():
    """The video-DiT shard (4096 rows, 8 chunks of 4096; 1 GiB of dS per chunk) with 2 GiB of
    room for dS: two chunks per dQ pass.  Against the oracle on kv-head group 0 and against
    the run with the recommended workspace (one dQ pass over all 8 chunks)."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w, Sq=lens[0])
    d = dev()
    gq, gk, gv, gdo = (t.to(d) for t in (q, k, v, do))
    ch = ra.Chunks(lens, ra.ring_order(w.n_chunks, 0))
    out, lse = ra.ring_fwd(gq, gk, gv, ch)
    lo = ra.ring_bwd_workspace_bytes(gq, gk, minimum=True)
    small = _bwd_with(gq, gk, gv, out, gdo, lse, ch, lo + (2 << 30))
    full = _bwd_with(gq, gk, gv, out, gdo, lse, ch, ra.ring_bwd_workspace_bytes(gq, gk))
    heads = [0, 1, 2, 3]
    ref = oracle_by_head(np64(q), np64(k), np64(v), np64(do), heads)
    check_bf16("out", np64(out[:, :, heads]), ref["out"])
    assert max_abs(np64(lse[:, heads]), ref["lse"]) <= LSE_TOL_BF16
    check_bf16("dq (2 GiB)", np64(small[0][:, :, heads]), ref["dq"])
    check_bf16("dk (2 GiB)", np64(small[1][:, :, 0]), ref["dk"][:, :, 0])
    check_bf16("dv (2 GiB)", np64(small[2][:, :, 0]), ref["dv"][:, :, 0])
    for a, b in zip(small, full):
        assert rel(np64(a), np64(b)) <= 5e-3


@pytest.mark.slow
def test_full_q_with_2gib_ds_budget_slices_chunks():
    """Full Q (32768 rows; 8 GiB of dS per chunk) with 2 GiB of room for dS: every chunk is
    swept in query-row slices of 8192, the dK/dV rows of a chunk are summed over its slices
    in fp32.  Against the run with the recommended workspace (8 slices of 4096 rows, each
    running every chunk and one dQ pass), and through the key sums that hold at any size
    (rows of P sum to 1, rows of dS to 0)."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w)
    d = dev()
    gq, gk, gv, gdo = (t.to(d) for t in (q, k, v, do))
    ch = ra.Chunks(lens, list(range(w.n_chunks)))
    out, lse = ra.ring_fwd(gq, gk, gv, ch)
    lo = ra.ring_bwd_workspace_bytes(gq, gk, minimum=True)
    small = _bwd_with(gq, gk, gv, out, gdo, lse, ch, lo + (2 << 30))
    full = _bwd_with(gq, gk, gv, out, gdo, lse, ch, ra.ring_bwd_workspace_bytes(gq, gk))
    for name, a, b in zip(("dq", "dk", "dv"), small, full):
        r = rel(np64(a), np64(b))
        print(name, "2 GiB vs recommended", r)
        assert r <= 5e-3
    dkn, dvn, dof = np64(small[1]), np64(small[2]), np64(do)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        want = dof[:, :, g * G:(g + 1) * G].sum(axis=(1, 2))
        check_bf16("key-sum of dV", dvn[:, :, g].sum(axis=1), want)
        assert np.linalg.norm(dkn[:, :, g].sum(axis=1)) <= 2e-2 * np.linalg.norm(dkn[:, :, g])
