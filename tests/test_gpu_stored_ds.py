"""The bf16 chunk step by the stored-dS route (the dK/dV kernel writes dS, a second
kernel forms dQ from it) against the oracle, against the recompute route and
against the ring sweep that uses it.

The route computes the chunk step of the diffusers issue "Ring attention backward uses
stale iteration-0 KV" (section "Expected behavior": every backward step against its own
chunk); only the way dQ = scale dS K is reached differs.  Inputs come from the seeded
generators in ``workloads``.
"""
import numpy as np
import pytest
import torch

import context_attention_lse_kv_amd as ra
import oracle
import workloads as W
from parity import BF16_TOL, check_bf16, LSE_TOL_BF16, dev, max_abs, np64, oracle_by_head, rel

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, S, Sq, Hq, Hkv, D, chunk lens, order, mask recipe (None: no mask)
    ("d128_gqa_ragged", 1, 1000, 320, 8, 2, 128, (384, 616), (1, 0), None),
    ("d64_b2", 2, 512, 200, 4, 4, 64, (256, 256), (0, 1), None),
    ("d128_gqa_masked", 2, 640, 256, 4, 2, 128, (300, 340), (0, 1),
     dict(p_keep=0.8, valid_len=(640, 450), masked_ranges=[(0, 0, 100)])),
    ("d128_ragged_rows_and_keys", 1, 700, 200, 8, 2, 128, (350, 350), (1, 0), None),
    ("tiny_17_rows_37_keys", 1, 37, 17, 4, 1, 128, (20, 17), (0, 1), None),
]


def _inputs(case):
    name, B, S, Sq, Hq, Hkv, D, lens, order, recipe = case
    seed = 1200 + 10 * CASES.index(case)
    q = W.randn((B, Sq, Hq, D), seed, "bf16")
    k = W.randn((B, S, Hkv, D), seed + 1, "bf16")
    v = W.randn((B, S, Hkv, D), seed + 2, "bf16")
    do = W.randn((B, Sq, Hq, D), seed + 3, "bf16")
    m = None if recipe is None else W.make_key_mask(B, S, seed + 4, **recipe)
    return q, k, v, do, m


def _chunk_steps(gq, gk, gv, gdo, out, lse, gm, lens, order, route):
    """Backward of every chunk through the chunk entry points; route 'ds' or 'recompute'."""
    d = gq.device
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    delta = torch.empty_like(lse)
    ra.bwd_delta(out, gdo, delta)
    dq = torch.zeros(gq.shape, dtype=torch.float32, device=d)
    dk = torch.zeros(gk.shape, dtype=torch.float32, device=d)
    dv = torch.zeros(gv.shape, dtype=torch.float32, device=d)
    for c in order:
        sl = slice(int(starts[c]), int(starts[c] + lens[c]))
        km = None if gm is None else gm[:, sl]
        if route == "ds":
            ds = torch.empty(ra.bwd_ds_bytes(gq, gk[:, sl]), dtype=torch.uint8, device=d)
            ra.bwd_chunk_dkdv_ds(gq, gk[:, sl], gv[:, sl], gdo, lse, delta, dk[:, sl], dv[:, sl], 1, ds, kmask=km)
            ra.bwd_chunk_dq_ds(gq, gk[:, sl], ds, dq)
        else:
            ra.bwd_chunk(gq, gk[:, sl], gv[:, sl], gdo, lse, delta, dq, dk[:, sl], dv[:, sl], 1, kmask=km)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stored_ds_route_matches_oracle_and_ring(case):
    name, B, S, Sq, Hq, Hkv, D, lens, order, recipe = case
    q, k, v, do, m = _inputs(case)
    d = dev()
    gq, gk, gv, gdo = (x.to(d) for x in (q, k, v, do))
    gm = None if m is None else m.to(d)
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(gq, gk, gv, ch, kmask=gm)
    dq_r, dk_r, dv_r = ra.ring_bwd(gq, gk, gv, out, gdo, lse, ch, grad_dtype=torch.float32, kmask=gm)
    dq, dk, dv = _chunk_steps(gq, gk, gv, gdo, out, lse, gm, lens, order, "ds")
    # the ring runs these very kernels in this order (one query slice): dK/dV bit for bit;
    # its dQ pass sweeps the dS of several chunks at once, so dQ sums their products in the
    # kernel's fp32 accumulator before one add to dq (the chunk entry point adds per
    # chunk): equal up to fp32 rounding
    for a, b in ((dk, dk_r), (dv, dv_r)):
        assert torch.equal(a, b)
    dq_rel = ((dq - dq_r).norm() / dq_r.norm()).item()
    assert dq_rel < 1e-6, dq_rel
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    mn = None if m is None else m.numpy().astype(np.uint8)
    g = oracle.attention_backward(qn, kn, vn, don, kmask=mn)
    for a, b in zip((dq, dk, dv), g):
        check_bf16('grad', np64(a), b)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stored_ds_route_agrees_with_recompute_route(case):
    """dK/dV: same kernel, bit for bit; dQ: the two routes round P differently (fp16
    on the way to the stored dS, fp32 in the recompute), so they agree to ~1e-3."""
    name, B, S, Sq, Hq, Hkv, D, lens, order, recipe = case
    q, k, v, do, m = _inputs(case)
    d = dev()
    gq, gk, gv, gdo = (x.to(d) for x in (q, k, v, do))
    gm = None if m is None else m.to(d)
    out, lse = ra.ring_fwd(gq, gk, gv, ra.Chunks(lens, order), kmask=gm)
    a = _chunk_steps(gq, gk, gv, gdo, out, lse, gm, lens, order, "ds")
    b = _chunk_steps(gq, gk, gv, gdo, out, lse, gm, lens, order, "recompute")
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    r = ((a[0] - b[0]).norm() / b[0].norm()).item()
    assert r < 5e-3, r


def test_stored_ds_masked_keys_store_zero_and_values_never_read():
    """Masked keys contribute nothing to dQ: changing K and V at masked keys leaves every
    gradient of the unmasked keys and dQ unchanged."""
    case = next(c for c in CASES if c[0] == "d128_gqa_masked")
    name, B, S, Sq, Hq, Hkv, D, lens, order, recipe = case
    q, k, v, do, m = _inputs(case)
    d = dev()
    gq, gk, gv, gdo, gm = (x.to(d) for x in (q, k, v, do, m))
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(gq, gk, gv, ch, kmask=gm)
    res = _chunk_steps(gq, gk, gv, gdo, out, lse, gm, lens, order, "ds")
    gk2, gv2 = gk.clone(), gv.clone()
    dead = ~gm
    gk2[dead] = 7.0
    gv2[dead] = -3.0
    res2 = _chunk_steps(gq, gk2, gv2, gdo, out, lse, gm, lens, order, "ds")
    assert torch.equal(res[0], res2[0])
    assert torch.equal(res[1][gm], res2[1][gm]) and torch.equal(res[2][gm], res2[2][gm])
    assert not res2[1][dead].any() and not res2[2][dead].any()


def test_ring_bwd_sweeps_query_slices_when_ds_exceeds_region():
    """Full Q (32768 rows) against the whole 32k sequence as one chunk: its dS (64 GiB) is 8x
    the region, so the ring backward runs the stored-dS route in 8 query slices of 4096 rows.
    dQ on sampled rows against the oracle; dK/dV against the 8-chunk ring (one slice per
    chunk), which reaches the same sums in another order."""
    w = W.VIDEO_DIT_GQA
    q, k, v, do = W.make_inputs(w)
    d = dev()
    gq, gk, gv, gdo = (x.to(d) for x in (q, k, v, do))
    assert ra.bwd_ds_bytes(gq, gk) == 64 << 30  # 32768 x 32768 x 32 heads x 2 B
    assert ra.ring_bwd_workspace_bytes(gq, gk, torch.float32, torch.float32) < (8 << 30) + (64 << 20)
    one = ra.Chunks([w.S], [0])
    out, lse = ra.ring_fwd(gq, gk, gv, one)
    dq, dk, dv = ra.ring_bwd(gq, gk, gv, out, gdo, lse, one, grad_dtype=torch.float32)
    eight = ra.Chunks(ra.split_sizes(w.S, w.n_chunks), list(range(w.n_chunks)))
    out8, lse8 = ra.ring_fwd(gq, gk, gv, eight)
    dq8, dk8, dv8 = ra.ring_bwd(gq, gk, gv, out8, gdo, lse8, eight, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in ((dk, dk8), (dv, dv8), (dq, dq8)):
        r = ((a - b).norm() / b.norm()).item()
        assert r < 5e-3, r
    rows = torch.as_tensor(np.sort(np.random.default_rng(7).choice(w.S, 64, replace=False)))
    heads = [3, 17, 30]
    qn, kn, vn, don = (np64(t) for t in (q[:, rows], k, v, do[:, rows]))
    ref = oracle_by_head(qn, kn, vn, don, heads)
    sel = lambda t: np64(t.cpu()[:, rows][:, :, heads])
    check_bf16('out', sel(out), ref["out"])
    assert max_abs(np64(lse.cpu()[:, heads][:, :, rows]), ref["lse"]) <= LSE_TOL_BF16
    check_bf16('dq', sel(dq), ref["dq"])


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_direct_bf16_dkdv_equals_accumulate_then_cast(case):
    """bf16 dk/dv with accumulate = 0 are written directly by the kernel; they equal the fp32
    accumulate path cast to bf16 bit for bit (0 + x = x, both round the same fp32 value)."""
    name, B, S, Sq, Hq, Hkv, D, lens, order, recipe = case
    q, k, v, do, m = _inputs(case)
    d = dev()
    gq, gk, gv, gdo = (x.to(d) for x in (q, k, v, do))
    gm = None if m is None else m.to(d)
    out, lse = ra.ring_fwd(gq, gk, gv, ra.Chunks(lens, order), kmask=gm)
    delta = torch.empty_like(lse)
    ra.bwd_delta(out, gdo, delta)
    c = lens[0]
    kc, vc = gk[:, :c], gv[:, :c]
    km = None if gm is None else gm[:, :c]
    ds = torch.empty(ra.bwd_ds_bytes(gq, kc), dtype=torch.uint8, device=d)
    dk32 = torch.empty(kc.shape, dtype=torch.float32, device=d)
    dv32 = torch.empty_like(dk32)
    ra.bwd_chunk_dkdv_ds(gq, kc, vc, gdo, lse, delta, dk32, dv32, 0, ds, kmask=km)
    dk16 = torch.full(kc.shape, float("nan"), dtype=torch.bfloat16, device=d)
    dv16 = torch.full_like(dk16, float("nan"))
    ra.bwd_chunk_dkdv_ds(gq, kc, vc, gdo, lse, delta, dk16, dv16, 0, ds, kmask=km)
    torch.cuda.synchronize()
    assert torch.equal(dk16, dk32.to(torch.bfloat16)) and torch.equal(dv16, dv32.to(torch.bfloat16))
