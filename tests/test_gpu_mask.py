"""Key-validity (key-padding) mask on the GPU against the oracle's masked attention.

The mask reading (masked keys leave every softmax of their batch; a batch with no
valid key gets out 0, lse -inf and zero gradients) follows the diffusers PR "Fix Flux
Context Parallel Bug", where padding to a divisible length is noted to change the
image because padded tokens are attended, and masking is the proposed remedy.
Inputs and masks come from the seeded generators in ``workloads``.
"""
import numpy as np
import pytest
import torch

import context_attention_lse_kv_amd as ra
import oracle
import workloads as W
from parity import BF16_TOL, check_bf16, F32_TOL, LSE_TOL_BF16, dev, max_abs, np64, oracle_by_head, rel

pytestmark = pytest.mark.gpu


def _ring(q, k, v, do, lens, order, kmask):
    d = dev()
    gq, gk, gv, gdo = (x.to(d) for x in (q, k, v, do))
    gm = None if kmask is None else kmask.to(d)
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(gq, gk, gv, ch, kmask=gm)
    dq, dk, dv = ra.ring_bwd(gq, gk, gv, out, gdo, lse, ch, kmask=gm)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _check(got, ref, tol, lse_tol):
    out, lse, dq, dk, dv = (np64(x) for x in got)
    r_out, r_lse, r_dq, r_dk, r_dv = ref
    for t in (out, lse, dq, dk, dv):
        assert not np.isnan(t).any()
    assert np.array_equal(np.isneginf(lse), np.isneginf(r_lse))
    fin = np.isfinite(r_lse)
    if fin.any():
        assert max_abs(lse[fin], r_lse[fin]) <= lse_tol
    for name, a, b in (("out", out, r_out), ("dq", dq, r_dq), ("dk", dk, r_dk), ("dv", dv, r_dv)):
        if tol == BF16_TOL:
            check_bf16(name, a, b)
        else:
            assert rel(a, b) <= tol, rel(a, b)


CASES = [
    # name, B, S, Sq, Hq, Hkv, D, dtype, chunk lens, order, mask recipe
    ("d64_ring2_tail", 2, 512, 512, 8, 8, 64, "bf16", (256, 256), (1, 0),
     dict(p_keep=0.7, valid_len=(512, 300))),
    ("d128_gqa_uneven_chunk_masked", 2, 640, 320, 8, 2, 128, "bf16", (214, 213, 213), (2, 1, 0),
     dict(p_keep=0.85, valid_len=(640, 500), masked_ranges=[(0, 214, 427)])),
    ("f32_tiny", 1, 256, 256, 2, 2, 64, "f32", (128, 128), (0, 1), dict(p_keep=0.6)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_masked_ring_matches_oracle(case):
    name, B, S, Sq, Hq, Hkv, D, dt, lens, order, recipe = case
    seed = 900 + CASES.index(case)
    q = W.randn((B, Sq, Hq, D), seed, dt)
    k = W.randn((B, S, Hkv, D), seed + 1, dt)
    v = W.randn((B, S, Hkv, D), seed + 2, dt)
    do = W.randn((B, Sq, Hq, D), seed + 3, dt)
    m = W.make_key_mask(B, S, seed + 4, **recipe)
    got = _ring(q, k, v, do, lens, order, m)
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    mn = m.numpy().astype(np.uint8)
    o, l = oracle.attention_forward(qn, kn, vn, kmask=mn)
    g = oracle.attention_backward(qn, kn, vn, don, kmask=mn)
    tol, lse_tol = (BF16_TOL, LSE_TOL_BF16) if dt == "bf16" else (F32_TOL, F32_TOL)
    _check(got, (o, l, *g), tol, lse_tol)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_masked_batch_without_valid_key(dt):
    B, S, Sq, Hq, Hkv, D = 3, 384, 200, 4, 2, 64
    q, k, v, do = (W.randn(s, 950 + i, dt) for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                   (B, S, Hkv, D), (B, Sq, Hq, D)]))
    m = W.make_key_mask(B, S, 955, p_keep=0.9)
    m[1] = False
    out, lse, dq, dk, dv = (np64(x) for x in _ring(q, k, v, do, (128, 128, 128), (0, 2, 1), m))
    assert np.all(np.isneginf(lse[1])) and np.all(out[1] == 0)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    for t in (out, dq, dk, dv):
        assert not np.isnan(t).any()
    sel = [0, 2]
    qn, kn, vn, don = (np64(t)[sel] for t in (q, k, v, do))
    mn = m.numpy().astype(np.uint8)[sel]
    o, l = oracle.attention_forward(qn, kn, vn, kmask=mn)
    g = oracle.attention_backward(qn, kn, vn, don, kmask=mn)
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    assert max_abs(lse[sel], l) <= (LSE_TOL_BF16 if dt == "bf16" else F32_TOL)
    for name, a, b in zip(("out", "dq", "dk", "dv"), (out[sel], dq[sel], dk[sel], dv[sel]), (o, *g)):
        if dt == "bf16":
            check_bf16(name, a, b)
        else:
            assert rel(a, b) <= tol


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_masked_key_values_never_read(dt):
    """Replacing masked keys' K/V by huge values changes nothing, bit for bit."""
    B, S, Sq, Hq, Hkv, D = 2, 300, 130, 8, 2, 128
    q, k, v, do = (W.randn(s, 960 + i, dt) for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                   (B, S, Hkv, D), (B, Sq, Hq, D)]))
    m = W.make_key_mask(B, S, 965, p_keep=0.6, valid_len=(300, 257))
    a = _ring(q, k, v, do, (100, 100, 100), (1, 0, 2), m)
    k2, v2 = k.clone(), v.clone()
    big = W.randn(k.shape, 966, dt, mult=300.0)
    k2[~m] = big[~m]
    v2[~m] = big.flip(0)[~m]
    b = _ring(q, k2, v2, do, (100, 100, 100), (1, 0, 2), m)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dk, dv = np64(a[3]), np64(a[4])
    mm = ~m.numpy()
    assert np.all(dk[mm] == 0) and np.all(dv[mm] == 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_all_ones_mask_equals_no_mask(dt):
    B, S, Sq, Hq, Hkv, D = 2, 512, 256, 8, 8, 64
    q, k, v, do = (W.randn(s, 970 + i, dt) for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                   (B, S, Hkv, D), (B, Sq, Hq, D)]))
    ones = torch.ones((B, S), dtype=torch.bool)
    a = _ring(q, k, v, do, (256, 256), (1, 0), ones)
    b = _ring(q, k, v, do, (256, 256), (1, 0), None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_masked_chunk_entry_points_match_ring():
    """fwd_chunk/bwd_chunk(_dkdv/_dq) with the chunk's mask slice reproduce the masked ring
    (bit for bit except dQ, which the two reach by different routes)."""
    B, S, Sq, Hq, Hkv, D = 2, 400, 160, 4, 2, 128
    q, k, v, do = (W.randn(s, 980 + i, "bf16") for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                      (B, S, Hkv, D), (B, Sq, Hq, D)]))
    m = W.make_key_mask(B, S, 985, p_keep=0.75, masked_ranges=[(1, 0, 200)])
    lens, order = (200, 200), (0, 1)
    out_r, lse_r, dq_r, dk_r, dv_r = _ring(q, k, v, do, lens, order, m)
    d = dev()
    gq, gk, gv, gdo, gm = (x.to(d) for x in (q, k, v, do, m))
    out = torch.empty(q.shape, dtype=torch.float32, device=d)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=d)
    starts = (0, 200)
    for i, c in enumerate(order):
        sl = slice(starts[c], starts[c] + lens[c])
        ra.fwd_chunk(gq, gk[:, sl], gv[:, sl], out, lse, merge=i > 0, kmask=gm[:, sl])
    outb = out.to(torch.bfloat16)
    assert torch.equal(outb, out_r) and torch.equal(lse, lse_r)
    delta = torch.empty_like(lse)
    ra.bwd_delta(outb, gdo, delta)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=d)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=d)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=d)
    for c in order:
        sl = slice(starts[c], starts[c] + lens[c])
        if c == 0:
            ra.bwd_chunk(gq, gk[:, sl], gv[:, sl], gdo, lse, delta, dq, dk[:, sl], dv[:, sl], 1, kmask=gm[:, sl])
        else:
            ra.bwd_chunk_dkdv(gq, gk[:, sl], gv[:, sl], gdo, lse, delta, dk[:, sl], dv[:, sl], 1, kmask=gm[:, sl])
            ra.bwd_chunk_dq(gq, gk[:, sl], gv[:, sl], gdo, lse, delta, dq, kmask=gm[:, sl])
    torch.cuda.synchronize()
    # dK/dV come from the same kernel in both; the ring forms dQ from the dS that kernel
    # stored (fp16 P), the chunk entry point recomputes it (fp32 P): equal up to rounding
    for a, b in ((dk, dk_r), (dv, dv_r)):
        assert torch.equal(a.to(torch.bfloat16), b)
    rel = ((dq.to(torch.bfloat16).float() - dq_r.float()).norm() / dq_r.float().norm()).item()
    assert rel < 5e-3, rel


@pytest.mark.parametrize("lens,order,masked", [
    ((192, 192), (0, 1), [(0, 192, 384)]),      # batch 0: every key of the last chunk masked
    ((192, 0, 192), (2, 0, 1), [(1, 0, 192)]),  # last chunk in order empty, batch 1's keys of the one before masked
    ((384,), (0,), [(0, 0, 384)]),              # one chunk, batch 0 without a valid key
])
def test_masked_bf16_output_is_rne_of_fp32(lens, order, masked):
    """The bf16 output that the sweep's last non-empty step writes itself equals the fp32
    output rounded to nearest even, also for rows whose keys in that step are all masked."""
    B, S, Sq, Hq, Hkv, D = 2, 384, 150, 4, 2, 128
    q, k, v = (W.randn(s, 995 + i, "bf16") for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)]))
    m = W.make_key_mask(B, S, 999, p_keep=0.8, masked_ranges=masked)
    d = dev()
    gq, gk, gv, gm = (x.to(d) for x in (q, k, v, m))
    ch = ra.Chunks(lens, order)
    o32, l32 = ra.ring_fwd(gq, gk, gv, ch, kmask=gm, out_dtype=torch.float32)
    o16, l16 = ra.ring_fwd(gq, gk, gv, ch, kmask=gm, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(l16, l32)
    assert not torch.isnan(o16).any()


def test_masked_video_shard():
    """The video-DiT GQA rank-0 shard with right padding (valid 30000 of 32768 keys) and
    5 % of the other keys masked; oracle on two kv-head groups."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w, Sq=lens[0])
    m = W.make_key_mask(w.B, w.S, 990, p_keep=0.95, valid_len=(30000,))
    out, lse, dq, dk, dv = _ring(q, k, v, do, lens, ra.ring_order(w.n_chunks, 0), m)
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    mn = m.numpy().astype(np.uint8)
    for grp in (1, 6):
        heads = list(range(4 * grp, 4 * grp + 4))
        ref = oracle_by_head(qn, kn, vn, don, heads, kmask=mn)
        check_bf16('out', np64(out[:, :, heads]), ref["out"])
        assert max_abs(np64(lse[:, heads]), ref["lse"]) <= LSE_TOL_BF16
        check_bf16('dq', np64(dq[:, :, heads]), ref["dq"])
        check_bf16('dk', np64(dk[:, :, grp]), ref["dk"][:, :, grp])
        check_bf16('dv', np64(dv[:, :, grp]), ref["dv"][:, :, grp])
