"""GPU parity of the HIP ring-attention path against the CPU fp64 oracle.

Every case feeds the same seeded inputs (``workloads``) to both sides and
compares element by element with the relative Frobenius error of the diffusers
issue "Ring attention backward uses stale iteration-0 KV" (section
Reproduction).  Tolerances: bf16 max rel err of out/dq/dk/dv <= 2e-2 and LSE
abs err <= 1e-3; fp32 path <= 1e-5; exchange bit-exact.
"""
import numpy as np
import pytest
import torch

import context_attention_lse_kv_amd as ra
import oracle
import workloads as W
from oracle_pins import golden
from parity import (BF16_TOL, F32_TOL, LSE_TOL_BF16, check_bf16, dev, max_abs, np64, oracle_by_head,
                    oracle_grads_by_head, rel)

pytestmark = pytest.mark.gpu


def to_dev(*ts):
    d = dev()
    return [t.to(d) for t in ts]


def ring(q, k, v, dout, lens, order, out_dtype=None, grad_dtype=torch.float32, layout="bshd", scale=None):
    ch = ra.Chunks(lens, order)
    out, lse = ra.ring_fwd(q, k, v, ch, scale=scale, out_dtype=out_dtype, layout=layout)
    dq, dk, dv = ra.ring_bwd(q, k, v, out, dout, lse, ch, scale=scale, grad_dtype=grad_dtype, layout=layout)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def shard_rows(lens, r):
    s = sum(lens[:r])
    return slice(s, s + lens[r])


# ------------------------------------------------------------------ tiny fp32 (B1 S256 H2 D64, 2 chunks)
def test_tiny_f32_full_and_shards():
    w = W.TINY_F32
    q, k, v, do = W.make_inputs(w)
    lens = ra.split_sizes(w.S, w.n_chunks)
    assert tuple(lens) == w.chunk_lens
    ref_o, ref_l = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), scale=1 / 8)
    ref_dq, ref_dk, ref_dv = oracle.attention_backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale=1 / 8)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, lens, [0, 1], scale=1 / 8)
    assert rel(np64(out), ref_o) <= F32_TOL
    assert max_abs(np64(lse), ref_l) <= F32_TOL
    for got, ref in ((dq, ref_dq), (dk, ref_dk), (dv, ref_dv)):
        assert rel(np64(got), ref) <= F32_TOL
    dk_sum = np.zeros(ref_dk.shape)
    dv_sum = np.zeros(ref_dv.shape)
    for r in range(2):
        rows = shard_rows(lens, r)
        o_r, l_r, dq_r, dk_r, dv_r = ring(gq[:, rows], gk, gv, gdo[:, rows], lens, ra.ring_order(2, r), scale=1 / 8)
        assert rel(np64(o_r), ref_o[:, rows]) <= F32_TOL
        assert max_abs(np64(l_r), ref_l[:, :, rows]) <= F32_TOL
        assert rel(np64(dq_r), ref_dq[:, rows]) <= F32_TOL
        c_dq, c_dk, c_dv = oracle.attention_backward(q.numpy()[:, rows], k.numpy(), v.numpy(), do.numpy()[:, rows],
                                                     scale=1 / 8)
        assert rel(np64(dk_r), c_dk) <= F32_TOL and rel(np64(dv_r), c_dv) <= F32_TOL
        dk_sum += np64(dk_r)
        dv_sum += np64(dv_r)
    assert rel(dk_sum, ref_dk) <= F32_TOL and rel(dv_sum, ref_dv) <= F32_TOL


# ------------------------------------------------------------------ bf16 ring (B2 S512 H8 D64, ring 2/4)
@pytest.mark.parametrize("w", [W.BF16_RING2, W.BF16_RING4], ids=lambda w: w.name)
def test_bf16_ring_every_rank(w):
    q, k, v, do = W.make_inputs(w)
    R = w.n_chunks
    lens = ra.split_sizes(w.S, R)
    assert tuple(lens) == w.chunk_lens
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    ref_o, ref_l = oracle.attention_forward(qn, kn, vn)
    ref_dq, ref_dk, ref_dv = oracle.attention_backward(qn, kn, vn, don)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    dk_sum = np.zeros(ref_dk.shape)
    dv_sum = np.zeros(ref_dv.shape)
    for r in range(R):
        rows = shard_rows(lens, r)
        out, lse, dq, dk, dv = ring(gq[:, rows], gk, gv, gdo[:, rows], lens, ra.ring_order(R, r))
        assert out.dtype == torch.bfloat16
        check_bf16('out', np64(out), ref_o[:, rows])
        assert max_abs(np64(lse), ref_l[:, :, rows]) <= LSE_TOL_BF16
        check_bf16('dq', np64(dq), ref_dq[:, rows])
        _, c_dk, c_dv = oracle.attention_backward(qn[:, rows], kn, vn, don[:, rows])
        check_bf16('dk', np64(dk), c_dk)
        check_bf16('dv', np64(dv), c_dv)
        dk_sum += np64(dk)
        dv_sum += np64(dv)
    check_bf16('dk (sum over ranks)', dk_sum, ref_dk)
    check_bf16('dv (sum over ranks)', dv_sum, ref_dv)


def test_bf16_gradients_in_bf16():
    w = W.BF16_RING2
    q, k, v, do = W.make_inputs(w)
    lens = ra.split_sizes(w.S, 2)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    rows = shard_rows(lens, 1)
    _, _, dq32, dk32, dv32 = ring(gq[:, rows], gk, gv, gdo[:, rows], lens, ra.ring_order(2, 1))
    _, _, dq16, dk16, dv16 = ring(gq[:, rows], gk, gv, gdo[:, rows], lens, ra.ring_order(2, 1),
                                  grad_dtype=torch.bfloat16)
    for a, b in ((dq32, dq16), (dk32, dk16), (dv32, dv16)):
        assert b.dtype == torch.bfloat16
        # the bf16 gradient is the fp32 accumulator rounded to nearest even
        assert rel(np64(b), np64(a)) <= 4e-3


def test_stale_kv_negative_control():
    """The defect of the diffusers issue ("Root cause"): every backward step recomputed
    against the step-0 (local) chunk.  Composed here from correct chunk steps fed the
    wrong chunk; it must miss the gate by orders of magnitude, while the correct
    composition of the same calls passes."""
    for w in (W.BF16_RING2, W.BF16_RING4):
        q, k, v, do = W.make_inputs(w)
        R = w.n_chunks
        lens = ra.split_sizes(w.S, R)
        qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
        ref_dq, ref_dk, ref_dv = oracle.attention_backward(qn, kn, vn, don)
        gq, gk, gv, gdo = to_dev(q, k, v, do)
        errs = {"dq": [], "dk": [], "dv": []}
        good = {"dq": [], "dk": [], "dv": []}
        dk_all = {True: torch.zeros(gk.shape, dtype=torch.float32, device=gk.device),
                  False: torch.zeros(gk.shape, dtype=torch.float32, device=gk.device)}
        dv_all = {True: torch.zeros_like(dk_all[True]), False: torch.zeros_like(dk_all[True])}
        for r in range(R):
            rows = shard_rows(lens, r)
            order = ra.ring_order(R, r)
            qs, dos = gq[:, rows].contiguous(), gdo[:, rows].contiguous()
            out, lse = ra.ring_fwd(qs, gk, gv, ra.Chunks(lens, order), out_dtype=torch.float32)
            delta = torch.empty_like(lse)
            ra.bwd_delta(out, dos, delta)
            for stale in (True, False):
                dq = torch.zeros(qs.shape, dtype=torch.float32, device=qs.device)
                for c in order:
                    src = order[0] if stale else c   # stale: the chunk saved at step 0
                    kr, sr = shard_rows(lens, c), shard_rows(lens, src)
                    ra.bwd_chunk(qs, gk[:, sr], gv[:, sr], dos, lse, delta, dq, dk_all[stale][:, kr],
                                 dv_all[stale][:, kr], accumulate=1)
                torch.cuda.synchronize()
                (errs if stale else good)["dq"].append(rel(np64(dq), ref_dq[:, rows]))
        for stale in (True, False):
            tgt = errs if stale else good
            tgt["dk"].append(rel(np64(dk_all[stale]), ref_dk))
            tgt["dv"].append(rel(np64(dv_all[stale]), ref_dv))
        print(w.name, "stale-KV rel err", {k_: max(v_) for k_, v_ in errs.items()},
              "correct", {k_: max(v_) for k_, v_ in good.items()})
        for name in ("dq", "dk", "dv"):
            assert max(good[name]) <= BF16_TOL
            assert max(errs[name]) > 0.2, (name, errs[name])


# ------------------------------------------------------------------ uneven + seq-first + Ulysses exchange
@pytest.mark.parametrize("R", [3, 2])
def test_uneven_seqfirst_ulysses(R):
    w = W.UNEVEN_SEQFIRST
    q, k, v, do = W.make_inputs(w)          # [S, B, H, D]
    S, B, H, D = q.shape
    seq_lens = ra.split_sizes(S, R)
    heads = ra.split_sizes(H, R)
    chunk_lens = ra.split_sizes(S, w.n_chunks)
    assert tuple(chunk_lens) == w.chunk_lens == (334, 333, 333)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    offs = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
    shard = lambda x: [x[offs[i]:offs[i + 1]] for i in range(R)]
    qh, kh, vh, doh = (ra.seq_to_head(shard(x), heads) for x in (gq, gk, gv, gdo))
    # the exchange is bit-exact against the oracle's index slicing
    for name, x, xs in (("q", q, qh), ("dout", do, doh)):
        ref = oracle.seq_to_head([t.view(torch.int16).numpy() for t in shard(x)], heads)
        for r in range(R):
            assert np.array_equal(xs[r].cpu().view(torch.int16).numpy(), ref[r]), (name, r)
    outs, dqs, dks, dvs = [], [], [], []
    for r in range(R):
        # each simulated rank: full-sequence attention on its head group, swept over the 3 chunks
        out, lse, dq, dk, dv = ring(qh[r], kh[r], vh[r], doh[r], chunk_lens, ra.ring_order(w.n_chunks, r % w.n_chunks),
                                    grad_dtype=torch.bfloat16, layout="sbhd")
        outs.append(out); dqs.append(dq); dks.append(dk); dvs.append(dv)
    out_s, dq_s, dk_s, dv_s = (ra.head_to_seq(x, seq_lens) for x in (outs, dqs, dks, dvs))
    torch.cuda.synchronize()
    cat = lambda xs: np64(torch.cat(xs, dim=0))
    bf = lambda x: np.ascontiguousarray(np.transpose(np64(x), (1, 0, 2, 3)))
    ref_o, _ = oracle.attention_forward(bf(q), bf(k), bf(v))
    ref_dq, ref_dk, ref_dv = oracle.attention_backward(bf(q), bf(k), bf(v), bf(do))
    sf = lambda x: np.transpose(x, (1, 0, 2, 3))
    check_bf16('out', cat(out_s), sf(ref_o))
    check_bf16('dq', cat(dq_s), sf(ref_dq))
    check_bf16('dk', cat(dk_s), sf(ref_dk))
    check_bf16('dv', cat(dv_s), sf(ref_dv))
    for xs, n in ((out_s, seq_lens), (dq_s, seq_lens)):
        assert [x.shape[0] for x in xs] == n and all(x.shape[2] == H for x in xs)


def test_exchange_bit_exact_properties():
    """Slot rule, inverse, gradient 2x (DeepSpeed PR "_DimZeroAllToAll ...", Testing)
    and the shapes of the DeepSpeed issue "DistributedAttention ...", last comment."""
    d = dev()
    g = golden()["ulysses_exchange_shapes"]
    S_loc, B, H, D = g["local_shape_sbhd"]
    for dtype in (torch.float32, torch.bfloat16):
        shards = [W.randn((S_loc, B, H, D), seed=20 + i, dtype="f32").to(dtype).to(d) for i in range(g["ranks"])]
        ys = ra.seq_to_head(shards, ra.split_sizes(H, g["ranks"]))
        assert all(list(y.shape) == g["exchanged_shape_sbhd"] for y in ys)
        back = ra.head_to_seq(ys, [S_loc] * g["ranks"])
        assert all(list(b.shape) == g["out_shape_sbhd"] for b in back)
        for x, b in zip(shards, back):
            assert torch.equal(x, b)
        grads = ra.head_to_seq([2 * y for y in ys], [S_loc] * g["ranks"])
        for x, gr in zip(shards, grads):
            assert torch.equal(gr, 2 * x)
    # uneven seq and head splits, batch-first layout, bitwise against the oracle (16-byte
    # vectors per row: 8 for bf16 D64, 16 for bf16 D128, 32 for fp32 D128)
    for D, dt, bits in ((64, "bf16", torch.int16), (128, "bf16", torch.int16), (128, "f32", torch.int32)):
        for (seq_lens, heads) in (([334, 333, 333], [3, 3, 2]), ([5, 0, 4, 3], [1, 2, 2, 3])):
            H = sum(heads)
            xs = [W.randn((2, s, H, D), seed=30 + i, dtype=dt).to(d) for i, s in enumerate(seq_lens)]
            ys = ra.seq_to_head(xs, heads, layout="bshd")
            ref = oracle.seq_to_head([np.transpose(x.cpu().view(bits).numpy(), (1, 0, 2, 3)) for x in xs], heads)
            for y, rr in zip(ys, ref):
                assert np.array_equal(np.transpose(y.cpu().view(bits).numpy(), (1, 0, 2, 3)), rr)
            back = ra.head_to_seq(ys, seq_lens, layout="bshd")
            for x, b in zip(xs, back):
                assert torch.equal(x, b)


# ------------------------------------------------------------------ image-DiT forward (D128, 4 chunks)
def test_image_dit_fwd_full_and_shard():
    w = W.IMAGE_DIT_FWD
    q, k, v, _ = W.make_inputs(w)
    lens = ra.split_sizes(w.S, w.n_chunks)
    assert tuple(lens) == w.chunk_lens
    gq, gk, gv = to_dev(q, k, v)
    qn, kn, vn = np64(q), np64(k), np64(v)
    # full Q (the four shards in one sweep): rows sampled, all heads
    out, lse = ra.ring_fwd(gq, gk, gv, ra.Chunks(lens, [0, 1, 2, 3]))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(w.S, 384, replace=False))
    ref = oracle_by_head(qn[:, rows], kn, vn, None, range(w.Hq), backward=False)
    check_bf16('out (full Q, sampled rows)', np64(out)[:, rows], ref["out"])
    assert max_abs(np64(lse)[:, :, rows], ref["lse"]) <= LSE_TOL_BF16
    # rank-0 shard (1152 rows), ring order 0,3,2,1: every element
    sl = shard_rows(lens, 0)
    out0, lse0 = ra.ring_fwd(gq[:, sl], gk, gv, ra.Chunks(lens, ra.ring_order(4, 0)))
    torch.cuda.synchronize()
    ref0 = oracle_by_head(qn[:, sl], kn, vn, None, range(w.Hq), backward=False)
    check_bf16('out (rank-0 shard)', np64(out0), ref0["out"])
    assert max_abs(np64(lse0), ref0["lse"]) <= LSE_TOL_BF16
    # the shard's rows of the full-Q sweep agree with the shard sweep to bf16 rounding
    assert rel(np64(out)[:, sl], np64(out0)) <= 1e-2


# ------------------------------------------------------------------ video-DiT GQA (S32k, Hq32/Hkv8, D128)
@pytest.mark.slow
def test_video_dit_gqa_shard():
    """Rank 0's shard (rows [0,4096)) swept over the 8 chunks in ring order 0,7,...,1,
    exactly as the bench times it; oracle on two whole kv-head groups (8 query heads)."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    assert tuple(lens) == w.chunk_lens
    q, k, v, do = W.make_inputs(w, Sq=lens[0])
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, lens, ra.ring_order(w.n_chunks, 0))
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    for grp in (0, 5):
        heads = list(range(4 * grp, 4 * grp + 4))
        ref = oracle_by_head(qn, kn, vn, don, heads)
        check_bf16('out', np64(out[:, :, heads]), ref["out"])
        assert max_abs(np64(lse[:, heads]), ref["lse"]) <= LSE_TOL_BF16
        check_bf16('dq', np64(dq[:, :, heads]), ref["dq"])
        check_bf16('dk', np64(dk[:, :, grp]), ref["dk"][:, :, grp])
        check_bf16('dv', np64(dv[:, :, grp]), ref["dv"][:, :, grp])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_video_dit_gqa_full_q():
    """Full Q (32768 rows) swept over the 8 chunks.  Against the oracle: out/lse on 96
    sampled rows of 4 heads; dq, dk and dv of one whole kv-head group (its 4 query heads,
    every row and key), element by element, as the diffusers issue "Ring attention
    backward uses stale iteration-0 KV" (section Reproduction) compares each gradient
    with the full-sequence reference.  The other kv heads' dK/dV through properties that
    hold at any size (rows of P sum to 1, rows of dS sum to 0)."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, lens, list(range(w.n_chunks)))
    rows = torch.as_tensor(np.sort(np.random.default_rng(1).choice(w.S, 96, replace=False)))
    heads = torch.as_tensor([0, 13, 22, 31])
    qn, kn, vn, don = (np64(t) for t in (q[:, rows], k, v, do[:, rows]))
    ref = oracle_by_head(qn, kn, vn, don, heads.tolist(), backward=False)
    sel = lambda t: np64(t.cpu()[:, rows][:, :, heads])
    check_bf16('out (sampled rows)', sel(out), ref["out"])
    assert max_abs(np64(lse.cpu()[:, heads][:, :, rows]), ref["lse"]) <= LSE_TOL_BF16
    dkn, dvn, dof = np64(dk), np64(dv), np64(do)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        want = dof[:, :, g * G:(g + 1) * G].sum(axis=(1, 2))
        check_bf16('key-sum of dV', dvn[:, :, g].sum(axis=1), want)
        assert np.linalg.norm(dkn[:, :, g].sum(axis=1)) <= BF16_TOL * np.linalg.norm(dkn[:, :, g])
    grp = 5
    gh = list(range(G * grp, G * grp + G))
    # the group on its own: its 4 query heads against kv head grp (kv head 0 of the slice)
    qn, don = np64(q[:, :, gh]), np64(do[:, :, gh])
    kn, vn = np64(k[:, :, grp:grp + 1]), np64(v[:, :, grp:grp + 1])
    rdq, rdk, rdv = oracle_grads_by_head(qn, kn, vn, don, list(range(G)), row_block=512)
    check_bf16('dq (kv group 5, all rows)', np64(dq[:, :, gh]), rdq)
    check_bf16('dk (kv group 5, all keys)', dkn[:, :, grp], rdk[:, :, 0])
    check_bf16('dv (kv group 5, all keys)', dvn[:, :, grp], rdv[:, :, 0])


# ------------------------------------------------------------------ single entry points
def test_fwd_chunk_and_merge_lse():
    d = dev()
    B, S, Hq, Hkv, D = 2, 300, 6, 2, 128
    q = W.randn((B, 77, Hq, D), 1, "bf16"); k = W.randn((B, S, Hkv, D), 2, "bf16"); v = W.randn((B, S, Hkv, D), 3, "bf16")
    gq, gk, gv = to_dev(q, k, v)
    o_full, l_full = oracle.attention_forward(np64(q), np64(k), np64(v))
    parts = [(0, 113), (113, 300)]
    outs, lses = [], []
    for a, b in parts:
        o = torch.empty(gq.shape, dtype=torch.float32, device=d)
        l = torch.empty((B, Hq, 77), dtype=torch.float32, device=d)
        ra.fwd_chunk(gq, gk[:, a:b], gv[:, a:b], o, l, merge=0)
        outs.append(o); lses.append(l)
        ro, rl = oracle.attention_forward(np64(q), np64(k)[:, a:b], np64(v)[:, a:b])
        torch.cuda.synchronize()
        assert rel(np64(o), ro) <= 5e-3 and max_abs(np64(l), rl) <= LSE_TOL_BF16
    # standalone merge
    m_o, m_l = outs[0].clone(), lses[0].clone()
    ra.merge_lse(m_o, m_l, outs[1], lses[1])
    # fused merge epilogue
    f_o, f_l = outs[0].clone(), lses[0].clone()
    ra.fwd_chunk(gq, gk[:, 113:], gv[:, 113:], f_o, f_l, merge=1)
    torch.cuda.synchronize()
    for o, l in ((m_o, m_l), (f_o, f_l)):
        assert rel(np64(o), o_full) <= 5e-3 and max_abs(np64(l), l_full) <= LSE_TOL_BF16
    # merge against the empty partial (lse = -inf) is the identity; both empty gives (0, -inf)
    e_o = torch.zeros_like(outs[0]); e_l = torch.full_like(lses[0], float("-inf"))
    i_o, i_l = outs[0].clone(), lses[0].clone()
    ra.merge_lse(i_o, i_l, e_o, e_l)
    z_o, z_l = e_o.clone(), e_l.clone()
    ra.merge_lse(z_o, z_l, e_o, e_l)
    torch.cuda.synchronize()
    assert torch.equal(i_o, outs[0]) and torch.equal(i_l, lses[0])
    assert torch.all(z_o == 0) and torch.all(torch.isneginf(z_l))


def test_bwd_chunk_halves_match_whole_step():
    """ra_bwd_chunk_dkdv + ra_bwd_chunk_dq reproduce ra_bwd_chunk, and each matches the
    oracle's gradients of a one-chunk sweep (bf16 and fp32 paths, GQA, odd sizes)."""
    d = dev()
    for dt, tol in (("bf16", BF16_TOL), ("f32", F32_TOL)):
        B, Sq, Sk, Hq, Hkv, D = 1, 150, 203, 4, 2, 128
        q = W.randn((B, Sq, Hq, D), 40, dt); k = W.randn((B, Sk, Hkv, D), 41, dt)
        v = W.randn((B, Sk, Hkv, D), 42, dt); do = W.randn((B, Sq, Hq, D), 43, dt)
        gq, gk, gv, gdo = to_dev(q, k, v, do)
        out, lse = ra.ring_fwd(gq, gk, gv, ra.Chunks([Sk]), out_dtype=torch.float32)
        delta = torch.empty_like(lse)
        ra.bwd_delta(out, gdo, delta)
        z = lambda t: torch.zeros(t.shape, dtype=torch.float32, device=d)
        dq1, dk1, dv1 = z(gq), z(gk), z(gk)
        ra.bwd_chunk(gq, gk, gv, gdo, lse, delta, dq1, dk1, dv1, accumulate=0)
        dq2, dk2, dv2 = z(gq), z(gk), z(gk)
        ra.bwd_chunk_dkdv(gq, gk, gv, gdo, lse, delta, dk2, dv2, accumulate=0)
        ra.bwd_chunk_dq(gq, gk, gv, gdo, lse, delta, dq2)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq2)  # same kernel, single writer per row: bit-identical
        assert rel(np64(dk1), np64(dk2)) <= 1e-6 and rel(np64(dv1), np64(dv2)) <= 1e-6  # atomics reorder sums
        ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do))
        for got, r in zip((dq2, dk2, dv2), ref):
            assert rel(np64(got), r) <= tol


def test_bwd_delta_against_oracle():
    d = dev()
    for odt, ddt in ((torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16), (torch.float32, torch.float32)):
        o = W.randn((2, 129, 5, 64), 4, "f32").to(odt)
        do = W.randn((2, 129, 5, 64), 5, "f32").to(ddt)
        delta = torch.empty((2, 5, 129), dtype=torch.float32, device=d)
        ra.bwd_delta(o.to(d), do.to(d), delta)
        torch.cuda.synchronize()
        assert rel(np64(delta), oracle.attention_delta(np64(o), np64(do))) <= 1e-6


def test_edge_cases():
    d = dev()
    # one query row against one key
    q = W.randn((1, 1, 2, 64), 6, "bf16"); k = W.randn((1, 1, 1, 64), 7, "bf16"); v = W.randn((1, 1, 1, 64), 8, "bf16")
    do = W.randn((1, 1, 2, 64), 9, "bf16")
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, [1], [0], out_dtype=torch.float32)
    ro, rl = oracle.attention_forward(np64(q), np64(k), np64(v))
    assert rel(np64(out), ro) <= 1e-6 and max_abs(np64(lse), rl) <= LSE_TOL_BF16
    # one key: P = 1, so dQ and dK vanish up to fp32 rounding of exp2/log
    assert np.abs(np64(dq)).max() < 1e-4 and np.abs(np64(dk)).max() < 1e-4
    # an empty chunk anywhere in the sweep, odd sizes, GQA, D=128, tails in every tile
    B, Sq, Sk, Hq, Hkv, D = 2, 77, 201, 6, 2, 128
    q = W.randn((B, Sq, Hq, D), 10, "bf16"); k = W.randn((B, Sk, Hkv, D), 11, "bf16")
    v = W.randn((B, Sk, Hkv, D), 12, "bf16"); do = W.randn((B, Sq, Hq, D), 13, "bf16")
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    ref_o, ref_l = oracle.attention_forward(np64(q), np64(k), np64(v))
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do))
    for lens, order in (([0, 100, 101], [0, 1, 2]), ([100, 0, 101], [1, 2, 0]), ([201, 0], [1, 0]), ([1] * 3 + [198], [3, 1, 0, 2])):
        out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, lens, order)
        check_bf16('out', np64(out), ref_o)
        assert max_abs(np64(lse), ref_l) <= LSE_TOL_BF16
        for got, r in zip((dq, dk, dv), ref):
            check_bf16('grad', np64(got), r)
    # no keys at all: lse = -inf, out = 0, gradients 0
    k0 = torch.empty((B, 0, Hkv, D), dtype=torch.bfloat16, device=d)
    out, lse, dq, dk, dv = ring(gq, k0, k0, gdo, [0], [0])
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse)) and torch.all(dq == 0)
    # no queries: nothing to do, nothing breaks
    q0 = torch.empty((B, 0, Hq, D), dtype=torch.bfloat16, device=d)
    out, lse, dq, dk, dv = ring(q0, gk, gv, q0, [201], [0])
    assert out.shape[1] == 0 and torch.all(dk == 0)
    # strided (non-contiguous) inputs: heads interleaved in a wider buffer, no copies made
    wide = torch.zeros((B, Sq, 2 * Hq, D), dtype=torch.bfloat16, device=d)
    wide[:, :, ::2] = gq
    qs = wide[:, :, ::2]
    assert not qs.is_contiguous()
    out, lse, dq, dk, dv = ring(qs, gk, gv, gdo, [201], [0])
    check_bf16('out', np64(out), ref_o)


def _strided_like(t, row_stride):
    """A device view of `t` ([1, S, H, D]) whose rows lie `row_stride` elements apart in one
    large buffer (heads adjacent within a row); the gaps between rows are never read."""
    _, S, H, D = t.shape
    buf = torch.empty((S - 1) * row_stride + H * D, dtype=t.dtype, device=dev())
    view = buf.as_strided((1, S, H, D), (S * row_stride, row_stride, D, 1))
    view.copy_(t.to(dev()))
    return view


@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float32])
def test_largest_accepted_slice_span(grad_dtype):
    """q, k, v, dout whose (batch, head) slices span just under 2^31 bytes (the largest the
    bf16 kernels' 32-bit buffer offsets accept, tile slack included): ragged tiles, GQA, two
    chunks, against the oracle."""
    Sq, Sk, Hq, Hkv, D = 200, 300, 2, 1, 128
    q = W.randn((1, Sq, Hq, D), 41, "bf16"); k = W.randn((1, Sk, Hkv, D), 42, "bf16")
    v = W.randn((1, Sk, Hkv, D), 43, "bf16"); do = W.randn((1, Sq, Hq, D), 44, "bf16")
    # largest row strides (multiples of 8 elements) with ((S + 128) * sS + D) * 2 < 2^31
    sq = ((2**30 - D) // (Sq + 128)) // 8 * 8
    sk = ((2**30 - D) // (Sk + 128)) // 8 * 8
    for S, st in ((Sq, sq), (Sk, sk)):
        span = ((S + 128) * st + D) * 2
        assert 2**31 - 2 * (S + 128) * 16 < span < 2**31
    gq, gdo = _strided_like(q, sq), _strided_like(do, sq)
    gk, gv = _strided_like(k, sk), _strided_like(v, sk)
    ref_o, ref_l = oracle.attention_forward(np64(q), np64(k), np64(v))
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(do))
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, [150, 150], [1, 0], grad_dtype=grad_dtype)
    check_bf16('out', np64(out), ref_o)
    assert max_abs(np64(lse), ref_l) <= LSE_TOL_BF16
    for name, got, r in zip(('dq', 'dk', 'dv'), (dq, dk, dv), ref):
        check_bf16(name, np64(got), r)


def test_fp32_path_d128_gqa():
    B, Sq, Sk, Hq, Hkv, D = 1, 45, 130, 4, 2, 128
    q = W.randn((B, Sq, Hq, D), 14); k = W.randn((B, Sk, Hkv, D), 15); v = W.randn((B, Sk, Hkv, D), 16)
    do = W.randn((B, Sq, Hq, D), 17)
    gq, gk, gv, gdo = to_dev(q, k, v, do)
    out, lse, dq, dk, dv = ring(gq, gk, gv, gdo, [65, 65], [1, 0])
    ref_o, ref_l = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy())
    ref = oracle.attention_backward(q.numpy(), k.numpy(), v.numpy(), do.numpy())
    assert rel(np64(out), ref_o) <= F32_TOL and max_abs(np64(lse), ref_l) <= F32_TOL
    for got, r in zip((dq, dk, dv), ref):
        assert rel(np64(got), r) <= F32_TOL


def test_bf16_output_is_rne_of_fp32_and_forward_is_deterministic():
    w = W.BF16_RING4
    q, k, v, _ = W.make_inputs(w)
    gq, gk, gv = to_dev(q, k, v)
    lens = ra.split_sizes(w.S, 4)
    ch = ra.Chunks(lens, ra.ring_order(4, 2))
    o32, l32 = ra.ring_fwd(gq, gk, gv, ch, out_dtype=torch.float32)
    o16, l16 = ra.ring_fwd(gq, gk, gv, ch, out_dtype=torch.bfloat16)
    o32b, l32b = ra.ring_fwd(gq, gk, gv, ch, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(o32, o32b) and torch.equal(l32, l32b) and torch.equal(l16, l32)


def test_gpu_refusals_raise():
    d = dev()
    q = torch.zeros((1, 8, 6, 64), dtype=torch.bfloat16, device=d)
    k = torch.zeros((1, 8, 4, 64), dtype=torch.bfloat16, device=d)
    with pytest.raises(RuntimeError, match="Number of heads in key/value must divide number of heads in query"):
        ra.ring_fwd(q, k, k, ra.Chunks([8]))
    with pytest.raises(ValueError):
        ra.ring_fwd(q.cpu(), k.cpu(), k.cpu(), ra.Chunks([8]))


# ------------------------------------------------------------------ forward tile counts
# Chunk lengths around the 64-key tile edges: no full tile, one, two, three, five full
# tiles, with and without a partial last tile.  The forward pipelines the full tiles
# (scores of tile T + 1 overlap P and P V of tile T) and runs a partial tile after the
# loop, so each count takes a different path through that control flow.  With the key
# mask, a sweep also ends early at the last tile that holds a valid key.
TILE_EDGE_KEYS = (1, 63, 64, 65, 128, 129, 192, 193, 320, 333)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("masked", [False, True], ids=["dense", "masked"])
def test_forward_at_tile_edges(D, masked):
    B, Sq, Hq, Hkv = 2, 70, 4, 2
    for n, Sk in enumerate(TILE_EDGE_KEYS):
        seed = 1200 + 10 * n + D
        S = Sk + 64  # the sweep: this chunk, then a full 64-key chunk merged into it
        q = W.randn((B, Sq, Hq, D), seed, "bf16")
        k = W.randn((B, S, Hkv, D), seed + 1, "bf16")
        v = W.randn((B, S, Hkv, D), seed + 2, "bf16")
        # batch 0: keys from Sk - 70 on masked (whole tiles at the end of the chunk with
        # no valid key); batch 1: the first keys masked
        m = (W.make_key_mask(B, S, seed + 3, p_keep=0.7, valid_len=(max(1, Sk - 70), S),
                             masked_ranges=[(1, 0, min(Sk, 130))]) if masked else None)
        gq, gk, gv = to_dev(q, k, v)
        gm = m.to(dev()) if masked else None
        for lens, order in (((Sk,), (0,)), ((Sk, 64), (1, 0))):
            if len(lens) == 1:
                kk, vv, mm = gk[:, :Sk], gv[:, :Sk], (gm[:, :Sk] if masked else None)
            else:
                kk, vv, mm = gk, gv, gm
            out, lse = ra.ring_fwd(gq, kk, vv, ra.Chunks(list(lens), list(order)), out_dtype=torch.float32, kmask=mm)
            torch.cuda.synchronize()
            kn, vn = np64(kk.cpu()), np64(vv.cpu())
            mn = mm.cpu().numpy().astype(np.uint8) if masked else None
            ref_o, ref_l = oracle.attention_forward(np64(q), kn, vn, kmask=mn)
            o, l = np64(out), np64(lse)
            assert not np.isnan(o).any(), (Sk, lens)
            assert np.array_equal(np.isneginf(l), np.isneginf(ref_l)), (Sk, lens)
            fin = np.isfinite(ref_l)
            if fin.any():
                assert max_abs(l[fin], ref_l[fin]) <= LSE_TOL_BF16, (Sk, lens)
            if np.any(ref_o != 0):
                check_bf16('out', o, ref_o)
            assert np.all(o[np.broadcast_to(~fin.transpose(0, 2, 1)[..., None], o.shape)] == 0), (Sk, lens)
