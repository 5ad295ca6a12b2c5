"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes a namespace ``o`` that provides the oracle's
functions and raises AssertionError when the oracle disagrees with what the
pages or the mathematics fix.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with a
planted mistake and requires that some pin fails.

Pins used (none of them retypes the oracle's own formula):
  closed forms   - one key; zero query; identical keys; no keys
  library        - torch CPU float64 scaled_dot_product_attention + autograd,
                   torch.logsumexp (the reference routine of the diffusers
                   issue "Ring attention backward uses stale iteration-0 KV",
                   section Reproduction)
  finite diff.   - central differences of L = sum(dout * out) in float64
  invariants     - chunked forward + LSE merge equals the full forward for any
                   split/order/empty chunk; sum over keys of dK is 0; sum over
                   keys of dV equals the sum of dO over the group's queries;
                   GQA equals MHA with repeated K/V and its dK/dV are the
                   head-group sums
  key mask       - torch SDPA with a boolean attn_mask (+ autograd); one valid
                   key; masked keys' values irrelevant and their dK/dV zero;
                   no valid key gives the empty-softmax result; finite
                   differences; chunk+merge with per-chunk mask slices
  exchange       - slot rule and gradient 2x of the DeepSpeed PR
                   "_DimZeroAllToAll silently fails to send grads", Testing;
                   shapes of the DeepSpeed issue "DistributedAttention ...
                   not divisible by world size", last comment
"""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_fixtures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ----------------------------------------------------------------------------- closed forms
def pin_single_key(o):
    r = _rng(1)
    q = r.standard_normal((2, 7, 4, 5)); k = r.standard_normal((2, 1, 2, 5)); v = r.standard_normal((2, 1, 2, 5))
    out, lse = o.attention_forward(q, k, v, scale=0.3)
    for h in range(4):
        g = h // 2
        assert np.allclose(out[:, :, h, :], np.broadcast_to(v[:, 0:1, g, :], (2, 7, 5)), rtol=0, atol=1e-14)
        s = 0.3 * np.einsum("bsd,bd->bs", q[:, :, h, :], k[:, 0, g, :])
        assert np.allclose(lse[:, h, :], s, rtol=0, atol=1e-13)
    dq, dk, dv = o.attention_backward(q, k, v, r.standard_normal(q.shape), scale=0.3)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    # one key: out = v, so dV = sum over the group's queries of dO
    d = r.standard_normal(q.shape)
    _, _, dv = o.attention_backward(q, k, v, d, scale=0.3)
    for g in range(2):
        want = d[:, :, 2 * g:2 * g + 2, :].sum(axis=(1, 2))
        assert np.allclose(dv[:, 0, g, :], want, rtol=0, atol=1e-12)


def pin_zero_query(o):
    r = _rng(2)
    Sk = 9
    q = np.zeros((1, 3, 2, 4)); k = r.standard_normal((1, Sk, 2, 4)); v = r.standard_normal((1, Sk, 2, 4))
    out, lse = o.attention_forward(q, k, v)
    assert np.all(np.abs(lse - math.log(Sk)) < 1e-15)
    for h in range(2):
        assert np.allclose(out[0, :, h, :], v[0, :, h, :].mean(axis=0), rtol=0, atol=1e-14)


def pin_equal_keys(o):
    r = _rng(3)
    Sk, D = 6, 8
    q = r.standard_normal((1, 4, 1, D)); k1 = r.standard_normal(D)
    k = np.broadcast_to(k1, (1, Sk, 1, D)).copy(); v = r.standard_normal((1, Sk, 1, D))
    scale = 0.25
    out, lse = o.attention_forward(q, k, v, scale=scale)
    want_lse = scale * (q[0, :, 0, :] @ k1) + math.log(Sk)
    assert np.allclose(lse[0, 0], want_lse, rtol=0, atol=1e-13)
    assert np.allclose(out[0, :, 0, :], np.broadcast_to(v[0, :, 0, :].mean(axis=0), (4, D)), rtol=0, atol=1e-14)


def pin_no_keys(o):
    q = np.ones((1, 3, 2, 4)); k = np.zeros((1, 0, 2, 4)); v = np.zeros((1, 0, 2, 4))
    out, lse = o.attention_forward(q, k, v)
    assert np.all(np.isneginf(lse)) and np.all(out == 0)
    dq, dk, dv = o.attention_backward(q, k, v, np.ones_like(q))
    assert np.all(dq == 0) and dk.shape == k.shape and dv.shape == v.shape


def pin_default_scale(o):
    # SDPA default scale is 1/sqrt(D) (diffusers issue, section Reproduction, reference call)
    r = _rng(4)
    q = r.standard_normal((1, 5, 1, 16)); k = r.standard_normal((1, 7, 1, 16)); v = r.standard_normal((1, 7, 1, 16))
    a, la = o.attention_forward(q, k, v)
    b, lb = o.attention_forward(q, k, v, scale=0.25)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ----------------------------------------------------------------------------- library routine
def _torch_sdpa(q, k, v, scale, dout):
    G = q.shape[2] // k.shape[2]
    qt = torch.tensor(q, dtype=torch.float64).transpose(1, 2).contiguous().requires_grad_(True)
    kt = torch.tensor(k, dtype=torch.float64).transpose(1, 2).contiguous().requires_grad_(True)
    vt = torch.tensor(v, dtype=torch.float64).transpose(1, 2).contiguous().requires_grad_(True)
    out = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=(G > 1))
    kr = kt.detach().repeat_interleave(G, dim=1)
    lse = torch.logsumexp(scale * (qt.detach() @ kr.transpose(-1, -2)), dim=-1)  # [B,H,S]
    dq, dk, dv = torch.autograd.grad(out, (qt, kt, vt), torch.tensor(dout).transpose(1, 2))
    tr = lambda t: t.detach().transpose(1, 2).numpy()
    return tr(out), lse.numpy(), tr(dq), tr(dk), tr(dv)


def pin_torch_sdpa(o):
    r = _rng(5)
    for (B, Sq, Sk, Hq, Hkv, D, scale) in [(2, 33, 47, 4, 4, 16, 0.25), (1, 40, 29, 6, 2, 8, None), (2, 17, 64, 8, 1, 32, 0.1)]:
        q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
        v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
        sc = scale if scale is not None else 1.0 / math.sqrt(D)
        t_out, t_lse, t_dq, t_dk, t_dv = _torch_sdpa(q, k, v, sc, d)
        out, lse = o.attention_forward(q, k, v, scale=scale)
        dq, dk, dv = o.attention_backward(q, k, v, d, scale=scale)
        assert _rel(out, t_out) < 1e-12, _rel(out, t_out)
        assert np.abs(lse - t_lse).max() < 1e-12
        for a, b in ((dq, t_dq), (dk, t_dk), (dv, t_dv)):
            assert _rel(a, b) < 1e-11, _rel(a, b)


# ----------------------------------------------------------------------------- finite differences
def pin_finite_differences(o):
    r = _rng(6)
    B, Sq, Sk, Hq, Hkv, D = 1, 5, 6, 4, 2, 3
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
    scale = 0.7

    def L(q_, k_, v_):
        return float((o.attention_forward(q_, k_, v_, scale=scale)[0] * d).sum())

    dq, dk, dv = o.attention_backward(q, k, v, d, scale=scale)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        base = args[which]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = base.copy(); plus[idx] += h
            minus = base.copy(); minus[idx] -= h
            ap = list(args); ap[which] = plus
            am = list(args); am[which] = minus
            fd[idx] = (L(*ap) - L(*am)) / (2 * h)
        assert _rel(grad, fd) < 1e-6, (which, _rel(grad, fd))


# ----------------------------------------------------------------------------- invariants
def _chunked_forward(o, q, k, v, lens, order, scale):
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    acc_out = np.zeros(q.shape); acc_lse = np.full((q.shape[0], q.shape[2], q.shape[1]), -np.inf)
    for j in order:
        sl = slice(starts[j], starts[j] + lens[j])
        po, pl = o.attention_forward(q, k[:, sl], v[:, sl], scale=scale)
        acc_out, acc_lse = o.merge_lse(acc_out, acc_lse, po, pl)
    return acc_out, acc_lse


def pin_chunk_merge_invariance(o):
    r = _rng(7)
    B, Sq, Sk, Hq, Hkv, D = 2, 11, 23, 4, 2, 8
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D)); v = r.standard_normal((B, Sk, Hkv, D))
    full_out, full_lse = o.attention_forward(q, k, v, scale=0.4)
    cases = [([12, 11], [0, 1]), ([8, 8, 7], [2, 0, 1]), ([5, 0, 18], [1, 2, 0]), ([23, 0], [1, 0]),
             ([3, 4, 5, 6, 5], [4, 3, 2, 1, 0]), ([1] * 23, list(range(22, -1, -1)))]
    for lens, order in cases:
        out, lse = _chunked_forward(o, q, k, v, lens, order, 0.4)
        assert np.abs(out - full_out).max() < 1e-12, (lens, order)
        assert np.abs(lse - full_lse).max() < 1e-12, (lens, order)


def pin_merge_closed_forms(o):
    r = _rng(8)
    oa = r.standard_normal((1, 4, 2, 3)); la = r.standard_normal((1, 2, 4))
    empty_o = np.zeros_like(oa); empty_l = np.full_like(la, -np.inf)
    out, lse = o.merge_lse(oa, la, empty_o, empty_l)
    assert np.array_equal(out, oa) and np.array_equal(lse, la)
    out, lse = o.merge_lse(empty_o, empty_l, oa, la)
    assert np.array_equal(out, oa) and np.array_equal(lse, la)
    out, lse = o.merge_lse(empty_o, empty_l, empty_o, empty_l)
    assert np.all(np.isneginf(lse)) and np.all(out == 0) and not np.any(np.isnan(out))
    out, lse = o.merge_lse(oa, la, oa, la)
    assert np.allclose(lse, la + math.log(2), rtol=0, atol=1e-14) and np.allclose(out, oa, rtol=0, atol=1e-14)
    # disjoint weights: a side with much larger lse dominates
    ob = r.standard_normal(oa.shape)
    out, lse = o.merge_lse(oa, la + 800.0, ob, la)
    assert np.allclose(out, oa, rtol=0, atol=1e-14)


def pin_gradient_invariants(o):
    r = _rng(9)
    B, Sq, Sk, Hq, Hkv, D = 2, 13, 17, 6, 3, 5
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
    dq, dk, dv = o.attention_backward(q, k, v, d, scale=0.5)
    # rows of dS sum to zero  =>  sum over keys of dK vanishes
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    # rows of P sum to one  =>  sum over keys of dV = sum over the group's queries of dO
    G = Hq // Hkv
    for g in range(Hkv):
        want = d[:, :, g * G:(g + 1) * G, :].sum(axis=(1, 2))
        assert np.allclose(dv[:, :, g, :].sum(axis=1), want, rtol=0, atol=1e-11)
    # adding the same vector c to every key adds scale*<q_i, c> to every score of row i:
    # the softmax, out and dQ are unchanged and lse moves by exactly that row constant
    c = r.standard_normal(D)
    out1, lse1 = o.attention_forward(q, k, v, scale=0.5)
    out2, lse2 = o.attention_forward(q, k + c, v, scale=0.5)
    assert np.abs(out1 - out2).max() < 1e-12
    shift = 0.5 * np.einsum("bshd,d->bhs", q, c)
    assert np.abs((lse2 - lse1) - shift).max() < 1e-12
    dq2, _, dv2 = o.attention_backward(q, k + c, v, d, scale=0.5)
    assert np.abs(dq2 - dq).max() < 1e-12 and np.abs(dv2 - dv).max() < 1e-12


def pin_gqa_group_sums(o):
    r = _rng(10)
    B, Sq, Sk, Hq, Hkv, D = 1, 9, 14, 8, 2, 6
    G = Hq // Hkv
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o_g, l_g = o.attention_forward(q, k, v)
    o_m, l_m = o.attention_forward(q, kr, vr)
    assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)
    dq_g, dk_g, dv_g = o.attention_backward(q, k, v, d)
    dq_m, dk_m, dv_m = o.attention_backward(q, kr, vr, d)
    assert np.abs(dq_g - dq_m).max() < 1e-13
    for g in range(Hkv):
        assert np.abs(dk_g[:, :, g] - dk_m[:, :, g * G:(g + 1) * G].sum(axis=2)).max() < 1e-13
        assert np.abs(dv_g[:, :, g] - dv_m[:, :, g * G:(g + 1) * G].sum(axis=2)).max() < 1e-13


def pin_rejects_bad_gqa(o):
    q = np.zeros((1, 2, 6, 4)); k = np.zeros((1, 2, 4, 4))
    try:
        o.attention_forward(q, k, k)
    except ValueError as e:
        assert golden()["gqa_divisibility_error"]["message"] in str(e)
        return
    raise AssertionError("H_q % H_kv != 0 must be refused")


def pin_delta_identity(o):
    """delta = rowsum(dout * out) equals rowsum(P * dP) with P from torch.softmax (library)."""
    r = _rng(14)
    B, Sq, Sk, Hq, Hkv, D = 2, 7, 9, 4, 2, 6
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
    out, _ = o.attention_forward(q, k, v, scale=0.3)
    delta = o.attention_delta(out, d)
    assert delta.shape == (B, Hq, Sq)
    qt = torch.tensor(q).transpose(1, 2); kt = torch.tensor(k).transpose(1, 2).repeat_interleave(2, dim=1)
    vt = torch.tensor(v).transpose(1, 2).repeat_interleave(2, dim=1); dt = torch.tensor(d).transpose(1, 2)
    P = torch.softmax(0.3 * qt @ kt.transpose(-1, -2), dim=-1)
    want = (P * (dt @ vt.transpose(-1, -2))).sum(-1).numpy()
    assert np.abs(delta - want).max() < 1e-12


# ----------------------------------------------------------------------------- exchange
def pin_split_sizes(o):
    assert o.split_sizes(1000, 3) == [334, 333, 333]   # the uneven workload's stated split
    assert o.split_sizes(8, 3) == [3, 3, 2]
    assert o.split_sizes(4608, 4) == [1152] * 4
    assert o.split_sizes(2, 4) == [1, 1, 0, 0]
    g = golden()["even_shard_rule"]
    sizes = o.split_sizes(g["S"], g["world"])
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    assert [[int(s), int(s + n)] for s, n in zip(starts, sizes)] == g["shards"]
    for n in range(0, 40):
        for p in range(1, 9):
            s = o.split_sizes(n, p)
            assert sum(s) == n and max(s) - min(s) <= 1 and s == sorted(s, reverse=True)


def _tag_shards(seq_lens, B, H, D):
    """Shards whose every element encodes its own (global row, b, head, d)."""
    S = sum(seq_lens)
    full = np.arange(S * B * H * D, dtype=np.float64).reshape(S, B, H, D)
    off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
    return full, [full[off[i]:off[i + 1]] for i in range(len(seq_lens))]


def pin_exchange_slot_rule(o):
    for seq_lens, heads in [([5, 5], [4, 4]), ([334, 333, 333], [3, 3, 2]), ([3, 2, 2, 1], [1, 2, 2, 3])]:
        B, D = 2, 3
        H = sum(heads)
        full, shards = _tag_shards(seq_lens, B, H, D)
        ys = o.seq_to_head(shards, heads)
        hoff = np.concatenate([[0], np.cumsum(heads)]).astype(int)
        soff = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
        for r, y in enumerate(ys):
            assert y.shape == (sum(seq_lens), B, heads[r], D)
            # slot i of rank r's output is the slot rank r owns in rank i's input
            for i in range(len(seq_lens)):
                assert np.array_equal(y[soff[i]:soff[i + 1]], shards[i][:, :, hoff[r]:hoff[r + 1], :])
            assert np.array_equal(y, full[:, :, hoff[r]:hoff[r + 1], :])
        back = o.head_to_seq(ys, seq_lens)
        for x, bk in zip(shards, back):
            assert np.array_equal(x, bk)


def pin_exchange_gradient_2x(o):
    """d/dx sum(exchange(x)**2) = 2x: the backward is the transposed exchange (head->seq)."""
    g = golden()["exchange_nonzero_gradient_counts"]
    n = g["elements_per_rank"]
    r = _rng(11)
    for R_str, want_nonzero in g["ranks_to_nonzero"].items():
        R = int(R_str)
        # dim-zero exchange of n elements per rank: one sequence row per rank, n elements split in R slots
        xs = [r.standard_normal((1, 1, n, 1)) for _ in range(R)]
        ys = o.seq_to_head(xs, [n // R] * R)
        grads = o.head_to_seq([2.0 * y for y in ys], [1] * R)
        nz = 0
        for x, gr in zip(xs, grads):
            assert np.array_equal(gr, 2.0 * x)
            nz += int(np.count_nonzero(gr))
        assert nz == want_nonzero
    # the same with explicit permutation matrices on a small uneven case (brute force)
    seq_lens, heads, B, D = [3, 2, 2], [2, 1, 1], 1, 2
    H = sum(heads)
    nel = sum(seq_lens) * B * H * D
    cols = []
    for e in range(nel):
        basis = np.zeros(nel); basis[e] = 1.0
        full = basis.reshape(sum(seq_lens), B, H, D)
        off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
        ys = o.seq_to_head([full[off[i]:off[i + 1]] for i in range(3)], heads)
        cols.append(np.concatenate([y.ravel() for y in ys]))
    P = np.stack(cols, axis=1)
    assert np.array_equal(P.T @ P, np.eye(nel))  # a permutation
    x = r.standard_normal(nel)
    assert np.array_equal(P.T @ (2 * (P @ x)), 2 * x)


def pin_page_exchange_shapes(o):
    g = golden()["ulysses_exchange_shapes"]
    R = g["ranks"]
    S_loc, B, H, D = g["local_shape_sbhd"]
    r = _rng(12)
    shards = [r.random((S_loc, B, H, D)) for _ in range(R)]
    ys = o.seq_to_head(shards, o.split_sizes(H, R))
    for y in ys:
        assert list(y.shape) == g["exchanged_shape_sbhd"]
    back = o.head_to_seq(ys, [S_loc] * R)
    for b in back:
        assert list(b.shape) == g["out_shape_sbhd"]


def pin_ulysses_composition(o):
    """exchange -> per-rank attention on its heads over the full sequence -> inverse
    equals direct attention, bit for bit (max abs diff 0.0 when both arms use the same
    local attention; DeepSpeed issue 'DistributedAttention ...', last comment)."""
    r = _rng(13)
    S, B, H, D = 20, 2, 8, 4
    for R in (2, 3):
        q, k, v = (r.standard_normal((S, B, H, D)) for _ in range(3))
        seq_lens, heads = o.split_sizes(S, R), o.split_sizes(H, R)
        off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
        sh = lambda x: [x[off[i]:off[i + 1]] for i in range(R)]
        qh, kh, vh = o.seq_to_head(sh(q), heads), o.seq_to_head(sh(k), heads), o.seq_to_head(sh(v), heads)
        outs = []
        for rr in range(R):
            bf = lambda x: np.ascontiguousarray(np.transpose(x, (1, 0, 2, 3)))
            out_b, _ = o.attention_forward(bf(qh[rr]), bf(kh[rr]), bf(vh[rr]))
            outs.append(np.ascontiguousarray(np.transpose(out_b, (1, 0, 2, 3))))
        got = np.concatenate(o.head_to_seq(outs, seq_lens), axis=0)
        bf = lambda x: np.ascontiguousarray(np.transpose(x, (1, 0, 2, 3)))
        direct_b, _ = o.attention_forward(bf(q), bf(k), bf(v))
        direct = np.transpose(direct_b, (1, 0, 2, 3))
        assert np.abs(got - direct).max() == golden()["ulysses_exchange_shapes"]["max_abs_diff_same_adapter"]


# ----------------------------------------------------------------------------- key mask
def _mask_case(seed, B, Sq, Sk, Hq, Hkv, D):
    r = _rng(seed)
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, D)); d = r.standard_normal((B, Sq, Hq, D))
    m = (r.random((B, Sk)) < 0.6).astype(np.uint8)
    m[:, 0] = 1  # every batch keeps at least one key (torch SDPA gives NaN otherwise)
    return q, k, v, d, m


def pin_mask_torch_sdpa(o):
    for seed, (B, Sq, Sk, Hq, Hkv, D, scale) in enumerate([(3, 9, 21, 4, 2, 8, 0.3), (2, 16, 40, 6, 6, 16, None)]):
        q, k, v, d, m = _mask_case(30 + seed, B, Sq, Sk, Hq, Hkv, D)
        sc = scale if scale is not None else 1.0 / math.sqrt(D)
        G = Hq // Hkv
        qt = torch.tensor(q).transpose(1, 2).contiguous().requires_grad_(True)
        kt = torch.tensor(k).transpose(1, 2).contiguous().requires_grad_(True)
        vt = torch.tensor(v).transpose(1, 2).contiguous().requires_grad_(True)
        am = torch.tensor(m.astype(bool))[:, None, None, :]  # True = attend
        out_t = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=sc, enable_gqa=(G > 1))
        sco = sc * (qt.detach() @ kt.detach().repeat_interleave(G, dim=1).transpose(-1, -2))
        lse_t = torch.logsumexp(sco.masked_fill(~am, float("-inf")), dim=-1)
        g_t = torch.autograd.grad(out_t, (qt, kt, vt), torch.tensor(d).transpose(1, 2))
        out, lse = o.attention_forward(q, k, v, scale=scale, kmask=m)
        dq, dk, dv = o.attention_backward(q, k, v, d, scale=scale, kmask=m)
        tr = lambda t: t.detach().transpose(1, 2).numpy()
        assert _rel(out, tr(out_t)) < 1e-12
        assert np.abs(lse - lse_t.numpy()).max() < 1e-12
        for a, b in ((dq, g_t[0]), (dk, g_t[1]), (dv, g_t[2])):
            assert _rel(a, tr(b)) < 1e-11, _rel(a, tr(b))


def pin_mask_single_valid_key(o):
    r = _rng(33)
    B, Sq, Sk, Hq, Hkv, D = 2, 6, 7, 4, 2, 5
    q = r.standard_normal((B, Sq, Hq, D)); k = r.standard_normal((B, Sk, Hkv, D)); v = r.standard_normal((B, Sk, Hkv, D))
    d = r.standard_normal(q.shape)
    m = np.zeros((B, Sk), np.uint8); m[0, 3] = 1; m[1, 5] = 1
    out, lse = o.attention_forward(q, k, v, scale=0.4, kmask=m)
    dq, dk, dv = o.attention_backward(q, k, v, d, scale=0.4, kmask=m)
    for b, j in ((0, 3), (1, 5)):
        for h in range(Hq):
            g = h // 2
            assert np.allclose(out[b, :, h, :], np.broadcast_to(v[b, j, g, :], (Sq, D)), rtol=0, atol=1e-14)
            assert np.allclose(lse[b, h, :], 0.4 * (q[b, :, h, :] @ k[b, j, g, :]), rtol=0, atol=1e-13)
        for g in range(Hkv):
            assert np.allclose(dv[b, j, g, :], d[b, :, 2 * g:2 * g + 2, :].sum(axis=(0, 1)), rtol=0, atol=1e-12)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    keep = np.zeros((B, Sk), bool); keep[0, 3] = keep[1, 5] = True
    assert np.all(dv[~keep] == 0)


def pin_mask_values_irrelevant(o):
    q, k, v, d, m = _mask_case(34, 2, 8, 15, 4, 2, 8)
    out, lse = o.attention_forward(q, k, v, kmask=m)
    grads = o.attention_backward(q, k, v, d, kmask=m)
    r = _rng(35)
    k2, v2 = k.copy(), v.copy()
    k2[m == 0] = 1e3 * r.standard_normal(k2[m == 0].shape); v2[m == 0] = r.standard_normal(v2[m == 0].shape)
    out2, lse2 = o.attention_forward(q, k2, v2, kmask=m)
    grads2 = o.attention_backward(q, k2, v2, d, kmask=m)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    for a, b in zip(grads, grads2):
        assert np.array_equal(a, b)
    assert np.all(grads[1][m == 0] == 0) and np.all(grads[2][m == 0] == 0)
    # all-ones mask = no mask
    ones = np.ones_like(m)
    a, la = o.attention_forward(q, k, v, kmask=ones)
    b, lb = o.attention_forward(q, k, v)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def pin_mask_no_valid_key(o):
    q, k, v, d, m = _mask_case(36, 3, 5, 9, 2, 1, 4)
    m[1, :] = 0
    out, lse = o.attention_forward(q, k, v, kmask=m)
    dq, dk, dv = o.attention_backward(q, k, v, d, kmask=m)
    assert np.all(np.isneginf(lse[1])) and np.all(out[1] == 0)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    assert np.all(np.isfinite(lse[[0, 2]])) and not np.any(np.isnan(out))
    # the other batches match a run without batch 1
    sel = [0, 2]
    o2, l2 = o.attention_forward(q[sel], k[sel], v[sel], kmask=m[sel])
    assert np.array_equal(o2, out[sel]) and np.array_equal(l2, lse[sel])


def pin_mask_finite_differences(o):
    q, k, v, d, m = _mask_case(37, 1, 4, 6, 2, 1, 3)
    m[0] = [1, 0, 1, 1, 0, 1]
    scale = 0.8

    def L(q_, k_, v_):
        return float((o.attention_forward(q_, k_, v_, scale=scale, kmask=m)[0] * d).sum())

    grads = o.attention_backward(q, k, v, d, scale=scale, kmask=m)
    h = 1e-6
    for which, grad in enumerate(grads):
        args = [q, k, v]
        base = args[which]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = base.copy(); plus[idx] += h
            minus = base.copy(); minus[idx] -= h
            ap = list(args); ap[which] = plus
            am = list(args); am[which] = minus
            fd[idx] = (L(*ap) - L(*am)) / (2 * h)
        assert _rel(grad, fd) < 1e-6, (which, _rel(grad, fd))


def pin_mask_chunk_merge(o):
    q, k, v, d, m = _mask_case(38, 2, 7, 20, 2, 2, 4)
    m[0, 8:15] = 0  # the second chunk is fully masked for batch 0
    full_out, full_lse = o.attention_forward(q, k, v, scale=0.5, kmask=m)
    lens, order = [8, 7, 5], [1, 2, 0]
    starts = [0, 8, 15]
    acc_out = np.zeros(q.shape); acc_lse = np.full((q.shape[0], q.shape[2], q.shape[1]), -np.inf)
    for j in order:
        sl = slice(starts[j], starts[j] + lens[j])
        po, pl = o.attention_forward(q, k[:, sl], v[:, sl], scale=0.5, kmask=m[:, sl])
        acc_out, acc_lse = o.merge_lse(acc_out, acc_lse, po, pl)
    assert np.abs(acc_out - full_out).max() < 1e-12 and np.abs(acc_lse - full_lse).max() < 1e-12


ALL_PINS = [
    pin_mask_torch_sdpa, pin_mask_single_valid_key, pin_mask_values_irrelevant, pin_mask_no_valid_key,
    pin_mask_finite_differences, pin_mask_chunk_merge,
    pin_single_key, pin_zero_query, pin_equal_keys, pin_no_keys, pin_default_scale,
    pin_torch_sdpa, pin_finite_differences, pin_chunk_merge_invariance, pin_merge_closed_forms,
    pin_gradient_invariants, pin_gqa_group_sums, pin_rejects_bad_gqa, pin_delta_identity,
    pin_split_sizes, pin_exchange_slot_rule, pin_exchange_gradient_2x, pin_page_exchange_shapes,
    pin_ulysses_composition,
]
