"""Differentiable custom ops (``ring_attention`` and the Ulysses exchange) on the GPU:
eager autograd against the ring backward and the oracle, and torch.compile against
eager.  The compiled Ulysses composition reproduces the situation of the DeepSpeed PR
"_DimZeroAllToAll silently fails to send grads under torch.compile" (an exchange inside
a compiled region) and requires the gradient to survive compilation unchanged.
Compiled graphs use the ``aot_eager`` backend: the tracing (dynamo + AOT autograd) is
what that PR's defect lives in, and no kernels are generated for it."""
import numpy as np
import pytest
import torch

import context_attention_lse_kv_amd as ra
import oracle
import workloads as W
from parity import BF16_TOL, check_bf16, LSE_TOL_BF16, dev, max_abs, np64, rel

pytestmark = pytest.mark.gpu


def _leaves(*ts):
    d = dev()
    return [t.to(d).requires_grad_(True) for t in ts]


def _grads(fn, leaves, dout):
    for t in leaves:
        t.grad = None
    out = fn(*leaves)
    outs = out if isinstance(out, (list, tuple)) else [out]
    douts = dout if isinstance(dout, (list, tuple)) else [dout]
    loss = sum((o.float() * d).sum() for o, d in zip(outs, douts))
    loss.backward()
    return [o.detach() for o in outs], [t.grad.detach().clone() for t in leaves]


def test_autograd_matches_ring_bwd_and_oracle():
    B, S, Sq, Hq, Hkv, D = 2, 512, 256, 8, 2, 128
    q, k, v, do = (W.randn(s, 1100 + i, "bf16") for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                        (B, S, Hkv, D), (B, Sq, Hq, D)]))
    ch = ra.Chunks((256, 256), (1, 0))
    gdo = do.to(dev()).float()
    (out,), grads = _grads(lambda a, b, c: ra.ring_attention(a, b, c, ch), _leaves(q, k, v), gdo)
    # the same kernels through the plain binding
    gq, gk, gv = (t.to(dev()) for t in (q, k, v))
    out_r, lse_r = ra.ring_fwd(gq, gk, gv, ch)
    dq_r, dk_r, dv_r = ra.ring_bwd(gq, gk, gv, out_r, do.to(dev()), lse_r, ch)
    assert torch.equal(out, out_r)
    for a, b in zip(grads, (dq_r, dk_r, dv_r)):
        assert torch.equal(a, b)
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    o, _ = oracle.attention_forward(qn, kn, vn)
    g = oracle.attention_backward(qn, kn, vn, don)
    check_bf16('out', np64(out), o)
    for a, b in zip(grads, g):
        check_bf16('grad', np64(a), b)


def test_autograd_backward_workspace_cap():
    """``bwd_workspace_bytes`` caps the backward's workspace: at the minimum every chunk takes
    the recompute route, with room for one chunk's dS the chunks run one dQ pass each; both
    give the gradients of the uncapped backward up to rounding, and the oracle's."""
    B, S, Sq, Hq, Hkv, D = 2, 600, 200, 8, 2, 64
    q, k, v, do = (W.randn(s, 1120 + i, "bf16") for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                        (B, S, Hkv, D), (B, Sq, Hq, D)]))
    ch = ra.Chunks((200, 200, 200), (1, 0, 2))
    gdo = do.to(dev()).float()
    gq, gk = q.to(dev()), k.to(dev())
    lo = ra.ring_bwd_workspace_bytes(gq, gk, minimum=True)
    one = lo + ra.bwd_ds_bytes(gq, gk[:, :200]) + 4096
    assert ra.ring_bwd_plan(gq, gk, ch, lo)["rows"] == [0, 0, 0]
    assert ra.ring_bwd_plan(gq, gk, ch, one)["accumulators"] == ["dq"]
    _, full = _grads(lambda a, b, c: ra.ring_attention(a, b, c, ch), _leaves(q, k, v), gdo)
    qn, kn, vn, don = (np64(t) for t in (q, k, v, do))
    g = oracle.attention_backward(qn, kn, vn, don)
    for cap in (1, one):
        _, capped = _grads(lambda a, b, c: ra.ring_attention(a, b, c, ch, bwd_workspace_bytes=cap),
                           _leaves(q, k, v), gdo)
        for a, b, r in zip(capped, full, g):
            assert rel(np64(a), np64(b)) <= 5e-3
            check_bf16(f"grad (cap {cap})", np64(a), r)


@pytest.mark.parametrize("masked", [False, True])
def test_compiled_equals_eager(masked):
    B, S, Sq, Hq, Hkv, D = 2, 384, 192, 4, 2, 64
    q, k, v, do = (W.randn(s, 1110 + i, "bf16") for i, s in enumerate([(B, Sq, Hq, D), (B, S, Hkv, D),
                                                                        (B, S, Hkv, D), (B, Sq, Hq, D)]))
    m = W.make_key_mask(B, S, 1115, p_keep=0.8).to(dev()) if masked else None
    ch = ra.Chunks((128, 128, 128), (2, 1, 0))
    gdo = do.to(dev()).float()

    def fn(a, b, c):
        return ra.ring_attention(a, b, c, ch, kmask=m)

    (oe,), ge = _grads(fn, _leaves(q, k, v), gdo)
    torch._dynamo.reset()
    cfn = torch.compile(fn, backend="aot_eager", fullgraph=True)
    (oc,), gc = _grads(cfn, _leaves(q, k, v), gdo)
    assert torch.equal(oe, oc)
    for a, b in zip(ge, gc):
        assert torch.equal(a, b)
        assert a.abs().sum() > 0


def test_compiled_ulysses_exchange_keeps_gradients():
    """Seq-first shards of R = 3 simulated ranks (334/333/333 rows; heads 3/3/2):
    exchange seq->head, attention per head group over the whole sequence (swept over
    chunks 334/333/333), exchange head->seq.  Compiled gradients must equal eager ones
    and the oracle's full-sequence gradients."""
    w = W.UNEVEN_SEQFIRST
    q, k, v, do = W.make_inputs(w)            # [S, B, H, D]
    seq = ra.split_sizes(w.S, 3)
    heads = ra.split_sizes(w.Hq, 3)
    cut = lambda t: list(torch.split(t, seq, dim=0))
    qs, ks, vs, dos = cut(q), cut(k), cut(v), cut(do)
    gdo = [x.to(dev()).float() for x in dos]

    def model(*flat):
        R = len(seq)
        qx = ra.seq_to_head_exchange(list(flat[:R]), heads)
        kx = ra.seq_to_head_exchange(list(flat[R:2 * R]), heads)
        vx = ra.seq_to_head_exchange(list(flat[2 * R:]), heads)
        outs = [ra.ring_attention(qx[r], kx[r], vx[r], seq, layout="sbhd") for r in range(R)]
        return ra.head_to_seq_exchange(outs, seq)

    oe, ge = _grads(model, _leaves(*qs, *ks, *vs), gdo)
    torch._dynamo.reset()
    cmodel = torch.compile(model, backend="aot_eager", fullgraph=True)
    oc, gc = _grads(cmodel, _leaves(*qs, *ks, *vs), gdo)
    for a, b in zip(oe + ge, oc + gc):
        assert torch.equal(a, b)
    for g in gc:
        assert g.abs().sum() > 0  # the defect of the page: compiled gradients were exactly zero
    # oracle: full-sequence attention in [B, S, H, D]
    to_b = lambda t: np.transpose(np64(t), (1, 0, 2, 3))
    o, _ = oracle.attention_forward(to_b(q), to_b(k), to_b(v))
    gq, gk, gv = oracle.attention_backward(to_b(q), to_b(k), to_b(v), to_b(do))
    cat = lambda ts: np.transpose(np64(torch.cat(ts, dim=0)), (1, 0, 2, 3))
    R = len(seq)
    check_bf16('out', cat(oc), o)
    check_bf16('dq', cat(gc[:R]), gq)
    check_bf16('dk', cat(gc[R:2 * R]), gk)
    check_bf16('dv', cat(gc[2 * R:]), gv)


def test_allgather_single_chunk_sweep():
    """The all-gather-K/V variant (one fused sweep over the resident key sequence, no
    per-step merge) agrees with the 8-chunk ring and with the oracle."""
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w, Sq=1024)
    gq, gk, gv, gdo = (t.to(dev()) for t in (q, k, v, do))
    one = ra.Chunks([w.S])
    ring = ra.Chunks(lens, ra.ring_order(w.n_chunks, 0))
    o1, l1 = ra.ring_fwd(gq, gk, gv, one)
    g1 = ra.ring_bwd(gq, gk, gv, o1, gdo, l1, one)
    o8, l8 = ra.ring_fwd(gq, gk, gv, ring)
    g8 = ra.ring_bwd(gq, gk, gv, o8, gdo, l8, ring)
    assert rel(np64(o1), np64(o8)) <= BF16_TOL and max_abs(np64(l1), np64(l8)) <= LSE_TOL_BF16
    for a, b in zip(g1, g8):
        assert rel(np64(a), np64(b)) <= BF16_TOL
    qn, kn, vn, don = (np64(t) for t in (q[:, :, :4], k[:, :, :1], v[:, :, :1], do[:, :, :4]))
    o, l = oracle.attention_forward(qn, kn, vn)
    gq_, gk_, gv_ = oracle.attention_backward(qn, kn, vn, don)
    check_bf16('out', np64(o1[:, :, :4]), o)
    assert max_abs(np64(l1[:, :4]), l) <= LSE_TOL_BF16
    check_bf16('dq', np64(g1[0][:, :, :4]), gq_)
    # dK/dV of kv head 0 receive the sum over its 4 query heads, all included above
    check_bf16('dk', np64(g1[1][:, :, :1]), gk_)
    check_bf16('dv', np64(g1[2][:, :, :1]), gv_)
