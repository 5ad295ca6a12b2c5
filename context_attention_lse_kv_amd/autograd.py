"""Differentiable, torch.compile-safe entry points of the ring-attention library.

DeepSpeed PR "_DimZeroAllToAll silently fails to send grads under torch.compile": a
sequence/head exchange written as a torch.autograd.Function whose forward fills a
pre-allocated buffer through an operation that writes into an output argument lost
its gradient under torch.compile - the tracer inlines the function's body and sees no
data dependence between input and output, so the hand-written backward never ran.
The fix there is an exchange that returns its result.

Here every differentiable call is a ``torch.library`` custom op that RETURNS fresh
tensors (``mutates_args=()``: no argument is written), with a fake implementation
that gives only shapes for tracing and a registered backward that is itself a custom
op.  Compiled graphs keep these ops as opaque nodes, so the input-output dependence
and the backward survive compilation.  The ops only marshal arguments into the HIP
library (``ops``); every step of the computation runs in its kernels.

The log-sum-exp returned by ``ring_attention(..., return_lse=True)`` is an auxiliary
output and is not differentiable (it is marked so; a loss that uses it receives no
gradient through it).
"""
import math
from typing import List, Optional, Tuple

import torch

from . import ops

Tensor = torch.Tensor


def _dims(q, layout):
    if layout == "bshd":
        B, S, H, _ = q.shape
    else:
        S, B, H, _ = q.shape
    return B, S, H


# ------------------------------------------------------------------ attention
@torch.library.custom_op("ra::ring_attn_fwd", mutates_args=())
def _ring_attn_fwd(q: Tensor, k: Tensor, v: Tensor, lens: List[int], order: List[int], scale: float,
                   kmask: Optional[Tensor], layout: str, bwd_ws: int) -> Tuple[Tensor, Tensor]:
    out, lse = ops.ring_fwd(q, k, v, ops.Chunks(lens, order), scale=scale, layout=layout, kmask=kmask)
    return out, lse


@_ring_attn_fwd.register_fake
def _ring_attn_fwd_fake(q, k, v, lens, order, scale, kmask, layout, bwd_ws):
    B, Sq, H = _dims(q, layout)
    return q.new_empty(q.shape), q.new_empty((B, H, Sq), dtype=torch.float32)


@torch.library.custom_op("ra::ring_attn_bwd", mutates_args=())
def _ring_attn_bwd(q: Tensor, k: Tensor, v: Tensor, out: Tensor, dout: Tensor, lse: Tensor, lens: List[int],
                   order: List[int], scale: float, kmask: Optional[Tensor], layout: str,
                   bwd_ws: int) -> Tuple[Tensor, Tensor, Tensor]:
    ws = None
    if bwd_ws > 0:
        # a cap on the backward's workspace: the library plans its sweep from the room it gets
        # (never below the size it accepts with any chunk table)
        lo = ops.ring_bwd_workspace_bytes(q, k, layout=layout, minimum=True)
        hi = ops.ring_bwd_workspace_bytes(q, k, layout=layout)
        n = max(lo, min(hi, int(bwd_ws)))
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)[:n] if n else None
    dq, dk, dv = ops.ring_bwd(q, k, v, out, dout, lse, ops.Chunks(lens, order), scale=scale, layout=layout,
                              kmask=kmask, workspace=ws)
    return dq, dk, dv


@_ring_attn_bwd.register_fake
def _ring_attn_bwd_fake(q, k, v, out, dout, lse, lens, order, scale, kmask, layout, bwd_ws):
    return q.new_empty(q.shape), k.new_empty(k.shape), v.new_empty(v.shape)


def _ring_attn_setup(ctx, inputs, output):
    q, k, v, lens, order, scale, kmask, layout, bwd_ws = inputs
    out, lse = output
    ctx.save_for_backward(q, k, v, out, lse, kmask)
    ctx.args = (list(lens), list(order), float(scale), layout, int(bwd_ws))
    ctx.mark_non_differentiable(lse)


def _ring_attn_backward(ctx, grad_out, grad_lse):
    q, k, v, out, lse, kmask = ctx.saved_tensors
    lens, order, scale, layout, bwd_ws = ctx.args
    # the kernels need D contiguous; an incoming gradient may be a broadcast view
    dq, dk, dv = _ring_attn_bwd(q, k, v, out, grad_out.contiguous(), lse, lens, order, scale, kmask, layout,
                                bwd_ws)
    return dq, dk, dv, None, None, None, None, None, None


torch.library.register_autograd("ra::ring_attn_fwd", _ring_attn_backward, setup_context=_ring_attn_setup)


def ring_attention(q, k, v, chunks, scale=None, kmask=None, layout="bshd", return_lse=False,
                   bwd_workspace_bytes=0):
    """Ring attention of the query shard ``q`` over the chunks of (k, v), differentiable
    in q, k, v (backward: one chunk step per forward step, each against its own chunk).

    ``chunks``: an ``ops.Chunks`` or a list of chunk lengths (swept in order).  A single
    chunk covering the whole key sequence is the all-gather variant: one fused sweep
    with no per-step merge.  ``kmask``: optional key-validity mask [B, S_k].
    ``bwd_workspace_bytes``: a cap on the device workspace the backward allocates (0: the
    size at which it runs fastest, up to 8 GiB of stored dS); with less room the backward
    groups fewer chunks per dQ pass, sweeps query-row slices or recomputes, with the same
    result up to rounding.  Never below the minimum the library accepts.
    """
    # plain lists only here (no ctypes objects), so that a compiled graph traces through
    if isinstance(chunks, ops.Chunks):
        lens, order = list(chunks.lens), list(chunks.order)
    else:
        lens = [int(n) for n in chunks]
        order = list(range(len(lens)))
    sc = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    out, lse = _ring_attn_fwd(q, k, v, lens, order, sc, kmask, layout, int(bwd_workspace_bytes))
    return (out, lse) if return_lse else out


# ------------------------------------------------------------------ Ulysses exchange
@torch.library.custom_op("ra::seq_head_exchange", mutates_args=())
def _exchange(xs: List[Tensor], sizes: List[int], direction: int, layout: str) -> List[Tensor]:
    if direction == 0:
        return list(ops.seq_to_head(list(xs), list(sizes), layout))
    return list(ops.head_to_seq(list(xs), list(sizes), layout))


@_exchange.register_fake
def _exchange_fake(xs, sizes, direction, layout):
    x0 = xs[0]
    sd = 1 if layout == "bshd" else 0
    outs = []
    if direction == 0:  # sizes = head counts; every output spans the whole sequence
        S = sum(x.shape[sd] for x in xs)
        for h in sizes:
            shape = list(x0.shape)
            shape[sd], shape[2] = S, h
            outs.append(x0.new_empty(shape))
    else:  # sizes = sequence lengths; every output has all heads
        H = sum(x.shape[2] for x in xs)
        for s in sizes:
            shape = list(x0.shape)
            shape[sd], shape[2] = s, H
            outs.append(x0.new_empty(shape))
    return outs


def _exchange_setup(ctx, inputs, output):
    xs, sizes, direction, layout = inputs
    sd = 1 if layout == "bshd" else 0
    # the inverse exchange needs the sizes the forward's inputs had along the split axis
    ctx.inv = ([int(x.shape[sd]) for x in xs] if direction == 0 else [int(x.shape[2]) for x in xs],
               1 - direction, layout)


def _exchange_backward(ctx, grads):
    sizes, direction, layout = ctx.inv
    return _exchange([g.contiguous() for g in grads], sizes, direction, layout), None, None, None


torch.library.register_autograd("ra::seq_head_exchange", _exchange_backward, setup_context=_exchange_setup)


def seq_to_head_exchange(shards, head_counts, layout="sbhd"):
    """Differentiable seq->head exchange of R simulated ranks (returns new tensors; its
    backward is the head->seq exchange of the gradients)."""
    return _exchange(list(shards), [int(h) for h in head_counts], 0, layout)


def head_to_seq_exchange(parts, seq_lens, layout="sbhd"):
    """Differentiable head->seq exchange (inverse of ``seq_to_head_exchange``)."""
    return _exchange(list(parts), [int(s) for s in seq_lens], 1, layout)
