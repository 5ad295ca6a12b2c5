"""Sequence <-> head exchange of Ulysses-style sequence parallelism, as index slicing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P4] "Testcase": ``DistributedAttention`` exchanges q, k, v with the
sequence-head all-to-all (scatter the head axis, gather the sequence axis) on
sequence-first tensors [S, B, H, D], runs attention locally on the full
sequence with a subset of heads, and exchanges the output back (gather the head
axis, scatter the sequence axis).  [P2] "Testing" fixes what an exchange
delivers: slot i of a rank's output holds the slot that this rank owns in rank
i's input.  On one device all R simulated ranks are present, so the exchange
is a permutation of the stacked data:

  seq->head: input of rank i is x_i [s_i, B, H, D] (its sequence shard);
             output of rank r is y_r [S, B, h_r, D] with
             y_r[off_i + t, b, c, d] = x_i[t, b, hoff_r + c, d].
  head->seq: the inverse.

Uneven splits ([P4] "Describe the bug": S not divisible by world size) follow
``split_sizes``.
"""
import numpy as np


def split_sizes(n, parts):
    """Sizes of ``parts`` consecutive pieces of ``n`` items, the first n % parts one larger.

    This is the reading taken for uneven sequence and head splits (the rule of
    ``torch.tensor_split``): 1000 over 3 gives 334/333/333, 8 over 3 gives 3/3/2.
    Pieces may be empty when parts > n.
    """
    if parts <= 0 or n < 0:
        raise ValueError("need parts > 0 and n >= 0")
    base, extra = divmod(n, parts)
    return [base + (1 if i < extra else 0) for i in range(parts)]


def _offsets(sizes):
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
    return off


def seq_to_head(shards, head_counts):
    """shards: list of R arrays [s_i, B, H, D]; returns list of R arrays [S, B, h_r, D]."""
    R = len(shards)
    if len(head_counts) != R:
        raise ValueError("one head count per rank")
    H = shards[0].shape[2]
    if sum(head_counts) != H:
        raise ValueError("head counts must sum to H")
    hoff = _offsets(head_counts)
    out = []
    for r in range(R):
        pieces = [x[:, :, hoff[r]:hoff[r + 1], :] for x in shards]
        out.append(np.concatenate(pieces, axis=0))
    return out


def head_to_seq(parts, seq_lens):
    """parts: list of R arrays [S, B, h_r, D]; returns list of R arrays [s_i, B, H, D]."""
    R = len(parts)
    if len(seq_lens) != R:
        raise ValueError("one sequence length per rank")
    S = parts[0].shape[0]
    if sum(seq_lens) != S:
        raise ValueError("sequence lengths must sum to S")
    soff = _offsets(seq_lens)
    out = []
    for i in range(R):
        pieces = [y[soff[i]:soff[i + 1]] for y in parts]
        out.append(np.concatenate(pieces, axis=2))
    return out
