"""fp64 full-sequence softmax attention, its analytic backward, and the LSE merge.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed and where the pages fix it:

* [P1] "Root cause": ring attention keeps Q local while K/V chunks rotate; the
  attention op of each ring step returns an output together with its
  log-sum-exp, and [P1] "How it surfaces per backend" (table, ``native`` row)
  states that ring needs that LSE to merge partial results.
* [P1] "Reproduction": the reference every CP result is compared against is a
  single-process full-sequence softmax attention (SDPA, default scale
  1/sqrt(D), no mask, no dropout, non-causal) and its autograd gradients.
  This oracle is that reference written out in fp64: it has no chunks, no ring
  and no merge inside the forward/backward.
* [P1] "Expected behavior": ring backward gradients must equal the gradients of
  that full-sequence reference.
* [P1] "How it surfaces per backend" (``_native_flash`` row) and [P2] (GQA
  example, 24 query / 4 key-value heads): the number of key/value heads
  divides the number of query heads.  Reading taken: query head h uses
  key/value head h // (H_q / H_kv) (contiguous groups).

* [P3] (comments on padding tokens to a divisible length): padding changes
  the result because padded tokens are attended, and a mask is the proposed
  way out.  Reading taken: an optional key-validity mask ``kmask`` [B, S_k]
  (nonzero = the key takes part) removes masked keys from every softmax of
  that batch; a batch with no valid key behaves like an empty key set
  (lse = -inf, out = 0, zero gradients), and masked keys get dK = dV = 0.

Layouts: q, dout, out are [B, S_q, H_q, D]; k, v are [B, S_k, H_kv, D]
(batch-first as in [P1] "Reproduction"); lse is [B, H_q, S_q], natural log.
Inputs are any real arrays; they are upcast to float64.

Rows of the query are independent of each other in this definition, so the
functions may process query rows in groups (``row_block``) purely to bound
memory; each row's arithmetic is the same whatever the group size.
"""
import numpy as np


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, _, Hq, D = q.shape
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("batch and head dim of q and k/v must agree")
    Hkv = k.shape[2]
    if Hkv == 0 or Hq % Hkv != 0:
        # same condition as the error text quoted in [P1] "How it surfaces per backend"
        raise ValueError("Number of heads in key/value must divide number of heads in query")
    return B, Hq, Hkv, Hq // Hkv


def _key_sets(kmask, B, Sk):
    """Indices of the keys each batch attends to (all keys without a mask)."""
    if kmask is None:
        return [np.arange(Sk)] * B
    kmask = np.asarray(kmask)
    if kmask.shape != (B, Sk):
        raise ValueError("kmask must be [B, S_k]")
    return [np.flatnonzero(kmask[b]) for b in range(B)]


def attention_forward(q, k, v, scale=None, row_block=4096, kmask=None):
    """Full softmax attention of every query row against every (valid) key.

    For each batch b, query head h (key/value head g = h // G) and query row i:
        s_ij   = scale * <q_i, k_j>
        lse_i  = log(sum_j exp(s_ij))                (natural log)
        out_i  = sum_j exp(s_ij - lse_i) * v_j
    j runs over the keys of batch b that ``kmask`` keeps (all keys without it).
    With no keys (S_k = 0, or all masked) the softmax is empty: lse = -inf and
    out = 0, which is the identity element of the LSE merge below.
    Returns (out [B,S_q,H_q,D] float64, lse [B,H_q,S_q] float64).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Hkv, G = _check_shapes(q, k, v)
    Sq, D, Sk = q.shape[1], q.shape[3], k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    keys = _key_sets(kmask, B, Sk)
    if Sk == 0 or Sq == 0:
        return out, lse
    for b in range(B):
        if keys[b].size == 0:
            continue
        for h in range(Hq):
            g = h // G
            kg, vg = k[b, keys[b], g, :], v[b, keys[b], g, :]
            for r0 in range(0, Sq, row_block):
                rows = slice(r0, min(Sq, r0 + row_block))
                s = scale * (q[b, rows, h, :] @ kg.T)
                m = s.max(axis=1)
                l_row = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                p = np.exp(s - l_row[:, None])
                out[b, rows, h, :] = p @ vg
                lse[b, h, rows] = l_row
    return out, lse


def attention_backward(q, k, v, dout, scale=None, row_block=4096, kmask=None):
    """Analytic gradients of L = sum(dout * out) for ``attention_forward``.

    Softmax-Jacobian form, per (b, h, g = h // G) and rows:
        P   = exp(s - lse)
        dV += P^T dO
        dP  = dO V^T
        dS  = P * (dP - rowsum(P * dP))
        dQ  = scale * dS K
        dK += scale * dS^T Q
    dK and dV of a key/value head sum the contributions of every query head
    of its group; with ``kmask`` the sums run over the valid keys only and
    masked keys get zero dK and dV.  Returns (dq, dk, dv) in float64 with the
    shapes of q, k, v.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, Hq, Hkv, G = _check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    Sq, D, Sk = q.shape[1], q.shape[3], k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    keys = _key_sets(kmask, B, Sk)
    if Sk == 0 or Sq == 0:
        return dq, dk, dv
    for b in range(B):
        kb = keys[b]
        if kb.size == 0:
            continue
        for h in range(Hq):
            g = h // G
            kg, vg = k[b, kb, g, :], v[b, kb, g, :]
            for r0 in range(0, Sq, row_block):
                rows = slice(r0, min(Sq, r0 + row_block))
                qr, dor = q[b, rows, h, :], dout[b, rows, h, :]
                s = scale * (qr @ kg.T)
                m = s.max(axis=1)
                l_row = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                p = np.exp(s - l_row[:, None])
                dv[b, kb, g, :] += p.T @ dor
                dp = dor @ vg.T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, rows, h, :] = scale * (ds @ kg)
                dk[b, kb, g, :] += scale * (ds.T @ qr)
    return dq, dk, dv


def attention_delta(out, dout):
    """Per-row dot product of the output gradient with the output, [B, H, S].

    delta_i = sum_d dout_id * out_id.  For out = attention_forward(q, k, v) this
    equals rowsum(P * dP) of ``attention_backward`` (since out_i = sum_j P_ij v_j
    and dP_ij = <dout_i, v_j>), which is how the backward consumes it.
    """
    out, dout = _as64(out), _as64(dout)
    if out.shape != dout.shape or out.ndim != 4:
        raise ValueError("out and dout must both be [B, S, H, D]")
    return np.transpose((out * dout).sum(axis=3), (0, 2, 1)).copy()


def merge_lse(out_a, lse_a, out_b, lse_b):
    """Merge two partial attention results over disjoint key sets.

    [P1] "How it surfaces per backend": ring needs each step's LSE to merge
    partial results.  With lse = log(exp(lse_a) + exp(lse_b)), the merged
    output is the softmax-weighted combination
        out = exp(lse_a - lse) * out_a + exp(lse_b - lse) * out_b.
    A side with lse = -inf (no keys) contributes nothing; both sides -inf give
    lse = -inf and out = 0.
    out_* are [B,S,H,D]; lse_* are [B,H,S].
    """
    out_a, lse_a, out_b, lse_b = map(_as64, (out_a, lse_a, out_b, lse_b))
    with np.errstate(invalid="ignore"):
        lse = np.logaddexp(lse_a, lse_b)
    both_empty = np.isneginf(lse_a) & np.isneginf(lse_b)
    safe = np.where(both_empty, 0.0, lse)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - safe))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - safe))
    # weights are [B,H,S]; outputs are [B,S,H,D]
    wa = np.transpose(wa, (0, 2, 1))[..., None]
    wb = np.transpose(wb, (0, 2, 1))[..., None]
    out = wa * out_a + wb * out_b
    lse = np.where(both_empty, -np.inf, lse)
    return out, lse
