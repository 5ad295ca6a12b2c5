"""Python binding of the ring-attention library on torch tensors.

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the HIP kernels behind the C ABI
(include/ra.h).  Layouts are described by strides, never copied: ``layout``
"bshd" means the tensor is indexed [B, S, H, D], "sbhd" means [S, B, H, D]
(sequence-first, as in the DeepSpeed DistributedAttention issue's testcase).
"""
import ctypes
import math

import torch

from . import _abi
from ._abi import RaChunks, RaKMask, RaLse, RaTensor, check, lib

_DT = {torch.bfloat16: _abi.RA_BF16, torch.float32: _abi.RA_F32}


def _dev_check(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("ring attention runs on the GPU only: every tensor must be on a HIP device")


def tensor_desc(t, layout="bshd"):
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    if t.dtype not in _DT:
        raise ValueError(f"dtype {t.dtype} not supported (bf16 or fp32)")
    if t.stride(3) != 1:
        raise ValueError("the head dim D must be contiguous (stride 1)")
    if layout == "bshd":
        B, S, H, D = t.shape
        sB, sS, sH = t.stride(0), t.stride(1), t.stride(2)
    elif layout == "sbhd":
        S, B, H, D = t.shape
        sB, sS, sH = t.stride(1), t.stride(0), t.stride(2)
    else:
        raise ValueError("layout must be 'bshd' or 'sbhd'")
    return RaTensor(t.data_ptr(), _DT[t.dtype], B, S, H, D, sB, sS, sH)


def rows_desc(t):
    """fp32 [B, H, S] statistic (LSE or delta)."""
    if t.dim() != 3 or t.dtype != torch.float32 or (t.numel() > 0 and t.stride(2) != 1):
        raise ValueError("row statistics are fp32 [B, H, S] with S contiguous")
    return RaLse(t.data_ptr(), t.shape[0], t.shape[1], t.shape[2], t.stride(0), t.stride(1))


def kmask_desc(m):
    """Key-validity mask [B, S_k] (bool or uint8 on the GPU, S contiguous; nonzero = the key
    takes part), or None."""
    if m is None:
        return None
    if m.dim() != 2 or m.dtype not in (torch.bool, torch.uint8) or (m.numel() > 0 and m.stride(1) != 1):
        raise ValueError("kmask is a bool/uint8 [B, S_k] tensor with S contiguous")
    if not m.is_cuda:
        raise ValueError("kmask must be on the GPU")
    return ctypes.byref(RaKMask(m.data_ptr(), m.shape[0], m.shape[1], m.stride(0)))


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _arr(xs):
    return (ctypes.c_int32 * len(xs))(*[int(x) for x in xs])


def split_sizes(n, parts):
    out = (ctypes.c_int32 * parts)()
    check(lib().ra_split_sizes(n, parts, out), "ra_split_sizes")
    return list(out)


def ring_order(R, rank):
    out = (ctypes.c_int32 * R)()
    check(lib().ra_ring_order(R, rank, out), "ra_ring_order")
    return list(out)


class Chunks:
    """Chunk table: lengths (tiling [0, S_k) in order) and a sweep order."""

    def __init__(self, lens, order=None):
        lens = [int(x) for x in lens]
        starts, at = [], 0
        for n in lens:
            starts.append(at)
            at += n
        self.lens, self.starts = lens, starts
        self.order = list(range(len(lens))) if order is None else [int(o) for o in order]
        self._keep = (_arr(starts), _arr(lens), _arr(self.order))
        self.c = RaChunks(len(lens), *self._keep)

    def __len__(self):
        return len(self.lens)


def fwd_chunk(q, k, v, out, lse, merge, scale=None, layout="bshd", kmask=None):
    _dev_check(q, k, v, out, lse)
    dq, dk, dv, do = (tensor_desc(x, layout) for x in (q, k, v, out))
    dl = rows_desc(lse)
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_fwd_chunk(dq, dk, dv, sc, do, dl, int(merge), _stream(q)), "ra_fwd_chunk")
    else:
        check(lib().ra_fwd_chunk_masked(dq, dk, dv, kmask_desc(kmask), sc, do, dl, int(merge), _stream(q)),
              "ra_fwd_chunk_masked")


def merge_lse(out_acc, lse_acc, out_part, lse_part, layout="bshd"):
    _dev_check(out_acc, lse_acc, out_part, lse_part)
    check(lib().ra_merge_lse(tensor_desc(out_acc, layout), rows_desc(lse_acc), tensor_desc(out_part, layout),
                             rows_desc(lse_part), _stream(out_acc)), "ra_merge_lse")


def bwd_delta(out, dout, delta, layout="bshd"):
    _dev_check(out, dout, delta)
    check(lib().ra_bwd_delta(tensor_desc(out, layout), tensor_desc(dout, layout), rows_desc(delta), _stream(out)),
          "ra_bwd_delta")


def bwd_chunk(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, accumulate, scale=None, layout="bshd", kmask=None):
    _dev_check(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc)
    d = [tensor_desc(x, layout) for x in (q, k, v, dout)]
    a = [tensor_desc(x, layout) for x in (dq_acc, dk_acc, dv_acc)]
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_bwd_chunk(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta), sc,
                                 a[0], a[1], a[2], int(accumulate), _stream(q)), "ra_bwd_chunk")
    else:
        check(lib().ra_bwd_chunk_masked(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta), kmask_desc(kmask), sc,
                                        a[0], a[1], a[2], int(accumulate), _stream(q)), "ra_bwd_chunk_masked")


def bwd_chunk_dkdv(q, k, v, dout, lse, delta, dk_acc, dv_acc, accumulate, scale=None, layout="bshd", kmask=None):
    _dev_check(q, k, v, dout, lse, delta, dk_acc, dv_acc)
    d = [tensor_desc(x, layout) for x in (q, k, v, dout, dk_acc, dv_acc)]
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_bwd_chunk_dkdv(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta), sc, d[4], d[5],
                                      int(accumulate), _stream(q)), "ra_bwd_chunk_dkdv")
    else:
        check(lib().ra_bwd_chunk_dkdv_masked(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta),
                                             kmask_desc(kmask), sc, d[4], d[5], int(accumulate), _stream(q)),
              "ra_bwd_chunk_dkdv_masked")


def bwd_chunk_dq(q, k, v, dout, lse, delta, dq_acc, scale=None, layout="bshd", kmask=None):
    _dev_check(q, k, v, dout, lse, delta, dq_acc)
    d = [tensor_desc(x, layout) for x in (q, k, v, dout, dq_acc)]
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_bwd_chunk_dq(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta), sc, d[4], _stream(q)),
              "ra_bwd_chunk_dq")
    else:
        check(lib().ra_bwd_chunk_dq_masked(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta),
                                           kmask_desc(kmask), sc, d[4], _stream(q)), "ra_bwd_chunk_dq_masked")


def bwd_ds_bytes(q, k, layout="bshd"):
    """Bytes of the dS buffer ``bwd_chunk_dkdv_ds`` writes for these q rows and chunk k."""
    return lib().ra_bwd_ds_bytes(tensor_desc(q, layout), tensor_desc(k, layout))


def bwd_chunk_dkdv_ds(q, k, v, dout, lse, delta, dk_acc, dv_acc, accumulate, ds, scale=None, layout="bshd",
                      kmask=None):
    """dK/dV half of the bf16 chunk step that also stores dS into ``ds`` (a device
    buffer of at least ``bwd_ds_bytes(q, k)`` bytes) for ``bwd_chunk_dq_ds``."""
    _dev_check(q, k, v, dout, lse, delta, dk_acc, dv_acc, ds)
    d = [tensor_desc(x, layout) for x in (q, k, v, dout, dk_acc, dv_acc)]
    nbytes = ds.numel() * ds.element_size()
    m = kmask_desc(kmask) if kmask is not None else None
    check(lib().ra_bwd_chunk_dkdv_ds(d[0], d[1], d[2], d[3], rows_desc(lse), rows_desc(delta), m,
                                     _scale(scale, q.shape[-1]), d[4], d[5], int(accumulate),
                                     ctypes.c_void_p(ds.data_ptr()), nbytes, _stream(q)), "ra_bwd_chunk_dkdv_ds")


def bwd_chunk_dq_ds(q, k, ds, dq_acc, scale=None, layout="bshd"):
    """dq_acc += scale dS K from the dS that ``bwd_chunk_dkdv_ds`` stored for the same
    q rows and chunk k."""
    _dev_check(q, k, ds, dq_acc)
    dq_, dk_, dd = (tensor_desc(x, layout) for x in (q, k, dq_acc))
    nbytes = ds.numel() * ds.element_size()
    check(lib().ra_bwd_chunk_dq_ds(dq_, dk_, ctypes.c_void_p(ds.data_ptr()), nbytes, _scale(scale, q.shape[-1]),
                                   dd, _stream(q)), "ra_bwd_chunk_dq_ds")


def _rows_shape(q, layout):
    if layout == "bshd":
        B, S, H, _ = q.shape
    else:
        S, B, H, _ = q.shape
    return (B, H, S)


def ring_fwd(q, k, v, chunks, scale=None, out=None, lse=None, out_dtype=None, layout="bshd", workspace=None,
             kmask=None):
    """Sweep the local query shard q over every chunk of (k, v) in ``chunks.order``.

    Returns (out, lse); out has q's layout and ``out_dtype`` (default q.dtype), lse is
    fp32 [B, H_q, S_q].  ``kmask``: optional key-validity mask [B, S_k] of the whole
    key sequence (nonzero = the key takes part).
    """
    _dev_check(q, k, v)
    if not isinstance(chunks, Chunks):
        chunks = Chunks(chunks)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(_rows_shape(q, layout), dtype=torch.float32, device=q.device)
    tq, tk, tv, to = (tensor_desc(x, layout) for x in (q, k, v, out))
    need = lib().ra_ring_fwd_workspace_bytes(tq, to)
    ws = _workspace(workspace, need, q.device)
    wsp = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_ring_fwd(tq, tk, tv, ctypes.byref(chunks.c), sc, to, rows_desc(lse), wsp, need, _stream(q)),
              "ra_ring_fwd")
    else:
        check(lib().ra_ring_fwd_masked(tq, tk, tv, kmask_desc(kmask), ctypes.byref(chunks.c), sc, to, rows_desc(lse),
                                       wsp, need, _stream(q)), "ra_ring_fwd_masked")
    return out, lse


def ring_bwd(q, k, v, out, dout, lse, chunks, scale=None, grad_dtype=None, layout="bshd", workspace=None,
             dq=None, dk=None, dv=None, kmask=None):
    """Backward sweep in the forward's chunk order; returns (dq, dk, dv) (written into
    dq/dk/dv when given).  ``kmask``: the forward's key-validity mask, if any."""
    _dev_check(q, k, v, out, dout, lse)
    if not isinstance(chunks, Chunks):
        chunks = Chunks(chunks)
    gd = grad_dtype or q.dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=gd, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=gd, device=q.device) if dv is None else dv
    t = [tensor_desc(x, layout) for x in (q, k, v, out, dout, dq, dk, dv)]
    if workspace is None:
        need = lib().ra_ring_bwd_workspace_bytes(t[0], t[1], t[5], t[6], t[7])
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    # the library plans from the room the workspace gives (at least the minimum size)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    wsp = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    sc = _scale(scale, q.shape[-1])
    if kmask is None:
        check(lib().ra_ring_bwd(t[0], t[1], t[2], t[3], t[4], rows_desc(lse), ctypes.byref(chunks.c), sc,
                                t[5], t[6], t[7], wsp, nbytes, _stream(q)), "ra_ring_bwd")
    else:
        check(lib().ra_ring_bwd_masked(t[0], t[1], t[2], t[3], t[4], rows_desc(lse), kmask_desc(kmask),
                                       ctypes.byref(chunks.c), sc, t[5], t[6], t[7], wsp, nbytes, _stream(q)),
              "ra_ring_bwd_masked")
    return dq, dk, dv


def ring_bwd_workspace_bytes(q, k, dq_dtype=None, dk_dtype=None, layout="bshd", minimum=False):
    """Workspace bytes for ``ring_bwd`` with these q, k (gradients of dtype ``dq_dtype`` /
    ``dk_dtype``, default q's dtype): the size at which it runs fastest (delta, the fp32
    accumulators its plan needs and, on the bf16 path, the dS region), or with
    ``minimum`` the least it accepts."""
    tq, tk = tensor_desc(q, layout), tensor_desc(k, layout)
    tdq, tdk = tensor_desc(q, layout), tensor_desc(k, layout)
    tdq.dtype = _DT[dq_dtype or q.dtype]
    tdk.dtype = _DT[dk_dtype or k.dtype]
    fn = lib().ra_ring_bwd_workspace_min_bytes if minimum else lib().ra_ring_bwd_workspace_bytes
    return fn(tq, tk, tdq, tdk, tdk)


def ring_bwd_plan(q, k, chunks, workspace_bytes, dq_dtype=None, dk_dtype=None, layout="bshd"):
    """The plan ``ring_bwd`` runs with a workspace of ``workspace_bytes`` bytes (host-side,
    no launch): a dict with ``slice_rows`` (query rows per slice when the sweep runs slice
    by slice, else 0), ``rows`` (per chunk in sweep order: query rows per dK/dV launch on the
    stored-dS route, 0 on the recompute route, -1 for an empty chunk) and ``accumulators``
    (the gradients that get an fp32 accumulator in the workspace)."""
    if not isinstance(chunks, Chunks):
        chunks = Chunks(chunks)
    tq, tk = tensor_desc(q, layout), tensor_desc(k, layout)
    tdq, tdk = tensor_desc(q, layout), tensor_desc(k, layout)
    tdq.dtype = _DT[dq_dtype or q.dtype]
    tdk.dtype = _DT[dk_dtype or k.dtype]
    n = chunks.c.n
    sr, rows, accs = ctypes.c_int32(0), (ctypes.c_int32 * max(n, 1))(), ctypes.c_uint32(0)
    check(lib().ra_ring_bwd_plan(tq, tk, tdq, tdk, tdk, ctypes.byref(chunks.c), int(workspace_bytes),
                                 ctypes.byref(sr), rows, ctypes.byref(accs)), "ra_ring_bwd_plan")
    return {"slice_rows": sr.value, "rows": [rows[i] for i in range(n)],
            "accumulators": [g for b, g in ((1, "dq"), (2, "dk"), (4, "dv")) if accs.value & b]}


def _workspace(ws, need, device):
    if need == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace of {need} bytes needed")
        return ws
    return torch.empty(need, dtype=torch.uint8, device=device)


def seq_head_permute(inputs, outputs, direction, layout="bshd"):
    """Exchange of R simulated ranks (direction 0: seq->head, 1: head->seq) into ``outputs``."""
    _dev_check(*inputs, *outputs)
    R = len(inputs)
    tin = (RaTensor * R)(*[tensor_desc(x, layout) for x in inputs])
    tout = (RaTensor * len(outputs))(*[tensor_desc(x, layout) for x in outputs])
    check(lib().ra_seq_head_permute(tin, R, tout, len(outputs), int(direction), _stream(inputs[0])),
          "ra_seq_head_permute")
    return outputs


def seq_to_head(shards, head_counts, layout="sbhd"):
    """shards[i]: rank i's sequence shard; returns rank r's head group over the whole sequence."""
    S = sum(x.shape[0 if layout == "sbhd" else 1] for x in shards)
    outs = []
    for h in head_counts:
        x0 = shards[0]
        shape = (S, x0.shape[1], h, x0.shape[3]) if layout == "sbhd" else (x0.shape[0], S, h, x0.shape[3])
        outs.append(torch.empty(shape, dtype=x0.dtype, device=x0.device))
    return seq_head_permute(shards, outs, 0, layout)


def head_to_seq(parts, seq_lens, layout="sbhd"):
    """parts[r]: rank r's head group; returns rank i's sequence shard with all heads."""
    H = sum(x.shape[2] for x in parts)
    outs = []
    for s in seq_lens:
        x0 = parts[0]
        shape = (s, x0.shape[1], H, x0.shape[3]) if layout == "sbhd" else (x0.shape[0], s, H, x0.shape[3])
        outs.append(torch.empty(shape, dtype=x0.dtype, device=x0.device))
    return seq_head_permute(parts, outs, 1, layout)
