"""The C ABI without a GPU: the library loads, exports every symbol include/ra.h
declares, its host helpers agree with the oracle's, and every malformed call is
refused with a status before anything is launched (no call here reaches HIP)."""
import ctypes
import os
import re

import pytest

import oracle
from oracle_pins import golden

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

abi = pytest.importorskip("context_attention_lse_kv_amd._abi")


def _lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libra.so is not built (run python -m context_attention_lse_kv_amd.build)")
    return abi.lib()


def declared_symbols():
    with open(os.path.join(ROOT, "include", "ra.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**(ra_[a-z0-9_]+)\s*\(", src, flags=re.M)))


def test_header_declares_what_binding_lists():
    assert declared_symbols() == sorted(abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_split_sizes_matches_oracle():
    lib = _lib()
    for n in list(range(0, 50)) + [512, 1000, 4608, 32768, 32769]:
        for parts in range(1, 10):
            buf = (ctypes.c_int32 * parts)()
            assert lib.ra_split_sizes(n, parts, buf) == abi.RA_OK
            assert list(buf) == oracle.split_sizes(n, parts)


def test_ring_order_starts_local_and_walks_back():
    lib = _lib()
    for R in range(1, 9):
        for rank in range(R):
            buf = (ctypes.c_int32 * R)()
            assert lib.ra_ring_order(R, rank, buf) == abi.RA_OK
            assert list(buf) == [(rank - i) % R for i in range(R)]
    buf = (ctypes.c_int32 * 8)()
    lib.ra_ring_order(8, 0, buf)
    assert list(buf) == [0, 7, 6, 5, 4, 3, 2, 1]


# ------------------------------------------------------------------ validation (no launch)
FAKE = 1 << 20  # 16-byte aligned fake device address: never dereferenced on the error paths below


def T(B, S, H, D, dtype=abi.RA_BF16, data=FAKE, strides=None):
    sB, sS, sH = strides if strides else (S * H * D, H * D, D)
    return abi.RaTensor(data, dtype, B, S, H, D, sB, sS, sH)


def Lrows(B, H, S, data=FAKE):
    return abi.RaLse(data, B, H, S, H * S, S)


def fwd(q, k, v, out, lse, merge=0, scale=0.125):
    lib = _lib()
    st = lib.ra_fwd_chunk(q, k, v, scale, out, lse, merge, None)
    return st, lib.ra_last_error().decode()


def good(Sq=64, Sk=64, Hq=8, Hkv=8, D=64):
    return (T(1, Sq, Hq, D), T(1, Sk, Hkv, D), T(1, Sk, Hkv, D), T(1, Sq, Hq, D, abi.RA_F32), Lrows(1, Hq, Sq))


def test_gqa_divisibility_refused_with_page_message():
    q, k, v, o, l = good(Hq=6, Hkv=4)
    st, msg = fwd(q, k, v, o, l)
    assert st == abi.RA_E_SHAPE
    assert golden()["gqa_divisibility_error"]["message"] in msg


@pytest.mark.parametrize("case, status", [
    ("null_q", abi.RA_E_ARG), ("null_data", abi.RA_E_ARG), ("bad_dtype", abi.RA_E_DTYPE),
    ("mixed_dtype", abi.RA_E_DTYPE), ("d96", abi.RA_E_UNSUPPORTED), ("misaligned_ptr", abi.RA_E_ALIGN),
    ("misaligned_stride", abi.RA_E_ALIGN), ("batch_mismatch", abi.RA_E_SHAPE), ("headdim_mismatch", abi.RA_E_SHAPE),
    ("out_bf16", abi.RA_E_DTYPE), ("out_shape", abi.RA_E_SHAPE), ("lse_shape", abi.RA_E_SHAPE),
    ("bad_merge", abi.RA_E_ARG), ("neg_scale", abi.RA_E_ARG), ("nan_scale", abi.RA_E_ARG), ("tiny_scale", abi.RA_E_ARG),
    ("overlap", abi.RA_E_ARG), ("neg_stride", abi.RA_E_ARG), ("zero_heads", abi.RA_E_SHAPE),
])
def test_fwd_chunk_refuses(case, status):
    q, k, v, o, l = good()
    merge, scale = 0, 0.125
    if case == "null_q":
        st = _lib().ra_fwd_chunk(None, k, v, scale, o, l, 0, None)
        assert st == status
        return
    if case == "null_data": q.data = None
    if case == "bad_dtype": q.dtype = 7
    if case == "mixed_dtype": k.dtype = abi.RA_F32
    if case == "d96": q, k, v, o = T(1, 64, 8, 96), T(1, 64, 8, 96), T(1, 64, 8, 96), T(1, 64, 8, 96, abi.RA_F32)
    if case == "misaligned_ptr": v.data = FAKE + 8
    if case == "misaligned_stride": q.sS = 8 * 64 + 4
    if case == "batch_mismatch": k.B = 2
    if case == "headdim_mismatch": k = T(1, 64, 8, 128)
    if case == "out_bf16": o.dtype = abi.RA_BF16
    if case == "out_shape": o.S = 63
    if case == "lse_shape": l.S = 65
    if case == "bad_merge": merge = 2
    if case == "neg_scale": scale = -1.0
    if case == "nan_scale": scale = float("nan")
    if case == "tiny_scale": scale = 2.0 ** -101
    if case == "overlap": q.sS = 8  # rows alias each other's heads
    if case == "neg_stride": q.sH = -64
    if case == "zero_heads": q.H = 0
    st, msg = fwd(q, k, v, o, l, merge, scale)
    assert st == status, (case, msg)
    assert msg


def chunks(lens, order):
    starts = [sum(lens[:i]) for i in range(len(lens))]
    keep = ((ctypes.c_int32 * len(lens))(*starts), (ctypes.c_int32 * len(lens))(*lens),
            (ctypes.c_int32 * len(order))(*order))
    c = abi.RaChunks(len(lens), *keep)
    c._keep = keep
    return c


@pytest.mark.parametrize("lens, order, status", [
    ([32, 32], [0, 0], abi.RA_E_ARG),        # order not a permutation
    ([32, 32], [1, 2], abi.RA_E_ARG),
    ([32, 31], [0, 1], abi.RA_E_SHAPE),      # does not cover S_k
    ([32, 40], [0, 1], abi.RA_E_SHAPE),      # runs past S_k
    ([-1, 65], [0, 1], abi.RA_E_ARG),
])
def test_ring_fwd_refuses_bad_chunk_tables(lens, order, status):
    lib = _lib()
    q, k, v, o, l = good()
    c = chunks(lens, order)
    st = lib.ra_ring_fwd(q, k, v, ctypes.byref(c), 0.125, o, l, None, 0, None)
    assert st == status, lib.ra_last_error()


def test_ring_fwd_refuses_gapped_tiling():
    lib = _lib()
    q, k, v, o, l = good()
    starts, lens, order = (ctypes.c_int32 * 2)(0, 40), (ctypes.c_int32 * 2)(32, 24), (ctypes.c_int32 * 2)(0, 1)
    c = abi.RaChunks(2, starts, lens, order)
    assert lib.ra_ring_fwd(q, k, v, ctypes.byref(c), 0.125, o, l, None, 0, None) == abi.RA_E_SHAPE


def test_ring_fwd_needs_workspace_for_bf16_out():
    lib = _lib()
    q, k, v, _, l = good()
    o = T(1, 64, 8, 64, abi.RA_BF16)
    need = lib.ra_ring_fwd_workspace_bytes(q, o)
    assert need >= 64 * 8 * 64 * 4
    c = chunks([32, 32], [0, 1])
    assert lib.ra_ring_fwd(q, k, v, ctypes.byref(c), 0.125, o, l, None, 0, None) == abi.RA_E_WORKSPACE
    assert lib.ra_ring_fwd(q, k, v, ctypes.byref(c), 0.125, o, l, FAKE, need - 1, None) == abi.RA_E_WORKSPACE
    assert lib.ra_ring_fwd_workspace_bytes(q, T(1, 64, 8, 64, abi.RA_F32)) == 0


def _region(lib, q, k):
    """The recommended dS room: the whole key sequence as one chunk plus the 7 key tiles of
    128 that splitting it into up to 8 chunks can add (each chunk's dS is whole tiles)."""
    return lib.ra_bwd_ds_bytes(q, k) + 7 * lib.ra_bwd_ds_bytes(q, T(k.B, 128, k.H, k.D, k.dtype))


def test_ring_bwd_workspace_sizes():
    """Recommended size: delta + the dS region (+ only the accumulators that plan needs);
    minimum: delta + an fp32 accumulator for every bf16 gradient, no dS region."""
    lib = _lib()
    q, k = T(1, 100, 8, 64), T(1, 300, 2, 64)
    f = lambda t: T(t.B, t.S, t.H, t.D, abi.RA_F32)
    r256 = lambda n: (n + 255) // 256 * 256
    delta = r256(8 * 100 * 4)
    ds = _region(lib, q, k)
    accs = r256(100 * 8 * 64 * 4) + 2 * r256(300 * 2 * 64 * 4)
    # fp32 gradients are their own accumulators
    assert lib.ra_ring_bwd_workspace_bytes(q, k, f(q), f(k), f(k)) == delta + ds
    assert lib.ra_ring_bwd_workspace_min_bytes(q, k, f(q), f(k), f(k)) == delta
    # bf16 gradients: the whole dS fits the region, so one dQ pass writes dq and each dK/dV
    # launch writes its rows in bf16 directly; the minimum carries every accumulator
    assert lib.ra_ring_bwd_workspace_bytes(q, k, q, k, k) == delta + ds
    assert lib.ra_ring_bwd_workspace_min_bytes(q, k, q, k, k) == delta + accs
    # fp32 inputs: no dS route at all
    q32, k32 = f(q), f(k)
    assert lib.ra_ring_bwd_workspace_bytes(q32, k32, q32, k32, k32) == delta
    assert lib.ra_ring_bwd_workspace_min_bytes(q32, k32, q, k, k) == delta + accs
    # the video shard: 8 GiB of dS, no accumulators in the recommended plan
    bq, bk = T(1, 4096, 32, 128), T(1, 32768, 8, 128)
    assert lib.ra_ring_bwd_workspace_bytes(bq, bk, bq, bk, bk) == r256(32 * 4096 * 4) + (8 << 30)


def _plan(q, k, c, ws, dq=None, dk=None):
    lib = _lib()
    sr, rows, accs = ctypes.c_int32(-9), (ctypes.c_int32 * c.n)(), ctypes.c_uint32(99)
    st = lib.ra_ring_bwd_plan(q, k, dq or q, dk or k, dk or k, ctypes.byref(c), ws, ctypes.byref(sr), rows,
                              ctypes.byref(accs))
    assert st == abi.RA_OK, lib.ra_last_error().decode()
    return sr.value, list(rows), [g for b, g in ((1, "dq"), (2, "dk"), (4, "dv")) if accs.value & b]


def test_ring_bwd_plans():
    """The backward's plan for the video-DiT workload (8 chunks of 4096 keys, Hq 32 / Hkv 8,
    D 128; 16 MiB of dS per 64 query rows and chunk) under the sizes the sweep is run with."""
    lib = _lib()
    r256 = lambda n: (n + 255) // 256 * 256
    k = T(1, 32768, 8, 128)
    c = chunks([4096] * 8, [0, 7, 6, 5, 4, 3, 2, 1])
    shard, full = T(1, 4096, 32, 128), T(1, 32768, 32, 128)
    acc_kv = 2 * r256(32768 * 8 * 128 * 4)
    # rank-0 shard, recommended: the whole dS (8 GiB) in one region, one dQ pass, no accumulators
    rec = lib.ra_ring_bwd_workspace_bytes(shard, k, shard, k, k)
    assert _plan(shard, k, c, rec) == (0, [4096] * 8, [])
    # ... with 2 GiB of dS room: chunk by chunk, two chunks' dS per dQ pass (fp32 dQ accumulator)
    lo = lib.ra_ring_bwd_workspace_min_bytes(shard, k, shard, k, k)
    assert _plan(shard, k, c, lo + (2 << 30)) == (0, [4096] * 8, ["dq"])
    # ... with the minimum: every chunk on the recompute route
    assert _plan(shard, k, c, lo) == (0, [0] * 8, ["dq", "dk", "dv"])
    # full Q, recommended: 8 GiB of dS hold every chunk for 4096 rows, so the sweep runs in 8
    # slices of 4096 rows (dQ of each slice written once; dK/dV summed over slices in fp32)
    rec_full = lib.ra_ring_bwd_workspace_bytes(full, k, full, k, k)
    assert rec_full == r256(32 * 32768 * 4) + acc_kv + (8 << 30)
    assert _plan(full, k, c, rec_full) == (4096, [4096] * 8, ["dk", "dv"])
    # ... with 2 GiB of room a slice of every chunk would be 1024 rows: chunk by chunk, each
    # chunk in 4 slices of 8192 rows
    lo_full = lib.ra_ring_bwd_workspace_min_bytes(full, k, full, k, k)
    assert _plan(full, k, c, lo_full + (2 << 30)) == (0, [8192] * 8, ["dq", "dk", "dv"])
    # fp32 gradients are their own accumulators
    f = lambda t: T(t.B, t.S, t.H, t.D, abi.RA_F32)
    rec32 = lib.ra_ring_bwd_workspace_bytes(full, k, f(full), f(k), f(k))
    assert rec32 == r256(32 * 32768 * 4) + (8 << 30)
    assert _plan(full, k, c, rec32, f(full), f(k)) == (4096, [4096] * 8, [])
    # more room than that: longer slices (the room the unneeded accumulators leave)
    assert _plan(full, k, c, rec_full, f(full), f(k)) == (4224, [4224] * 8, [])
    # fp32 inputs have no dS route; an empty chunk is reported as -1
    c3 = chunks([0, 100, 200], [2, 0, 1])
    q32, k32 = f(T(1, 64, 4, 64)), f(T(1, 300, 2, 64))
    assert _plan(q32, k32, c3, 1 << 20) == (0, [0, -1, 0], [])
    # refusals: a chunk table that does not tile the keys, an unknown gradient dtype, GQA
    # heads that do not divide
    sr = ctypes.c_int32()
    bad = chunks([4096] * 7, list(range(7)))
    assert lib.ra_ring_bwd_plan(full, k, None, None, None, ctypes.byref(bad), rec_full, ctypes.byref(sr), None,
                                None) == abi.RA_E_SHAPE
    assert lib.ra_ring_bwd_plan(full, k, T(1, 32768, 32, 128, 7), None, None, ctypes.byref(c), rec_full,
                                ctypes.byref(sr), None, None) == abi.RA_E_DTYPE
    assert lib.ra_ring_bwd_plan(T(1, 4096, 30, 128), k, None, None, None, ctypes.byref(c), rec_full,
                                ctypes.byref(sr), None, None) == abi.RA_E_SHAPE
    # below what the plan needs
    assert lib.ra_ring_bwd_plan(full, k, full, k, k, ctypes.byref(c), 4096, ctypes.byref(sr), None, None) == \
        abi.RA_E_WORKSPACE


def test_ring_bwd_refuses_below_minimum_workspace():
    lib = _lib()
    q, k, v = T(1, 100, 8, 64), T(1, 300, 2, 64), T(1, 300, 2, 64)
    l = Lrows(1, 8, 100)
    c = chunks([150, 150], [1, 0])
    need = lib.ra_ring_bwd_workspace_min_bytes(q, k, q, k, k)
    st = lib.ra_ring_bwd(q, k, v, q, q, l, ctypes.byref(c), 0.125, q, k, v, FAKE, need - 256, None)
    assert st == abi.RA_E_WORKSPACE and str(need) in lib.ra_last_error().decode()
    assert lib.ra_ring_bwd(q, k, v, q, q, l, ctypes.byref(c), 0.125, q, k, v, None, 0, None) == abi.RA_E_WORKSPACE
    assert lib.ra_ring_bwd(q, k, v, q, q, l, ctypes.byref(c), 0.125, q, k, v, FAKE + 16, need, None) == abi.RA_E_ALIGN


def test_bwd_ds_bytes_and_ring_ds_region():
    """dS blocks: 4 KiB per (batch, query head, 64 query rows, 32 keys counted in whole
    128-key tiles); the ring backward reserves min(8 GiB, that for the whole key sequence plus
    the tile rounding of up to 8 chunks) for bf16 inputs and nothing for fp32."""
    lib = _lib()
    q, k = T(2, 100, 8, 64), T(2, 300, 2, 64)
    assert lib.ra_bwd_ds_bytes(q, k) == 2 * 8 * 2 * (4 * 3) * 4096
    assert lib.ra_bwd_ds_bytes(T(1, 4096, 32, 128), T(1, 4096, 8, 128)) == 1 << 30
    assert lib.ra_bwd_ds_bytes(T(2, 100, 8, 64, abi.RA_F32), T(2, 300, 2, 64, abi.RA_F32)) == 0
    assert lib.ra_bwd_ds_bytes(T(2, 0, 8, 64), k) == 0
    f = lambda t: T(t.B, t.S, t.H, t.D, abi.RA_F32)
    with_ds = lib.ra_ring_bwd_workspace_bytes(q, k, f(q), f(k), f(k))
    q32, k32 = f(q), f(k)
    without = lib.ra_ring_bwd_workspace_bytes(q32, k32, q32, k32, k32)
    assert with_ds - without == _region(lib, q, k)
    # the room runs any table of up to 8 chunks as one group: 300 keys as 8 ragged chunks take
    # 8 key tiles where one chunk takes 3
    c8 = chunks([38, 37, 38, 37, 37, 38, 37, 38], list(range(8)))
    assert _plan(q, k, c8, with_ds, f(q), f(k)) == (0, [100] * 8, [])
    need = sum(lib.ra_bwd_ds_bytes(q, T(2, n, 2, 64)) for n in [38, 37, 38, 37, 37, 38, 37, 38])
    assert lib.ra_bwd_ds_bytes(q, k) < need <= _region(lib, q, k)
    big_q, big_k = T(1, 32768, 32, 128), T(1, 32768, 8, 128)
    fq, fk = f(big_q), f(big_k)
    assert lib.ra_ring_bwd_workspace_bytes(big_q, big_k, fq, fk, fk) - \
        lib.ra_ring_bwd_workspace_bytes(fq, fk, fq, fk, fk) == 8 << 30  # the 8 GiB cap of the region


def test_stored_ds_entry_points_refuse():
    lib = _lib()
    q, k, v = T(1, 64, 8, 64), T(1, 64, 2, 64), T(1, 64, 2, 64)
    l = Lrows(1, 8, 64)
    acc_k = T(1, 64, 2, 64, abi.RA_F32)
    acc_q = T(1, 64, 8, 64, abi.RA_F32)
    need = lib.ra_bwd_ds_bytes(q, k)

    def kv(ds, nbytes, **kw):
        a = dict(q=q, k=k, v=v, acc=acc_k, acc_v=acc_k, accumulate=1)
        a.update(kw)
        st = lib.ra_bwd_chunk_dkdv_ds(a["q"], a["k"], a["v"], a["q"], l, l, None, 0.125, a["acc"], a["acc_v"],
                                      a["accumulate"], ds, nbytes, None)
        return st

    assert kv(None, 0) == abi.RA_E_WORKSPACE
    assert kv(FAKE, need - 1) == abi.RA_E_WORKSPACE
    assert kv(FAKE + 16, need) == abi.RA_E_ALIGN
    assert kv(FAKE, need, accumulate=2) == abi.RA_E_ARG
    assert kv(FAKE, need, acc=T(1, 64, 2, 64)) == abi.RA_E_DTYPE
    q32, k32 = T(1, 64, 8, 64, abi.RA_F32), T(1, 64, 2, 64, abi.RA_F32)
    assert kv(FAKE, need, q=q32, k=k32, v=k32) == abi.RA_E_DTYPE
    # bf16 dk/dv are final outputs: only with accumulate = 0, and of the shape of k
    assert kv(FAKE, need, acc=T(1, 64, 2, 64), acc_v=T(1, 64, 2, 64), accumulate=1) == abi.RA_E_DTYPE
    assert kv(FAKE, need, acc=T(1, 64, 2, 128), acc_v=T(1, 64, 2, 128), accumulate=0) == abi.RA_E_SHAPE
    assert lib.ra_bwd_chunk_dq_ds(q, k, None, 0, 0.125, acc_q, None) == abi.RA_E_WORKSPACE
    assert lib.ra_bwd_chunk_dq_ds(q, k, FAKE, need - 256, 0.125, acc_q, None) == abi.RA_E_WORKSPACE
    assert lib.ra_bwd_chunk_dq_ds(q, T(1, 64, 3, 64), FAKE, need, 0.125, acc_q, None) == abi.RA_E_SHAPE
    assert lib.ra_bwd_chunk_dq_ds(q, k, FAKE, need, -1.0, acc_q, None) == abi.RA_E_ARG
    assert lib.ra_bwd_chunk_dq_ds(q, k, FAKE, need, 0.125, T(1, 64, 8, 64), None) == abi.RA_E_DTYPE
    assert lib.ra_bwd_chunk_dq_ds(q32, k32, FAKE, need, 0.125, acc_q, None) == abi.RA_E_DTYPE


def test_bwd_chunk_refuses_bf16_accumulators():
    lib = _lib()
    q, k, v = T(1, 64, 8, 64), T(1, 64, 2, 64), T(1, 64, 2, 64)
    l = Lrows(1, 8, 64)
    st = lib.ra_bwd_chunk(q, k, v, q, l, l, 0.125, T(1, 64, 8, 64), T(1, 64, 2, 64, abi.RA_F32),
                          T(1, 64, 2, 64, abi.RA_F32), 0, None)
    assert st == abi.RA_E_DTYPE


def test_permute_refusals():
    lib = _lib()
    A = abi.RaTensor * 2
    ins = A(T(2, 5, 8, 64, data=FAKE), T(2, 5, 8, 64, data=FAKE + (1 << 16)))
    outs = A(T(2, 10, 4, 64, data=FAKE + (2 << 16)), T(2, 10, 4, 64, data=FAKE + (3 << 16)))
    bad = A(T(2, 10, 4, 64, data=FAKE + (2 << 16)), T(2, 10, 3, 64, data=FAKE + (3 << 16)))
    assert lib.ra_seq_head_permute(ins, 2, bad, 2, 0, None) == abi.RA_E_SHAPE   # heads sum to 7
    assert lib.ra_seq_head_permute(ins, 2, outs, 2, 2, None) == abi.RA_E_ARG    # bad direction
    assert lib.ra_seq_head_permute(ins, 2, outs, 1, 0, None) == abi.RA_E_ARG    # rank count mismatch
    alias = A(T(2, 10, 4, 64, data=FAKE), T(2, 10, 4, 64, data=FAKE + (3 << 16)))
    assert lib.ra_seq_head_permute(ins, 2, alias, 2, 0, None) == abi.RA_E_ARG   # out aliases in
    short = A(T(2, 9, 4, 64, data=FAKE + (2 << 16)), T(2, 9, 4, 64, data=FAKE + (3 << 16)))
    assert lib.ra_seq_head_permute(ins, 2, short, 2, 0, None) == abi.RA_E_SHAPE  # 5 + 5 != 9


def test_status_strings():
    lib = _lib()
    for i, name in enumerate(abi.STATUS_NAMES):
        assert lib.ra_status_string(i).decode() == name


# ------------------------------------------------------------------ key mask (no launch)
def K(B, S, data=FAKE, sB=None):
    return abi.RaKMask(data, B, S, S if sB is None else sB)


@pytest.mark.parametrize("case, status", [
    ("batch", abi.RA_E_SHAPE), ("keys", abi.RA_E_SHAPE), ("null_data", abi.RA_E_ARG),
    ("neg_stride", abi.RA_E_ARG), ("rows_overlap", abi.RA_E_ARG),
])
def test_masked_entry_points_refuse_bad_masks(case, status):
    lib = _lib()
    B, Sq, Sk = 2, 64, 96
    q, k, v, o, l = T(B, Sq, 8, 64), T(B, Sk, 8, 64), T(B, Sk, 8, 64), T(B, Sq, 8, 64, abi.RA_F32), Lrows(B, 8, Sq)
    m = K(B, Sk)
    if case == "batch": m.B = 1
    if case == "keys": m.S = Sk - 1
    if case == "null_data": m.data = None
    if case == "neg_stride": m.sB = -Sk
    if case == "rows_overlap": m.sB = Sk - 1
    assert lib.ra_fwd_chunk_masked(q, k, v, ctypes.byref(m), 0.125, o, l, 0, None) == status, lib.ra_last_error()
    c = chunks([48, 48], [1, 0])
    assert lib.ra_ring_fwd_masked(q, k, v, ctypes.byref(m), ctypes.byref(c), 0.125, o, l, None, 0, None) == status
    acc = T(B, Sq, 8, 64, abi.RA_F32)
    kacc = T(B, Sk, 8, 64, abi.RA_F32)
    st = lib.ra_bwd_chunk_masked(q, k, v, q, l, l, ctypes.byref(m), 0.125, acc, kacc, kacc, 1, None)
    assert st == status
    assert lib.ra_bwd_chunk_dq_masked(q, k, v, q, l, l, ctypes.byref(m), 0.125, acc, None) == status
    assert lib.ra_bwd_chunk_dkdv_masked(q, k, v, q, l, l, ctypes.byref(m), 0.125, kacc, kacc, 1, None) == status


def test_masked_entry_points_validate_the_rest_as_before():
    """A NULL mask is no mask: the masked entry points refuse exactly what the plain ones do."""
    lib = _lib()
    q, k, v, o, l = good(Hq=6, Hkv=4)
    assert lib.ra_fwd_chunk_masked(q, k, v, None, 0.125, o, l, 0, None) == abi.RA_E_SHAPE
    assert golden()["gqa_divisibility_error"]["message"] in lib.ra_last_error().decode()


def test_bwd_refuses_dout_slice_past_32bit_span():
    """The bf16 backward kernels address a (batch, head) slice of dout with 32-bit buffer
    offsets, as for q: a dout whose own strides make one slice span 2^31 bytes or more is
    refused before any launch, even when q's slices are small."""
    lib = _lib()
    B, S, Hq, Hkv, D = 1, 40000, 4, 4, 128
    q, k, v = T(B, S, Hq, D), T(B, S, Hkv, D), T(B, S, Hkv, D)
    wide = T(B, S, Hq, D, strides=(S * 65536, 65536, D))  # 5.2 GB per slice
    l = Lrows(B, Hq, S)
    acc_q, acc_k = T(B, S, Hq, D, abi.RA_F32), T(B, S, Hkv, D, abi.RA_F32)
    st = lib.ra_bwd_chunk(q, k, v, wide, l, l, 0.125, acc_q, acc_k, acc_k, 1, None)
    assert st == abi.RA_E_UNSUPPORTED and "dout" in lib.ra_last_error().decode()
    assert lib.ra_bwd_chunk(q, k, v, q, l, l, 0.125, acc_q, acc_k, acc_k, 2, None) == abi.RA_E_ARG  # same call, dout ok
    need = lib.ra_bwd_ds_bytes(q, k)
    st = lib.ra_bwd_chunk_dkdv_ds(q, k, v, wide, l, l, None, 0.125, acc_k, acc_k, 1, FAKE, need, None)
    assert st == abi.RA_E_UNSUPPORTED
    c = chunks([20000, 20000], [0, 1])
    o = T(B, S, Hq, D)
    st = lib.ra_ring_bwd(q, k, v, o, wide, l, ctypes.byref(c), 0.125, o, k, v, None, 0, None)
    assert st == abi.RA_E_UNSUPPORTED and "dout" in lib.ra_last_error().decode()
