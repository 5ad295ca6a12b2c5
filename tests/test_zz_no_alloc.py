"""ra_ring_fwd_noalloc through the C ABI against ra_ring_fwd (the same sweep with a
caller workspace): bit-identical outputs on two calls in a row, the second with a
smaller input, so the shared device scratch is reused with stale contents from the
first call; an fp32 output (no scratch); and the refusal past the scratch's size."""
import ctypes

import pytest
import torch

import context_attention_lse_kv_amd as ra
import workloads as W
from context_attention_lse_kv_amd import _abi, ops
from parity import dev

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, ch, out, lse, kmask=None):
    lib = _abi.lib()
    st = lib.ra_ring_fwd_noalloc(ops.tensor_desc(q), ops.tensor_desc(k), ops.tensor_desc(v),
                                 ops.kmask_desc(kmask), ctypes.byref(ch.c), 1.0 / q.shape[-1] ** 0.5,
                                 ops.tensor_desc(out), ops.rows_desc(lse), ops._stream(q))
    return st


def _case(B, Sq, Sk, Hq, Hkv, D, lens, order, seed, out_dtype=torch.bfloat16, masked=False):
    d = dev()
    q = W.randn((B, Sq, Hq, D), seed, "bf16").to(d)
    k = W.randn((B, Sk, Hkv, D), seed + 1, "bf16").to(d)
    v = W.randn((B, Sk, Hkv, D), seed + 2, "bf16").to(d)
    km = W.make_key_mask(B, Sk, seed + 3, p_keep=0.8).to(d) if masked else None
    ch = ra.Chunks(lens, order)
    ref_o, ref_l = ra.ring_fwd(q, k, v, ch, out_dtype=out_dtype, kmask=km)
    out = torch.full(q.shape, 7.0, dtype=out_dtype, device=d)
    lse = torch.full((B, Hq, Sq), 7.0, dtype=torch.float32, device=d)
    st = _noalloc(q, k, v, ch, out, lse, km)
    torch.cuda.synchronize()
    assert st == _abi.RA_OK, _abi.lib().ra_last_error()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_noalloc_forward_matches_workspace_forward_twice():
    # the video-DiT shard: 4096 rows x 32 heads x 128 = the whole 64 MiB of scratch
    lens = [4096] * 8
    _case(1, 4096, 32768, 32, 8, 128, lens, ra.ring_order(8, 0), 500)
    # second call, smaller: the scratch holds the first call's running output
    _case(2, 300, 700, 8, 2, 64, [250, 250, 200], [2, 0, 1], 510, masked=True)
    # fp32 output: no scratch at all
    _case(1, 77, 201, 6, 2, 128, [100, 0, 101], [1, 0, 2], 520, out_dtype=torch.float32)


def test_noalloc_refuses_past_its_scratch():
    d = dev()
    q = torch.zeros((1, 4097, 32, 128), dtype=torch.bfloat16, device=d)  # 64 MiB + one row of fp32
    k = torch.zeros((1, 64, 8, 128), dtype=torch.bfloat16, device=d)
    out = torch.empty_like(q)
    lse = torch.empty((1, 32, 4097), dtype=torch.float32, device=d)
    st = _noalloc(q, k, k, ra.Chunks([64]), out, lse)
    assert st == _abi.RA_E_WORKSPACE
    assert "ra_ring_fwd with a workspace" in _abi.lib().ra_last_error().decode()
