"""The ring sweeps captured in a HIP graph and replayed.

Both sweeps enqueue kernels only (no allocation, no memset, no host synchronisation:
every scratch buffer is a caller workspace), so a caller can capture a whole
forward + backward step once and replay it.  Each replay is checked bit for bit against
the eager sweeps on the same inputs; new inputs are written into the captured buffers
between replays, with eager work and synchronisations in between.  Shapes follow the
bf16 ring workload (B2, S512, H8, D64, ring 4) and a small GQA one at D 128 with uneven
chunks; inputs come from the seeded generators in ``workloads``.
"""
import pytest
import torch

import context_attention_lse_kv_amd as ra
import workloads as W
from parity import dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, S, Sq, Hq, Hkv, D, chunk lens, order
    ("bf16_ring4_shard", 2, 512, 128, 8, 8, 64, (128, 128, 128, 128), (0, 3, 2, 1)),
    ("gqa_d128_uneven", 1, 1000, 320, 8, 2, 128, (334, 333, 333), (1, 0, 2)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ring_step_replays_from_hip_graph(case):
    name, B, S, Sq, Hq, Hkv, D, lens, order = case
    d = dev()
    seed = 1500 + 10 * CASES.index(case)
    shapes = [(B, Sq, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D), (B, Sq, Hq, D)]
    q, k, v, do = (W.randn(s, seed + i, "bf16").to(d) for i, s in enumerate(shapes))
    ch = ra.Chunks(lens, order)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=d)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=d)
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.bfloat16, device=d) for t in (q, k, v))
    fws = torch.empty(q.numel() * 4 + 256, dtype=torch.uint8, device=d)
    bws = torch.empty(ra.ring_bwd_workspace_bytes(q, k), dtype=torch.uint8, device=d)

    def step():
        ra.ring_fwd(q, k, v, ch, out=out, lse=lse, workspace=fws)
        ra.ring_bwd(q, k, v, out, do, lse, ch, workspace=bws, dq=dq, dk=dk, dv=dv)

    def eager_result():
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in (out, lse, dq, dk, dv)]

    ref0 = eager_result()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture's side stream, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        if rep > 0:
            # new inputs into the captured buffers (eager work), then the eager reference
            for t, i in zip((q, k, v, do), range(4)):
                t.copy_(W.randn(t.shape, seed + 100 * rep + i, "bf16").to(d))
            ref = eager_result()
            for t in (out, lse, dq, dk, dv):
                t.fill_(float("nan"))  # the replay must rewrite every output
            torch.cuda.synchronize()
        else:
            ref = ref0
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (name, rep)
