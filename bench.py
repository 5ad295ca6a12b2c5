"""Benchmark of the ring-attention hot path on one MI355X.

One step = one ring forward sweep + one ring backward sweep of one rank's
share: the video-DiT GQA workload (B1, S 32768, H_q 32, H_kv 8, D 128, bf16)
with the local query shard of 4096 rows swept over the 8 key/value chunks of
4096 in ring order 0,7,6,...,1.  Inputs are resident in HBM before the timed
region; the timed region covers every launch of both sweeps (delta, chunk
steps, merges, finalisation casts).

Prints ONE JSON line.  ``value`` is fwd+bwd TFLOP/s with the attention flop
count 4*B*Hq*Sq*Sk*D (forward) + 10*B*Hq*Sq*Sk*D (backward, five products
including the recompute).  ``roofline`` describes the dominant kernel (the
dK/dV kernel of the backward chunk step): the backward sweep's 8 launches,
issued as in the sweep right after a forward sweep, timed with HIP events on
the stream they run on;
``cpu_baseline`` times the CPU fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import context_attention_lse_kv_amd as ra  # noqa: E402
import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 flop/clk/CU (dense MFMA)
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "ring attn fwd+bwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"


def flops(B, Hq, Sq, Sk, D):
    return 4.0 * B * Hq * Sq * Sk * D, 10.0 * B * Hq * Sq * Sk * D


def timed(fn, steps, warmup, per_step=None):
    """Mean seconds per call over `steps` calls between two synchronisations.  With
    `per_step` (a list), a HIP event pair around each call on the current stream also
    records every call's duration in ms (events do not synchronise the timed region)."""
    for _ in range(warmup):
        fn()
    ev = []
    s = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if per_step is not None:
            a = torch.cuda.Event(enable_timing=True)
            a.record(s)
        fn()
        if per_step is not None:
            b = torch.cuda.Event(enable_timing=True)
            b.record(s)
            ev.append((a, b))
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    if per_step is not None:
        per_step.extend(a.elapsed_time(b) for a, b in ev)
    return t


def setup(Sq_rows, full):
    w = W.VIDEO_DIT_GQA
    lens = ra.split_sizes(w.S, w.n_chunks)
    q, k, v, do = W.make_inputs(w, Sq=w.S if full else Sq_rows)
    d = torch.device("cuda", 0)
    gq, gk, gv, gdo = (t.to(d) for t in (q, k, v, do))
    order = list(range(w.n_chunks)) if full else ra.ring_order(w.n_chunks, 0)
    return w, lens, order, gq, gk, gv, gdo


MASK_RECIPE = dict(p_keep=0.95, valid_len=(30000,))  # right padding past 30000 keys + 5 % random holes


def run_workload(full, steps, warmup, masked=False, single=False):
    w, lens, order, q, k, v, do = setup(4096, full)
    if single:  # all-gather variant: one fused sweep over the resident key sequence
        lens, order = [w.S], [0]
    ch = ra.Chunks(lens, order)
    km = W.make_key_mask(w.B, w.S, 990, **MASK_RECIPE).to(q.device) if masked else None
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((w.B, w.Hq, q.shape[1]), dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.bfloat16, device=q.device) for t in (q, k, v))
    # workspaces allocated once, outside the timed region
    fws = torch.empty(q.numel() * 4 + 256, dtype=torch.uint8, device=q.device)
    bws = torch.empty(ra.ring_bwd_workspace_bytes(q, k), dtype=torch.uint8, device=q.device)

    def fwd():
        ra.ring_fwd(q, k, v, ch, out=out, lse=lse, workspace=fws, kmask=km)

    def bwd():
        ra.ring_bwd(q, k, v, out, do, lse, ch, workspace=bws, dq=dq, dk=dk, dv=dv, kmask=km)

    def step():
        fwd()
        bwd()

    step_ms = []
    t_step = timed(step, steps, warmup, step_ms)
    t_fwd = timed(fwd, max(3, steps // 2), 1)
    t_bwd = timed(bwd, max(3, steps // 2), 1)
    f_f, f_b = flops(w.B, w.Hq, q.shape[1], w.S, w.D)
    return dict(w=w, lens=lens, order=order, q=q, k=k, v=v, do=do, out=out, lse=lse, dq=dq, dk=dk, dv=dv,
                t_step=t_step, t_fwd=t_fwd, t_bwd=t_bwd, f_f=f_f, f_b=f_b, km=km, step=step, fwd=fwd, bwd=bwd,
                bws=bws, step_ms=step_ms)


def plan_record(r):
    """The backward plan the timed sweep ran with its workspace (host-side query of the
    library): query rows per slice when it ran slice by slice (else 0), query rows per dK/dV
    launch of each chunk in sweep order, and the gradients given an fp32 accumulator."""
    pl = ra.ring_bwd_plan(r["q"], r["k"], ra.Chunks(r["lens"], r["order"]), r["bws"].numel())
    return {"workspace_bytes": int(r["bws"].numel()), **pl}


def dominant_kernel(r, launches=8, back_to_back=True, lead_steps=3):
    """The dK/dV half of the backward chunk step as the ring backward runs it (one
    kernel launch per call: it stores the step's dS for the dQ pass and writes the
    chunk's final bf16 dK/dV rows).  It executes S = Q K^T, dP = dO V^T, dV = P^T dO and
    dK = dS^T Q: 8*D flop per (query row, key) pair per head.

    The ring backward of the shard runs its 8 dK/dV launches back to back (their dS go
    to consecutive parts of the dS region; one dQ pass over all of them follows), so the
    timed launches run back to back too, between one HIP event pair on the stream (no
    event between them, as in the ring); the result is the interval over the number of
    launches.  The board's clock settles only under sustained load (after an idle gap it
    boosts, overshoots its power limit and throttles for a few milliseconds), so
    `lead_steps` whole ring steps are queued right before the timed launches, with no
    host synchronisation in between.
    `back_to_back=False` puts a dQ pass of the same chunk before each timed launch
    instead (the order of the per-chunk entry points), each launch between its own event
    pair."""
    q, k, v, do, out, lse = r["q"], r["k"], r["v"], r["do"], r["out"], r["lse"]
    c = r["lens"][0]
    kc, vc = k[:, :c], v[:, :c]
    delta = torch.empty_like(lse)
    ra.bwd_delta(out, do, delta)
    # bf16 dk/dv with accumulate = 0: the kernel writes the chunk's final rows, as in the ring
    dk = torch.empty(kc.shape, dtype=torch.bfloat16, device=q.device)
    dv = torch.empty_like(dk)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    ds = torch.empty(ra.bwd_ds_bytes(q, kc), dtype=torch.uint8, device=q.device)
    w = r["w"]
    f = 8.0 * w.B * w.Hq * q.shape[1] * c * w.D
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    torch.cuda.synchronize()
    for _ in range(lead_steps):
        r["step"]()
    if back_to_back:
        ev[0][0].record(s)
        for _ in range(launches):
            ra.bwd_chunk_dkdv_ds(q, kc, vc, do, lse, delta, dk, dv, 0, ds)
        ev[0][1].record(s)
        torch.cuda.synchronize()
        return ev[0][0].elapsed_time(ev[0][1]) / launches / 1e3, f
    for i in range(launches):
        ra.bwd_chunk_dq_ds(q, kc, ds, dq)
        ev[i][0].record(s)
        ra.bwd_chunk_dkdv_ds(q, kc, vc, do, lse, delta, dk, dv, 0, ds)
        ev[i][1].record(s)
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in ev) / launches / 1e3
    return t, f


def forward_kernel(r, lead_steps=3):
    """The forward chunk step as the ring sweep runs it after its first step: one launch of
    fwd_bf16_kernel<128, MERGE> per chunk, each merging its partial into the running fp32
    (output, LSE) state in its epilogue.  The shard's 7 merging launches (chunks in ring
    order after the local one) run back to back between one HIP event pair on the stream,
    after `lead_steps` whole ring steps queued without a host synchronisation (the clock
    settles only under sustained load); the result is the interval over the number of
    launches.  4*D flop per (query row, key, head)."""
    q, k, v = r["q"], r["k"], r["v"]
    lens, order = r["lens"], r["order"]
    starts = [sum(lens[:i]) for i in range(len(lens))]
    acc = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty_like(r["lse"])
    c0 = order[0]
    ra.fwd_chunk(q, k[:, starts[c0]:starts[c0] + lens[c0]], v[:, starts[c0]:starts[c0] + lens[c0]], acc, lse, merge=0)
    s = torch.cuda.current_stream()
    rest = order[1:]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(lead_steps):
        r["step"]()
    a.record(s)
    for c in rest:
        ra.fwd_chunk(q, k[:, starts[c]:starts[c] + lens[c]], v[:, starts[c]:starts[c] + lens[c]], acc, lse, merge=1)
    b.record(s)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / len(rest) / 1e3
    w = r["w"]
    return t, 4.0 * w.B * w.Hq * q.shape[1] * lens[rest[0]] * w.D


def backward_windows(r, reps=4):
    """HIP-event timing of the shard's backward sweep and of its parts, each rep right
    after a forward sweep, as in the step.  Rep i times (a) the whole ring backward sweep
    (one library call: delta, the 8 dK/dV launches, the dQ pass over all 8 chunks' dS),
    then, after another forward sweep, (b) the same sweep's delta and 8 dK/dV launches
    issued through the per-chunk entry points: the chunks in ring order, each writing its
    final bf16 dK/dV rows and its dS into consecutive parts of the sweep's dS region.
    Returns medians in seconds: the sweep, delta + the 8 dK/dV launches, and the mean
    dK/dV launch (the 8 launches back to back between one event pair)."""
    q, k, v, do, out, lse = r["q"], r["k"], r["v"], r["do"], r["out"], r["lse"]
    lens, order, bws = r["lens"], r["order"], r["bws"]
    starts = [sum(lens[:i]) for i in range(len(lens))]
    delta = torch.empty_like(lse)
    dk, dv = r["dk"], r["dv"]
    off = (lse.numel() * 4 + 255) // 256 * 256  # the sweep's delta rows come first in its workspace
    ds_parts = []
    for c in order:
        n = ra.bwd_ds_bytes(q, k[:, starts[c]:starts[c] + lens[c]])
        ds_parts.append(bws[off:off + n])
        off += n
    s = torch.cuda.current_stream()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    sweeps, parts, kvs = [], [], []
    torch.cuda.synchronize()
    for _ in range(reps):
        r["fwd"]()
        a, b = mk(), mk()
        a.record(s)
        r["bwd"]()
        b.record(s)
        r["fwd"]()
        e0, e1, e2 = mk(), mk(), mk()
        e0.record(s)
        ra.bwd_delta(out, do, delta)
        e1.record(s)
        for c, ds in zip(order, ds_parts):
            sl = slice(starts[c], starts[c] + lens[c])
            ra.bwd_chunk_dkdv_ds(q, k[:, sl], v[:, sl], do, lse, delta, dk[:, sl], dv[:, sl], 0, ds)
        e2.record(s)
        torch.cuda.synchronize()
        sweeps.append(a.elapsed_time(b))
        parts.append(e0.elapsed_time(e2))
        kvs.append(e1.elapsed_time(e2) / len(order))
    med = lambda xs: sorted(xs)[len(xs) // 2] / 1e3
    return med(sweeps), med(parts), med(kvs)


def image_dit_fwd(steps=20, warmup=3):
    """The image-DiT inference workload (B1, S 4608, H 24, D 128, inputs N(0,1) x 0.5): the
    forward ring sweep of the full query sequence over 4 chunks of 1152 keys, LSE-merged,
    4*B*H*S*S*D flop per sweep."""
    w = W.IMAGE_DIT_FWD
    q, k, v, _ = W.make_inputs(w)
    d = torch.device("cuda", 0)
    q, k, v = (t.to(d) for t in (q, k, v))
    ch = ra.Chunks(ra.split_sizes(w.S, w.n_chunks), list(range(w.n_chunks)))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=d)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=d)
    fws = torch.empty(q.numel() * 4 + 256, dtype=torch.uint8, device=d)
    t = timed(lambda: ra.ring_fwd(q, k, v, ch, out=out, lse=lse, workspace=fws), steps, warmup)
    # the same attention as one fused sweep over the resident keys (the all-gather variant):
    # no per-step merge, 72 key tiles per workgroup instead of 18
    one = ra.Chunks([w.S], [0])
    t1 = timed(lambda: ra.ring_fwd(q, k, v, one, out=out, lse=lse, workspace=fws), steps, warmup)
    f = 4.0 * w.B * w.Hq * w.S * w.S * w.D
    return {"B": w.B, "S": w.S, "H": w.Hq, "D": w.D, "chunks": ra.split_sizes(w.S, w.n_chunks),
            "ms_per_sweep": round(t * 1e3, 4), "tflops": round(f / t / 1e12, 2),
            "pct_of_peak": round(100.0 * f / t / 1e12 / PEAK_BF16_TFLOPS, 2),
            "allgather_single_sweep": {"ms": round(t1 * 1e3, 4), "tflops": round(f / t1 / 1e12, 2),
                                       "pct_of_peak": round(100.0 * f / t1 / 1e12 / PEAK_BF16_TFLOPS, 2)}}




def hbm_kernels(r, reps=10):
    """The HBM-bound kernels of the path at the video shard's sizes, timed with HIP events
    on the current stream: the in-device Ulysses exchange of the whole 32k sequence over 8
    simulated ranks (seq -> head, the 4096-row query shard as every rank's input), the
    standalone LSE merge of two fp32 partials and the backward's delta.  Bytes are the
    algorithmic reads + writes of one launch."""
    q, out, do, lse = r["q"], r["out"], r["do"], r["lse"]
    B, Sq, Hq, D = q.shape
    R = 8
    parts = [torch.empty((B, Sq * R, Hq // R, D), dtype=q.dtype, device=q.device) for _ in range(R)]
    o_acc = torch.randn(q.shape, dtype=torch.float32, device=q.device)
    o_part = torch.randn(q.shape, dtype=torch.float32, device=q.device)
    l_acc, l_part = torch.randn_like(lse), torch.randn_like(lse)
    delta = torch.empty_like(lse)
    cases = {
        "ulysses_exchange_8_ranks": (lambda: ra.seq_head_permute([q] * R, parts, 0, "bshd"), 2 * R * q.numel() * 2),
        "merge_lse": (lambda: ra.merge_lse(o_acc, l_acc, o_part, l_part), 3 * o_acc.numel() * 4 + 3 * lse.numel() * 4),
        "bwd_delta": (lambda: ra.bwd_delta(out, do, delta), 2 * out.numel() * 2 + lse.numel() * 4),
    }
    res = {}
    s = torch.cuda.current_stream()
    for name, (fn, nbytes) in cases.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(reps):
            fn()
        b.record(s)
        b.synchronize()
        t = a.elapsed_time(b) / reps / 1e3
        gbps = nbytes / t / 1e9
        res[name] = {"ms": round(t * 1e3, 4), "bytes": int(nbytes), "GB/s": round(gbps, 1),
                     "frac": round(gbps / HBM_PEAK_GBPS, 3)}
    return res


KERNEL_SRC = os.path.join(ROOT, "context_attention_lse_kv_amd", "csrc", "attn_bf16.hip")
PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(profile):
    """HBM bytes per launch of a kernel from its committed counter profile (the
    machine-readable lines at its end), or None when the kernel source has changed since
    the counters were taken (or the profile holds no counter figure)."""
    import hashlib
    try:
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
        vals = {}
        with open(os.path.join(PROFILES, profile)) as f:
            for line in f:
                if ":" in line:
                    k, _, v = line.partition(":")
                    vals[k.strip()] = v.strip()
        if vals.get("kernel_source_sha256_16") != sha:
            return None
        return int(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def roofline_entry(kernel, flop, seconds, method_bytes, profile, note=None):
    """One matrix-core kernel against the bf16 MFMA peak.  `method_bytes`: the HBM bytes
    the method itself needs for the launch (its inputs read once, its outputs written
    once); `traffic`: what the hardware counters measured for it (FETCH_SIZE + WRITE_SIZE,
    calibrated), and `traffic_ratio` = traffic / method_bytes (well above 1: bytes the
    route moves that the method does not need)."""
    achieved = flop / seconds / 1e12
    traffic = measured_traffic(profile)
    e = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(seconds * 1e3, 4),
         "method_flop": flop, "method_bytes": int(method_bytes), "traffic": traffic,
         "traffic_ratio": None if traffic is None else round(traffic / method_bytes, 2)}
    if note:
        e["note"] = note
    return e


def hbm_roofline_entry(kernel, nbytes, seconds, flop, profile, note=None):
    """One HBM-bound kernel against the HBM peak: `nbytes` = the bytes its algorithm moves
    per launch (each input byte read once, each output byte written once), `traffic` the
    counters' figure for it, as in roofline_entry."""
    gbps = nbytes / seconds / 1e9
    traffic = measured_traffic(profile)
    e = {"bound": "hbm", "kernel": kernel, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(gbps / HBM_PEAK_GBPS, 4), "avg_launch_ms": round(seconds * 1e3, 4), "bytes": int(nbytes),
         "flop": flop, "tflops": round(flop / seconds / 1e12, 2), "traffic": traffic,
         "traffic_ratio": None if traffic is None else round(traffic / nbytes, 3)}
    if note:
        e["note"] = note
    return e


def snapshot(r, groups=2):
    """Host copies of the timed step's results for the first `groups` kv-head groups (their
    query heads' out, lse, dq; their kv heads' dk, dv), for the parity check of the CPU
    baseline leg."""
    w = r["w"]
    nh = groups * (w.Hq // w.Hkv)
    f = lambda t: t.float().cpu()
    return {"groups": groups, "out": f(r["out"][:, :, :nh]), "lse": r["lse"][:, :nh].cpu(),
            "dq": f(r["dq"][:, :, :nh]), "dk": f(r["dk"][:, :, :groups]), "dv": f(r["dv"][:, :, :groups])}


def cpu_baseline(snap, target_s=10.0):
    """The CPU fp64 oracle, as it stands, on a bounded sample of the workload: whole
    kv-head groups of the rank-0 shard (each group = its 4 query heads, 4096 rows each,
    against all 32768 keys of the group's kv head), forward + backward, one group after
    another until at least `target_s` seconds have been spent (at most the groups in
    `snap`).  Its results are compared with the timed step's (`snap`): the parity record
    carries the whole-tensor relative error of the diffusers issue "Ring attention
    backward uses stale iteration-0 KV" (section Reproduction), the worst single D-vector
    and the max-abs error of out/dq/dk/dv, and the LSE's max abs error, against the gates
    (bf16 2e-2, LSE 1e-3)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = W.VIDEO_DIT_GQA
    q, k, v, do = W.make_inputs(w, Sq=4096)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    G = w.Hq // w.Hkv
    ref = {"out": [], "lse": [], "dq": [], "dk": [], "dv": []}
    groups, spent = 0, 0.0
    while groups < snap["groups"] and (groups == 0 or spent < target_s):
        g = groups
        kn, vn = f64(k[:, :, g:g + 1]), f64(v[:, :, g:g + 1])
        dk_g, dv_g = 0.0, 0.0
        for h in range(g * G, (g + 1) * G):
            qn, don = f64(q[:, :, h:h + 1]), f64(do[:, :, h:h + 1])
            t0 = time.perf_counter()
            o, l = oracle.attention_forward(qn, kn, vn, row_block=256)
            dq_, dk_, dv_ = oracle.attention_backward(qn, kn, vn, don, row_block=256)
            spent += time.perf_counter() - t0
            ref["out"].append(o[:, :, 0]); ref["lse"].append(l[:, 0]); ref["dq"].append(dq_[:, :, 0])
            dk_g = dk_g + dk_[:, :, 0]
            dv_g = dv_g + dv_[:, :, 0]
        ref["dk"].append(dk_g); ref["dv"].append(dv_g)
        groups += 1
    heads = groups * G
    fl = 14.0 * heads * q.shape[1] * w.S * w.D

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    def worst_vec(a, b):
        e = np.linalg.norm((a - b).reshape(-1, a.shape[-1]), axis=1)
        n = np.linalg.norm(b.reshape(-1, b.shape[-1]), axis=1)
        return float((e / np.maximum(n, 0.25 * np.sqrt(np.mean(n * n)))).max())

    par = {"sample": f"kv-head groups 0..{groups - 1} (query heads 0..{heads - 1}) of the timed step", "tensors": {}}
    for name, axis in (("out", 2), ("dq", 2), ("dk", 2), ("dv", 2)):
        want = np.stack(ref[name], axis=axis)
        got = snap[name].numpy().astype(np.float64)[:, :, :want.shape[2]]
        par["tensors"][name] = {"rel": round(rel(got, want), 6), "worst_vector": round(worst_vec(got, want), 6),
                                "max_abs": round(float(np.abs(got - want).max()), 6)}
    want_l = np.stack(ref["lse"], axis=1)
    got_l = snap["lse"].numpy().astype(np.float64)[:, :heads]
    par["lse_max_abs"] = round(float(np.abs(got_l - want_l).max()), 8)
    par["gates"] = {"rel": 2e-2, "worst_vector": 2e-2, "lse_max_abs": 1e-3}
    par["pass"] = bool(all(t["rel"] <= 2e-2 and t["worst_vector"] <= 2e-2 for t in par["tensors"].values())
                       and par["lse_max_abs"] <= 1e-3)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(fl / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host": {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": threads},
            "sample": f"oracle fwd+bwd (numpy fp64) of kv-head groups 0..{groups - 1} (query heads 0..{heads - 1}) "
                      f"of the rank-0 shard ({q.shape[1]} rows each, all {w.S} keys of the group's kv head); "
                      f"{spent:.1f} s wall; same 14*Sq*Sk*D flop count",
            "parity": par}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full", action="store_true", help="skip the full-Q sweep (extra field)")
    ap.add_argument("--no-masked", action="store_true", help="skip the key-masked sweep (extra field)")
    ap.add_argument("--no-allgather", action="store_true", help="skip the single fused sweep (extra field)")
    ap.add_argument("--no-image", action="store_true", help="skip the image-DiT forward sweep (extra field)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only launch the dominant kernel (for hardware-counter runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB, 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU and has no collectives)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (HIP device)", file=sys.stderr)
        sys.exit(2)

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "launches": 3}))
        return
    if args.kernel_only:
        r = run_workload(False, 1, 0)
        t_k, f_k = dominant_kernel(r, launches=args.steps, back_to_back=True, lead_steps=0)
        print(json.dumps({"kernel_only": True, "avg_launch_ms": round(t_k * 1e3, 4),
                          "tflops": round(f_k / t_k / 1e12, 2)}))
        return
    r = run_workload(False, args.steps, args.warmup)
    total = r["f_f"] + r["f_b"]
    value = total / r["t_step"] / 1e12
    w = r["w"]
    B, Sq, Hq, Hkv, D, Sc = w.B, int(r["q"].shape[1]), w.Hq, w.Hkv, w.D, r["lens"][0]
    n_ch = len(r["lens"])
    # the method's HBM bytes per launch: inputs read once, outputs written once (bf16 = 2 B, fp32 = 4 B)
    q_b, kv_b, st_b = B * Sq * Hq * D * 2, B * Sc * Hkv * D * 2, B * Hq * Sq * 4
    f_k = 8.0 * B * Hq * Sq * Sc * D
    t_bwd_ev, t_delta_kv, t_k = backward_windows(r)
    t_after_dq, _ = dominant_kernel(r, back_to_back=False)
    t_f, f_f1 = forward_kernel(r)
    snap = None if args.no_cpu_baseline else snapshot(r)
    dkdv = roofline_entry(
        "bwd_kv_bf16_kernel<128> (dK/dV of one ring step, storing dS: 4096 q rows x 4096 keys x 32 heads)",
        f_k, t_k, 2 * q_b + 2 * kv_b + 2 * st_b + 2 * kv_b, "bwd_kv_bf16_video_dit_shard.md",
        note="method bytes: Q, dO, K_j, V_j, lse, delta read; dK_j, dV_j (bf16) written.  The dS this route "
             "stores for the dQ pass (2 B per query row, key and head) is route traffic, not method bytes")
    dkdv["avg_launch_ms_after_dq_pass"] = round(t_after_dq * 1e3, 4)
    fwd = roofline_entry(
        "fwd_bf16_kernel<128, merge> (one ring step merging into the running state: 4096 q rows x 4096 keys x 32 heads)",
        f_f1, t_f, q_b + 2 * kv_b + 2 * (2 * q_b + st_b), "fwd_bf16_video_dit_shard.md",
        note="method bytes: Q, K_j, V_j read; the running fp32 output and LSE read and written (the LSE merge)")
    # the dQ pass: one launch per backward sweep over the dS of all chunks; its time is the sweep's
    # HIP-event time minus the same sweep's delta and 8 dK/dV launches (backward_windows)
    res_hbm = hbm_kernels(r)
    t_dq = t_bwd_ev - t_delta_kv
    ds_b = n_ch * B * Hq * Sq * Sc * 2  # the stored dS of every chunk (bf16)
    dqp = hbm_roofline_entry(
        "bwd_dqs_bf16_kernel<128> (dQ of the whole backward sweep from the stored dS of its 8 chunks)",
        ds_b + n_ch * kv_b + q_b, t_dq, 2.0 * B * Hq * Sq * w.S * D, "bwd_dqs_bf16_video_dit_shard.md",
        note="time derived: backward sweep (HIP events) minus the same sweep's delta and dK/dV launches "
             "(issued through the per-chunk entry points); bytes: the stored dS and K of every chunk read, "
             "dq (bf16) written")
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["t_step"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "video_dit_gqa_rank0_shard", "B": 1, "S": w.S, "Sq": Sq,
                   "Hq": Hq, "Hkv": Hkv, "D": D, "chunks": r["lens"], "order": r["order"],
                   "inputs": "N(0,1) seed 777, bf16"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(r["f_f"] / r["t_fwd"] / 1e12, 2),
        "bwd_tflops": round(r["f_b"] / r["t_bwd"] / 1e12, 2),
        "step_ms_events": {"median": round(sorted(r["step_ms"])[len(r["step_ms"]) // 2], 4),
                           "min": round(min(r["step_ms"]), 4), "max": round(max(r["step_ms"]), 4)},
        "fwd_ms": round(r["t_fwd"] * 1e3, 4),
        "bwd_ms": round(r["t_bwd"] * 1e3, 4),
        "roofline": dkdv,
        "rooflines": [dkdv, fwd, dqp],
        "bwd_plan": plan_record(r),
    }
    res["hbm_kernels"] = res_hbm
    del r
    torch.cuda.empty_cache()
    if not args.no_full:
        rf = run_workload(True, max(3, args.steps // 4), 1)
        tf = rf["f_f"] + rf["f_b"]
        res["full_q"] = {"Sq": int(rf["q"].shape[1]), "ms_per_step": round(rf["t_step"] * 1e3, 3),
                         "tflops": round(tf / rf["t_step"] / 1e12, 2),
                         "pct_of_peak": round(100.0 * tf / rf["t_step"] / 1e12 / PEAK_BF16_TFLOPS, 2),
                         "fwd_tflops": round(rf["f_f"] / rf["t_fwd"] / 1e12, 2),
                         "bwd_tflops": round(rf["f_b"] / rf["t_bwd"] / 1e12, 2),
                         "bwd_plan": plan_record(rf)}
        del rf
        torch.cuda.empty_cache()
    if not args.no_masked:
        rm = run_workload(False, max(3, args.steps // 2), 1, masked=True)
        tm = rm["f_f"] + rm["f_b"]
        res["masked"] = {"mask": "keys >= 30000 of 32768 masked (right padding) + 5 % random holes, seed 990",
                         "valid_key_fraction": round(float(rm["km"].float().mean()), 4),
                         "ms_per_step": round(rm["t_step"] * 1e3, 3),
                         "tflops_dense_count": round(tm / rm["t_step"] / 1e12, 2),
                         "fwd_tflops": round(rm["f_f"] / rm["t_fwd"] / 1e12, 2),
                         "bwd_tflops": round(rm["f_b"] / rm["t_bwd"] / 1e12, 2)}
        del rm
        torch.cuda.empty_cache()
    if not args.no_allgather:
        ra_ = run_workload(False, max(3, args.steps // 2), 1, single=True)
        ta = ra_["f_f"] + ra_["f_b"]
        res["allgather"] = {"chunks": [ra_["w"].S], "ms_per_step": round(ra_["t_step"] * 1e3, 3),
                            "tflops": round(ta / ra_["t_step"] / 1e12, 2),
                            "pct_of_peak": round(100.0 * ta / ra_["t_step"] / 1e12 / PEAK_BF16_TFLOPS, 2),
                            "fwd_tflops": round(ra_["f_f"] / ra_["t_fwd"] / 1e12, 2),
                            "bwd_tflops": round(ra_["f_b"] / ra_["t_bwd"] / 1e12, 2)}
        del ra_
        torch.cuda.empty_cache()
    if not args.no_image:
        res["image_dit_fwd"] = image_dit_fwd()
        torch.cuda.empty_cache()
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(snap)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
