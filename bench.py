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
dK/dV kernel of the backward chunk step), timed per launch with HIP events on
the stream it runs on, each launch placed as in the backward sweep;
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
HBM_PEAK_GBS = 8000.0
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
    return dict(w=w, lens=lens, order=order, q=q, k=k, v=v, do=do, out=out, lse=lse, t_step=t_step, t_fwd=t_fwd,
                t_bwd=t_bwd, f_f=f_f, f_b=f_b, km=km, step=step, step_ms=step_ms)


def dominant_kernel(r, launches=8, back_to_back=True, lead_steps=3):
    """The dK/dV half of the backward chunk step as the ring backward runs it (one
    kernel launch per call: it stores the step's dS for the dQ pass and writes the
    chunk's final bf16 dK/dV rows).  It executes S = Q K^T, dP = dO V^T, dV = P^T dO and
    dK = dS^T Q: 8*D flop per (query row, key) pair per head.

    The ring backward of the shard runs its 8 dK/dV launches back to back (their dS go
    to consecutive parts of the dS region; one dQ pass over all of them follows), so the
    timed launches run back to back too, each between a HIP event pair on the stream;
    the result is the mean of the per-launch event intervals.  The board's clock settles
    only under sustained load (after an idle gap it boosts, overshoots its power limit
    and throttles for a few milliseconds), so `lead_steps` whole ring steps are queued
    right before the timed launches, with no host synchronisation in between.
    `back_to_back=False` puts a dQ pass of the same chunk before each timed launch
    instead (the order of the per-chunk entry points)."""
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
    for i in range(launches):
        if not back_to_back:
            ra.bwd_chunk_dq_ds(q, kc, ds, dq)
        ev[i][0].record(s)
        ra.bwd_chunk_dkdv_ds(q, kc, vc, do, lse, delta, dk, dv, 0, ds)
        ev[i][1].record(s)
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in ev) / launches / 1e3
    return t, f


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


HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


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
PROFILE = os.path.join(ROOT, "profiles", "bwd_kv_bf16_video_dit_shard.md")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter profile,
    or None when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
        vals = {}
        with open(PROFILE) as f:
            for line in f:
                if ":" in line:
                    k, _, v = line.partition(":")
                    vals[k.strip()] = v.strip()
        if vals.get("kernel_source_sha256_16") != sha:
            return None
        return int(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(target_s=10.0):
    """The CPU fp64 oracle, as it stands, on a bounded sample of the workload: whole
    query heads of the rank-0 shard (4096 rows each, against all 32768 keys of the
    head's kv head), forward + backward, one head after another until at least
    `target_s` seconds have been spent."""
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
    heads, spent = 0, 0.0
    while spent < target_s and heads < w.Hq:
        h = heads
        qn, don = f64(q[:, :, h:h + 1]), f64(do[:, :, h:h + 1])
        kn, vn = f64(k[:, :, h // G:h // G + 1]), f64(v[:, :, h // G:h // G + 1])
        t0 = time.perf_counter()
        oracle.attention_forward(qn, kn, vn, row_block=256)
        oracle.attention_backward(qn, kn, vn, don, row_block=256)
        spent += time.perf_counter() - t0
        heads += 1
    fl = 14.0 * heads * q.shape[1] * w.S * w.D
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(fl / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host": {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": threads},
            "sample": f"oracle fwd+bwd (numpy fp64) of query heads 0..{heads - 1} of the rank-0 shard "
                      f"({q.shape[1]} rows each, all {w.S} keys of the head's kv head); {spent:.1f} s wall; "
                      f"same 14*Sq*Sk*D flop count"}


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
    t_k, f_k = dominant_kernel(r)
    t_after_dq, _ = dominant_kernel(r, back_to_back=False)
    achieved = f_k / t_k / 1e12
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
        "config": {"workload": "video_dit_gqa_rank0_shard", "B": 1, "S": r["w"].S, "Sq": int(r["q"].shape[1]),
                   "Hq": r["w"].Hq, "Hkv": r["w"].Hkv, "D": r["w"].D, "chunks": r["lens"], "order": r["order"],
                   "inputs": "N(0,1) seed 777, bf16"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(r["f_f"] / r["t_fwd"] / 1e12, 2),
        "bwd_tflops": round(r["f_b"] / r["t_bwd"] / 1e12, 2),
        "step_ms_events": {"median": round(sorted(r["step_ms"])[len(r["step_ms"]) // 2], 4),
                           "min": round(min(r["step_ms"]), 4), "max": round(max(r["step_ms"]), 4)},
        "fwd_ms": round(r["t_fwd"] * 1e3, 4),
        "bwd_ms": round(r["t_bwd"] * 1e3, 4),
        "roofline": {"bound": "mfma", "kernel": "bwd_kv_bf16_kernel<128> (dK/dV of one ring step, storing dS: 4096 q rows x 4096 keys x 32 heads)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(t_k * 1e3, 4),
                     "avg_launch_ms_after_dq_pass": round(t_after_dq * 1e3, 4),
                     "traffic": measured_traffic()},
    }
    res["hbm_kernels"] = hbm_kernels(r)
    del r
    torch.cuda.empty_cache()
    if not args.no_full:
        rf = run_workload(True, max(3, args.steps // 4), 1)
        tf = rf["f_f"] + rf["f_b"]
        res["full_q"] = {"Sq": int(rf["q"].shape[1]), "ms_per_step": round(rf["t_step"] * 1e3, 3),
                         "tflops": round(tf / rf["t_step"] / 1e12, 2),
                         "pct_of_peak": round(100.0 * tf / rf["t_step"] / 1e12 / PEAK_BF16_TFLOPS, 2),
                         "fwd_tflops": round(rf["f_f"] / rf["t_fwd"] / 1e12, 2),
                         "bwd_tflops": round(rf["f_b"] / rf["t_bwd"] / 1e12, 2)}
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
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
