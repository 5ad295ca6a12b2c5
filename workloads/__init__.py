"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds shapes and random numbers only - none of the method's
arithmetic - so that the HIP path and the CPU oracle can be fed the very same
values without sharing any code.

Recipe (same for every workload): a CPU ``torch.Generator`` seeded with
``seed`` (777 by default, the seed of the gradient-parity reproduction in the
diffusers issue "Ring attention backward uses stale iteration-0 KV",
section "Reproduction") draws q, k, v, dout in that order as N(0, 1) float32,
each optionally multiplied by ``mult`` (0.5 for the image-DiT workload), and is
then rounded to the workload dtype.  The oracle receives these exact rounded
values upcast to float64; the GPU receives them by copy.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int            # full sequence length (keys)
    Hq: int
    Hkv: int
    D: int
    dtype: str        # "bf16" | "f32"
    n_chunks: int     # K/V chunks the ring sweeps
    chunk_lens: Tuple[int, ...]   # lengths stated for the workload (data, not computed)
    seq_first: bool = False
    mult: float = 1.0
    fwd_only: bool = False
    note: str = ""


# The five workloads.  chunk_lens are written out as data; each side derives its own
# split and the tests check both against these numbers.
TINY_F32 = Workload("tiny_f32_ring", 1, 256, 2, 2, 64, "f32", 2, (128, 128),
                    note="B1 S256 H2/2 D64 fp32, 2 chunks of 128, scale 1/8")
BF16_RING2 = Workload("bf16_ring2", 2, 512, 8, 8, 64, "bf16", 2, (256, 256),
                      note="B2 S512 H8 D64 bf16, ring 2, Q shard = S/2")
BF16_RING4 = Workload("bf16_ring4", 2, 512, 8, 8, 64, "bf16", 4, (128, 128, 128, 128),
                      note="B2 S512 H8 D64 bf16, ring 4, Q shard = S/4")
UNEVEN_SEQFIRST = Workload("uneven_seqfirst_ulysses", 2, 1000, 8, 8, 64, "bf16", 3, (334, 333, 333),
                           seq_first=True,
                           note="[S,B,H,D] S1000 B2 H8 D64 bf16, chunks 334/333/333, Ulysses permute")
IMAGE_DIT_FWD = Workload("image_dit_fwd", 1, 4608, 24, 24, 128, "bf16", 4, (1152,) * 4,
                         mult=0.5, fwd_only=True,
                         note="B1 S4608 (4096 image + 512 text) H24 D128 bf16, x0.5, 4 chunks, fwd")
VIDEO_DIT_GQA = Workload("video_dit_gqa", 1, 32768, 32, 8, 128, "bf16", 8, (4096,) * 8,
                         note="B1 S32768 Hq32 Hkv8 D128 bf16, 8 chunks of 4096, Q shard 4096 / full Q")

ALL = [TINY_F32, BF16_RING2, BF16_RING4, UNEVEN_SEQFIRST, IMAGE_DIT_FWD, VIDEO_DIT_GQA]


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_inputs(w: Workload, seed: int = 777, Sq: Optional[int] = None):
    """Return CPU tensors (q, k, v, dout) of workload ``w``.

    q and dout have ``Sq`` rows (default: the full S); k, v have S rows.
    Layout is [B,S,H,D], or [S,B,H,D] when ``w.seq_first``.
    """
    g = torch.Generator().manual_seed(seed)
    Sq = w.S if Sq is None else Sq
    if w.seq_first:
        qs, ks = (Sq, w.B, w.Hq, w.D), (w.S, w.B, w.Hkv, w.D)
    else:
        qs, ks = (w.B, Sq, w.Hq, w.D), (w.B, w.S, w.Hkv, w.D)
    dt = torch_dtype(w.dtype)
    out = []
    for shape in (qs, ks, ks, qs):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.mult != 1.0:
            t = t * w.mult
        out.append(t.to(dt))
    return tuple(out)


def randn(shape, seed, dtype="f32", mult=1.0):
    """One seeded N(0,1) tensor (for small ad-hoc test shapes)."""
    g = torch.Generator().manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        t = t * mult
    return t.to(torch_dtype(dtype))


def make_key_mask(B, S, seed, p_keep=0.8, valid_len=None, masked_ranges=()):
    """Seeded key-validity mask [B, S] (bool, True = the key takes part), CPU.

    Each key is kept with probability ``p_keep`` (independent draws from a CPU
    ``torch.Generator`` seeded with ``seed``); ``valid_len[b]`` additionally masks
    keys >= valid_len[b] of batch b (right padding, as a padded text sequence would
    have); ``masked_ranges`` is a list of (b, start, stop) key ranges masked as a
    whole.  Shapes and random numbers only.
    """
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((B, S), generator=g) < p_keep
    if valid_len is not None:
        for b, n in enumerate(valid_len):
            m[b, int(n):] = False
    for b, a, z in masked_ranges:
        m[b, a:z] = False
    return m
