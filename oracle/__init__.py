"""Plain, slow, CPU fp64 oracle for blockwise ring attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports it and
shares no code with it; the only thing both sides use is the seeded input
generator in ``workloads``, which holds none of the method's arithmetic.

Pages cited (the four pages of the reference text):
  [P1] diffusers issue "Ring attention backward uses stale iteration-0 KV from
       ctx.saved_tensors - silent gradient corruption when training with
       context parallelism"
  [P2] DeepSpeed PR "[bugfix] _DimZeroAllToAll silently fails to send grads
       under torch.compile"
  [P3] diffusers PR "Fix Flux Context Parallel Bug (Incoherent Image Generation)"
  [P4] DeepSpeed issue "[BUG] DistributedAttention produces numerically
       incorrect results vs its own SeqAllToAll-equivalent baseline when
       sequence length is not divisible by world size"

Every public function is pinned by ``tests/test_oracle_pins.py`` (closed forms,
finite differences, a library routine, invariants, page fixtures); none is
"parity unpinned".
"""
from .attention import attention_backward, attention_delta, attention_forward, merge_lse
from .permute import split_sizes, seq_to_head, head_to_seq

__all__ = [
    "attention_forward",
    "attention_backward",
    "merge_lse",
    "attention_delta",
    "split_sizes",
    "seq_to_head",
    "head_to_seq",
]
