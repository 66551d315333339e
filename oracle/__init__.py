"""CPU oracle for position-free paged prefill attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library
(no kernels, headers, tables or helpers); the only thing both sides consume is
the seeded input generator in ``workload``, which holds none of the method's
arithmetic.

What it computes is the plain definition from "MiniPIC: Flexible
Position-Independent Caching in <100LOC":

* §3.2.1 (score equation): score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d),
  with k~_j the unrotated key stored in the cache and pi(j) the per-request
  logical position of key j.
* §3.2.2: softmax over the visible keys, then the weighted sum of the V rows,
  which are unchanged.
* §3.1.1 and §3.3.1: the block-level attention structure that SSep, PDep and
  padding induce (``mask.py`` states the reading).

Everything is evaluated in float64 on the values the GPU receives, upcast
exactly. Every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, a library attention routine, invariants the pages fix
and brute force on tiny inputs.
"""
from .rope import inv_freq, rotate, rope_angles
from .mask import block_mask
from .attention import prefill_attention, workload_reference, visible_pair_count

__all__ = ["inv_freq", "rotate", "rope_angles", "block_mask", "prefill_attention",
           "workload_reference", "visible_pair_count"]
