"""CPU fp64 oracle for fused ring + current causal attention.

TEST INFRASTRUCTURE, not product code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library never imports it,
links it or shares code with it; the only thing both sides share is the seeded
input generator in ``workloads/``, which holds none of the method's arithmetic.

The method is the one described on the vLLM tpu-inference pull request "PCP:
in-kernel ring cache phase, fused with the current phase" (its Summary and
Design sections): one launch walks the P striped cache shards ("ring rounds")
and then the causal current chunk through a single online softmax, with no
LSE merge.  What that launch computes has a plain definition -- softmax
attention of every real chunk row over [whole cache ; current tokens up to
and including itself] -- and ``attention.attention_rows`` is that definition
written out in fp64.  ``attention.ring_online`` follows the method's own
steps (shard visits in ring order, then current blocks, one running
(m, l, acc)) so that the two can pin each other.  ``stripe`` holds the shard
map that the strided KV-cache write uses.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (brute force, closed forms, hand-worked fixtures,
invariances); see the docstring of each test module.  Pad-row outputs are
"parity unpinned": the pages say pad rows are discarded by the caller, so
there is nothing to compare them with.
"""
from .stripe import (shard_lengths, stripe_position, stripe, destripe,
                     kv_cache_write_ref)
from .attention import (bf16_bits_to_f64, attention_rows, ring_attention,
                        ring_online, two_pass_merge, rank_positions, zigzag_pieces)

__all__ = ["shard_lengths", "stripe_position", "stripe", "destripe",
           "kv_cache_write_ref", "bf16_bits_to_f64", "attention_rows",
           "ring_attention", "ring_online", "two_pass_merge", "rank_positions",
           "zigzag_pieces"]
