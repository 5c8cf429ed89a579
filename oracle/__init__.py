"""CPU oracle for the paged-attention hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the HIP library never does.
"""

from .reference import (BLOCK_SIZE, blocks_needed, chunk_plan, gather_sequence,
                        kv_block_bytes, prefill_steps, ref_cache_write, ref_forward)

__all__ = ["BLOCK_SIZE", "blocks_needed", "chunk_plan", "gather_sequence", "kv_block_bytes",
           "prefill_steps", "ref_cache_write", "ref_forward"]
