"""CPU oracle for the paged-attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
library (no kernels, headers, helpers or constant tables); the only module both
sides see is ``workloads``, which draws seeded inputs and does none of the
arithmetic below.

Sources (the three web pages on "Inside vLLM: Anatomy of a High-Throughput LLM
Inference System"; cited by page and section, never by listing line):

* English/Chinese copy at s.sunxiunan.com, section "Scheduler" (allocate_slots,
  16-token blocks, ceil(17/16) = 2), section "Run forward pass" (slot_mapping is
  built in "prepare inputs"; all sequences are flattened into one super
  sequence, and positions plus attention masks keep every sequence to its own
  tokens), section "Chunked prefill" (a prompt of two full 8-token chunks and a
  2-token tail needs at least three engine steps), section "Prefix Caching"
  (the forward pass fills the paged KV memory of the blocks just allocated).
* Chinese translation at uml.org.cn, section "LLM Engine 构造函数" (bytes of one
  KV block of a standard, non-MLA layer: 2 for K and V, times block_size, times
  num_kv_heads, times head_size, times the dtype's bytes).
* chengshu blog copy of part 2, sections "Chunked prefill" and "Prefix Caching"
  (same chunk example; only full blocks are cached).

The pages define attention only as "each sequence attends to its own tokens"
in a causal decoder; the plainest reading, used here, is exact softmax
attention of every query token over the keys of its own sequence at positions
up to and including its own position (bottom-right causal alignment when the
sequence already holds cached context). Everything is computed in float64 by
default; ``dtype=torch.float32`` gives the single-precision variant.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
something other than itself (brute force, closed forms, SDPA with an explicit
mask, invariants, the pages' printed numbers). No function is "parity
unpinned".
"""

from __future__ import annotations

from typing import Iterable, Optional

import torch

# Default KV-cache block size in tokens (page 1, section "Scheduler").
BLOCK_SIZE = 16


# ---------------------------------------------------------------------------
# Numbers the pages print
# ---------------------------------------------------------------------------

def kv_block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    """Bytes of one KV-cache block of one standard attention layer.

    Chinese translation (uml.org.cn), section "LLM Engine 构造函数": a factor 2
    for key and value, times block_size, num_kv_heads, head_size and the
    element size (2 for bf16).
    """
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks allocate_slots takes for ``num_tokens`` new tokens: the ceiling
    of tokens over block size (page 1, section "Scheduler", allocate_slots step
    1: 17 new tokens need 2 blocks)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return -(-num_tokens // block_size)


def prefill_steps(prompt_tokens: int, chunk_tokens: int) -> int:
    """Fewest engine steps a chunked prefill of ``prompt_tokens`` takes when
    each step may add at most ``chunk_tokens`` new tokens (page 1, section
    "Chunked prefill": x-y-z with n = 8 and a 2-token z takes at least 3 steps;
    equality holds when the request is scheduled every step)."""
    if prompt_tokens < 0 or chunk_tokens <= 0:
        raise ValueError("prompt_tokens must be >= 0 and chunk_tokens > 0")
    return -(-prompt_tokens // chunk_tokens)


def chunk_plan(prompt_tokens: int, chunk_tokens: int) -> list[int]:
    """New tokens scheduled in each step of that chunked prefill: every step
    is capped at ``chunk_tokens`` (page 1, section "Chunked prefill": the
    number of new tokens is reset to the threshold when it exceeds it)."""
    plan = []
    left = prompt_tokens
    while left > 0:
        take = min(left, chunk_tokens)
        plan.append(take)
        left -= take
    return plan


# ---------------------------------------------------------------------------
# KV-cache write (the forward pass populates the paged KV memory)
# ---------------------------------------------------------------------------

def ref_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Write each new token's key and value into its slot of the paged cache.

    Page 1, section "Run forward pass" (slot_mapping is built while preparing
    inputs) and section "Prefix Caching" (the forward pass populates the KV
    blocks allocated for the request). Reading: slot s names row ``s % B`` of
    block ``s // B`` (B = block size); a negative slot marks a padding token
    that is not written. The copy is of bits, so it is exact.

    k, v: [T, Hkv, D]; slot_mapping: int64 [T]; caches [NB, B, Hkv, D], updated
    in place. Raises on a slot past the pool or on two tokens sharing a slot.
    """
    T = k.shape[0]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    seen = set()
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        if slot >= nb * bs:
            raise ValueError(f"slot {slot} of token {t} is outside the pool of {nb * bs} slots")
        if slot in seen:
            raise ValueError(f"slot {slot} is written by two tokens")
        seen.add(slot)
        block, offset = divmod(slot, bs)
        k_cache[block, offset] = k[t]
        v_cache[block, offset] = v[t]


# ---------------------------------------------------------------------------
# Paged attention over the flattened batch
# ---------------------------------------------------------------------------

def gather_sequence(cache: torch.Tensor, block_table_row: torch.Tensor, length: int) -> torch.Tensor:
    """Contiguous [length, Hkv, D] view of one sequence's cached tokens,
    gathered block by block through its block table (the "paging")."""
    bs = cache.shape[1]
    nb = blocks_needed(length, bs)
    ids = block_table_row[:nb].to(torch.long)
    if nb and (int(ids.min()) < 0 or int(ids.max()) >= cache.shape[0]):
        raise ValueError("block table names a block outside the pool")
    blocks = cache.index_select(0, ids)                 # [nb, bs, Hkv, D]
    return blocks.reshape(nb * bs, cache.shape[2], cache.shape[3])[:length]


def visible_keys(context_len: int, query_rows: torch.Tensor, seq_len: int) -> torch.Tensor:
    """Mask [R, L]: key j is visible to query row i of a sequence with
    ``context_len`` earlier tokens iff j <= context_len + i, i.e. the query at
    absolute position c + i sees itself and everything before it."""
    key_pos = torch.arange(seq_len)
    return key_pos[None, :] <= (context_len + query_rows)[:, None]


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``q_head``: the query heads are split into
    ``num_kv_heads`` groups of consecutive heads, one group per KV head."""
    return q_head // (num_q_heads // num_kv_heads)


def ref_forward(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_table: torch.Tensor, seq_lens: torch.Tensor,
                query_start_loc: torch.Tensor, scale: float,
                dtype: torch.dtype = torch.float64,
                tokens: Optional[Iterable[int]] = None) -> torch.Tensor:
    """Exact attention of the flattened batch over its paged KV cache.

    Page 1, section "Run forward pass" step 3: the sequences of one step are
    concatenated into one super sequence and masks keep each sequence to its
    own tokens. Sequence s owns query rows ``query_start_loc[s] ..
    query_start_loc[s+1]-1`` and ``seq_lens[s]`` cached tokens (its earlier
    context plus the rows just written). Query row i of the sequence sits at
    position ``c + i`` with ``c = seq_lens[s] - q_len`` and sees keys 0..c+i.
    Query head h reads KV head ``h // (Hq // Hkv)``.

    q: [T, Hq, D]; caches [NB, B, Hkv, D]; block_table int [S, MB];
    seq_lens int [S]; query_start_loc int [S+1]. Returns [T, Hq, D] in
    ``dtype``; with ``tokens`` only those flattened rows are computed and every
    other row is NaN.
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    S = seq_lens.shape[0]
    qsl = [int(x) for x in query_start_loc]
    lens = [int(x) for x in seq_lens]
    if len(qsl) != S + 1 or qsl[0] != 0 or qsl[-1] != T:
        raise ValueError("query_start_loc must run from 0 to T with S+1 entries")

    want = None if tokens is None else sorted(set(int(t) for t in tokens))
    out = torch.full((T, Hq, D), float("nan"), dtype=dtype)
    for s in range(S):
        t0, t1 = qsl[s], qsl[s + 1]
        ql = t1 - t0
        if ql < 0:
            raise ValueError("query_start_loc must not decrease")
        if ql == 0:
            continue
        rows = list(range(ql)) if want is None else [t - t0 for t in want if t0 <= t < t1]
        if not rows:
            continue
        L = lens[s]
        c = L - ql
        if c < 0:
            raise ValueError(f"sequence {s} has more query rows than cached tokens")
        K = gather_sequence(k_cache, block_table[s], L).to(dtype)   # [L, Hkv, D]
        V = gather_sequence(v_cache, block_table[s], L).to(dtype)
        ri = torch.tensor(rows, dtype=torch.long)
        Q = q[t0 + ri].to(dtype)                                     # [R, Hq, D]
        visible = visible_keys(c, ri, L)                             # [R, L]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            scores = scale * (Q[:, h, :] @ K[:, g, :].T)             # [R, L]
            scores = scores.masked_fill(~visible, float("-inf"))
            p = torch.softmax(scores, dim=-1)
            out[t0 + ri, h, :] = p @ V[:, g, :]
    return out

