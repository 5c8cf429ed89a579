"""Seeded synthetic inputs for the paged-attention hot path.

This module only draws inputs: lengths, block placement, the slot of every new
token, and N(0, 1) bf16 values. It holds none of the arithmetic of the method
(no cache write, no attention). Both the oracle and the HIP library are fed
from it, and it imports neither.

The five named workloads follow the configurations the work is graded on:

1. tiny: 2 prefill sequences of 5 and 8 tokens, 32 q / 4 kv heads, D 64,
   a 64-block pool placed by a seeded permutation.
2. decode: 64 sequences with 1 query token, context U{512..2048}, 32 q / 4 kv
   heads, D 64, 100k-block pool, random placement.
3. mixed: 256 decode rows (context U{256..8192}) then 4 chunked-prefill rows
   of 1984 tokens with prior context U{0..4096} (8192 new tokens in all),
   32 q / 8 kv heads, D 128.
4. long decode: 16 sequences at context 32768, 64 q / 8 kv heads, D 128.
5. prefix-shared decode: 256 rows whose tables share the same 256 blocks
   (a 4096-token prefix) followed by 8 private blocks (a 128-token suffix whose
   last token is this step's query), 32 q / 8 kv heads, D 128.

Reading of the pages used to place tokens: a sequence's cached tokens fill its
table's blocks in order, 16 per block; its new (query) tokens are its last
``q_len`` positions and go to slot ``table[pos // 16] * 16 + pos % 16``
(page 1, section "Run forward pass": block tables and slot_mapping are built
while preparing inputs).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

BLOCK_SIZE = 16
# Large finite value written into every cache row no sequence may read.
POISON = 30000.0
# Seeds: configuration i draws lengths and placement from 1000+i and values
# from 2000+i.
SEED_LAYOUT_BASE = 1000
SEED_VALUES_BASE = 2000


@dataclass(frozen=True)
class Spec:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q_lens: Tuple[int, ...]
    seq_lens: Tuple[int, ...]
    shared_prefix_blocks: int = 0
    block_size: int = BLOCK_SIZE
    seed_layout: int = 0
    seed_values: int = 0
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return len(self.q_lens)

    @property
    def num_tokens(self) -> int:
        return sum(self.q_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def ctx_lens(self) -> Tuple[int, ...]:
        return tuple(L - q for L, q in zip(self.seq_lens, self.q_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_size)

    def check(self) -> None:
        if self.num_q_heads % self.num_kv_heads:
            raise ValueError("q heads must be a multiple of kv heads")
        if len(self.q_lens) != len(self.seq_lens):
            raise ValueError("q_lens and seq_lens differ in length")
        for ql, L in zip(self.q_lens, self.seq_lens):
            if not (0 <= ql <= L <= self.max_blocks_per_seq * self.block_size):
                raise ValueError(f"bad row q_len={ql} seq_len={L}")
        need = self.shared_prefix_blocks + sum(
            -(-L // self.block_size) - self.shared_prefix_blocks for L in self.seq_lens)
        if need > self.num_blocks:
            raise ValueError(f"pool of {self.num_blocks} blocks is too small ({need} needed)")


def _uniform(g: torch.Generator, lo: int, hi: int, n: int) -> List[int]:
    """n integers uniform on lo..hi inclusive."""
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def config(i: int) -> Spec:
    """The named workload i (1..5)."""
    g = torch.Generator().manual_seed(SEED_LAYOUT_BASE + i)
    common = dict(seed_layout=SEED_LAYOUT_BASE + i, seed_values=SEED_VALUES_BASE + i)
    if i == 1:
        return Spec("tiny", 32, 4, 64, num_blocks=64, max_blocks_per_seq=4,
                    q_lens=(5, 8), seq_lens=(5, 8),
                    description="2 prefill sequences of 5 and 8 tokens; 32q/4kv, D64; 64-block pool",
                    **common)
    if i == 2:
        L = _uniform(g, 512, 2048, 64)
        return Spec("decode", 32, 4, 64, num_blocks=100_000, max_blocks_per_seq=128,
                    q_lens=(1,) * 64, seq_lens=tuple(L),
                    description="64 decode rows, context U[512,2048]; 32q/4kv, D64; 100k-block pool",
                    **common)
    if i == 3:
        dec = _uniform(g, 256, 8192, 256)
        ctx = _uniform(g, 0, 4096, 4)
        return Spec("mixed", 32, 8, 128, num_blocks=150_000, max_blocks_per_seq=512,
                    q_lens=(1,) * 256 + (1984,) * 4,
                    seq_lens=tuple(dec) + tuple(c + 1984 for c in ctx),
                    description=("256 decode rows (context U[256,8192]) + 4 prefill chunks of 1984 "
                                 "tokens (prior context U[0,4096]); 32q/8kv, D128; 150k-block pool"),
                    **common)
    if i == 4:
        return Spec("long_decode", 64, 8, 128, num_blocks=65_536, max_blocks_per_seq=2048,
                    q_lens=(1,) * 16, seq_lens=(32768,) * 16,
                    description="16 decode rows at context 32768; 64q/8kv, D128; 65536-block pool",
                    **common)
    if i == 5:
        return Spec("prefix_shared", 32, 8, 128, num_blocks=65_536, max_blocks_per_seq=264,
                    q_lens=(1,) * 256, seq_lens=(4224,) * 256, shared_prefix_blocks=256,
                    description=("256 decode rows sharing 256 prefix blocks (4096 tokens) + 8 private "
                                 "blocks (128 tokens); 32q/8kv, D128; 65536-block pool"),
                    **common)
    raise ValueError(f"no workload {i}")


def spec_decode(q_len: int = 4) -> Spec:
    """Rows verifying speculated tokens: 256 rows of q_len query tokens each,
    prior contexts drawn like the mixed step's decode rows (U[256, 8192]),
    32q/8kv, D128, 150k-block pool."""
    g = torch.Generator().manual_seed(SEED_LAYOUT_BASE + 6)
    ctx = _uniform(g, 256, 8192, 256)
    return Spec("spec_decode", 32, 8, 128, num_blocks=150_000, max_blocks_per_seq=520,
                q_lens=(q_len,) * 256, seq_lens=tuple(c + q_len for c in ctx),
                description=(f"256 rows of {q_len} query tokens (speculative verify), prior "
                             "context U[256,8192]; 32q/8kv, D128; 150k-block pool"),
                seed_layout=SEED_LAYOUT_BASE + 6, seed_values=SEED_VALUES_BASE + 6)


def custom(name: str, num_q_heads: int, num_kv_heads: int, head_size: int,
           rows: Sequence[Tuple[int, int]], seed: int, num_blocks: Optional[int] = None,
           max_blocks_per_seq: Optional[int] = None, shared_prefix_blocks: int = 0) -> Spec:
    """A workload from explicit rows of (q_len, prior context length)."""
    q_lens = tuple(int(q) for q, _ in rows)
    seq_lens = tuple(int(q) + int(c) for q, c in rows)
    mb = max_blocks_per_seq or max(1, max(-(-L // BLOCK_SIZE) for L in seq_lens))
    need = shared_prefix_blocks + sum(-(-L // BLOCK_SIZE) - shared_prefix_blocks for L in seq_lens)
    nb = num_blocks or max(8, 2 * need)
    spec = Spec(name, num_q_heads, num_kv_heads, head_size, num_blocks=nb, max_blocks_per_seq=mb,
                q_lens=q_lens, seq_lens=seq_lens, shared_prefix_blocks=shared_prefix_blocks,
                seed_layout=seed, seed_values=seed + 1)
    spec.check()
    return spec


@dataclass
class Layout:
    block_table: torch.Tensor        # int32 [S, MB], padding entries = table_pad
    slot_mapping: torch.Tensor       # int64 [T]
    query_start_loc: torch.Tensor    # int32 [S+1]
    seq_lens: torch.Tensor           # int32 [S]
    context_slots: torch.Tensor      # int64 [*] slots holding earlier context (readable before the write)


def build_layout(spec: Spec, table_pad: int = -1) -> Layout:
    """Block placement (one seeded permutation of the pool, consumed sequence
    by sequence), the per-token slots of this step's new tokens, and the slots
    of every sequence's earlier context. CPU tensors."""
    spec.check()
    bs = spec.block_size
    S, MB = spec.num_seqs, spec.max_blocks_per_seq
    g = torch.Generator().manual_seed(spec.seed_layout * 7919 + 17)
    perm = torch.randperm(spec.num_blocks, generator=g)
    table = torch.full((S, MB), table_pad, dtype=torch.int32)
    used = 0
    shared = perm[:spec.shared_prefix_blocks]
    used += spec.shared_prefix_blocks
    for s, L in enumerate(spec.seq_lens):
        nb = -(-L // bs)
        own = nb - spec.shared_prefix_blocks
        if own < 0:
            raise ValueError("sequence shorter than the shared prefix")
        table[s, :spec.shared_prefix_blocks] = shared.to(torch.int32)
        table[s, spec.shared_prefix_blocks:nb] = perm[used:used + own].to(torch.int32)
        used += own
    slots = []
    ctx_slots = []
    for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
        row = table[s].to(torch.int64)
        pos_new = torch.arange(L - ql, L, dtype=torch.int64)
        slots.append(row[pos_new // bs] * bs + pos_new % bs)
        pos_old = torch.arange(0, L - ql, dtype=torch.int64)
        ctx_slots.append(row[pos_old // bs] * bs + pos_old % bs)
    qsl = torch.zeros(S + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(spec.q_lens, dtype=torch.int64), 0).to(torch.int32)
    return Layout(block_table=table,
                  slot_mapping=torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int64),
                  query_start_loc=qsl,
                  seq_lens=torch.tensor(spec.seq_lens, dtype=torch.int32),
                  context_slots=torch.unique(torch.cat(ctx_slots)) if ctx_slots
                  else torch.zeros(0, dtype=torch.int64))


@dataclass
class Case:
    spec: Spec
    q: torch.Tensor              # bf16 [T, Hq, D]
    k: torch.Tensor              # bf16 [T, Hkv, D]  this step's new keys
    v: torch.Tensor              # bf16 [T, Hkv, D]
    slot_mapping: torch.Tensor   # int64 [T]
    k_cache: torch.Tensor        # bf16 [NB, 16, Hkv, D] earlier context only; all else poisoned
    v_cache: torch.Tensor
    block_table: torch.Tensor    # int32 [S, MB]
    seq_lens: torch.Tensor       # int32 [S]
    query_start_loc: torch.Tensor  # int32 [S+1]
    scale: float
    context_slots: torch.Tensor = field(repr=False, default=None)


def make_case(spec: Spec, device: str = "cpu", poison: float = POISON, table_pad: int = -1,
              values_seed: Optional[int] = None) -> Case:
    """Materialise a workload on ``device``.

    Every cache row outside the sequences' earlier context holds ``poison``
    (a large finite value, or NaN), including the rows this step's tokens
    will be written to, so a missed write or a read past a sequence shows up
    in the output.
    """
    lay = build_layout(spec, table_pad=table_pad)
    T, Hq, Hkv, D = spec.num_tokens, spec.num_q_heads, spec.num_kv_heads, spec.head_size
    NB, bs = spec.num_blocks, spec.block_size
    gen = torch.Generator(device=device).manual_seed(spec.seed_values if values_seed is None
                                                     else values_seed)
    bf = torch.bfloat16

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).to(bf)

    q = randn(T, Hq, D)
    k = randn(T, Hkv, D)
    v = randn(T, Hkv, D)
    k_cache = torch.empty((NB, bs, Hkv, D), dtype=bf, device=device)
    v_cache = torch.empty((NB, bs, Hkv, D), dtype=bf, device=device)
    # Fill block by block-chunk to bound the float32 staging buffer.
    chunk = max(1, (1 << 26) // (bs * Hkv * D))
    for cache in (k_cache, v_cache):
        for b0 in range(0, NB, chunk):
            b1 = min(NB, b0 + chunk)
            cache[b0:b1] = randn(b1 - b0, bs, Hkv, D)
    live = torch.zeros(NB * bs, dtype=torch.bool)
    live[lay.context_slots] = True
    dead = (~live).to(device)
    for cache in (k_cache, v_cache):
        flat = cache.view(NB * bs, Hkv, D)
        flat[dead] = torch.tensor(poison, dtype=bf, device=device)
    return Case(spec=spec, q=q, k=k, v=v,
                slot_mapping=lay.slot_mapping.to(device),
                k_cache=k_cache, v_cache=v_cache,
                block_table=lay.block_table.to(device),
                seq_lens=lay.seq_lens.to(device),
                query_start_loc=lay.query_start_loc.to(device),
                scale=spec.scale, context_slots=lay.context_slots)


def sequences_subset(case: Case, seqs: Sequence[int]):
    """CPU copies of just what sequences ``seqs`` read, with the pool
    compacted to their blocks and their tables renumbered. Returns
    (q, k_cache, v_cache, block_table, seq_lens, query_start_loc, token_map)
    where token_map[i] is the flattened row (in the full batch) of row i of
    the subset. Plumbing only: nothing here computes attention."""
    bs = case.spec.block_size
    qsl = case.query_start_loc.cpu().tolist()
    lens = case.seq_lens.cpu().tolist()
    bt = case.block_table.cpu()
    ids = []
    for s in seqs:
        nb = -(-lens[s] // bs)
        ids.append(bt[s, :nb].to(torch.int64))
    uniq = torch.unique(torch.cat(ids)) if ids else torch.zeros(0, dtype=torch.int64)
    remap = {int(b): i for i, b in enumerate(uniq.tolist())}
    idx = uniq.to(case.k_cache.device)
    kc = case.k_cache.index_select(0, idx).cpu()
    vc = case.v_cache.index_select(0, idx).cpu()
    nbmax = max(1, max(-(-lens[s] // bs) for s in seqs))
    table = torch.full((len(seqs), nbmax), -1, dtype=torch.int32)
    token_map = []
    new_qsl = [0]
    for i, s in enumerate(seqs):
        nb = -(-lens[s] // bs)
        table[i, :nb] = torch.tensor([remap[int(b)] for b in bt[s, :nb].tolist()], dtype=torch.int32)
        token_map.extend(range(qsl[s], qsl[s + 1]))
        new_qsl.append(new_qsl[-1] + qsl[s + 1] - qsl[s])
    tm = torch.tensor(token_map, dtype=torch.int64)
    q = case.q.index_select(0, tm.to(case.q.device)).cpu()
    return (q, kc, vc, table, torch.tensor([lens[s] for s in seqs], dtype=torch.int32),
            torch.tensor(new_qsl, dtype=torch.int32), tm)
