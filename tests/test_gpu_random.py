"""Seeded random batches through the C ABI against the CPU oracle: each case
draws head counts, head size, a mix of rows (empty, decode, a few query
tokens, chunks with and without prior context), the length hints (tight,
none, loose), the decode schedule flag, the serial flag and the entry point
(pa_write_and_forward, or pa_cache_write then pa_forward_ex); and random
shared-prefix batches through both shared-prefix entry points. Every row
with query tokens is checked against the oracle to the same bar as the
other parity tests, and the pool's written blocks bit for bit."""

import random

import pytest
import torch

import paged_attention_kv_amd as pa
import workloads as wl
from oracle_view import OracleView, assert_close, assert_pool_written

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

HEADS = [(8, 8), (16, 8), (32, 8), (32, 4), (64, 4), (16, 1), (32, 16)]
QLENS = [0, 1, 1, 1, 1, 2, 3, 4, 7, 16, 33, 64, 130, 700]


def draw_case(seed):
    r = random.Random(seed)
    hq, hkv = r.choice(HEADS)
    d = r.choice([64, 128])
    short = r.random() < 0.25  # every row within 128 keys
    nrows = r.randint(1, 40)
    rows = []
    for _ in range(nrows):
        ql = r.choice(QLENS)
        cmax = 128 - max(ql, 1) if short else 3000
        if cmax < 0:
            ql, cmax = r.choice([1, 2, 5, 40]), 60
        c = r.choice([0, r.randint(0, cmax), r.randint(0, cmax), cmax])
        # at least 8 earlier keys, so that every query token sees 9 or
        # more: with a few keys an output is nearly one V value, and bf16
        # rounding of a value past 4 in magnitude alone can exceed the bar
        # (a 16-token prompt's sixth token, 6 keys: exact 4.199, correctly
        # rounded 4.1875, the kernel's output)
        rows.append((ql, max(c, 8)))
    if all(q == 0 for q, _ in rows):
        rows[0] = (1, rows[0][1])
    opts = dict(
        hints=r.choice(["tight", "tight", "none", "loose"]),
        schedule=r.choice([None, None, "even", "partitioned"]),
        serial=r.random() < 0.25,
        fused=r.random() < 0.6,
    )
    return hq, hkv, d, rows, opts


@pytest.mark.parametrize("seed", range(64))
def test_random_batch_against_the_oracle(seed):
    hq, hkv, d, rows, opts = draw_case(7000 + seed)
    spec = wl.custom(f"random{seed}", hq, hkv, d, rows=rows, seed=7100 + seed)
    print(f"\n[case] random {seed}: Hq={hq} Hkv={hkv} D={d} {opts} rows={rows}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, [s for s in range(spec.num_seqs) if spec.q_lens[s] > 0])
    k0, v0 = case.k_cache.clone(), case.v_cache.clone()
    hints = {}
    if opts["hints"] == "tight":
        hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
    elif opts["hints"] == "loose":
        cap = spec.max_blocks_per_seq * spec.block_size
        hints = dict(max_query_len=min(2 * max(spec.q_lens), spec.num_tokens),
                     max_seq_len=min(2 * max(spec.seq_lens), cap))
    kw = dict(decode_schedule=opts["schedule"], serial=opts["serial"], **hints)
    if opts["fused"]:
        out = pa.write_and_forward(case.k, case.v, case.slot_mapping, case.k_cache, case.v_cache,
                                   case.q, case.block_table, case.seq_lens,
                                   case.query_start_loc, case.scale, **kw)
    else:
        pa.cache_write(case.k, case.v, case.slot_mapping, case.k_cache, case.v_cache)
        out = pa.forward(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                         case.query_start_loc, case.scale, **kw)
    torch.cuda.synchronize()
    assert_pool_written(case.k_cache, case.v_cache, k0, v0, case.k, case.v, case.slot_mapping)
    r, want = view.expect()
    assert_close(out.cpu()[r], want, spec.name)


@pytest.mark.parametrize("seed", range(16))
def test_random_shared_prefix_batch_against_the_oracle(seed):
    """Seeded random shared-prefix batches (head counts, head size, prefix
    length, row count, each row's own tokens past the prefix), through
    pa_write_and_forward_shared_prefix or pa_cache_write then
    pa_forward_shared_prefix: every row against the oracle, the pool bit
    for bit."""
    r = random.Random(9000 + seed)
    hq, hkv = r.choice(HEADS)
    d = r.choice([64, 128])
    pb = r.choice([1, 2, 7, 16, 33, 64])
    own = [r.choice([1, 2, 15, 16, 17, r.randint(1, 600)]) for _ in range(r.randint(1, 300))]
    rows = [(1, 16 * pb + n - 1) for n in own]
    spec = wl.custom(f"random_sp{seed}", hq, hkv, d, rows=rows, seed=9100 + seed,
                     shared_prefix_blocks=pb)
    fused = r.random() < 0.5
    print(f"\n[case] random shared prefix {seed}: Hq={hq} Hkv={hkv} D={d} prefix={pb} "
          f"rows={len(rows)} fused={fused}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    k0, v0 = case.k_cache.clone(), case.v_cache.clone()
    args = (case.q, case.block_table, case.seq_lens, case.query_start_loc, case.scale, pb)
    if fused:
        out = pa.write_and_forward_shared_prefix(case.k, case.v, case.slot_mapping, case.k_cache,
                                                 case.v_cache, *args,
                                                 max_seq_len=max(spec.seq_lens))
    else:
        pa.cache_write(case.k, case.v, case.slot_mapping, case.k_cache, case.v_cache)
        out = pa.forward_shared_prefix(case.q, case.k_cache, case.v_cache, *args[1:],
                                       max_seq_len=max(spec.seq_lens))
    torch.cuda.synchronize()
    assert_pool_written(case.k_cache, case.v_cache, k0, v0, case.k, case.v, case.slot_mapping)
    rr, want = view.expect()
    assert_close(out.cpu()[rr], want, spec.name)
