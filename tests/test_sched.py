"""The native block manager and step planner (include/pa_sched.h) on the CPU.

Pins from the pages ('Inside vLLM: Anatomy of a High-Throughput LLM Inference
System'; numbers in tests/golden/pages_examples.json): ceil(17/16) = 2
blocks (section 'Scheduler', allocate_slots), the x-y-z prompt taking three
steps at 8 tokens per chunk (section 'Chunked prefill'), decode rows first
under a token budget (section 'Scheduler'), reuse of a cached prefix, its
reference counts and lazy invalidation (section 'Prefix Caching'), and the
slot mapping of section 'Run forward pass'. Every planned step is checked
against the definitions (slots from tables, lengths from counts) and the
pool's books are checked against a count of the live requests' blocks."""

import json
import os
import random

import numpy as np
import pytest

import paged_attention_kv_amd as pa
from paged_attention_kv_amd.sched import Scheduler

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))
BS = 16


def check_step(st, inp):
    """The step's inputs agree with their definitions."""
    S, T = inp.num_seqs, inp.num_tokens
    assert inp.query_start_loc[0] == 0 and inp.query_start_loc[S] == T
    assert (np.diff(inp.query_start_loc) >= 1).all()
    for s in range(S):
        t0, t1 = inp.query_start_loc[s], inp.query_start_loc[s + 1]
        L = int(inp.seq_lens[s])
        nb = -(-L // BS)
        row = inp.block_table[s]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        assert len(set(row[:nb].tolist())) == nb
        pos = inp.positions[t0:t1]
        assert (pos == np.arange(L - (t1 - t0), L)).all()
        for t in range(t0, t1):
            p = int(inp.positions[t])
            assert inp.slot_mapping[t] == row[p // BS] * BS + p % BS
    # slots written this step are distinct
    assert len(set(inp.slot_mapping.tolist())) == T


def check_books(sch, live, num_blocks):
    """Free blocks + blocks held by live requests account for the pool, and
    every block's reference count is the number of live requests holding
    it."""
    held = {}
    for rid in live:
        for b in sch.request_blocks(rid):
            held[b] = held.get(b, 0) + 1
    st = sch.stats()
    for b in range(num_blocks):
        assert sch.block_ref_count(b) == held.get(b, 0), b
    assert st.num_free_blocks == num_blocks - len(held)


def run_to_end(sch, live, num_blocks, max_steps=10_000, on_step=None):
    steps = 0
    while live and steps < max_steps:
        inp = sch.schedule()
        if inp.num_seqs == 0:
            raise AssertionError("planner made no progress")
        check_step(sch, inp)
        if on_step:
            on_step(inp)
        sch.update([int(x) % 50_000 for x in inp.request_ids * 7 + steps])
        steps += 1
        done = set(live) - {r for r in live if _alive(sch, r)}
        live.difference_update(done)
        check_books(sch, live, num_blocks)
    return steps


def _alive(sch, rid):
    try:
        sch.request_computed(rid)
        return True
    except KeyError:
        return False


def test_seventeen_tokens_take_two_blocks():
    g = GOLDEN["allocate_slots"]
    sch = Scheduler(64, max_num_batched_tokens=256)
    sch.add_request(1, list(range(g["new_tokens"])), max_new_tokens=2)
    inp = sch.schedule()
    assert inp.num_seqs == 1 and inp.num_tokens == g["new_tokens"]
    assert len(sch.request_blocks(1)) == g["blocks"] == -(-g["new_tokens"] // g["block_size"])


def test_chunked_prefill_of_x_y_z_takes_three_steps():
    g = GOLDEN["chunked_prefill"]
    n = g["chunk_tokens"]
    prompt_len = g["full_chunks"] * n + g["tail_tokens"]
    sch = Scheduler(64, max_num_batched_tokens=256, long_prefill_token_threshold=n)
    sch.add_request(7, list(range(100, 100 + prompt_len)), max_new_tokens=1)
    counts = []
    while _alive(sch, 7):
        inp = sch.schedule()
        counts.append(int(inp.num_tokens))
        check_step(sch, inp)
        sch.update([5])
    assert counts == [n, n, g["tail_tokens"]]
    assert len(counts) == g["min_engine_steps"]


def test_decode_rows_first_and_the_token_budget():
    sch = Scheduler(1024, max_num_batched_tokens=40)
    sch.add_request(1, list(range(30)), max_new_tokens=5)   # prefilled in step 0
    inp = sch.schedule()
    assert inp.request_ids.tolist() == [1] and inp.num_tokens == 30
    sch.update([9])
    sch.add_request(2, list(range(100)), max_new_tokens=3)  # longer than the budget
    inp = sch.schedule()
    # the decode row of request 1 comes first, then a 39-token chunk of 2
    assert inp.request_ids.tolist() == [1, 2]
    assert np.diff(inp.query_start_loc).tolist() == [1, 39]
    assert inp.num_tokens <= 40
    check_step(sch, inp)


def test_prefix_cache_reuse_reference_counts_and_lazy_invalidation():
    # a long prefix of n full blocks, section 'Prefix Caching'
    n = 4
    prefix = list(range(1000, 1000 + n * BS))
    NB = 32
    sch = Scheduler(NB, max_num_batched_tokens=512)
    sch.add_request(1, prefix + [1, 2, 3], max_new_tokens=1)
    sch.schedule()
    a_blocks = sch.request_blocks(1)[:n]
    assert sch.stats().prefix_hit_tokens == 0          # first request: no hits
    sch.update([4])                                     # done: blocks back to the pool
    assert not _alive(sch, 1)
    assert all(sch.block_ref_count(b) == 0 for b in a_blocks)
    assert sch.stats().num_cached_blocks == n           # still cached while free
    # second request with the same prefix: all n blocks reused, taken out of the queue
    sch.add_request(2, prefix + [7, 8], max_new_tokens=3)
    inp = sch.schedule()
    assert sch.stats().prefix_hit_tokens == n * BS
    assert sch.request_blocks(2)[:n] == a_blocks
    assert inp.num_tokens == 2 and int(inp.positions[0]) == n * BS
    assert all(sch.block_ref_count(b) == 1 for b in a_blocks)
    sch.update([9])
    # a third live request sharing the prefix: reference count 2
    sch.add_request(3, prefix + [5], max_new_tokens=1)
    sch.schedule()
    assert all(sch.block_ref_count(b) == 2 for b in a_blocks)
    sch.update([1, 2])
    sch.finish_request(2)
    assert not _alive(sch, 3)
    # the blocks are free again but cached; new requests that take every
    # free block invalidate them as they are handed out
    sch.add_request(4, list(range(5000, 5000 + NB * BS - 1)), max_new_tokens=1)
    sch.schedule()
    assert sch.stats().num_cached_blocks == 0
    sch.update([0])
    sch.add_request(5, prefix + [3], max_new_tokens=1)
    sch.schedule()
    assert sch.stats().prefix_hit_tokens == 2 * n * BS  # no new hits for request 5


def test_a_fully_cached_prompt_still_computes_its_last_token():
    prefix = list(range(64))  # exactly 4 blocks
    sch = Scheduler(16, max_num_batched_tokens=512)
    sch.add_request(1, prefix, max_new_tokens=1)
    sch.schedule()
    sch.update([0])
    sch.add_request(2, prefix, max_new_tokens=1)
    inp = sch.schedule()
    # 3 blocks reused, the 4th recomputed (the last token must produce logits)
    assert sch.stats().prefix_hit_tokens == 3 * BS
    assert inp.num_tokens == BS


def test_preemption_recomputes_and_every_request_finishes():
    NB = 12
    sch = Scheduler(NB, max_num_batched_tokens=64, long_prefill_token_threshold=24)
    live = set()
    for r in range(6):
        sch.add_request(r, [r * 1000 + i for i in range(40)], max_new_tokens=30)
        live.add(r)
    steps = run_to_end(sch, live, NB)
    st = sch.stats()
    assert st.num_finished == 6 and st.num_preemptions > 0
    assert st.num_free_blocks == NB and st.num_running == 0 and st.num_waiting == 0
    assert steps < 1000


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_workload_books_and_steps(seed):
    rng = random.Random(seed)
    NB = 96
    sch = Scheduler(NB, max_num_batched_tokens=rng.choice([32, 64, 200]),
                    max_num_seqs=rng.choice([4, 16]),
                    long_prefill_token_threshold=rng.choice([0, 8, 40]),
                    enable_prefix_caching=rng.random() < 0.7)
    prefixes = [[rng.randrange(50_000) for _ in range(BS * rng.randrange(1, 5))] for _ in range(3)]
    live = set()
    for r in range(40):
        p = rng.choice(prefixes) if rng.random() < 0.6 else []
        p = p + [rng.randrange(50_000) for _ in range(rng.randrange(1, 60))]
        sch.add_request(r, p, max_new_tokens=rng.randrange(1, 20))
        live.add(r)
    run_to_end(sch, live, NB)
    st = sch.stats()
    assert st.num_finished == 40 and st.num_free_blocks == NB


def test_argument_errors():
    assert Scheduler(8, 16) is not None
    with pytest.raises(ValueError):
        Scheduler(0, 16)
    sch = Scheduler(8, 16)
    with pytest.raises(pa.PaError):
        sch.add_request(1, [], 1)
    sch.add_request(1, [1, 2], 1)
    with pytest.raises(pa.PaError):
        sch.add_request(1, [3], 1)           # id already live
    with pytest.raises(pa.PaError):
        sch.update([0])                       # no planned step
    sch.schedule()
    with pytest.raises(pa.PaError):
        sch.schedule()                        # the planned step was not updated


def test_shared_prefix_blocks_of_a_step():
    """pa_sched_shared_prefix_blocks on hand-made step inputs: the leading
    table entries every row shares with row 0, capped so every row keeps a
    key past the prefix, 0 when a row holds other than one query token."""
    from paged_attention_kv_amd.sched import StepInputs
    z = np.zeros(0, np.int64)

    def step(qls, lens, table):
        qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
        return StepInputs(np.arange(len(qls), dtype=np.int64), qsl, np.array(lens, np.int32),
                          np.array(table, np.int32), z, z.astype(np.int32), z.astype(np.int32))

    t = [[5, 6, 7, 8, 0], [5, 6, 7, 9, 1], [5, 6, 7, 8, 2]]
    assert step([1, 1, 1], [70, 70, 70], t).shared_prefix_blocks() == 3
    assert step([1, 1, 1], [70, 48, 70], t).shared_prefix_blocks() == 2   # row 1: 48 keys
    assert step([1, 1, 1], [70, 49, 70], t).shared_prefix_blocks() == 3
    assert step([1, 2, 1], [70, 70, 70], t).shared_prefix_blocks() == 0   # not decode rows
    assert step([1, 0, 1], [70, 70, 70], t).shared_prefix_blocks() == 0
    t2 = [[5, 6, 7], [4, 6, 7]]
    assert step([1, 1], [40, 40], t2).shared_prefix_blocks() == 0       # first blocks differ
    assert step([1], [40], [[5, 6, 7]]).shared_prefix_blocks() == 2      # one row: its own
    lib = pa.load_library()
    assert lib.pa_sched_shared_prefix_blocks(None, None, None, 3, 5) == 0


def test_decode_steps_of_requests_with_a_cached_prompt_share_its_blocks():
    """Requests whose prompts start with the same 3 full blocks: once every
    row decodes, the planned step's rows share those blocks (prefix caching
    hands the same blocks to each), and the shared-prefix count says so."""
    prefix = list(range(2000, 2000 + 3 * BS))
    sch = Scheduler(64, max_num_batched_tokens=512)
    # the first request computes the prefix; the others, admitted after,
    # find its blocks in the cache
    sch.add_request(0, prefix + [0, 1, 2], max_new_tokens=6)
    counts = []
    for step in range(5):
        if step == 1:
            for r in range(1, 4):
                sch.add_request(r, prefix + [r, r + 1, 2 * r + 2], max_new_tokens=4)
        inp = sch.schedule(table_cols=8)
        check_step(sch, inp)
        counts.append(inp.shared_prefix_blocks())
        sch.update([7] * inp.num_seqs)
    # prompt step, a step with the others' prompts beside request 0's
    # decode row, then decode steps of all four
    assert counts[:2] == [0, 0] and counts[2:] == [3, 3, 3], counts
