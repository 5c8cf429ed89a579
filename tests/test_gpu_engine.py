"""End to end on the GPU: the native step planner (block pool, prefix cache,
chunked prefill, preemption) feeds pa_write_and_forward step after step (and
pa_write_and_forward_shared_prefix on steps whose decode rows share a
cached prefix).

Every token's K, V and q are a fixed function of the tokens up to it (as in
a causal model), so a block reused from the prefix cache holds exactly the
values a recompute would write. After each step: every cache row that any
scheduled row reads holds its token's K/V bit-exactly, and every output row
matches the oracle run on the request's unpaged sequence (max abs <= 1e-2,
mean abs <= 1e-3)."""

import random

import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_amd as pa
from paged_attention_kv_amd.sched import Scheduler

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BS = 16


def token_values(tokens, pos, Hq, Hkv, D):
    """(q [Hq, D], k [Hkv, D], v [Hkv, D]) of position pos: seeded by a hash
    chain over tokens[0..pos], rounded to bf16."""
    h = 1469598103934665603
    for t in tokens[:pos + 1]:
        h = ((h ^ (int(t) & 0xFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    g = torch.Generator().manual_seed(h & 0x7FFFFFFFFFFFFFFF)
    x = torch.randn((Hq + 2 * Hkv) * D, generator=g).to(torch.bfloat16)
    x = x.view(Hq + 2 * Hkv, D)
    return x[:Hq], x[Hq:Hq + Hkv], x[Hq + Hkv:]


class Mirror:
    """The test's own copy of every request's tokens and of their values."""

    def __init__(self, Hq, Hkv, D):
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.tokens = {}
        self.vals = {}

    def add(self, rid, prompt):
        self.tokens[rid] = list(prompt)
        self.vals[rid] = []

    def values(self, rid, pos):
        vs = self.vals[rid]
        while len(vs) <= pos:
            vs.append(token_values(self.tokens[rid], len(vs), self.Hq, self.Hkv, self.D))
        return vs[pos]


def run_engine(Hq, Hkv, D, num_blocks, budget, threshold, caching, seed, n_req=12,
               new_tokens=(2, 10), one_prefix=False, shared_prefix_calls=False,
               first_alone_steps=0):
    rng = random.Random(seed)
    sch = Scheduler(num_blocks, max_num_batched_tokens=budget, max_num_seqs=8,
                    long_prefill_token_threshold=threshold, enable_prefix_caching=caching)
    mir = Mirror(Hq, Hkv, D)
    prefixes = [[rng.randrange(30_000) for _ in range(BS * rng.randrange(2, 4))] for _ in range(2)]
    pending = []
    for r in range(n_req):
        head = prefixes[0] if one_prefix else (rng.choice(prefixes) if rng.random() < 0.7 else [])
        p = head + [rng.randrange(30_000) for _ in range(rng.randrange(3, 50))]
        pending.append((r, p, rng.randrange(*new_tokens)))
    k_cache = torch.full((num_blocks, BS, Hkv, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    v_cache = torch.full_like(k_cache, float("nan"))
    scale = D ** -0.5
    MB = num_blocks
    live = set()
    steps = checked_rows = shared_steps = 0
    while pending or live:
        # requests arrive over the first steps
        while pending and (steps % 2 == 0 or not live) and \
                (steps >= first_alone_steps or not live):
            r, p, m = pending.pop(0)
            sch.add_request(r, p, m)
            mir.add(r, p)
            live.add(r)
            if steps % 4:
                break
        inp = sch.schedule(table_cols=MB)
        S, T = inp.num_seqs, inp.num_tokens
        assert S > 0, "the planner made no progress"
        q = torch.empty((T, Hq, D), dtype=torch.bfloat16)
        k = torch.empty((T, Hkv, D), dtype=torch.bfloat16)
        v = torch.empty((T, Hkv, D), dtype=torch.bfloat16)
        for s in range(S):
            rid = int(inp.request_ids[s])
            for t in range(inp.query_start_loc[s], inp.query_start_loc[s + 1]):
                q[t], k[t], v[t] = mir.values(rid, int(inp.positions[t]))
        dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)  # noqa: E731
        qsl = dev(inp.query_start_loc, torch.int32)
        lens = dev(inp.seq_lens, torch.int32)
        table = dev(inp.block_table, torch.int32)
        slots = dev(inp.slot_mapping, torch.int64)
        ql = np.diff(inp.query_start_loc)
        pb = inp.shared_prefix_blocks() if shared_prefix_calls else 0
        if pb > 0:
            # every row decodes and shares the leading pb blocks: the prefix
            # is attended once for all rows, the write in the same launch
            out = pa.write_and_forward_shared_prefix(k.to(DEV), v.to(DEV), slots, k_cache,
                                                     v_cache, q.to(DEV), table, lens, qsl,
                                                     scale, pb,
                                                     max_seq_len=int(inp.seq_lens.max()))
            shared_steps += 1
        else:
            out = pa.write_and_forward(k.to(DEV), v.to(DEV), slots, k_cache, v_cache, q.to(DEV),
                                       table, lens, qsl, scale, max_query_len=int(ql.max()),
                                       max_seq_len=int(inp.seq_lens.max()))
        torch.cuda.synchronize()
        out = out.cpu()
        kc, vc = k_cache.cpu(), v_cache.cpu()
        for s in range(S):
            rid = int(inp.request_ids[s])
            L = int(inp.seq_lens[s])
            nb = -(-L // BS)
            ids = inp.block_table[s, :nb]
            # the cache holds every visible token's K/V bit-exactly
            kk = kc[torch.from_numpy(ids).long()].reshape(nb * BS, Hkv, D)[:L]
            vv = vc[torch.from_numpy(ids).long()].reshape(nb * BS, Hkv, D)[:L]
            want_k = torch.stack([mir.values(rid, p)[1] for p in range(L)])
            want_v = torch.stack([mir.values(rid, p)[2] for p in range(L)])
            assert torch.equal(kk.view(torch.int16), want_k.view(torch.int16)), (steps, rid)
            assert torch.equal(vv.view(torch.int16), want_v.view(torch.int16)), (steps, rid)
            # the output rows match the oracle on the unpaged sequence
            n = int(ql[s])
            pad = nb * BS - L
            kd = torch.cat([want_k, torch.zeros(pad, Hkv, D, dtype=torch.bfloat16)]).view(nb, BS, Hkv, D)
            vd = torch.cat([want_v, torch.zeros(pad, Hkv, D, dtype=torch.bfloat16)]).view(nb, BS, Hkv, D)
            qd = torch.stack([mir.values(rid, p)[0] for p in range(L - n, L)])
            want = oracle.ref_forward(qd, kd, vd, torch.arange(nb, dtype=torch.int32)[None],
                                      torch.tensor([L], dtype=torch.int32),
                                      torch.tensor([0, n], dtype=torch.int32), scale)
            t0 = int(inp.query_start_loc[s])
            err = (out[t0:t0 + n].double() - want).abs()
            assert err.max().item() <= 1e-2 and err.mean().item() <= 1e-3, (steps, rid, err.max())
            checked_rows += 1
        # sample: rows that computed all their request's known tokens
        sampled = []
        for s in range(S):
            rid = int(inp.request_ids[s])
            tok = (rid * 7919 + steps * 104729) % 30_000
            sampled.append(tok)
            if int(inp.seq_lens[s]) == len(mir.tokens[rid]):
                mir.tokens[rid].append(tok)
        sch.update(sampled)
        for rid in list(live):
            try:
                sch.request_computed(rid)
            except KeyError:
                live.discard(rid)
        steps += 1
        assert steps < 2000
    st = sch.stats()
    print(f"\n  steps {steps}, rows checked {checked_rows}, prefix hits {st.prefix_hit_tokens} "
          f"tokens, preemptions {st.num_preemptions}, shared-prefix steps {shared_steps}",
          flush=True)
    assert st.num_finished == n_req and st.num_free_blocks == num_blocks
    st.shared_prefix_steps = shared_steps
    return st


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (32, 8, 128)])
def test_engine_steps_with_prefix_cache_and_chunked_prefill(Hq, Hkv, D):
    st = run_engine(Hq, Hkv, D, num_blocks=96, budget=80, threshold=24, caching=True, seed=D)
    assert st.prefix_hit_tokens > 0


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (32, 8, 128)])
def test_engine_decode_steps_through_the_shared_prefix_call(Hq, Hkv, D):
    """Every request starts with the same prompt prefix: the planner's
    steps whose rows all decode and share its cached blocks go through
    pa_write_and_forward_shared_prefix, and every row still matches the
    oracle and every cache row its token's K/V."""
    # the first request computes the prefix alone; the others find it cached
    st = run_engine(Hq, Hkv, D, num_blocks=96, budget=80, threshold=24, caching=True,
                    seed=31 + D, n_req=8, new_tokens=(24, 32), one_prefix=True,
                    shared_prefix_calls=True, first_alone_steps=6)
    assert st.prefix_hit_tokens > 0 and st.shared_prefix_steps >= 5


def test_engine_steps_under_preemption():
    # the longest request needs 9 of the 12 blocks; rows that keep decoding
    # run the pool dry
    st = run_engine(8, 2, 64, num_blocks=12, budget=64, threshold=16, caching=True, seed=5,
                    new_tokens=(20, 40))
    assert st.num_preemptions > 0


def test_engine_steps_without_prefix_cache():
    st = run_engine(16, 4, 128, num_blocks=64, budget=200, threshold=0, caching=False, seed=9)
    assert st.prefix_hit_tokens == 0
