"""Pins for the CPU oracle: each check compares it with something other than
itself (the pages' printed numbers, brute force on tiny inputs, a library
routine as a special case, closed forms, invariants), and the planted-mistake
tests at the end show that each plausible slip in the oracle trips a pin.

Everything here runs on the CPU."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.reference as ref
import workloads as wl

BF = torch.bfloat16


# ---------------------------------------------------------------------------
# Helpers that build paged inputs from contiguous ones, independently of the
# oracle's gather.
# ---------------------------------------------------------------------------

def paged_from_contiguous(K_seqs, V_seqs, spec, poison=wl.POISON):
    """Scatter per-sequence contiguous K/V ([L, Hkv, D] each) into a pool
    through the seeded block tables, one position at a time."""
    lay = wl.build_layout(spec)
    NB, bs, Hkv, D = spec.num_blocks, spec.block_size, spec.num_kv_heads, spec.head_size
    kc = torch.full((NB, bs, Hkv, D), poison, dtype=K_seqs[0].dtype)
    vc = torch.full((NB, bs, Hkv, D), poison, dtype=V_seqs[0].dtype)
    for s, L in enumerate(spec.seq_lens):
        for p in range(L):
            b = int(lay.block_table[s, p // bs])
            kc[b, p % bs] = K_seqs[s][p]
            vc[b, p % bs] = V_seqs[s][p]
    return kc, vc, lay


def brute_attention(q, K_seqs, V_seqs, spec):
    """Per query row, per head, per visible key: explicit loops in float64 on
    unpaged K/V. Returns [T, Hq, D] float64 numpy."""
    G = spec.group
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D))
    qn = q.to(torch.float64).numpy()
    t = 0
    for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
        Kn = K_seqs[s].to(torch.float64).numpy()
        Vn = V_seqs[s].to(torch.float64).numpy()
        c = L - ql
        for i in range(ql):
            for h in range(Hq):
                g = h // G
                scores = [spec.scale * float(np.dot(qn[t, h], Kn[j, g])) for j in range(c + i + 1)]
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                z = sum(w)
                acc = np.zeros(D)
                for j, wj in enumerate(w):
                    acc += wj * Vn[j, g]
                out[t, h] = acc / z
            t += 1
    return out


def random_seqs(spec, seed, dtype=BF):
    g = torch.Generator().manual_seed(seed)
    Ks, Vs = [], []
    for L in spec.seq_lens:
        Ks.append(torch.randn(L, spec.num_kv_heads, spec.head_size, generator=g).to(dtype))
        Vs.append(torch.randn(L, spec.num_kv_heads, spec.head_size, generator=g).to(dtype))
    q = torch.randn(spec.num_tokens, spec.num_q_heads, spec.head_size, generator=g).to(dtype)
    return q, Ks, Vs


def run_oracle(q, kc, vc, lay, spec, **kw):
    return oracle.ref_forward(q, kc, vc, lay.block_table, lay.seq_lens, lay.query_start_loc,
                              spec.scale, **kw)


SMALL_SPECS = [
    wl.config(1),
    wl.custom("mixed_small", 8, 2, 64, rows=[(1, 40), (7, 0), (0, 20), (5, 11), (1, 15), (17, 16)],
              seed=11),
    wl.custom("mha_small", 4, 4, 32, rows=[(3, 29), (1, 0), (16, 0)], seed=12),
    wl.custom("gqa8_small", 16, 2, 16, rows=[(2, 33), (9, 7)], seed=13),
]


# ---------------------------------------------------------------------------
# The pages' own numbers
# ---------------------------------------------------------------------------

def test_pages_allocate_slots_example(golden):
    ex = golden["allocate_slots"]
    assert oracle.blocks_needed(ex["new_tokens"], ex["block_size"]) == ex["blocks"]
    assert oracle.BLOCK_SIZE == ex["block_size"]
    # a few more values the ceiling fixes: the boundary cases of one block
    assert [oracle.blocks_needed(n) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 1, 1, 1, 2, 2, 3]


def test_pages_chunked_prefill_example(golden):
    ex = golden["chunked_prefill"]
    n = ex["chunk_tokens"]
    prompt = ex["full_chunks"] * n + ex["tail_tokens"]
    assert oracle.prefill_steps(prompt, n) == ex["min_engine_steps"]
    assert oracle.chunk_plan(prompt, n) == [n] * ex["full_chunks"] + [ex["tail_tokens"]]
    assert sum(oracle.chunk_plan(prompt, n)) == prompt


@pytest.mark.parametrize("hkv,d,expect", [(4, 64, 16384), (8, 128, 65536)])
def test_pages_block_bytes_formula(golden, hkv, d, expect):
    ex = golden["kv_block_bytes"]
    got = oracle.kv_block_bytes(ex["default_block_size"], hkv, d, ex["bf16_bytes"])
    # measured independently: bytes a [NB, 16, Hkv, D] bf16 K and V pool spend per block
    nb = 3
    kc = torch.empty((nb, ex["default_block_size"], hkv, d), dtype=BF)
    vc = torch.empty_like(kc)
    assert got == (kc.nbytes + vc.nbytes) // nb == expect


# ---------------------------------------------------------------------------
# KV write
# ---------------------------------------------------------------------------

def test_cache_write_matches_flat_scatter():
    spec = SMALL_SPECS[1]
    case = wl.make_case(spec)
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    oracle.ref_cache_write(case.k, case.v, case.slot_mapping, kc, vc)
    # independent: a vectorised scatter into the flat [slots, Hkv, D] view
    fk = case.k_cache.clone().view(-1, spec.num_kv_heads, spec.head_size)
    fv = case.v_cache.clone().view(-1, spec.num_kv_heads, spec.head_size)
    fk[case.slot_mapping] = case.k
    fv[case.slot_mapping] = case.v
    assert torch.equal(kc.view(torch.int16), fk.view_as(kc).view(torch.int16))
    assert torch.equal(vc.view(torch.int16), fv.view_as(vc).view(torch.int16))
    # nothing outside the written slots moved
    touched = torch.zeros(kc.shape[0] * kc.shape[1], dtype=torch.bool)
    touched[case.slot_mapping] = True
    before = case.k_cache.view(-1, spec.num_kv_heads, spec.head_size)
    after = kc.view(-1, spec.num_kv_heads, spec.head_size)
    assert torch.equal(before[~touched].view(torch.int16), after[~touched].view(torch.int16))


def test_cache_write_block_and_offset():
    # slot 17 of a 16-token block is row 1 of block 1; a negative slot is skipped
    kc = torch.zeros((4, 16, 1, 8), dtype=BF)
    vc = torch.zeros_like(kc)
    k = torch.arange(3 * 8, dtype=torch.float32).reshape(3, 1, 8).to(BF) + 1
    v = -k
    oracle.ref_cache_write(k, v, torch.tensor([17, -1, 63]), kc, vc)
    assert torch.equal(kc[1, 1], k[0]) and torch.equal(vc[1, 1], v[0])
    assert torch.equal(kc[3, 15], k[2]) and torch.equal(vc[3, 15], v[2])
    assert int((kc != 0).any(-1).any(-1).sum()) == 2


def test_cache_write_rejects_bad_slots():
    kc = torch.zeros((2, 16, 1, 8), dtype=BF)
    vc = torch.zeros_like(kc)
    k = torch.ones((2, 1, 8), dtype=BF)
    with pytest.raises(ValueError):
        oracle.ref_cache_write(k, k, torch.tensor([3, 3]), kc, vc)
    with pytest.raises(ValueError):
        oracle.ref_cache_write(k, k, torch.tensor([0, 32]), kc, vc)


# ---------------------------------------------------------------------------
# Attention: brute force, SDPA, precision
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("spec", SMALL_SPECS, ids=lambda s: s.name)
def test_forward_matches_brute_force_on_unpaged_kv(spec):
    q, Ks, Vs = random_seqs(spec, seed=5)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    want = brute_attention(q, Ks, Vs, spec)
    rows = np.concatenate([np.arange(a, b) for a, b in
                           zip(lay.query_start_loc[:-1].tolist(), lay.query_start_loc[1:].tolist())])
    assert rows.size == spec.num_tokens
    np.testing.assert_allclose(got.numpy(), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", SMALL_SPECS, ids=lambda s: s.name)
def test_forward_matches_sdpa_with_explicit_bottom_right_mask(spec):
    q, Ks, Vs = random_seqs(spec, seed=6)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    G = spec.group
    t0 = 0
    for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
        if ql == 0:
            continue
        c = L - ql
        Q = q[t0:t0 + ql].to(torch.float64).transpose(0, 1)                   # [Hq, ql, D]
        K = Ks[s].to(torch.float64).repeat_interleave(G, dim=1).transpose(0, 1)  # [Hq, L, D]
        V = Vs[s].to(torch.float64).repeat_interleave(G, dim=1).transpose(0, 1)
        mask = torch.ones(ql, L, dtype=torch.bool).tril(diagonal=c)            # j <= c + i
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=mask, scale=spec.scale).transpose(0, 1)
        torch.testing.assert_close(got[t0:t0 + ql], o, rtol=0, atol=1e-12)
        t0 += ql


def test_forward_rows_with_no_queries_are_left_alone():
    spec = SMALL_SPECS[1]   # has a row with q_len 0
    q, Ks, Vs = random_seqs(spec, seed=7)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    assert not torch.isnan(got).any()     # every flattened row belongs to a sequence


def test_float32_variant_within_1e5_of_float64():
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=8)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    a = run_oracle(q, kc, vc, lay, spec)
    b = run_oracle(q, kc, vc, lay, spec, dtype=torch.float32)
    assert b.dtype == torch.float32
    assert (a - b.double()).abs().max() < 1e-5


def test_token_subset_equals_full_rows():
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=9)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    full = run_oracle(q, kc, vc, lay, spec)
    pick = [0, 3, 9, spec.num_tokens - 1]
    part = run_oracle(q, kc, vc, lay, spec, tokens=pick)
    assert torch.equal(part[pick], full[pick])
    others = [t for t in range(spec.num_tokens) if t not in pick]
    assert torch.isnan(part[others]).all()


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_zero_query_gives_mean_of_visible_values():
    """q = 0 makes every visible score equal: row i is the plain mean of V over
    keys 0..c+i, which pins where the causal boundary falls."""
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=10)
    q.zero_()
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    G = spec.group
    t = 0
    for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
        c = L - ql
        for i in range(ql):
            for h in range(spec.num_q_heads):
                want = Vs[s][:c + i + 1, h // G].to(torch.float64).mean(0)
                torch.testing.assert_close(got[t, h], want, rtol=0, atol=1e-13)
            t += 1


def test_single_visible_key_returns_its_value_exactly():
    spec = wl.custom("first_token", 8, 2, 64, rows=[(1, 0), (4, 0)], seed=14)
    q, Ks, Vs = random_seqs(spec, seed=11)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    G = spec.group
    for h in range(spec.num_q_heads):
        assert torch.equal(got[0, h], Vs[0][0, h // G].to(torch.float64))
        assert torch.equal(got[1, h], Vs[1][0, h // G].to(torch.float64))   # row 0 of sequence 1


def test_identical_keys_give_mean_and_dominant_key_wins():
    spec = wl.custom("ties", 4, 1, 16, rows=[(1, 20)], seed=15)
    q, Ks, Vs = random_seqs(spec, seed=12, dtype=torch.float64)
    Ks[0][:] = Ks[0][0:1]                       # all keys equal
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    torch.testing.assert_close(got[0, 0], Vs[0][:, 0].mean(0), rtol=0, atol=1e-13)
    # now make key 7 dominant for query head 0: its value comes out
    Ks[0][:] = 0
    Ks[0][7, 0] = q[0, 0] * 200
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    torch.testing.assert_close(got[0, 0], Vs[0][7, 0], rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_weights_sum_to_one():
    """With V = 1 everywhere the output is the sum of the softmax weights."""
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=13)
    Vs = [torch.ones_like(v) for v in Vs]
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    got = run_oracle(q, kc, vc, lay, spec)
    torch.testing.assert_close(got, torch.ones_like(got), rtol=0, atol=1e-14)


def test_future_keys_do_not_leak_into_earlier_rows():
    spec = wl.custom("prefill", 8, 2, 32, rows=[(12, 5)], seed=16)
    q, Ks, Vs = random_seqs(spec, seed=14)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    base = run_oracle(q, kc, vc, lay, spec)
    c = 5
    for i in range(12):
        Ks2 = [Ks[0].clone()]
        Vs2 = [Vs[0].clone()]
        Ks2[0][c + i + 1:] = 7.0
        Vs2[0][c + i + 1:] = -7.0
        kc2, vc2, _ = paged_from_contiguous(Ks2, Vs2, spec)
        got = run_oracle(q, kc2, vc2, lay, spec)
        assert torch.equal(got[:i + 1], base[:i + 1])
        if i + 1 < 12:
            assert not torch.equal(got[i + 1:], base[i + 1:])


def test_other_sequences_do_not_leak():
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=15)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    base = run_oracle(q, kc, vc, lay, spec)
    qsl = lay.query_start_loc.tolist()
    Ks2 = [k.clone() for k in Ks]
    Vs2 = [v.clone() for v in Vs]
    Ks2[3] += 1.0
    Vs2[3] -= 1.0
    q2 = q.clone()
    q2[qsl[3]:qsl[4]] += 1.0
    kc2, vc2, _ = paged_from_contiguous(Ks2, Vs2, spec)
    got = run_oracle(q2, kc2, vc2, lay, spec)
    keep = [t for t in range(spec.num_tokens) if not qsl[3] <= t < qsl[4]]
    assert torch.equal(got[keep], base[keep])
    assert not torch.equal(got[qsl[3]:qsl[4]], base[qsl[3]:qsl[4]])


def test_block_placement_does_not_matter():
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=16)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    base = run_oracle(q, kc, vc, lay, spec)
    # the same logical content under another permutation of the pool
    perm = torch.randperm(spec.num_blocks, generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    kc2 = torch.empty_like(kc)
    vc2 = torch.empty_like(vc)
    kc2[inv] = kc
    vc2[inv] = vc
    table = lay.block_table.clone()
    used = table >= 0
    table[used] = inv[table[used].long()].to(torch.int32)
    got = oracle.ref_forward(q, kc2, vc2, table, lay.seq_lens, lay.query_start_loc, spec.scale)
    assert torch.equal(got, base)


def test_gqa_equals_mha_with_repeated_kv():
    spec = wl.custom("gqa", 8, 2, 32, rows=[(3, 9), (1, 30)], seed=17)
    mha = wl.custom("mha", 8, 8, 32, rows=[(3, 9), (1, 30)], seed=17)
    q, Ks, Vs = random_seqs(spec, seed=18)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    a = run_oracle(q, kc, vc, lay, spec)
    Ks8 = [k.repeat_interleave(4, dim=1) for k in Ks]
    Vs8 = [v.repeat_interleave(4, dim=1) for v in Vs]
    kc8, vc8, lay8 = paged_from_contiguous(Ks8, Vs8, mha)
    b = run_oracle(q, kc8, vc8, lay8, mha)
    assert torch.equal(a, b)


def test_chunked_prefill_equals_one_shot():
    """An 18-token prompt run as chunks of 8, 8 and 2 (the pages' x-y-z
    example), with the cache written between steps, gives the same rows as a
    single prefill of all 18 tokens."""
    Hq, Hkv, D, bs = 8, 2, 32, 16
    P = 18
    g = torch.Generator().manual_seed(21)
    q = torch.randn(P, Hq, D, generator=g).to(BF)
    k = torch.randn(P, Hkv, D, generator=g).to(BF)
    v = torch.randn(P, Hkv, D, generator=g).to(BF)
    table = torch.tensor([[5, 2]], dtype=torch.int32)
    scale = 1 / math.sqrt(D)

    def step(kc, vc, lo, hi):
        pos = torch.arange(lo, hi)
        slots = table[0, pos // bs].long() * bs + pos % bs
        oracle.ref_cache_write(k[lo:hi], v[lo:hi], slots, kc, vc)
        return oracle.ref_forward(q[lo:hi], kc, vc, table, torch.tensor([hi], dtype=torch.int32),
                                  torch.tensor([0, hi - lo], dtype=torch.int32), scale)

    kc = torch.full((8, bs, Hkv, D), wl.POISON, dtype=BF)
    vc = kc.clone()
    one = step(kc.clone(), vc.clone(), 0, P)
    outs = []
    lo = 0
    for n in oracle.chunk_plan(P, 8):
        outs.append(step(kc, vc, lo, lo + n))
        lo += n
    assert len(outs) == oracle.prefill_steps(P, 8) == 3
    torch.testing.assert_close(torch.cat(outs), one, rtol=0, atol=1e-14)


def test_oracle_rejects_inconsistent_metadata():
    spec = SMALL_SPECS[0]
    case = wl.make_case(spec)
    with pytest.raises(ValueError):
        oracle.ref_forward(case.q, case.k_cache, case.v_cache, case.block_table,
                           case.seq_lens, torch.tensor([0, 5, 12], dtype=torch.int32), case.scale)
    bad_lens = case.seq_lens.clone()
    bad_lens[0] = 4       # fewer cached tokens than query rows
    with pytest.raises(ValueError):
        oracle.ref_forward(case.q, case.k_cache, case.v_cache, case.block_table,
                           bad_lens, case.query_start_loc, case.scale)


# ---------------------------------------------------------------------------
# Planted mistakes: each one, put into the oracle, must trip a pin above.
# ---------------------------------------------------------------------------

def _mistake_top_left_mask(context_len, query_rows, seq_len):
    return torch.arange(seq_len)[None, :] <= query_rows[:, None]


def _mistake_off_by_one_mask(context_len, query_rows, seq_len):
    return torch.arange(seq_len)[None, :] < (context_len + query_rows)[:, None]


def _mistake_strided_gqa(q_head, num_q_heads, num_kv_heads):
    return q_head % num_kv_heads


def _mistake_gather_reversed(cache, row, length):
    bs = cache.shape[1]
    nb = oracle.blocks_needed(length, bs)
    ids = row[:nb].to(torch.long).flip(0)
    return cache.index_select(0, ids).reshape(nb * bs, cache.shape[2], cache.shape[3])[:length]


@pytest.mark.parametrize("name,mistake", [
    ("visible_keys", _mistake_top_left_mask),
    ("visible_keys", _mistake_off_by_one_mask),
    ("kv_head_of", _mistake_strided_gqa),
    ("gather_sequence", _mistake_gather_reversed),
])
def test_planted_mistake_is_caught(monkeypatch, name, mistake):
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=31)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    want = brute_attention(q, Ks, Vs, spec)
    monkeypatch.setattr(ref, name, mistake)
    got = run_oracle(q, kc, vc, lay, spec)
    assert not np.allclose(got.numpy(), want, rtol=0, atol=1e-6)


def test_planted_dropped_scale_is_caught():
    spec = SMALL_SPECS[1]
    q, Ks, Vs = random_seqs(spec, seed=32)
    kc, vc, lay = paged_from_contiguous(Ks, Vs, spec)
    want = brute_attention(q, Ks, Vs, spec)
    got = oracle.ref_forward(q, kc, vc, lay.block_table, lay.seq_lens, lay.query_start_loc, 1.0)
    assert not np.allclose(got.numpy(), want, rtol=0, atol=1e-6)
