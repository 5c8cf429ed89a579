"""A step captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches) and replayed: every replay, with new inputs copied into the
captured buffers and eager work in between, gives the same bits as the
eager call on the same inputs, and matches the oracle on them (whose inputs
are a CPU copy of the rows' blocks taken before the library was called, the
replay's own q, k and v written into it by the oracle). Covers the fused
decode launch, partitioned rows merged in the kernel (arrival counters, reset by the kernels
themselves, so replays start from zero) or by the combine launch, the even-share schedule, a mixed
step with prefill tiles and their device planner, rows of four query tokens
on both decode schedules, a batch of short rows run as few-key tiles, the
shared-prefix pass (with the step's write in its launch, and without), and
several steps in one graph."""

import pytest
import torch

import paged_attention_kv_amd as pa
import workloads as wl
from oracle_view import OracleView, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # name, Hq, Hkv, D, rows, schedule
    ("decode_fused", 32, 4, 64, [(1, 512 + 37 * i) for i in range(64)], "partitioned"),
    # rows split into partitions of 736 keys (merged in the kernel) and of
    # 2736 keys (merged by the combine launch)
    ("decode_long_rows", 64, 8, 128, [(1, 8000), (1, 3000), (1, 5)], "partitioned"),
    ("decode_long_rows_combine", 64, 8, 128, [(1, 30000), (1, 12000), (1, 5)], "partitioned"),
    ("even_shares", 32, 8, 128, [(1, 2000 + 61 * i) for i in range(200)], "even"),
    ("mixed", 32, 8, 128, [(1, 900), (300, 1000), (1, 33), (64, 0), (1, 4000)], None),
    # rows of four query tokens (speculative verify) on each decode schedule
    ("verify_even", 32, 8, 128, [(4, 1500 + 97 * i) for i in range(80)], "even"),
    ("verify_partitioned", 32, 8, 64, [(4, 300 + 53 * i) for i in range(40)], "partitioned"),
    # no row past 128 keys: the write with the planner, then every row as a
    # few-key tile (no decode launch)
    ("short_tiles", 32, 8, 128, [(1, 50), (20, 30), (1, 100), (7, 8), (1, 127), (40, 60)], None),
]


@pytest.mark.parametrize("name,hq,hkv,d,rows,schedule", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, hq, hkv, d, rows, schedule):
    spec = wl.custom(name, hq, hkv, d, rows=rows, seed=170 + len(rows))
    print(f"\n[case] graph replay {name}: S={spec.num_seqs} T={spec.num_tokens}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, [s for s in range(spec.num_seqs) if spec.q_lens[s] > 0])
    hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
    ws = torch.zeros(pa.forward_workspace_bytes(spec.num_tokens, spec.num_seqs, hq, hkv, d,
                                                spec.max_blocks_per_seq, **hints),
                     dtype=torch.uint8, device=DEV)
    q, k, v = case.q.clone(), case.k.clone(), case.v.clone()
    out = torch.empty_like(q)

    def step(o):
        pa.write_and_forward(k, v, case.slot_mapping, case.k_cache, case.v_cache, q,
                             case.block_table, case.seq_lens, case.query_start_loc, case.scale,
                             out=o, workspace=ws, decode_schedule=schedule, **hints)

    step(out)  # warm up (loads kernels) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    gen = torch.Generator(device=DEV).manual_seed(7)
    ref = torch.empty_like(out)
    for i in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        k.copy_(torch.randn(k.shape, generator=gen, device=DEV).to(k.dtype))
        v.copy_(torch.randn(v.shape, generator=gen, device=DEV).to(v.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step(ref)  # eager on the same inputs (rewrites the same cache rows)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        r, want = view.expect(q=q, k=k, v=v)
        assert_close(got.cpu()[r], want, f"{name} replay {i}")
        # eager work between replays
        _ = (q.float() @ q.float()[:1].transpose(1, 2).contiguous()).sum()
    assert int(ws[:pa.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


def test_graph_of_several_steps_matches_eager():
    """Three decode steps in one graph, each writing its own new tokens into
    the same slots and attending with its own queries: every replay gives
    the bits of the three eager steps run in the same order."""
    rows = [(1, 512 + 37 * i) for i in range(64)]
    spec = wl.custom("graph_loop", 32, 4, 64, rows=rows, seed=191)
    print(f"\n[case] graph of three steps: S={spec.num_seqs}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    hints = dict(max_query_len=1, max_seq_len=max(spec.seq_lens))
    gen = torch.Generator(device=DEV).manual_seed(11)

    def rnd(t):
        return torch.randn(t.shape, generator=gen, device=DEV).to(t.dtype)

    ins = [(rnd(case.q), rnd(case.k), rnd(case.v)) for _ in range(3)]
    outs = [torch.empty_like(case.q) for _ in range(3)]

    def steps(dst):
        for (q, k, v), o in zip(ins, dst):
            pa.write_and_forward(k, v, case.slot_mapping, case.k_cache, case.v_cache, q,
                                 case.block_table, case.seq_lens, case.query_start_loc,
                                 case.scale, out=o, **hints)

    steps(outs)  # kernels loaded and the workspace allocated outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(outs)
    refs = [torch.empty_like(case.q) for _ in range(3)]
    for r in range(3):
        for q, k, v in ins:
            q.copy_(rnd(q))
            k.copy_(rnd(k))
            v.copy_(rnd(v))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        steps(refs)
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.isfinite(got[i].float()).all()
            assert torch.equal(got[i].view(torch.int16), refs[i].view(torch.int16)), (r, i)
            q, k, v = ins[i]
            rows, want = view.expect(q=q, k=k, v=v)
            assert_close(got[i].cpu()[rows], want, f"replay {r} step {i}")
        _ = (case.q.float() @ case.q.float()[:1].transpose(1, 2).contiguous()).sum()


@pytest.mark.parametrize("fused", [False, True], ids=["forward", "write_and_forward"])
def test_graph_replays_of_the_shared_prefix_pass_match_eager(fused):
    """The shared-prefix pass (prefix tiles, then the rows' own blocks with
    the merge in the kernel) captured and replayed with new queries; with
    the step's write in the prefix launch, new keys and values too."""
    pb = 24
    rows = [(1, 16 * pb + own - 1) for own in (1, 17, 40, 200, 5, 64)]
    spec = wl.custom("prefix_graph", 32, 8, 128, rows=rows, seed=181, shared_prefix_blocks=pb)
    print(f"\n[case] graph replay shared-prefix pass: S={spec.num_seqs} fused={fused}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    q, k, v = case.q.clone(), case.k.clone(), case.v.clone()
    if not fused:
        pa.cache_write(k, v, case.slot_mapping, case.k_cache, case.v_cache)
    out = torch.empty_like(q)
    ms = max(spec.seq_lens)

    def step(o):
        if fused:
            pa.write_and_forward_shared_prefix(k, v, case.slot_mapping, case.k_cache,
                                               case.v_cache, q, case.block_table, case.seq_lens,
                                               case.query_start_loc, case.scale, pb, out=o,
                                               max_seq_len=ms)
        else:
            pa.forward_shared_prefix(q, case.k_cache, case.v_cache, case.block_table,
                                     case.seq_lens, case.query_start_loc, case.scale, pb, out=o,
                                     max_seq_len=ms)

    step(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    gen = torch.Generator(device=DEV).manual_seed(9)
    ref = torch.empty_like(out)
    for i in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        if fused:
            k.copy_(torch.randn(k.shape, generator=gen, device=DEV).to(k.dtype))
            v.copy_(torch.randn(v.shape, generator=gen, device=DEV).to(v.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step(ref)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        r, want = view.expect(q=q, k=k, v=v)
        assert_close(got.cpu()[r], want, f"shared prefix replay {i}")
        _ = (q.float() * 2).sum()


def test_implicit_workspace_does_not_grow_under_capture():
    """A call made under capture without a workspace of its own, whose sizes
    need more than the implicit per-device workspace holds, raises before
    launching anything (a larger workspace would leave graphs captured
    earlier pointing at the old one); outside capture the workspace grows and
    the old one is kept alive."""
    pa._workspaces.clear()
    small = wl.custom("ws_small", 32, 8, 128, rows=[(1, 100)], seed=300)
    big = wl.custom("ws_big", 32, 8, 128, rows=[(1, 8000)] + [(1, 5)] * 2999, seed=301)
    need = [pa.forward_workspace_bytes(s.num_tokens, s.num_seqs, 32, 8, 128,
                                       s.max_blocks_per_seq) for s in (small, big)]
    assert need[1] > need[0]
    cs = wl.make_case(small, device=DEV)
    cb = wl.make_case(big, device=DEV)

    def fwd(c):
        return pa.forward(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                          c.query_start_loc, c.scale)

    fwd(cs)
    torch.cuda.synchronize()
    first = pa._workspaces[torch.cuda.current_device()]
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="graph capture"):
        with torch.cuda.graph(g):
            fwd(cb)
    torch.cuda.synchronize()
    fwd(cb)  # outside capture: grows
    torch.cuda.synchronize()
    assert pa._workspaces[torch.cuda.current_device()].numel() >= need[1]
    assert any(w is first for w in pa._retired_workspaces)


def test_graph_of_a_large_mixed_step_keeps_one_stream():
    """A mixed batch large enough for its prefill to run on the library's
    second stream eagerly keeps every launch on the capturing stream under
    capture: each replay gives the bits of the eager call with
    PA_FORWARD_SERIAL and matches the oracle."""
    rows = [(1, 256 + (97 * i) % 1800) for i in range(300)] + [(700, 300), (900, 0)]
    spec = wl.custom("graph_mixed_large", 32, 8, 128, rows=rows, seed=440)
    assert spec.num_tokens - spec.num_seqs >= 1024
    print(f"\n[case] graph of a large mixed step: S={spec.num_seqs} T={spec.num_tokens}",
          flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
    ws = torch.zeros(pa.forward_workspace_bytes(spec.num_tokens, spec.num_seqs, 32, 8, 128,
                                                spec.max_blocks_per_seq, **hints),
                     dtype=torch.uint8, device=DEV)
    q, k, v = case.q.clone(), case.k.clone(), case.v.clone()
    out = torch.empty_like(q)

    def step(o, **kw):
        pa.write_and_forward(k, v, case.slot_mapping, case.k_cache, case.v_cache, q,
                             case.block_table, case.seq_lens, case.query_start_loc, case.scale,
                             out=o, workspace=ws, **hints, **kw)

    step(out)  # warm up outside the capture (kernels loaded, side stream made)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    gen = torch.Generator(device=DEV).manual_seed(9)
    ref = torch.empty_like(out)
    for i in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        k.copy_(torch.randn(k.shape, generator=gen, device=DEV).to(k.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step(ref, serial=True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        r, want = view.expect(q=q, k=k, v=v)
        assert_close(got.cpu()[r], want, f"large mixed replay {i}")
        _ = (q.float() * 2).sum()
    assert int(ws[:pa.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
