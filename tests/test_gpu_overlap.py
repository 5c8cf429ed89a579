"""Mixed batches whose prefill launches run beside the decode launch (the
prefill on the library's second stream, forked from and joined back to the
caller's stream): every row matches the oracle with the overlap and with
PA_FORWARD_SERIAL, the prefill rows are bit-identical either way (same
kernels, same tiles), and work queued on the caller's stream right after
the call, with no host synchronisation, already sees every row written."""

import pytest
import torch

import paged_attention_kv_amd as pa
import workloads as wl
from oracle_view import OracleView, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# 300 decode rows (the even-share schedule by size) + two prefill chunks and
# one more decode row: num_tokens - num_seqs = 1598 prefill tokens, above the
# overlap's threshold of 1024.
ROWS = ([(1, 256 + (97 * i) % 1800) for i in range(300)] +
        [(700, 300), (900, 0), (1, 3000)])
SHAPES = [(32, 8, 128), (32, 4, 64)]


def run(case, spec, **kw):
    hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
    return pa.write_and_forward(case.k, case.v, case.slot_mapping, case.k_cache, case.v_cache,
                                case.q, case.block_table, case.seq_lens, case.query_start_loc,
                                case.scale, **hints, **kw)


@pytest.mark.parametrize("hq,hkv,d", SHAPES, ids=[f"{a}q{b}kv_d{c}" for a, b, c in SHAPES])
def test_overlapped_mixed_batch_matches_oracle_and_serial(hq, hkv, d):
    spec = wl.custom("overlap", hq, hkv, d, rows=ROWS, seed=410 + d)
    assert spec.num_tokens - spec.num_seqs >= 1024
    print(f"\n[case] overlapped mixed batch {hq}q/{hkv}kv D{d}: S={spec.num_seqs} "
          f"T={spec.num_tokens}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    # (the fused write is off for mixed batches: each call writes the same
    # tokens into the same slots first, so the two calls see the same cache)
    got = run(case, spec)
    torch.cuda.synchronize()
    ser = run(case, spec, serial=True)
    torch.cuda.synchronize()
    rows, want = view.expect()
    got, ser = got.cpu(), ser.cpu()
    assert_close(got[rows], want, "overlapped")
    assert_close(ser[rows], want, "serial")
    pre = [t for s in range(spec.num_seqs) if spec.q_lens[s] > 1
           for t in range(int(case.query_start_loc[s]), int(case.query_start_loc[s + 1]))]
    assert torch.equal(got[pre].view(torch.int16), ser[pre].view(torch.int16))


def test_results_are_ordered_on_the_callers_stream():
    """The output starts as NaN; a copy queued on the current stream right
    after the call (no synchronisation in between) must hold every row."""
    spec = wl.custom("overlap_order", 32, 8, 128, rows=ROWS, seed=430)
    print(f"\n[case] overlap ordering: S={spec.num_seqs} T={spec.num_tokens}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    out = torch.full_like(case.q, float("nan"))
    copies = []
    for _ in range(3):
        out.fill_(float("nan"))
        run(case, spec, out=out)
        copies.append(out.clone())  # queued behind the call's join
    torch.cuda.synchronize()
    rows, want = view.expect()
    for i, c in enumerate(copies):
        c = c.cpu()
        assert torch.isfinite(c.float()).all(), f"copy {i} saw rows not yet written"
        assert_close(c[rows], want, f"copy {i}")


def test_prefill_tiles_wait_for_their_own_calls_write():
    """Calls queued back to back with different new tokens each time (no
    host synchronisation between them): each call's prefill rows, run on the
    second stream, see that call's own tokens written, not the last call's."""
    spec = wl.custom("overlap_fork", 32, 8, 128, rows=ROWS, seed=450)
    print(f"\n[case] overlap fork order: S={spec.num_seqs} T={spec.num_tokens}", flush=True)
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, range(spec.num_seqs))
    gen = torch.Generator(device=DEV).manual_seed(11)
    ins, outs = [], []
    for _ in range(3):
        k = torch.randn(case.k.shape, generator=gen, device=DEV).to(case.k.dtype)
        v = torch.randn(case.v.shape, generator=gen, device=DEV).to(case.v.dtype)
        q = torch.randn(case.q.shape, generator=gen, device=DEV).to(case.q.dtype)
        hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
        outs.append(pa.write_and_forward(k, v, case.slot_mapping, case.k_cache, case.v_cache, q,
                                         case.block_table, case.seq_lens, case.query_start_loc,
                                         case.scale, **hints).clone())
        ins.append((q, k, v))
    torch.cuda.synchronize()
    for i, ((q, k, v), o) in enumerate(zip(ins, outs)):
        rows, want = view.expect(q=q, k=k, v=v)
        assert_close(o.cpu()[rows], want, f"call {i}")
