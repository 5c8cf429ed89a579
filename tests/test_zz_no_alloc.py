"""pa_write_and_forward_noalloc (the library's fixed scratch array as the
workspace) against pa_write_and_forward with a caller's workspace: two calls
in a row, the second with a smaller batch, each on a fresh copy of the same
seeded inputs. Outputs and both caches are bit-identical (the same kernels
on the same inputs), the output matches the oracle, and the call allocates
nothing through torch."""

import pytest
import torch

import paged_attention_kv_amd as pa
import workloads as wl
from oracle_view import OracleView, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (name, Hq, Hkv, D, rows): the first batch uses the scratch array's counter
# region (long decode rows split into partitions of 1008 keys, short enough
# to be merged in the kernel), its partials and the prefill tile lists; the
# second is smaller, decode rows only (the write rides in the decode launch).
CALLS = [
    ("mixed_larger", 32, 8, 128, [(1, 4000), (1, 300), (40, 100), (1, 3100), (200, 0),
                                  (1, 17), (3, 60), (1, 2500)]),
    ("decode_smaller", 32, 8, 128, [(1, 50), (1, 2000), (1, 1), (1, 777)]),
]


def run(spec, noalloc):
    case = wl.make_case(spec, device=DEV)
    view = OracleView(case, [s for s in range(spec.num_seqs) if spec.q_lens[s] > 0])
    out = torch.empty_like(case.q)
    hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))
    args = (case.k, case.v, case.slot_mapping, case.k_cache, case.v_cache, case.q,
            case.block_table, case.seq_lens, case.query_start_loc, case.scale)
    if noalloc:
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        pa.profile_begin()
        pa.write_and_forward_noalloc(*args, out=out, **hints)
        torch.cuda.synchronize()
        launches = pa.profile_end()
        assert torch.cuda.memory_allocated() == before
        assert "combine" not in launches, launches  # split rows merged in the kernel
    else:
        ws = torch.zeros(pa.forward_workspace_bytes(spec.num_tokens, spec.num_seqs,
                                                    spec.num_q_heads, spec.num_kv_heads,
                                                    spec.head_size, spec.max_blocks_per_seq,
                                                    **hints),
                         dtype=torch.uint8, device=DEV)
        pa.write_and_forward(*args, out=out, workspace=ws, **hints)
        torch.cuda.synchronize()
    return case, view, out


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    for name, hq, hkv, d, rows in CALLS:
        spec = wl.custom(name, hq, hkv, d, rows=rows, seed=220 + len(rows))
        print(f"\n[case] noalloc {name}: S={spec.num_seqs} T={spec.num_tokens}", flush=True)
        ca, _, out_a = run(spec, noalloc=False)
        cb, view, out_b = run(spec, noalloc=True)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), name
        assert torch.equal(ca.k_cache.view(torch.int16), cb.k_cache.view(torch.int16)), name
        assert torch.equal(ca.v_cache.view(torch.int16), cb.v_cache.view(torch.int16)), name
        r, want = view.expect()
        assert_close(out_b.cpu()[r], want, f"noalloc {name}")
        del ca, cb


def test_noalloc_rejects_a_batch_past_its_scratch():
    S, Hq, Hkv, D, MB = 4000, 64, 8, 128, 2048
    need = pa.forward_workspace_bytes(S, S, Hq, Hkv, D, MB)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((16, 16, Hkv, D), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((S, MB), dtype=torch.int32, device=DEV)
    lens = torch.ones(S, dtype=torch.int32, device=DEV)
    qsl = torch.arange(S + 1, dtype=torch.int32, device=DEV)
    slots = torch.full((S,), -1, dtype=torch.int64, device=DEV)
    with pytest.raises(pa.PaError, match="fixed size"):
        pa.write_and_forward_noalloc(k, k, slots, kc, kc.clone(), q, table, lens, qsl, 0.1,
                                     out=torch.empty_like(q))
