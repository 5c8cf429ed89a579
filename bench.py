"""Benchmark of the paged-attention hot path on one MI355X.

One step = the whole hot path over one batch: the KV-cache write of the
step's new tokens (pa_cache_write) followed by paged attention of the
flattened batch (pa_forward). Inputs are synthetic, seeded, and resident in
HBM before the timed region starts.

Headline (one JSON line on stdout):
  * value: decode GB/s on the decode workload (64 sequences x 1 query token,
    context U[512, 2048], 32 q / 4 kv heads, D 64, 16-token blocks, 100k-block
    bf16 pool); bytes are algorithmic (each row's K and V context once, q, out,
    and the KV write), time is the whole step. Eight disjoint block-table sets
    drawn from the same pool rotate between steps so the 256 MiB Infinity
    Cache cannot hold a step's KV.
  * mixed_step: tokens/s of the 8192-token mixed chunked-prefill step (256
    decode rows + 4 x 1984-token chunks, 32 q / 8 kv heads, D 128).
  * roofline: the decode kernel's algorithmic bytes per launch over its
    average launch duration (HIP events on the launch stream), against
    8 TB/s.
  * cpu_baseline: the CPU oracle timed on this host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only decode|mixed]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = "paged-attn decode GB/s (% of 8 TB/s) + mixed-step tokens/s on 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATIONS = 8


# ---------------------------------------------------------------------------
# Algorithmic work (bytes and flops a step must move / do at minimum)
# ---------------------------------------------------------------------------

def attention_bytes(spec, rows=None) -> int:
    """K and V of each row's context once per KV head, q read, out written."""
    rows = range(spec.num_seqs) if rows is None else rows
    per_tok_kv = 2 * spec.num_kv_heads * spec.head_size * 2
    per_q = spec.num_q_heads * spec.head_size * 2
    b = 0
    for s in rows:
        if spec.q_lens[s] == 0:
            continue
        b += spec.seq_lens[s] * per_tok_kv + 2 * spec.q_lens[s] * per_q
    return b


def write_bytes(spec, rows=None) -> int:
    """Read k and v of the new tokens, write them into the cache."""
    rows = range(spec.num_seqs) if rows is None else rows
    n = sum(spec.q_lens[s] for s in rows)
    return n * spec.num_kv_heads * spec.head_size * 2 * 2 * 2


def attention_flops(spec, rows=None) -> int:
    """4 * D * Hq per visible (query, key) pair (QK^T and PV)."""
    rows = range(spec.num_seqs) if rows is None else rows
    pairs = 0
    for s in rows:
        ql, L = spec.q_lens[s], spec.seq_lens[s]
        c = L - ql
        pairs += ql * c + ql * (ql + 1) // 2
    return 4 * spec.head_size * spec.num_q_heads * pairs


# ---------------------------------------------------------------------------
# Inputs: one pool, R disjoint block-table sets
# ---------------------------------------------------------------------------

class StepInputs:
    def __init__(self, spec, rotations: int, device: str):
        self.spec = spec
        T, Hq, Hkv, D = spec.num_tokens, spec.num_q_heads, spec.num_kv_heads, spec.head_size
        NB, bs, S, MB = spec.num_blocks, spec.block_size, spec.num_seqs, spec.max_blocks_per_seq
        gen = torch.Generator(device=device).manual_seed(spec.seed_values)
        self.k_cache = torch.empty((NB, bs, Hkv, D), dtype=torch.bfloat16, device=device)
        self.v_cache = torch.empty_like(self.k_cache)
        chunk = max(1, (1 << 26) // (bs * Hkv * D))
        for cache in (self.k_cache, self.v_cache):
            for b0 in range(0, NB, chunk):
                b1 = min(NB, b0 + chunk)
                cache[b0:b1] = torch.randn((b1 - b0, bs, Hkv, D), generator=gen, device=device)
        nb_per_set = sum(-(-L // bs) for L in spec.seq_lens)
        if rotations * nb_per_set > NB:
            rotations = max(1, NB // nb_per_set)
        self.rotations = rotations
        perm = torch.randperm(NB, generator=torch.Generator().manual_seed(spec.seed_layout))
        self.sets = []
        used = 0
        for r in range(rotations):
            table = torch.full((S, MB), -1, dtype=torch.int32)
            slots = []
            for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
                nb = -(-L // bs)
                table[s, :nb] = perm[used:used + nb].to(torch.int32)
                used += nb
                pos = torch.arange(L - ql, L)
                slots.append(table[s, pos // bs].to(torch.int64) * bs + pos % bs)
            self.sets.append(dict(
                q=torch.randn((T, Hq, D), generator=gen, device=device).to(torch.bfloat16),
                k=torch.randn((T, Hkv, D), generator=gen, device=device).to(torch.bfloat16),
                v=torch.randn((T, Hkv, D), generator=gen, device=device).to(torch.bfloat16),
                slot_mapping=torch.cat(slots).to(device),
                block_table=table.to(device),
                out=torch.empty((T, Hq, D), dtype=torch.bfloat16, device=device)))
        self.seq_lens = torch.tensor(spec.seq_lens, dtype=torch.int32, device=device)
        qsl = [0]
        for ql in spec.q_lens:
            qsl.append(qsl[-1] + ql)
        self.qsl = torch.tensor(qsl, dtype=torch.int32, device=device)
        self.hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens))


def run_steps(pa, inp: StepInputs, steps: int, warmup: int, rows=None):
    """Time `steps` steps (write + forward); also HIP-event time of each
    pa_forward call on the launch stream. Returns (ms/step, ms/forward)."""
    spec = inp.spec
    if rows is not None:
        raise ValueError("sub-batch timing uses its own StepInputs")

    def step(i, ev=None):
        st = inp.sets[i % inp.rotations]
        pa.cache_write(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache)
        if ev is not None:
            ev[0].record()
        pa.forward(st["q"], inp.k_cache, inp.v_cache, st["block_table"], inp.seq_lens, inp.qsl,
                   spec.scale, out=st["out"], **inp.hints)
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    fwd = sorted(a.elapsed_time(b) for a, b in evs)
    return ms_step, sum(fwd) / len(fwd), fwd[len(fwd) // 2]


def sub_spec(spec, rows, name):
    """The same rows as a workload of their own (for attributing time)."""
    return wl.Spec(name, spec.num_q_heads, spec.num_kv_heads, spec.head_size,
                   num_blocks=spec.num_blocks, max_blocks_per_seq=spec.max_blocks_per_seq,
                   q_lens=tuple(spec.q_lens[s] for s in rows),
                   seq_lens=tuple(spec.seq_lens[s] for s in rows),
                   seed_layout=spec.seed_layout, seed_values=spec.seed_values)


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(spec, budget_s: float = 12.0):
    """Time the oracle (float64, as it stands) on all rows of the workload
    for about budget_s seconds of CPU work on this host."""
    import oracle
    case = wl.make_case(spec, device="cpu")
    q, kc, vc, table, lens, qsl, _ = wl.sequences_subset(case, list(range(spec.num_seqs)))
    k, v, slots = case.k, case.v, case.slot_mapping
    # the write touches the compacted pool: remap slots into it
    n = 0
    t_start = time.perf_counter()
    while True:
        kc2, vc2 = kc.clone(), vc.clone()
        oracle.ref_cache_write(k[:0], v[:0], slots[:0], kc2, vc2)
        oracle.ref_forward(q, kc2, vc2, table, lens, qsl, spec.scale)
        n += 1
        el = time.perf_counter() - t_start
        if el >= budget_s or n >= 1000:
            break
    per = el / n
    gbs = (attention_bytes(spec) + write_bytes(spec)) / per / 1e9
    return dict(value=round(gbs, 4), unit="GB/s", cores=torch.get_num_threads(), kind="oracle",
                sample=(f"all {spec.num_seqs} rows of the decode workload, oracle ref_forward in "
                        f"float64 (PyTorch CPU), {n} repetitions in {el:.1f} s "
                        f"({per * 1e3:.1f} ms per step)"),
                ms_per_step=round(per * 1e3, 3))


# ---------------------------------------------------------------------------

def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["decode", "mixed"], default=None)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path runs on a single MI355X)", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    import paged_attention_kv_amd as pa
    pa.load_library()
    dev = "cuda:0"
    result = {}

    if args.only in (None, "decode"):
        spec = wl.config(2)
        inp = StepInputs(spec, ROTATIONS, dev)
        ms_step, ms_fwd, ms_fwd_med = run_steps(pa, inp, args.steps, args.warmup)
        b_attn = attention_bytes(spec)
        b_step = b_attn + write_bytes(spec)
        gbs = b_step / (ms_step * 1e-3) / 1e9
        kern_gbs = b_attn / (ms_fwd * 1e-3) / 1e9
        result["decode"] = dict(ms_step=ms_step, gbs=gbs, ms_fwd=ms_fwd, ms_fwd_median=ms_fwd_med,
                                fwd_gbs=kern_gbs, bytes_step=b_step, bytes_fwd=b_attn,
                                rotations=inp.rotations)
        del inp
        torch.cuda.empty_cache()

    if args.only in (None, "mixed"):
        spec = wl.config(3)
        inp = StepInputs(spec, 1, dev)
        ms_step, ms_fwd, ms_fwd_med = run_steps(pa, inp, max(5, args.steps // 5),
                                                max(2, args.warmup // 2))
        dec_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] == 1]
        pre_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] > 1]
        del inp
        torch.cuda.empty_cache()
        sub = {}
        for name, rows in (("decode_rows", dec_rows), ("prefill_rows", pre_rows)):
            ss = sub_spec(spec, rows, name)
            si = StepInputs(ss, 1, dev)
            _, f_ms, _ = run_steps(pa, si, max(5, args.steps // 5), 2)
            sub[name] = dict(ms_fwd=f_ms, bytes=attention_bytes(ss), flops=attention_flops(ss))
            del si
            torch.cuda.empty_cache()
        tok_s = spec.num_tokens / (ms_step * 1e-3)
        result["mixed"] = dict(ms_step=ms_step, tokens_per_s=tok_s, ms_fwd=ms_fwd, sub=sub)

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 values, seeded lengths and block placement)"}
    if "decode" in result:
        d = result["decode"]
        line.update(value=round(d["gbs"], 2), unit="GB/s", ms_per_step=round(d["ms_step"], 5))
        line["config"] = {
            "workload": ("decode step: 64 sequences x 1 query token, context U[512,2048], "
                         "32 q / 4 kv heads, head_size 64, block 16, 100k-block bf16 pool; "
                         "KV write + paged attention"),
            "tokens": 64, "kv_bytes_per_step": d["bytes_step"],
            "block_table_rotations": d["rotations"],
            "pct_of_hbm_peak": round(100 * d["gbs"] / HBM_PEAK_GBS, 2)}
        line["roofline"] = {"bound": "hbm", "kernel": "pa_forward (decode_partition_kernel)",
                            "achieved": round(d["fwd_gbs"], 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(d["fwd_gbs"] / HBM_PEAK_GBS, 4),
                            "traffic": None,
                            "avg_launch_us": round(d["ms_fwd"] * 1e3, 3),
                            "median_launch_us": round(d["ms_fwd_median"] * 1e3, 3),
                            "algorithmic_bytes_per_launch": d["bytes_fwd"]}
    if "mixed" in result:
        m = result["mixed"]
        pre = m["sub"]["prefill_rows"]
        dec = m["sub"]["decode_rows"]
        line["mixed_step"] = {
            "workload": ("mixed chunked-prefill step, 8192 new tokens: 256 decode rows (context "
                         "U[256,8192]) + 4 chunks of 1984 tokens (prior context U[0,4096]); "
                         "32 q / 8 kv heads, head_size 128"),
            "tokens_per_s": round(m["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(m["ms_step"], 4), "ms_forward": round(m["ms_fwd"], 4),
            "prefill_rows": {"ms": round(pre["ms_fwd"], 4), "flops": pre["flops"],
                             "tflops": round(pre["flops"] / (pre["ms_fwd"] * 1e-3) / 1e12, 2),
                             "frac_of_bf16_peak": round(pre["flops"] / (pre["ms_fwd"] * 1e-3)
                                                        / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "decode_rows": {"ms": round(dec["ms_fwd"], 4), "bytes": dec["bytes"],
                            "gbs": round(dec["bytes"] / (dec["ms_fwd"] * 1e-3) / 1e9, 2),
                            "frac_of_hbm_peak": round(dec["bytes"] / (dec["ms_fwd"] * 1e-3)
                                                      / 1e9 / HBM_PEAK_GBS, 4)}}
        if "value" not in line:
            line.update(value=round(m["tokens_per_s"], 1), unit="tokens/s",
                        ms_per_step=round(m["ms_step"], 5),
                        config={"workload": line["mixed_step"]["workload"]})
    if not args.no_cpu and "decode" in result:
        line["cpu_baseline"] = cpu_baseline(wl.config(2))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
