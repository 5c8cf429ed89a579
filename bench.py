"""Benchmark of the paged-attention hot path on one MI355X.

One step = the whole hot path over one batch: the KV-cache write of the
step's new tokens and paged attention of the flattened batch, through
pa_write_and_forward (one launch for a batch of decode rows on the
partitioned schedule; a write launch and the forward launches otherwise).
Inputs are synthetic, seeded, and resident in HBM before the timed region
starts.

Headline (one JSON line on stdout):
  * value: decode GB/s on the decode workload (64 sequences x 1 query token,
    context U[512, 2048], 32 q / 4 kv heads, D 64, 16-token blocks, 100k-block
    bf16 pool); bytes are algorithmic (each row's K and V context once, q, out,
    and the KV write), time is the whole step. Eight disjoint block-table sets
    drawn from the same pool rotate between steps so the 256 MiB Infinity
    Cache cannot hold a step's KV.
  * mixed_step: tokens/s of the 8192-token mixed chunked-prefill step (256
    decode rows + 4 x 1984-token chunks, 32 q / 8 kv heads, D 128).
  * roofline: the decode kernel's algorithmic bytes per launch (with the
    KV write when the launch does it) over its average launch duration (HIP
    events on the launch stream), against 8 TB/s.
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
COPY_MIB = 512


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
        P = spec.shared_prefix_blocks
        nb_per_set = P + sum(-(-L // bs) - P for L in spec.seq_lens)
        if rotations * nb_per_set > NB:
            rotations = max(1, NB // nb_per_set)
        self.rotations = rotations
        perm = torch.randperm(NB, generator=torch.Generator().manual_seed(spec.seed_layout))
        self.sets = []
        used = 0
        for r in range(rotations):
            table = torch.full((S, MB), -1, dtype=torch.int32)
            slots = []
            shared = perm[used:used + P].to(torch.int32)
            used += P
            for s, (ql, L) in enumerate(zip(spec.q_lens, spec.seq_lens)):
                nb = -(-L // bs)
                table[s, :P] = shared
                table[s, P:nb] = perm[used:used + nb - P].to(torch.int32)
                used += nb - P
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
        self.hints = dict(max_query_len=max(spec.q_lens), max_seq_len=max(spec.seq_lens),
                          shared_blocks=spec.shared_prefix_blocks > 0)


FORWARD_KERNELS = ("decode", "combine", "prefill", "prefill_short", "plan", "prefix")


def run_steps(pa, inp: StepInputs, steps: int, warmup: int, shared_prefix: bool = False):
    """Time `steps` steps (KV write + forward). Pass 1 is bracketed by
    synchronize and timed with HIP events on the launch stream, with nothing
    else inside (the step time). Pass 2 repeats the steps with the library's
    kernel timing on (pa.profile_begin/end: HIP events around every kernel
    launch on its stream). Returns (ms per step, {kernel class: mean ms per
    launch}, {kernel class: launches per step}, ms of forward kernels per
    step)."""
    spec = inp.spec

    def step(i):
        st = inp.sets[i % inp.rotations]
        if shared_prefix:
            # the write, then the shared prefix attended once for all rows
            pa.cache_write(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache)
            pa.forward_shared_prefix(st["q"], inp.k_cache, inp.v_cache, st["block_table"],
                                     inp.seq_lens, inp.qsl, spec.scale, spec.shared_prefix_blocks,
                                     out=st["out"], max_seq_len=inp.hints["max_seq_len"])
            return
        pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                             st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                             out=st["out"], **inp.hints)

    for i in range(warmup):
        step(i)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    pa.profile_begin()
    for i in range(steps):
        step(i)
    per = pa.profile_end()
    mean = {k: v[1] / v[0] for k, v in per.items()}
    count = {k: v[0] / steps for k, v in per.items()}
    ms_fwd = sum(per[k][1] for k in FORWARD_KERNELS if k in per) / steps
    return ms_step, mean, count, ms_fwd


def run_graph_steps(pa, inp: StepInputs, steps: int, warmup: int) -> float:
    """The same steps captured once per block-table set in a HIP graph
    (torch.cuda.CUDAGraph over the library's launches) and replayed in turn;
    returns ms per step (HIP events around the replays on the current
    stream)."""
    spec = inp.spec
    graphs = []
    for r in range(inp.rotations):
        st = inp.sets[r]

        def step(st=st):
            pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                                 st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                                 out=st["out"], **inp.hints)
        step()  # kernels loaded and the workspace allocated outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def run_graph_loop(pa, inp: StepInputs, steps: int, warmup: int) -> float:
    """One HIP graph holding one step per block-table set, in order (the
    graph launch paid once per that many steps); returns ms per step (HIP
    events around the replays on the current stream)."""
    spec = inp.spec

    def all_sets():
        for st in inp.sets:
            pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                                 st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                                 out=st["out"], **inp.hints)

    all_sets()  # kernels loaded and the workspace allocated outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        all_sets()
    reps = max(1, steps // inp.rotations)
    for _ in range(max(1, warmup // inp.rotations)):
        g.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * inp.rotations)


PROBE_SHAPES = ((4, 16), (8, 16), (16, 16), (8, 8), (4, 32), (8, 32), (16, 32), (8, 64))


def run_read_probe(pa, inp: StepInputs, steps: int, warmup: int):
    """The library's read probe (every K and V block of the step's rows read
    whole, no arithmetic) over the same block-table rotations, for a few
    launch shapes (waves, table columns per workgroup); returns (best ms per
    launch, its shape, bytes per launch)."""
    spec = inp.spec
    blk = wl.BLOCK_SIZE * spec.num_kv_heads * spec.head_size * 2 * 2
    nbytes = sum(-(-L // wl.BLOCK_SIZE) for L in spec.seq_lens) * blk
    sink = torch.zeros(1, dtype=torch.int32, device=inp.k_cache.device)
    best = None
    for shape in PROBE_SHAPES:
        def launch(i):
            st = inp.sets[i % inp.rotations]
            pa.probe_block_read(inp.k_cache, inp.v_cache, st["block_table"], inp.seq_lens,
                                waves=shape[0], blocks_per_workgroup=shape[1], sink=sink)
        for i in range(warmup):
            launch(i)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            launch(i)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        if best is None or ms < best[0]:
            best = (ms, shape)
    return best[0], best[1], nbytes


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

def decode_source_hash() -> str:
    """Hash of the decode kernel's code (decode.hip and common.h with their
    comments removed and white space collapsed, so that an edit of a comment
    does not count as a change of the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("decode.hip", "common.h"):
        with open(os.path.join(ROOT, "paged_attention_kv_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size), or None when the summary is missing or was
    taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_decode.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("decode_code_sha256_16") != decode_source_hash():
        return None
    for key, k in rec.get("kernels", {}).items():
        name, _, wl = key.partition(" @ ")
        if kernel in name and wl.startswith(workload) and "write_bytes" in k:
            return int(k["read_bytes"] + k["write_bytes"])
    return None


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
    ap.add_argument("--only", choices=["decode", "mixed", "long", "prefix", "tiny", "copy",
                                       "mixed_decode", "mixed_prefill", "spec_decode"],
                    default=None)
    ap.add_argument("--all", action="store_true",
                    help="also time the long-decode, prefix-shared and tiny workloads")
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
    if args.only == "copy":
        # Calibration for the HBM byte counters: a plain device-to-device copy
        # of a known size (COPY_MIB read + COPY_MIB written per launch).
        n = COPY_MIB << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": COPY_MIB, "launches": args.warmup + args.steps}), flush=True)
        return 0

    if args.only in (None, "decode"):
        spec = wl.config(2)
        inp = StepInputs(spec, ROTATIONS, dev)
        ms_step, kmean, kcount, ms_fwd = run_steps(pa, inp, args.steps, args.warmup)
        b_attn = attention_bytes(spec)
        b_step = b_attn + write_bytes(spec)
        gbs = b_step / (ms_step * 1e-3) / 1e9
        ms_graph = run_graph_steps(pa, inp, args.steps, args.warmup)
        ms_graph_loop = run_graph_loop(pa, inp, args.steps, args.warmup)
        ms_probe, probe_shape, probe_bytes = run_read_probe(pa, inp, args.steps, args.warmup)
        fused = "cache_write" not in kcount  # the decode launch also wrote the new tokens
        one_launch = set(kcount) == {"decode"} and abs(kcount["decode"] - 1.0) < 1e-9
        # A step that is one launch: its duration is the events around the
        # whole timed region over the launches in it (gaps between launches
        # included, so never shorter than the kernel). Events around each
        # launch add their own packets to it and read longer.
        ms_dec = ms_step if one_launch else kmean["decode"]
        b_dec = b_step if fused else b_attn
        result["decode"] = dict(ms_step=ms_step, gbs=gbs, ms_fwd=ms_fwd, ms_decode_kernel=ms_dec,
                                kernel_gbs=b_dec / (ms_dec * 1e-3) / 1e9, bytes_step=b_step,
                                bytes_fwd=b_dec, fused=fused, rotations=inp.rotations,
                                ms_graph=ms_graph, ms_graph_loop=ms_graph_loop,
                                one_launch=one_launch,
                                probe=(ms_probe, probe_shape, probe_bytes),
                                kernels={k: round(v * 1e3, 3) for k, v in kmean.items()})
        del inp
        torch.cuda.empty_cache()

    if args.only in (None, "mixed"):
        spec = wl.config(3)
        inp = StepInputs(spec, 1, dev)
        ms_step, kmean_m, _, ms_fwd = run_steps(pa, inp, max(5, args.steps // 5),
                                                max(2, args.warmup // 2))
        dec_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] == 1]
        pre_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] > 1]
        del inp
        torch.cuda.empty_cache()
        sub = {}
        for name, rows in (("decode_rows", dec_rows), ("prefill_rows", pre_rows)):
            ss = sub_spec(spec, rows, name)
            si = StepInputs(ss, 1, dev)
            _, km, _, f_ms = run_steps(pa, si, max(5, args.steps // 5), 2)
            sub[name] = dict(ms_fwd=f_ms, bytes=attention_bytes(ss), flops=attention_flops(ss),
                             kernels={k: round(v * 1e3, 3) for k, v in km.items()})
            del si
            torch.cuda.empty_cache()
        tok_s = spec.num_tokens / (ms_step * 1e-3)
        result["mixed"] = dict(ms_step=ms_step, tokens_per_s=tok_s, ms_fwd=ms_fwd, sub=sub,
                               kernels={k: round(v * 1e3, 3) for k, v in kmean_m.items()})

    others = []
    if args.all or args.only in ("long", "prefix", "tiny", "mixed_decode", "mixed_prefill",
                                 "spec_decode"):
        m3 = wl.config(3)
        for name, i, rot in (("long", 4, 1), ("prefix", 5, ROTATIONS), ("tiny", 1, 1),
                             ("spec_decode", 6, 1), ("mixed_decode", 3, 1),
                             ("mixed_prefill", 3, 1)):
            if args.only != name and (args.only is not None or name.startswith("mixed_")):
                continue
            spec = wl.spec_decode(4) if name == "spec_decode" else wl.config(i)
            if name == "mixed_decode":
                spec = sub_spec(m3, [s for s in range(m3.num_seqs) if m3.q_lens[s] == 1], name)
            if name == "mixed_prefill":
                spec = sub_spec(m3, [s for s in range(m3.num_seqs) if m3.q_lens[s] > 1], name)
            inp = StepInputs(spec, rot, dev)
            ms_step, km, _, ms_fwd = run_steps(pa, inp, args.steps, args.warmup)
            b = attention_bytes(spec)
            entry = dict(workload=spec.description or spec.name, ms_per_step=round(ms_step, 5),
                         ms_forward_kernels=round(ms_fwd, 5), rotations=inp.rotations,
                         forward_gbs_logical=round(b / (ms_fwd * 1e-3) / 1e9, 2),
                         kernel_avg_us={k: round(v * 1e3, 3) for k, v in km.items()},
                         tokens_per_s=round(spec.num_tokens / (ms_step * 1e-3), 1))
            if i == 5:
                uniq = (spec.shared_prefix_blocks + spec.num_seqs * (
                    spec.max_blocks_per_seq - spec.shared_prefix_blocks)) * \
                    2 * spec.block_size * spec.num_kv_heads * spec.head_size * 2
                entry["forward_gbs_unique"] = round(uniq / (ms_fwd * 1e-3) / 1e9, 2)
                # the same step through pa_forward_shared_prefix
                ms2, km2, _, fwd2 = run_steps(pa, inp, args.steps, args.warmup, shared_prefix=True)
                entry["shared_prefix_pass"] = {
                    "ms_per_step": round(ms2, 5), "ms_forward_kernels": round(fwd2, 5),
                    "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in km2.items()},
                    "forward_gbs_logical": round(b / (fwd2 * 1e-3) / 1e9, 2),
                    "forward_gbs_unique": round(uniq / (fwd2 * 1e-3) / 1e9, 2),
                    "tokens_per_s": round(spec.num_tokens / (ms2 * 1e-3), 1)}
            if i == 4:
                entry["frac_of_hbm_peak"] = round(b / (ms_fwd * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                pms, pshape, pbytes = run_read_probe(pa, inp, max(5, args.steps // 5), 2)
                pgbs = pbytes / (pms * 1e-3) / 1e9
                entry["read_probe"] = {"us": round(pms * 1e3, 3), "gbs": round(pgbs, 1),
                                       "waves_blocks_per_wg": list(pshape),
                                       "forward_frac_of_probe": round(b / (ms_fwd * 1e-3) / 1e9
                                                                      / pgbs, 4)}
            if name == "spec_decode":
                entry["frac_of_hbm_peak"] = round(b / (ms_fwd * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                # the same rows without the tight hint: the prefill path
                inp.hints["max_query_len"] = None
                ms2, km2, _, fwd2 = run_steps(pa, inp, args.steps, args.warmup)
                entry["prefill_path"] = {
                    "ms_per_step": round(ms2, 5), "ms_forward_kernels": round(fwd2, 5),
                    "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in km2.items()},
                    "forward_gbs_logical": round(b / (fwd2 * 1e-3) / 1e9, 2)}
            others.append((name, entry))
            del inp
            torch.cuda.empty_cache()

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
            "graph_replay": {"ms_per_step": round(d["ms_graph"], 5),
                             "gbs": round(d["bytes_step"] / (d["ms_graph"] * 1e-3) / 1e9, 2),
                             "note": "the same step captured in a HIP graph per block-table "
                                     "set and replayed (value uses eager launches)"},
            "graph_of_rotations": {"ms_per_step": round(d["ms_graph_loop"], 5),
                                   "gbs": round(d["bytes_step"] / (d["ms_graph_loop"] * 1e-3) / 1e9,
                                                2),
                                   "steps_per_graph": d["rotations"],
                                   "note": "one graph holding one step per block-table set, "
                                           "replayed whole"},
            "block_table_rotations": d["rotations"],
            "pct_of_hbm_peak": round(100 * d["gbs"] / HBM_PEAK_GBS, 2)}
        kname = "decode_kernel<64, 2, true, %s, false>" % ("true" if d["fused"] else "false")
        line["roofline"] = {"bound": "hbm", "kernel": kname,
                            "achieved": round(d["kernel_gbs"], 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(d["kernel_gbs"] / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(kname, "decode ("),
                            "avg_launch_us": round(d["ms_decode_kernel"] * 1e3, 3),
                            "avg_launch_us_from": ("events around the timed region / launches"
                                                   if d["one_launch"] else
                                                   "events around each launch"),
                            "algorithmic_bytes_per_launch": d["bytes_fwd"],
                            "forward_kernels_us_per_step": round(d["ms_fwd"] * 1e3, 3),
                            "kernel_avg_us": d["kernels"]}
        pms, pshape, pbytes = d["probe"]
        pgbs = pbytes / (pms * 1e-3) / 1e9
        line["roofline"]["read_probe"] = {
            "what": "the same blocks read whole with no arithmetic (pa_probe_block_read), "
                    "best of %d launch shapes" % len(PROBE_SHAPES),
            "us": round(pms * 1e3, 3), "bytes": pbytes, "gbs": round(pgbs, 1),
            "frac_of_peak": round(pgbs / HBM_PEAK_GBS, 4),
            "waves_blocks_per_wg": list(pshape),
            "kernel_frac_of_probe": round(d["kernel_gbs"] / pgbs, 4)}
    if "mixed" in result:
        m = result["mixed"]
        pre = m["sub"]["prefill_rows"]
        dec = m["sub"]["decode_rows"]
        line["mixed_step"] = {
            "workload": ("mixed chunked-prefill step, 8192 new tokens: 256 decode rows (context "
                         "U[256,8192]) + 4 chunks of 1984 tokens (prior context U[0,4096]); "
                         "32 q / 8 kv heads, head_size 128"),
            "tokens_per_s": round(m["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(m["ms_step"], 4), "ms_forward_kernels": round(m["ms_fwd"], 4),
            "kernel_avg_us": m["kernels"],
            "prefill_rows": {"ms": round(pre["ms_fwd"], 4), "flops": pre["flops"],
                             "kernel_avg_us": pre["kernels"],
                             "tflops": round(pre["flops"] / (pre["ms_fwd"] * 1e-3) / 1e12, 2),
                             "frac_of_bf16_peak": round(pre["flops"] / (pre["ms_fwd"] * 1e-3)
                                                        / 1e12 / BF16_PEAK_TFLOPS, 4),
                             # the tile kernel alone (events around each launch)
                             "tile_kernel_frac_of_bf16_peak": round(
                                 pre["flops"] / (pre["kernels"]["prefill"] * 1e-6) / 1e12
                                 / BF16_PEAK_TFLOPS, 4) if "prefill" in pre["kernels"] else None},
            "decode_rows": {"ms": round(dec["ms_fwd"], 4), "bytes": dec["bytes"],
                            "kernel_avg_us": dec["kernels"],
                            "gbs": round(dec["bytes"] / (dec["ms_fwd"] * 1e-3) / 1e9, 2),
                            "frac_of_hbm_peak": round(dec["bytes"] / (dec["ms_fwd"] * 1e-3)
                                                      / 1e9 / HBM_PEAK_GBS, 4)}}
        if "value" not in line:
            line.update(value=round(m["tokens_per_s"], 1), unit="tokens/s",
                        ms_per_step=round(m["ms_step"], 5),
                        config={"workload": line["mixed_step"]["workload"]})
    for name, entry in others:
        line.setdefault("other_workloads", {})[name] = entry
    if "value" not in line and others:
        name, entry = others[0]
        line.update(value=entry["forward_gbs_logical"], unit="GB/s",
                    ms_per_step=entry["ms_per_step"], config={"workload": entry["workload"]})
    if not args.no_cpu and "decode" in result:
        line["cpu_baseline"] = cpu_baseline(wl.config(2))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
