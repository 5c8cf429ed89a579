"""Benchmark of the paged-attention hot path on one MI355X.

One step = the whole hot path over one batch: the KV-cache write of the
step's new tokens and paged attention of the flattened batch, through
pa_write_and_forward (one launch for a batch of decode rows on the
partitioned schedule; a write launch and the forward launches otherwise).
Inputs are synthetic, seeded, and resident in HBM before the timed region
starts.

One JSON line on stdout:
  * value: decode GB/s on the decode workload (64 sequences x 1 query token,
    context U[512, 2048], 32 q / 4 kv heads, D 64, 16-token blocks, 100k-block
    bf16 pool); bytes are algorithmic (each row's K and V context once, q, out,
    and the KV write), time is the whole step. Eight disjoint block-table sets
    drawn from the same pool rotate between steps so the 256 MiB Infinity
    Cache cannot hold a step's KV. config.step_us gives the median, p10 and
    p90 of single steps; config.graph_* the same step replayed from graphs.
  * roofline: the decode kernel's algorithmic bytes per launch (with the
    KV write when the launch does it) over its average launch duration (HIP
    events on the launch stream), against 8 TB/s, with the read probe.
  * mixed_step: tokens/s of the 8192-token mixed chunked-prefill step (256
    decode rows + 4 x 1984-token chunks, 32 q / 8 kv heads, D 128), and its
    decode rows (HBM roofline) and prefill rows (bf16 matrix-core roofline)
    timed apart.
  * workloads: the other named workloads, each with its roofline fraction:
    long_decode (16 x 32768), prefix_shared (256 rows sharing a 4096-token
    prefix, per-row path and shared-prefix pass), tiny (two short prompts)
    and spec_verify (256 rows of 4 query tokens).
  * cpu_baseline: the CPU oracle (float32) timed on this host on one step of
    the decode workload, all threads and one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--only decode|mixed|long|prefix|tiny|spec_decode|...]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
import types

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
MIXED_WARMUP = 40  # untimed steps before the mixed step is timed (see leg_mixed)
GRAPH_NOTE = ("the same step captured in a HIP graph per block-table set and replayed "
              "(value uses eager launches)")


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


# (write_plan: the KV write and the tile planner in one launch, counted with
# the planner)
FORWARD_KERNELS = ("decode", "combine", "prefill", "prefill_short", "plan", "prefix",
                   "write_plan")


def percentile(xs, f):
    """The f-quantile (0..1) of xs by linear interpolation between ranks."""
    v = sorted(xs)
    if not v:
        return float("nan")
    x = f * (len(v) - 1)
    lo = int(math.floor(x))
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def run_steps(pa, inp: StepInputs, steps: int, warmup: int, shared_prefix: bool = False,
              serial: bool = False):
    """Time `steps` steps (KV write + forward). Pass 1 is bracketed by
    synchronize and timed with HIP events on the launch stream, with nothing
    else inside: the step time. Pass 2 records an event between consecutive
    steps for the distribution of single steps (median, p10, p90; the events
    add their own packets, so these read a little longer). Pass 3 repeats
    the steps with the library's kernel timing on (pa.profile_begin/end: HIP
    events around every kernel launch on its stream). Returns a dict:
    ms_step, ms_median, ms_p10, ms_p90, kernels {class: mean ms per launch},
    counts {class: launches per step}, ms_fwd (forward kernels per step).
    serial: a mixed batch's launches stay on one stream (PA_FORWARD_SERIAL)."""
    spec = inp.spec

    def step(i):
        st = inp.sets[i % inp.rotations]
        if shared_prefix:
            # the shared prefix attended once for all rows, the write in its
            # launch; then the rows' own blocks
            pa.write_and_forward_shared_prefix(st["k"], st["v"], st["slot_mapping"], inp.k_cache,
                                               inp.v_cache, st["q"], st["block_table"],
                                               inp.seq_lens, inp.qsl, spec.scale,
                                               spec.shared_prefix_blocks, out=st["out"],
                                               max_seq_len=inp.hints["max_seq_len"])
            return
        pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                             st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                             out=st["out"], serial=serial, **inp.hints)

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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record()
        step(i)
    ev[steps].record()
    torch.cuda.synchronize()
    each = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    pa.profile_begin()
    for i in range(steps):
        step(i)
    per = pa.profile_end()
    return dict(ms_step=ms_step, ms_median=percentile(each, 0.5), ms_p10=percentile(each, 0.1),
                ms_p90=percentile(each, 0.9),
                kernels={k: v[1] / v[0] for k, v in per.items()},
                counts={k: v[0] / steps for k, v in per.items()},
                ms_fwd=sum(per[k][1] for k in FORWARD_KERNELS if k in per) / steps)


def dist_us(t):
    """Step-time distribution of a run_steps result, in microseconds."""
    return {"median": round(t["ms_median"] * 1e3, 3), "p10": round(t["ms_p10"] * 1e3, 3),
            "p90": round(t["ms_p90"] * 1e3, 3)}


def graph_workspace(pa, inp: StepInputs) -> torch.Tensor:
    """A workspace owned by the caller for captured steps (zeroed: its
    counter region must start at zero), kept alive with the graphs."""
    s = inp.spec
    n = pa.forward_workspace_bytes(s.num_tokens, s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                   s.head_size, s.max_blocks_per_seq,
                                   max_seq_len=inp.hints["max_seq_len"],
                                   max_query_len=inp.hints["max_query_len"])
    return torch.zeros(n, dtype=torch.uint8, device=inp.k_cache.device)


def run_graph_steps(pa, inp: StepInputs, steps: int, warmup: int) -> float:
    """The same steps captured once per block-table set in a HIP graph
    (torch.cuda.CUDAGraph over the library's launches) and replayed in turn;
    returns ms per step (HIP events around the replays on the current
    stream)."""
    spec = inp.spec
    ws = graph_workspace(pa, inp)
    graphs = []
    for r in range(inp.rotations):
        st = inp.sets[r]

        def step(st=st):
            pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                                 st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                                 out=st["out"], workspace=ws, **inp.hints)
        step()  # kernels loaded and the workspace allocated outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        graphs.append(g)
    # every graph replayed (uploaded, first-launch costs paid) before timing
    for i in range(max(warmup, 2 * len(graphs))):
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
    ws = graph_workspace(pa, inp)

    def all_sets():
        for st in inp.sets:
            pa.write_and_forward(st["k"], st["v"], st["slot_mapping"], inp.k_cache, inp.v_cache,
                                 st["q"], st["block_table"], inp.seq_lens, inp.qsl, spec.scale,
                                 out=st["out"], workspace=ws, **inp.hints)

    all_sets()  # kernels loaded and the workspace allocated outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        all_sets()
    reps = max(1, steps // inp.rotations)
    for _ in range(max(2, warmup // inp.rotations)):
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


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, budget_s: float = 6.0):
    """The oracle as it stands, in float32, on this host: one step of the
    workload (the KV write of its new tokens with ref_cache_write, then
    ref_forward over all rows) on a CPU copy of just the blocks the rows
    read. Timed with all of torch's threads and with one thread: one warm-up
    run, then runs until at least 3 and about budget_s seconds; the median
    run counts. Input generation and the copy are outside the timing."""
    import oracle
    case = wl.make_case(spec, device="cpu")
    q, kc, vc, table, lens, qsl, tmap = wl.sequences_subset(case, list(range(spec.num_seqs)))
    # the new tokens' slots in the compacted copy of the pool (plumbing: the
    # same block and row, renumbered the way sequences_subset renumbers)
    bs = spec.block_size
    bt = case.block_table
    used = torch.unique(torch.cat([bt[s_, :-(-L // bs)].to(torch.int64)
                                   for s_, L in enumerate(spec.seq_lens)]))
    slots = case.slot_mapping[tmap]
    local = torch.searchsorted(used, slots // bs) * bs + slots % bs
    k, v = case.k[tmap], case.v[tmap]
    nbytes = attention_bytes(spec) + write_bytes(spec)

    def one_step():
        oracle.ref_cache_write(k, v, local, kc, vc)
        oracle.ref_forward(q, kc, vc, table, lens, qsl, spec.scale, dtype=torch.float32)

    default_threads = torch.get_num_threads()
    runs = {}
    for threads in (default_threads, 1):
        torch.set_num_threads(threads)
        one_step()
        times = []
        t_start = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 200):
            t = time.perf_counter()
            one_step()
            times.append(time.perf_counter() - t)
        med = percentile(times, 0.5)
        runs[threads] = dict(ms_per_step=round(med * 1e3, 3), runs=len(times),
                             gbs=round(nbytes / med / 1e9, 4))
    torch.set_num_threads(default_threads)
    full, one = runs[default_threads], runs[1]
    return dict(value=full["gbs"], unit="GB/s", cores=default_threads, kind="oracle",
                sample=(f"one step of the decode workload: ref_cache_write of its {spec.num_tokens} "
                        f"new tokens and ref_forward of all {spec.num_seqs} rows in float32 "
                        f"(PyTorch CPU) on a copy of the blocks they read; median of "
                        f"{full['runs']} runs after a warm-up"),
                ms_per_step=full["ms_per_step"], cpu_model=cpu_model(),
                nproc=os.cpu_count(),
                one_thread={"value": one["gbs"], "ms_per_step": one["ms_per_step"],
                            "runs": one["runs"]})


# ---------------------------------------------------------------------------
# Workload legs
# ---------------------------------------------------------------------------

def progress(msg):
    """One line on stderr as each part of the run ends (stdout holds only the
    JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def frac(x, peak):
    return round(x / peak, 4)


def leg_decode(pa, args, dev):
    """Workload 2, the headline: the decode step through one
    pa_write_and_forward launch, graph replays, and the read probe."""
    spec = wl.config(2)
    inp = StepInputs(spec, ROTATIONS, dev)
    # The read probe and the graph forms are measured first: they read the
    # same blocks, so the eager steps timed last do not carry the first
    # launches' start-up (clocks, translations) of a fresh process, whatever
    # the warm-up count.
    ms_probe, probe_shape, probe_bytes = run_read_probe(pa, inp, args.steps, args.warmup)
    ms_graph = run_graph_steps(pa, inp, args.steps, args.warmup)
    ms_graph_loop = run_graph_loop(pa, inp, args.steps, args.warmup)
    t = run_steps(pa, inp, args.steps, args.warmup)
    b_attn = attention_bytes(spec)
    b_step = b_attn + write_bytes(spec)
    gbs = b_step / (t["ms_step"] * 1e-3) / 1e9
    kcount = t["counts"]
    fused = "cache_write" not in kcount  # the decode launch also wrote the new tokens
    one_launch = set(kcount) == {"decode"} and abs(kcount["decode"] - 1.0) < 1e-9
    # A step that is one launch: its duration is the events around the
    # whole timed region over the launches in it (gaps between launches
    # included, so never shorter than the kernel). Events around each
    # launch add their own packets to it and read longer.
    ms_dec = t["ms_step"] if one_launch else t["kernels"]["decode"]
    b_dec = b_step if fused else b_attn
    kernel_gbs = b_dec / (ms_dec * 1e-3) / 1e9
    config = {
        "workload": ("decode step: 64 sequences x 1 query token, context U[512,2048], "
                     "32 q / 4 kv heads, head_size 64, block 16, 100k-block bf16 pool; "
                     "KV write + paged attention"),
        "tokens": spec.num_tokens, "kv_bytes_per_step": b_step,
        "step_us": dist_us(t),
        "graph_replay": {"ms_per_step": round(ms_graph, 5),
                         "gbs": round(b_step / (ms_graph * 1e-3) / 1e9, 2),
                         "note": GRAPH_NOTE},
        "graph_of_rotations": {"ms_per_step": round(ms_graph_loop, 5),
                               "gbs": round(b_step / (ms_graph_loop * 1e-3) / 1e9, 2),
                               "steps_per_graph": inp.rotations,
                               "note": "one graph holding one step per block-table set, "
                                       "replayed whole"},
        "block_table_rotations": inp.rotations,
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    kname = "decode_kernel<64, 2, true, %s, false>" % ("true" if fused else "false")
    pgbs = probe_bytes / (ms_probe * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(kernel_gbs, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": frac(kernel_gbs, HBM_PEAK_GBS),
                "traffic": measured_traffic(kname, "decode ("),
                "avg_launch_us": round(ms_dec * 1e3, 3),
                "avg_launch_us_from": ("events around the timed region / launches"
                                       if one_launch else "events around each launch"),
                "algorithmic_bytes_per_launch": b_dec,
                "forward_kernels_us_per_step": round(t["ms_fwd"] * 1e3, 3),
                "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
                "read_probe": {
                    "what": "the same blocks read whole with no arithmetic "
                            "(pa_probe_block_read), best of %d launch shapes" % len(PROBE_SHAPES),
                    "us": round(ms_probe * 1e3, 3), "bytes": probe_bytes, "gbs": round(pgbs, 1),
                    "frac_of_peak": frac(pgbs, HBM_PEAK_GBS),
                    "waves_blocks_per_wg": list(probe_shape),
                    "kernel_frac_of_probe": round(kernel_gbs / pgbs, 4)}}
    return dict(value=round(gbs, 2), ms_step=t["ms_step"], config=config, roofline=roofline)


def leg_mixed(pa, args, dev):
    """Workload 3: the mixed chunked-prefill step (tokens/s), and its decode
    and prefill rows timed as batches of their own to attribute HBM and
    matrix-core use."""
    spec = wl.config(3)
    inp = StepInputs(spec, 1, dev)
    # With the prefill tiles running beside the decode launch, the first
    # ~20-30 steps after a start or an idle pause run 5-15% slower before the
    # step time settles; the leg times the settled steps.
    warm = max(args.warmup, MIXED_WARMUP)
    t = run_steps(pa, inp, args.steps, warm)
    t_ser = run_steps(pa, inp, args.steps, warm, serial=True)
    dec_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] == 1]
    pre_rows = [s for s in range(spec.num_seqs) if spec.q_lens[s] > 1]
    del inp
    torch.cuda.empty_cache()
    sub = {}
    for name, rows in (("decode_rows", dec_rows), ("prefill_rows", pre_rows)):
        ss = sub_spec(spec, rows, name)
        si = StepInputs(ss, 1, dev)
        st = run_steps(pa, si, args.steps, args.warmup)
        sub[name] = dict(t=st, bytes=attention_bytes(ss), flops=attention_flops(ss))
        del si
        torch.cuda.empty_cache()
    pre, dec = sub["prefill_rows"], sub["decode_rows"]
    pre_ms, dec_ms = pre["t"]["ms_fwd"], dec["t"]["ms_fwd"]
    pre_tf = pre["flops"] / (pre_ms * 1e-3) / 1e12
    tile_us = pre["t"]["kernels"].get("prefill", float("nan")) * 1e3
    dec_gbs = dec["bytes"] / (dec_ms * 1e-3) / 1e9
    return {
        "workload": ("mixed chunked-prefill step, 8192 new tokens: 256 decode rows (context "
                     "U[256,8192]) + 4 chunks of 1984 tokens (prior context U[0,4096]); "
                     "32 q / 8 kv heads, head_size 128"),
        "tokens_per_s": round(spec.num_tokens / (t["ms_step"] * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(t["ms_step"], 4), "step_us": dist_us(t),
        "ms_forward_kernels": round(t["ms_fwd"], 4),
        "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
        "warmup_steps": warm,
        "overlap": ("prefill launches on the library's second stream beside the decode "
                    "launch (160 even shares); ms_forward_kernels sums kernels that overlap"),
        "serial": {"ms_per_step": round(t_ser["ms_step"], 4), "step_us": dist_us(t_ser),
                   "tokens_per_s": round(spec.num_tokens / (t_ser["ms_step"] * 1e-3), 1),
                   "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t_ser["kernels"].items()},
                   "note": "the same step with PA_FORWARD_SERIAL (one stream, 256 shares)"},
        "prefill_rows": {
            "ms": round(pre_ms, 4), "flops": pre["flops"],
            "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in pre["t"]["kernels"].items()},
            "tflops": round(pre_tf, 2),
            "roofline": {"bound": "mfma", "kernel": "prefill_tile_kernel (all forward launches)",
                         "achieved": round(pre_tf, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": frac(pre_tf, BF16_PEAK_TFLOPS)},
            "tile_kernel_frac_of_bf16_peak": frac(pre["flops"] / (tile_us * 1e-6) / 1e12,
                                                  BF16_PEAK_TFLOPS)},
        "decode_rows": {
            "ms": round(dec_ms, 4), "bytes": dec["bytes"],
            "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in dec["t"]["kernels"].items()},
            "gbs": round(dec_gbs, 2),
            "roofline": {"bound": "hbm", "kernel": "decode_stream_kernel<128, 2, true>",
                         "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": frac(dec_gbs, HBM_PEAK_GBS)}}}


def leg_long(pa, args, dev):
    """Workload 4: 16 rows at context 32768, the rows shared out evenly."""
    spec = wl.config(4)
    inp = StepInputs(spec, 1, dev)
    t = run_steps(pa, inp, args.steps, args.warmup)
    b = attention_bytes(spec)
    gbs = b / (t["ms_fwd"] * 1e-3) / 1e9
    pms, pshape, pbytes = run_read_probe(pa, inp, args.steps, args.warmup)
    pgbs = pbytes / (pms * 1e-3) / 1e9
    return {
        "workload": spec.description, "ms_per_step": round(t["ms_step"], 5),
        "step_us": dist_us(t), "ms_forward_kernels": round(t["ms_fwd"], 5),
        "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
        "tokens_per_s": round(spec.num_tokens / (t["ms_step"] * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "decode_stream_kernel<128, 2, true>",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": frac(gbs, HBM_PEAK_GBS), "algorithmic_bytes_per_launch": b,
                     "kernel_trace": "profiles/decode_stream_kernel_long-decode-16x32768.md"},
        "read_probe": {"us": round(pms * 1e3, 3), "gbs": round(pgbs, 1),
                       "frac_of_peak": frac(pgbs, HBM_PEAK_GBS),
                       "waves_blocks_per_wg": list(pshape),
                       "forward_frac_of_probe": round(gbs / pgbs, 4)}}


def leg_prefix(pa, args, dev):
    """Workload 5: 256 rows sharing a 4096-token prefix, on the per-row path
    and through the shared-prefix pass."""
    spec = wl.config(5)
    inp = StepInputs(spec, ROTATIONS, dev)
    b = attention_bytes(spec)
    blk = 2 * spec.block_size * spec.num_kv_heads * spec.head_size * 2
    uniq = (spec.shared_prefix_blocks + spec.num_seqs * (
        spec.max_blocks_per_seq - spec.shared_prefix_blocks)) * blk
    pre_flops = (4 * spec.head_size * spec.num_q_heads * spec.num_seqs
                 * spec.shared_prefix_blocks * spec.block_size)
    out = {"workload": spec.description, "rotations": inp.rotations,
           "logical_bytes": b, "unique_bytes": uniq, "ms_per_step": None}
    for name, sp in (("per_row_path", False), ("shared_prefix_pass", True)):
        t = run_steps(pa, inp, args.steps, args.warmup, shared_prefix=sp)
        e = {"ms_per_step": round(t["ms_step"], 5), "step_us": dist_us(t),
             "ms_forward_kernels": round(t["ms_fwd"], 5),
             "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
             "forward_gbs_logical": round(b / (t["ms_fwd"] * 1e-3) / 1e9, 2),
             "forward_gbs_unique": round(uniq / (t["ms_fwd"] * 1e-3) / 1e9, 2),
             "tokens_per_s": round(spec.num_tokens / (t["ms_step"] * 1e-3), 1)}
        e["roofline"] = {"bound": "hbm", "achieved": e["forward_gbs_unique"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": frac(e["forward_gbs_unique"], HBM_PEAK_GBS),
                         "bytes": "unique (each shared block counted once)"}
        if sp and "prefix" in t["kernels"]:
            tf = pre_flops / (t["kernels"]["prefix"] * 1e-3) / 1e12
            e["prefix_kernel"] = {"bound": "mfma", "achieved": round(tf, 2),
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": frac(tf, BF16_PEAK_TFLOPS), "flops": pre_flops,
                                  "note": "its launch also writes the step's new tokens"}
        out[name] = e
    # the workload's step time is that of its faster path, the shared-prefix pass
    out["ms_per_step"] = out["shared_prefix_pass"]["ms_per_step"]
    # the rows' own blocks (past the prefix) read whole with no arithmetic:
    # the memory system's rate for the rows' pass of the shared-prefix call
    P = spec.shared_prefix_blocks
    own_spec = wl.Spec("own_blocks", spec.num_q_heads, spec.num_kv_heads, spec.head_size,
                       num_blocks=spec.num_blocks, max_blocks_per_seq=spec.max_blocks_per_seq - P,
                       q_lens=spec.q_lens,
                       seq_lens=tuple(L - P * spec.block_size for L in spec.seq_lens),
                       seed_layout=spec.seed_layout, seed_values=spec.seed_values)
    own = types.SimpleNamespace(
        spec=own_spec, k_cache=inp.k_cache, v_cache=inp.v_cache, rotations=inp.rotations,
        seq_lens=torch.tensor(own_spec.seq_lens, dtype=torch.int32, device=dev),
        sets=[{"block_table": st["block_table"][:, P:].contiguous()} for st in inp.sets])
    pms, pshape, pbytes = run_read_probe(pa, own, args.steps, args.warmup)
    rows_us = out["shared_prefix_pass"]["kernel_avg_us"].get("decode")
    out["own_blocks_read_probe"] = {
        "what": "the rows' own blocks past the prefix read whole with no arithmetic "
                "(pa_probe_block_read), best of %d launch shapes" % len(PROBE_SHAPES),
        "us": round(pms * 1e3, 3), "bytes": pbytes,
        "gbs": round(pbytes / (pms * 1e-3) / 1e9, 1),
        "rows_pass_us": rows_us,
        "note": "the rows' pass also reads the prefix chunks' partials and merges them"}
    return out


def leg_tiny(pa, args, dev):
    """Workload 1: two short prompts (launch-bound; parity is its point)."""
    spec = wl.config(1)
    inp = StepInputs(spec, 1, dev)
    t = run_steps(pa, inp, args.steps, args.warmup)
    ms_graph = run_graph_steps(pa, inp, args.steps, args.warmup)
    return {"workload": spec.description, "ms_per_step": round(t["ms_step"], 5),
            "step_us": dist_us(t), "ms_forward_kernels": round(t["ms_fwd"], 5),
            "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
            "launches_per_step": {k: round(v, 2) for k, v in t["counts"].items()},
            "bound": "launch", "flops": attention_flops(spec),
            "graph_replay": {"ms_per_step": round(ms_graph, 5),
                             "note": "the step's launches captured in one HIP graph and "
                                     "replayed (ms_per_step uses eager launches)"}}


def leg_spec(pa, args, dev):
    """Rows verifying 3 drafted tokens (4 query tokens each): on the decode
    path (the tight max_query_len hint) and on the prefill path."""
    spec = wl.spec_decode(4)
    inp = StepInputs(spec, 1, dev)
    b = attention_bytes(spec)
    t = run_steps(pa, inp, args.steps, args.warmup)
    gbs = b / (t["ms_fwd"] * 1e-3) / 1e9
    out = {"workload": spec.description, "ms_per_step": round(t["ms_step"], 5),
           "step_us": dist_us(t), "ms_forward_kernels": round(t["ms_fwd"], 5),
           "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()},
           "forward_gbs_logical": round(gbs, 2),
           "roofline": {"bound": "hbm", "kernel": "decode_stream_kernel<128, 2, true>",
                        "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": frac(gbs, HBM_PEAK_GBS)}}
    inp.hints["max_query_len"] = None
    t2 = run_steps(pa, inp, args.steps, args.warmup)
    out["prefill_path"] = {
        "ms_per_step": round(t2["ms_step"], 5), "ms_forward_kernels": round(t2["ms_fwd"], 5),
        "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t2["kernels"].items()},
        "forward_gbs_logical": round(b / (t2["ms_fwd"] * 1e-3) / 1e9, 2)}
    return out


def leg_sub(pa, args, dev, which):
    """Workload 3's decode rows or prefill rows alone (profiling runs)."""
    m3 = wl.config(3)
    rows = [s for s in range(m3.num_seqs) if (m3.q_lens[s] == 1) == (which == "mixed_decode")]
    spec = sub_spec(m3, rows, which)
    inp = StepInputs(spec, 1, dev)
    t = run_steps(pa, inp, args.steps, args.warmup)
    return {"workload": which, "ms_per_step": round(t["ms_step"], 5),
            "ms_forward_kernels": round(t["ms_fwd"], 5),
            "kernel_avg_us": {k: round(v * 1e3, 3) for k, v in t["kernels"].items()}}


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
                    help="accepted for compatibility: every workload runs by default")
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

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 values, seeded lengths and block placement)"}
    only = args.only
    if only in ("mixed_decode", "mixed_prefill"):
        line["workloads"] = {only: leg_sub(pa, args, dev, only)}
        print(json.dumps(line), flush=True)
        return 0
    if only in (None, "decode"):
        t_leg = time.perf_counter()
        d = leg_decode(pa, args, dev)
        progress(f"decode done in {time.perf_counter() - t_leg:.1f} s")
        line.update(value=d["value"], unit="GB/s", ms_per_step=round(d["ms_step"], 5),
                    config=d["config"], roofline=d["roofline"])
        torch.cuda.empty_cache()
    legs = (("mixed_step", "mixed", leg_mixed), ("long_decode", "long", leg_long),
            ("prefix_shared", "prefix", leg_prefix), ("tiny", "tiny", leg_tiny),
            ("spec_verify", "spec_decode", leg_spec))
    for key, name, fn in legs:
        if only not in (None, name):
            continue
        t_leg = time.perf_counter()
        entry = fn(pa, args, dev)
        progress(f"{key} done in {time.perf_counter() - t_leg:.1f} s")
        torch.cuda.empty_cache()
        if key == "mixed_step":
            line["mixed_step"] = entry
        else:
            line.setdefault("workloads", {})[key] = entry
    if "value" not in line:
        # a single-workload profiling run: its own rate stands as the value
        if "mixed_step" in line:
            m = line["mixed_step"]
            line.update(value=m["tokens_per_s"], unit="tokens/s", ms_per_step=m["ms_per_step"],
                        config={"workload": m["workload"]})
        else:
            (key, e), = line["workloads"].items()
            line.update(value=e["ms_per_step"], unit="ms", ms_per_step=e["ms_per_step"],
                        higher_is_better=False, config={"workload": e["workload"]})
    if not args.no_cpu and only in (None, "decode"):
        t_leg = time.perf_counter()
        line["cpu_baseline"] = cpu_baseline(wl.config(2))
        progress(f"cpu_baseline done in {time.perf_counter() - t_leg:.1f} s")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
