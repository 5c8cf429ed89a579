"""What the oracle is given in GPU parity tests.

``OracleView(case, seqs)`` copies to the CPU everything the listed rows read
(their query rows and the cache blocks their tables name), and it must be
made before any library call touches the case. Library output never reaches
the oracle through it: the step's new tokens are written into that copy by
the oracle's own ``ref_cache_write`` from the seeded k and v (or from the
k, v and q a test passes in), and ``ref_forward`` then runs on the copy.
Cache rows that no sequence has cached yet hold the workload's poison in the
copy, exactly as they did on the device before the call, so a row the
library reads past its sequence, or a new token it fails to take into
account, shows up as a mismatch.
"""

from __future__ import annotations

import torch

import oracle
import workloads as wl

# The bar for attention outputs (bf16 result against the oracle's float64).
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def assert_close(got, want, what=""):
    """Max abs error <= MAX_ABS and mean abs error <= MEAN_ABS, all finite."""
    got = got.detach().cpu().double()
    want = want.detach().cpu().double()
    assert got.shape == want.shape
    assert torch.isfinite(got).all(), f"{what}: non-finite output"
    err = (got - want).abs()
    mx, mean = err.max().item(), err.mean().item()
    print(f"  {what}: max abs {mx:.3e} mean abs {mean:.3e} over {got.numel()} values", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"


class OracleView:
    def __init__(self, case, seqs):
        self.case = case
        self.seqs = list(seqs)
        (self.q, self.kc, self.vc, self.table, self.lens, self.qsl,
         self.tmap) = wl.sequences_subset(case, self.seqs)
        bs = case.spec.block_size
        bt = case.block_table.cpu()
        lens = case.seq_lens.cpu().tolist()
        # the full pool's blocks read by these rows, in the order of the copy
        self.used = torch.unique(torch.cat([bt[s, :-(-lens[s] // bs)].to(torch.int64)
                                            for s in self.seqs]))

    def expect(self, tokens_per_seq=None, q=None, k=None, v=None, slot_mapping=None,
               dtype=torch.float64):
        """Oracle output of the rows (optionally only some query rows of
        each: {sequence: [row within the sequence, ...]}). q, k, v and
        slot_mapping default to the case's; pass the ones a test fed the
        library when it changed them after the view was made. Returns
        (flattened row indices of the full batch, [R, Hq, D] result)."""
        c = self.case
        bs = c.spec.block_size
        tm = self.tmap
        kk = (c.k if k is None else k).cpu()[tm]
        vv = (c.v if v is None else v).cpu()[tm]
        slots = (c.slot_mapping if slot_mapping is None else slot_mapping).cpu()[tm]
        keep = slots >= 0
        blk, off = slots[keep] // bs, slots[keep] % bs
        pos = torch.searchsorted(self.used, blk)
        assert bool((self.used[pos.clamp(max=len(self.used) - 1)] == blk).all()), \
            "a new token's slot lies outside the blocks its row reads"
        # the same slots every call, so earlier writes are simply overwritten
        oracle.ref_cache_write(kk[keep], vv[keep], pos * bs + off, self.kc, self.vc)
        qq = self.q if q is None else q.cpu()[tm]
        pick = None
        if tokens_per_seq is not None:
            pick = []
            for i, s in enumerate(self.seqs):
                base = int(self.qsl[i])
                pick.extend(base + r for r in tokens_per_seq.get(s, ()))
        want = oracle.ref_forward(qq, self.kc, self.vc, self.table, self.lens, self.qsl,
                                  c.scale, dtype=dtype, tokens=pick)
        rows = list(range(qq.shape[0])) if pick is None else pick
        return tm[rows], want[rows]


def assert_pool_written(k_cache, v_cache, k0, v0, k, v, slot_mapping, block_size=16):
    """After a call that wrote the step's tokens: the blocks holding the
    step's slots equal a CPU copy of their state before the call (k0, v0,
    taken before any library call) with ref_cache_write applied, bit for
    bit; every other block of the pool is unchanged."""
    slots = slot_mapping.cpu()
    blocks = torch.unique(slots[slots >= 0] // block_size)
    nb = k_cache.shape[0]
    remap = torch.full((nb,), -1, dtype=torch.int64)
    remap[blocks] = torch.arange(blocks.numel())
    sc = slots.clamp(min=0)
    local = torch.where(slots >= 0, remap[sc // block_size] * block_size + sc % block_size, slots)
    dev = k_cache.device
    kref = k0[blocks.to(dev)].cpu()
    vref = v0[blocks.to(dev)].cpu()
    oracle.ref_cache_write(k.cpu(), v.cpu(), local, kref, vref)
    assert torch.equal(k_cache[blocks.to(dev)].cpu().view(torch.int16), kref.view(torch.int16))
    assert torch.equal(v_cache[blocks.to(dev)].cpu().view(torch.int16), vref.view(torch.int16))
    rest = torch.ones(nb, dtype=torch.bool, device=dev)
    rest[blocks.to(dev)] = False
    assert torch.equal(k_cache[rest].view(torch.int16), k0[rest].view(torch.int16)), \
        "a K block outside the step's slots changed"
    assert torch.equal(v_cache[rest].view(torch.int16), v0[rest].view(torch.int16)), \
        "a V block outside the step's slots changed"
