"""Python handle on the native block manager and step planner
(include/pa_sched.h): argument marshalling only."""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import BLOCK_SIZE, PaError, SchedStats, load_library


@dataclass
class StepInputs:
    """One planned step's kernel inputs (host arrays)."""
    request_ids: np.ndarray      # int64 [S]
    query_start_loc: np.ndarray  # int32 [S+1]
    seq_lens: np.ndarray         # int32 [S]
    block_table: np.ndarray      # int32 [S, MB]
    slot_mapping: np.ndarray     # int64 [T]
    token_ids: np.ndarray        # int32 [T]
    positions: np.ndarray        # int32 [T]

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    def shared_prefix_blocks(self) -> int:
        """Leading blocks every row shares, when every row is a decode row
        (pa_sched_shared_prefix_blocks); above 0, the step can take the
        shared-prefix calls."""
        if self.num_seqs == 0:
            return 0
        qsl = np.ascontiguousarray(self.query_start_loc, dtype=np.int32)
        lens = np.ascontiguousarray(self.seq_lens, dtype=np.int32)
        table = np.ascontiguousarray(self.block_table, dtype=np.int32)
        return int(load_library().pa_sched_shared_prefix_blocks(
            _ptr(qsl), _ptr(lens), _ptr(table), self.num_seqs, table.shape[1]))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class Scheduler:
    """Block pool, prefix cache and step planner over ``num_blocks`` blocks."""

    def __init__(self, num_blocks: int, max_num_batched_tokens: int, max_num_seqs: int = 256,
                 long_prefill_token_threshold: int = 0, enable_prefix_caching: bool = True):
        self._lib = load_library()
        h = self._lib.pa_sched_create(num_blocks, BLOCK_SIZE, max_num_batched_tokens,
                                      max_num_seqs, long_prefill_token_threshold,
                                      1 if enable_prefix_caching else 0)
        if not h:
            raise ValueError(self._lib.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)

    def close(self) -> None:
        if self._h:
            self._lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, status: int) -> None:
        if status != 0:
            raise PaError(status, self._lib.pa_last_error().decode())

    def add_request(self, request_id: int, prompt: Sequence[int], max_new_tokens: int) -> None:
        p = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
        self._check(self._lib.pa_sched_add_request(self._h, request_id, _ptr(p), int(p.size),
                                                   max_new_tokens))

    def schedule(self, table_cols: Optional[int] = None) -> StepInputs:
        """Plans a step and returns its inputs (a step with no rows when
        nothing can run). ``table_cols`` widens the block table."""
        s, t, mb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_sched_schedule(self._h, ctypes.byref(s), ctypes.byref(t),
                                                ctypes.byref(mb)))
        S, T = s.value, t.value
        cols = max(1, mb.value, table_cols or 0)
        out = StepInputs(np.zeros(S, np.int64), np.zeros(S + 1, np.int32), np.zeros(S, np.int32),
                         np.zeros((S, cols), np.int32), np.zeros(T, np.int64),
                         np.zeros(T, np.int32), np.zeros(T, np.int32))
        self._check(self._lib.pa_sched_step_inputs(
            self._h, _ptr(out.request_ids), _ptr(out.query_start_loc), _ptr(out.seq_lens),
            _ptr(out.block_table), cols, _ptr(out.slot_mapping), _ptr(out.token_ids),
            _ptr(out.positions)))
        return out

    def update(self, sampled: Optional[Sequence[int]] = None) -> None:
        """Ends the planned step; ``sampled[i]`` is row i's new token."""
        if sampled is None:
            self._check(self._lib.pa_sched_update(self._h, None))
            return
        a = np.ascontiguousarray(np.asarray(sampled, dtype=np.int32))
        self._check(self._lib.pa_sched_update(self._h, _ptr(a)))

    def finish_request(self, request_id: int) -> None:
        self._check(self._lib.pa_sched_finish_request(self._h, request_id))

    def stats(self) -> SchedStats:
        st = SchedStats()
        self._check(self._lib.pa_sched_get_stats(self._h, ctypes.byref(st)))
        return st

    def request_blocks(self, request_id: int) -> list:
        n = self._lib.pa_sched_request_blocks(self._h, request_id, None, 0)
        if n < 0:
            raise KeyError(request_id)
        buf = np.zeros(max(n, 1), np.int32)
        self._lib.pa_sched_request_blocks(self._h, request_id, _ptr(buf), n)
        return buf[:n].tolist()

    def request_computed(self, request_id: int) -> int:
        n = self._lib.pa_sched_request_computed(self._h, request_id)
        if n < 0:
            raise KeyError(request_id)
        return int(n)

    def block_ref_count(self, block: int) -> int:
        return int(self._lib.pa_sched_block_ref_count(self._h, block))
