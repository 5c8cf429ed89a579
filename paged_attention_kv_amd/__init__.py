"""Paged attention and paged KV-cache write for MI355X (gfx950).

Python binding of ``libpa.so`` (the C ABI declared in ``include/pa.h``). The
binding only marshals arguments: it reads sizes from tensor shapes, passes
``data_ptr()`` values and the current HIP stream, and raises on a non-zero
status. Every step of the computation runs in the library's HIP kernels;
there is no fallback path, and importing a function that needs the library
raises if ``libpa.so`` has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["cache_write", "forward", "write_and_forward", "write_and_forward_noalloc",
           "forward_shared_prefix", "write_and_forward_shared_prefix",
           "validate_shared_prefix", "forward_workspace_bytes",
           "validate_inputs",
           "kv_block_bytes", "last_error", "version", "library_path", "load_library",
           "profile_begin", "profile_end", "PaError", "BLOCK_SIZE", "KERNEL_CLASSES"]

BLOCK_SIZE = 16
FORWARD_SHARED_BLOCKS = 1  # PA_FORWARD_SHARED_BLOCKS
WORKSPACE_COUNTER_BYTES = 256 * 1024  # PA_WORKSPACE_COUNTER_BYTES
FORWARD_DECODE_EVEN_SHARES = 2  # PA_FORWARD_DECODE_EVEN_SHARES
FORWARD_DECODE_PARTITIONED = 4  # PA_FORWARD_DECODE_PARTITIONED
FORWARD_SERIAL = 8  # PA_FORWARD_SERIAL
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # PA_NOALLOC_SCRATCH_BYTES
_SCHEDULE_FLAGS = {"even": FORWARD_DECODE_EVEN_SHARES, "partitioned": FORWARD_DECODE_PARTITIONED}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
          -4: "PA_ERR_ALIGN", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_HIP",
          -7: "PA_ERR_INVALID_DATA"}

# (name, restype, argtypes) of every symbol include/pa.h declares.
class SchedStats(ctypes.Structure):
    """pa_sched_stats (include/pa_sched.h)."""
    _fields_ = [("num_free_blocks", ctypes.c_int64), ("num_cached_blocks", ctypes.c_int64),
                ("num_waiting", ctypes.c_int32), ("num_running", ctypes.c_int32),
                ("num_finished", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("num_steps", ctypes.c_int64), ("prefix_hit_tokens", ctypes.c_int64),
                ("num_preemptions", ctypes.c_int64)]


SIGNATURES = {
    "pa_sched_create": (_P, [_I64, _I32, _I32, _I32, _I32, _I32]),
    "pa_sched_destroy": (None, [_P]),
    "pa_sched_add_request": (ctypes.c_int, [_P, _I64, _P, _I32, _I32]),
    "pa_sched_schedule": (ctypes.c_int, [_P, _P, _P, _P]),
    "pa_sched_step_inputs": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _P, _P]),
    "pa_sched_update": (ctypes.c_int, [_P, _P]),
    "pa_sched_finish_request": (ctypes.c_int, [_P, _I64]),
    "pa_sched_get_stats": (ctypes.c_int, [_P, ctypes.POINTER(SchedStats)]),
    "pa_sched_request_blocks": (_I32, [_P, _I64, _P, _I32]),
    "pa_sched_request_computed": (_I32, [_P, _I64]),
    "pa_sched_block_ref_count": (_I32, [_P, _I32]),
    "pa_sched_shared_prefix_blocks": (_I32, [_P, _P, _P, _I32, _I32]),
    "pa_kv_block_bytes": (_I64, [_I32, _I32, _I32, _I32]),
    "pa_cache_write": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _P]),
    "pa_forward_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_shared_prefix_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_forward_shared_prefix": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                                _I32, _I32, _I32, _I32, _I32, _I32, _I64, _I32,
                                                _I32, _P, _SZ, ctypes.c_uint32, _P]),
    "pa_write_and_forward_shared_prefix": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                          ctypes.c_float, _P, _I32, _I32, _I32,
                                                          _I32, _I32, _I32, _I64, _I32, _I32, _P,
                                                          _SZ, ctypes.c_uint32, _P]),
    "pa_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32, _I32,
                                  _I32, _I32, _I32, _I32, _I64, _I32, _I32, _P, _SZ, _P]),
    "pa_forward_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _I32,
                                     _I32, _I32, _I32, _I32, _I32, _I64, _I32, _I32, _P, _SZ,
                                     ctypes.c_uint32, _P]),
    "pa_write_and_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                            _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I64,
                                            _I32, _I32, _P, _SZ, ctypes.c_uint32, _P]),
    "pa_write_and_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                    ctypes.c_float, _P, _I32, _I32, _I32, _I32,
                                                    _I32, _I32, _I32, _I64, _I32, _I32,
                                                    ctypes.c_uint32, _P]),
    "pa_validate_inputs": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32,
                                          _I32, _I32, _P]),
    "pa_validate_shared_prefix": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P]),
    "pa_probe_block_read": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I64, _I32,
                                           _I32, _P, _P]),
    "pa_profile_begin": (ctypes.c_int, []),
    "pa_profile_end": (ctypes.c_int, [_P]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
}


# Kernel classes of the timing facility (PA_KERNEL_* in include/pa.h).
KERNEL_CLASSES = {0: "cache_write", 1: "decode", 2: "combine", 3: "prefill",
                  4: "prefill_short", 5: "plan", 6: "prefix", 7: "write_plan"}
_NCLASS = 8


class _Profile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * _NCLASS), ("total_ms", ctypes.c_double * _NCLASS)]


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libpa.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m paged_attention_kv_amd.build` "
                "(the paged-attention path has no fallback)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return load_library().pa_last_error().decode()


def version() -> str:
    return load_library().pa_version().decode()


def _check(status: int) -> None:
    if status != 0:
        raise PaError(status, last_error())


# torch's raw-stream query (one C call) where this torch has it; the public
# current_stream() builds a Stream object on every call (~2 us).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    """The HIP stream torch has current for t's device (t is on a device)."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev_tensor(name: str, t: torch.Tensor, dtype: torch.dtype, ndim: int) -> None:
    # the usual case in one pass; the checks below name what is wrong
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is dtype and t.dim() == ndim
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, not {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kv_block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    return int(load_library().pa_kv_block_bytes(block_size, num_kv_heads, head_size, dtype_bytes))


def cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Write this step's keys/values ([T, Hkv, D] bf16) into the paged caches
    ([NB, 16, Hkv, D] bf16) at ``slot_mapping`` (int64 [T], negative = skip)."""
    lib = load_library()
    for n, t in (("k", k), ("v", v)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(n, t, torch.bfloat16, 4)
    _dev_tensor("slot_mapping", slot_mapping, torch.int64, 1)
    T, Hkv, D = k.shape
    if v.shape != k.shape or slot_mapping.shape[0] != T:
        raise ValueError("k, v and slot_mapping disagree in shape")
    if k_cache.shape != v_cache.shape or tuple(k_cache.shape[2:]) != (Hkv, D):
        raise ValueError("cache shape must be [NB, 16, Hkv, D] matching k")
    _check(lib.pa_cache_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                              k_cache.data_ptr(), v_cache.data_ptr(), T, Hkv, D,
                              k_cache.shape[0], k_cache.shape[1], _stream(k_cache)))


def forward_workspace_bytes(num_tokens: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                            head_size: int, max_blocks_per_seq: int,
                            max_seq_len: Optional[int] = None,
                            max_query_len: Optional[int] = None) -> int:
    """Workspace bytes of a forward call with these sizes and hints (the
    same hints the call passes)."""
    n = load_library().pa_forward_workspace_bytes(num_tokens, num_seqs, num_q_heads, num_kv_heads,
                                                  head_size, max_blocks_per_seq,
                                                  max_query_len or 0, max_seq_len or 0)
    if n == 0:
        raise ValueError("unsupported sizes for pa_forward")
    return int(n)


_workspaces: dict = {}
# Workspaces replaced by larger ones stay alive for the life of the process:
# a graph captured earlier still holds their addresses.
_retired_workspaces: list = []


def _workspace(device: int, nbytes: int) -> torch.Tensor:
    """The implicit workspace of device index ``device``, grown to nbytes."""
    ws = _workspaces.get(device)
    if ws is not None and ws.numel() >= nbytes:
        return ws
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError(
            "the implicit workspace would have to grow during graph capture: pass a "
            "workspace (forward_workspace_bytes(...) bytes, its first "
            "WORKSPACE_COUNTER_BYTES zero) to calls made under capture")
    # zero-filled once: the leading counter region must start at zero
    # (every call leaves it zero)
    if ws is not None:
        _retired_workspaces.append(ws)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=torch.device("cuda", device))
    _workspaces[device] = ws
    return ws


_need_cache: dict = {}


def _workspace_need(*sizes) -> int:
    """pa_forward_workspace_bytes of these sizes (T, S, Hq, Hkv, D, MB, max
    query length, max sequence length hints), remembered per size tuple: the
    library's answer depends on nothing else."""
    n = _need_cache.get(sizes)
    if n is None:
        n = int(load_library().pa_forward_workspace_bytes(*sizes))
        if len(_need_cache) > 4096:
            _need_cache.clear()
        _need_cache[sizes] = n
    return n


def _forward_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out,
                  max_query_len, max_seq_len, workspace, shared_blocks, decode_schedule,
                  serial=False):
    """Checks and marshals the arguments shared by pa_forward_ex and
    pa_write_and_forward: returns (q .. out pointers and sizes .. stream), out."""
    lib = load_library()
    _dev_tensor("q", q, torch.bfloat16, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(n, t, torch.bfloat16, 4)
    _dev_tensor("block_table", block_table, torch.int32, 2)
    _dev_tensor("seq_lens", seq_lens, torch.int32, 1)
    _dev_tensor("query_start_loc", query_start_loc, torch.int32, 1)
    T, Hq, D = q.shape
    NB, bs, Hkv, Dc = k_cache.shape
    S, MB = block_table.shape
    if v_cache.shape != k_cache.shape or Dc != D:
        raise ValueError("caches must be [NB, 16, Hkv, D] with q's head size")
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens must be [S] and query_start_loc [S+1]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor("out", out, torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    flags = FORWARD_SHARED_BLOCKS if shared_blocks else 0
    if serial:
        flags |= FORWARD_SERIAL
    if decode_schedule is not None:
        if decode_schedule not in _SCHEDULE_FLAGS:
            raise ValueError(f"decode_schedule must be one of {sorted(_SCHEDULE_FLAGS)}")
        flags |= _SCHEDULE_FLAGS[decode_schedule]
    if workspace is None:
        workspace = _workspace(q.get_device(), _workspace_need(T, S, Hq, Hkv, D, MB,
                                                               max_query_len or 0,
                                                               max_seq_len or 0))
    elif not workspace.is_cuda or workspace.get_device() != q.get_device():
        raise ValueError("workspace must be on q's device")
    tail = (block_table.data_ptr(), seq_lens.data_ptr(), query_start_loc.data_ptr(), float(scale),
            out.data_ptr(), T, S, Hq, Hkv, D, bs, MB, NB, max_query_len or 0, max_seq_len or 0,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), flags, _stream(q))
    return tail, out


def forward(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
            block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
            scale: float, out: Optional[torch.Tensor] = None,
            max_query_len: Optional[int] = None, max_seq_len: Optional[int] = None,
            workspace: Optional[torch.Tensor] = None,
            shared_blocks: bool = False,
            decode_schedule: Optional[str] = None,
            serial: bool = False) -> torch.Tensor:
    """Paged attention of the flattened batch (q [T, Hq, D] bf16) over the
    paged caches; returns ``out`` ([T, Hq, D] bf16). ``max_query_len`` and
    ``max_seq_len`` are optional host upper bounds that shrink the launch
    grids; ``workspace`` (uint8, on the device, its first
    ``WORKSPACE_COUNTER_BYTES`` zero before its first use) is taken from a
    per-device cache when omitted. ``shared_blocks`` tells the library that
    some blocks appear in several rows' tables (prefix caching); results are
    the same either way. ``decode_schedule`` ("even" or "partitioned")
    forces the decode rows' schedule; by default the library picks.
    ``serial`` keeps a mixed batch's prefill and decode launches on the
    current stream one after the other (by default a large mixed batch runs
    them side by side, the prefill on a second stream of the library's,
    joined back before the call returns)."""
    tail, out = _forward_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                              out, max_query_len, max_seq_len, workspace, shared_blocks,
                              decode_schedule, serial)
    _check(load_library().pa_forward_ex(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                         *tail))
    return out


def _shared_prefix_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                        prefix_blocks, out, max_seq_len, workspace, shared_blocks):
    """Checks and marshals the arguments of the shared-prefix calls: returns
    the C call's arguments from ``q`` on, and ``out``."""
    lib = load_library()
    _dev_tensor("q", q, torch.bfloat16, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(n, t, torch.bfloat16, 4)
    _dev_tensor("block_table", block_table, torch.int32, 2)
    _dev_tensor("seq_lens", seq_lens, torch.int32, 1)
    _dev_tensor("query_start_loc", query_start_loc, torch.int32, 1)
    T, Hq, D = q.shape
    NB, bs, Hkv, Dc = k_cache.shape
    S, MB = block_table.shape
    if v_cache.shape != k_cache.shape or Dc != D:
        raise ValueError("caches must be [NB, 16, Hkv, D] with q's head size")
    if T != S or seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("one query token per row: q [S, Hq, D], seq_lens [S], "
                         "query_start_loc [S+1]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor("out", out, torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = lib.pa_shared_prefix_workspace_bytes(S, Hq, Hkv, D, MB, prefix_blocks,
                                                max_seq_len or 0)
    if need == 0:
        raise ValueError("unsupported sizes for the shared-prefix call")
    if workspace is None:
        workspace = _workspace(q.get_device(), need)
    elif not workspace.is_cuda or workspace.get_device() != q.get_device():
        raise ValueError("workspace must be on q's device")
    tail = (q.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
            query_start_loc.data_ptr(), float(scale), out.data_ptr(), S, Hq, Hkv, D, bs, MB, NB,
            prefix_blocks, max_seq_len or 0, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(),
            FORWARD_SHARED_BLOCKS if shared_blocks else 0, _stream(q))
    return tail, out


def forward_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor,
                          query_start_loc: torch.Tensor, scale: float, prefix_blocks: int,
                          out: Optional[torch.Tensor] = None,
                          max_seq_len: Optional[int] = None,
                          workspace: Optional[torch.Tensor] = None,
                          shared_blocks: bool = False) -> torch.Tensor:
    """Decode rows (one query token each) whose tables all start with the
    same ``prefix_blocks`` blocks (pa_forward_shared_prefix): the prefix is
    attended once for all rows, each row's own blocks after it separately,
    and the two merged. Returns ``out`` ([S, Hq, D] bf16)."""
    tail, out = _shared_prefix_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                                    scale, prefix_blocks, out, max_seq_len, workspace,
                                    shared_blocks)
    _check(load_library().pa_forward_shared_prefix(tail[0], k_cache.data_ptr(),
                                                   v_cache.data_ptr(), *tail[1:]))
    return out


def write_and_forward_shared_prefix(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                                    k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
                                    block_table: torch.Tensor, seq_lens: torch.Tensor,
                                    query_start_loc: torch.Tensor, scale: float,
                                    prefix_blocks: int, out: Optional[torch.Tensor] = None,
                                    max_seq_len: Optional[int] = None,
                                    workspace: Optional[torch.Tensor] = None,
                                    shared_blocks: bool = False) -> torch.Tensor:
    """``cache_write`` then ``forward_shared_prefix`` in one call
    (pa_write_and_forward_shared_prefix): the write rides in the prefix
    pass's launch. Returns ``out``."""
    for n, t in (("k", k), ("v", v)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("slot_mapping", slot_mapping, torch.int64, 1)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("k, v, slot_mapping and q disagree in token count")
    if tuple(k.shape[1:]) != tuple(k_cache.shape[2:]):
        raise ValueError("k must be [T, Hkv, D] matching the caches")
    tail, out = _shared_prefix_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                                    scale, prefix_blocks, out, max_seq_len, workspace,
                                    shared_blocks)
    _check(load_library().pa_write_and_forward_shared_prefix(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), *tail))
    return out


def write_and_forward(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor,
                      query_start_loc: torch.Tensor, scale: float,
                      out: Optional[torch.Tensor] = None,
                      max_query_len: Optional[int] = None, max_seq_len: Optional[int] = None,
                      workspace: Optional[torch.Tensor] = None,
                      shared_blocks: bool = False,
                      decode_schedule: Optional[str] = None,
                      serial: bool = False) -> torch.Tensor:
    """``cache_write`` then ``forward`` in one call (pa_write_and_forward):
    with ``max_query_len=1`` (decode rows only) one launch writes the new
    tokens and attends. ``serial`` as for ``forward``. Returns ``out``."""
    for n, t in (("k", k), ("v", v)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("slot_mapping", slot_mapping, torch.int64, 1)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("k, v, slot_mapping and q disagree in token count")
    if tuple(k.shape[1:]) != tuple(k_cache.shape[2:]):
        raise ValueError("k must be [T, Hkv, D] matching the caches")
    tail, out = _forward_args(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                              out, max_query_len, max_seq_len, workspace, shared_blocks,
                              decode_schedule, serial)
    _check(load_library().pa_write_and_forward(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                               k_cache.data_ptr(), v_cache.data_ptr(),
                                               q.data_ptr(), *tail))
    return out


def write_and_forward_noalloc(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                              k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor,
                              query_start_loc: torch.Tensor, scale: float, out: torch.Tensor,
                              max_query_len: Optional[int] = None,
                              max_seq_len: Optional[int] = None, shared_blocks: bool = False,
                              decode_schedule: Optional[str] = None) -> torch.Tensor:
    """``write_and_forward`` with the library's own fixed scratch array as
    the workspace (pa_write_and_forward_noalloc): nothing is allocated, by
    the library or here, so ``out`` must be given. For callers that cannot
    allocate (graph capture, serving loops); calls that overlap on one
    device race for the scratch."""
    lib = load_library()
    for n, t in (("k", k), ("v", v)):
        _dev_tensor(n, t, torch.bfloat16, 3)
    _dev_tensor("slot_mapping", slot_mapping, torch.int64, 1)
    _dev_tensor("q", q, torch.bfloat16, 3)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(n, t, torch.bfloat16, 4)
    _dev_tensor("block_table", block_table, torch.int32, 2)
    _dev_tensor("seq_lens", seq_lens, torch.int32, 1)
    _dev_tensor("query_start_loc", query_start_loc, torch.int32, 1)
    _dev_tensor("out", out, torch.bfloat16, 3)
    T, Hq, D = q.shape
    NB, bs, Hkv, Dc = k_cache.shape
    S, MB = block_table.shape
    if v_cache.shape != k_cache.shape or Dc != D or out.shape != q.shape:
        raise ValueError("caches must be [NB, 16, Hkv, D] with q's head size; out q's shape")
    if k.shape != v.shape or k.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("k, v, slot_mapping and q disagree in token count")
    if tuple(k.shape[1:]) != (Hkv, D):
        raise ValueError("k must be [T, Hkv, D] matching the caches")
    if seq_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens must be [S] and query_start_loc [S+1]")
    flags = FORWARD_SHARED_BLOCKS if shared_blocks else 0
    if decode_schedule is not None:
        if decode_schedule not in _SCHEDULE_FLAGS:
            raise ValueError(f"decode_schedule must be one of {sorted(_SCHEDULE_FLAGS)}")
        flags |= _SCHEDULE_FLAGS[decode_schedule]
    _check(lib.pa_write_and_forward_noalloc(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), q.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
        query_start_loc.data_ptr(), float(scale), out.data_ptr(), T, S, Hq, Hkv, D, bs, MB, NB,
        max_query_len or 0, max_seq_len or 0, flags, _stream(q)))
    return out


def validate_inputs(block_table: torch.Tensor, seq_lens: torch.Tensor,
                    query_start_loc: torch.Tensor, num_tokens: int, num_blocks: int,
                    slot_mapping: Optional[torch.Tensor] = None,
                    max_query_len: Optional[int] = None,
                    max_seq_len: Optional[int] = None) -> None:
    """Synchronously check the device metadata the hot path trusts; raises
    PaError(PA_ERR_INVALID_DATA) with the first problem found."""
    lib = load_library()
    S, MB = block_table.shape
    nw = 0 if slot_mapping is None else slot_mapping.shape[0]
    _check(lib.pa_validate_inputs(block_table.data_ptr(), seq_lens.data_ptr(),
                                  query_start_loc.data_ptr(),
                                  None if slot_mapping is None else slot_mapping.data_ptr(),
                                  num_tokens, S, MB, num_blocks, BLOCK_SIZE, nw,
                                  max_query_len or 0, max_seq_len or 0,
                                  _stream(block_table)))


def validate_shared_prefix(block_table: torch.Tensor, seq_lens: torch.Tensor, prefix_blocks: int,
                           slot_mapping: Optional[torch.Tensor] = None) -> None:
    """Synchronously check the shared-prefix calls' caller contract (every
    row's first ``prefix_blocks`` table entries equal row 0's, every row
    longer than the prefix, no new token's slot in a prefix block); raises
    PaError(PA_ERR_INVALID_DATA) naming the first row that breaks it."""
    lib = load_library()
    _dev_tensor("block_table", block_table, torch.int32, 2)
    _dev_tensor("seq_lens", seq_lens, torch.int32, 1)
    S, MB = block_table.shape
    if seq_lens.shape[0] != S:
        raise ValueError("seq_lens must have one entry per table row")
    if slot_mapping is not None:
        _dev_tensor("slot_mapping", slot_mapping, torch.int64, 1)
        if slot_mapping.shape[0] != S:
            raise ValueError("slot_mapping must hold one new token per row")
    _check(lib.pa_validate_shared_prefix(
        block_table.data_ptr(), seq_lens.data_ptr(),
        None if slot_mapping is None else slot_mapping.data_ptr(), S, MB, prefix_blocks,
        _stream(block_table)))


def probe_block_read(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, waves: int = 8, blocks_per_workgroup: int = 16,
                     sink: Optional[torch.Tensor] = None) -> None:
    """Read every K and V block the rows cover, whole, with no arithmetic (a
    measurement probe for the memory system on the decode read pattern; see
    pa_probe_block_read). Enqueued on the current stream."""
    lib = load_library()
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(n, t, torch.bfloat16, 4)
    _dev_tensor("block_table", block_table, torch.int32, 2)
    _dev_tensor("seq_lens", seq_lens, torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    S, MB = block_table.shape
    if seq_lens.shape[0] != S:
        raise ValueError("seq_lens must have one entry per table row")
    NB, _, Hkv, D = k_cache.shape
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=k_cache.device)
    _check(lib.pa_probe_block_read(k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                   seq_lens.data_ptr(), S, Hkv, D, MB, NB, waves,
                                   blocks_per_workgroup, sink.data_ptr(), _stream(k_cache)))


def profile_begin() -> None:
    """Start timing every kernel launch of the library with HIP events on its
    stream (measurement harnesses only; see pa_profile_begin)."""
    _check(load_library().pa_profile_begin())


def profile_end() -> dict:
    """Stop timing; wait for the recorded events and return
    {class name: (launches, total ms)} for every class that launched."""
    prof = _Profile()
    _check(load_library().pa_profile_end(ctypes.byref(prof)))
    return {KERNEL_CLASSES.get(c, str(c)): (int(prof.launches[c]), float(prof.total_ms[c]))
            for c in range(_NCLASS) if prof.launches[c]}
