"""The C ABI on the CPU: libpa.so loads, exports every symbol include/*.h
declares, and rejects bad host arguments before launching anything. No
kernel runs here (no GPU), only host-side argument checks and pure host
arithmetic."""

import ctypes
import os
import re

import pytest

import oracle
import paged_attention_kv_amd as pa
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

NULL = None
FAKE = 4096 * 16  # 16-byte aligned, never dereferenced: every call below fails before a launch


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(pa.SIGNATURES), "binding and header disagree"
    raw = ctypes.CDLL(pa.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} not exported"


def test_version(lib):
    assert "gfx950" in pa.version()


@pytest.mark.parametrize("hkv,d", [(4, 64), (8, 128), (1, 256), (2, 80)])
def test_block_bytes_matches_oracle(lib, hkv, d):
    assert pa.kv_block_bytes(16, hkv, d, 2) == oracle.kv_block_bytes(16, hkv, d, 2)
    assert pa.kv_block_bytes(0, hkv, d, 2) == -1


def cw(lib, **kw):
    a = dict(k=FAKE, v=FAKE, slot=FAKE, kc=FAKE, vc=FAKE, T=4, Hkv=4, D=64, NB=10, bs=16)
    a.update(kw)
    return lib.pa_cache_write(a["k"], a["v"], a["slot"], a["kc"], a["vc"], a["T"], a["Hkv"],
                              a["D"], a["NB"], a["bs"], None)


def test_cache_write_rejects_bad_arguments(lib):
    assert cw(lib, kc=NULL) == -1
    assert cw(lib, k=NULL) == -1
    assert cw(lib, T=-1) == -2
    assert cw(lib, Hkv=0) == -2
    assert cw(lib, NB=0) == -2
    assert cw(lib, bs=32) == -3
    assert "block_size" in pa.last_error()
    assert cw(lib, D=60) == -3
    assert cw(lib, k=FAKE + 8) == -4
    assert cw(lib, T=0) == 0          # nothing to write: no launch


def fw(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, qsl=FAKE, scale=0.125, out=FAKE, T=8, S=2,
             Hq=32, Hkv=4, D=64, bs=16, MB=4, NB=64, mq=0, ms=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.pa_forward(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["qsl"], a["scale"], a["out"],
                          a["T"], a["S"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["MB"], a["NB"],
                          a["mq"], a["ms"], a["ws"], a["wsb"], None)


def test_forward_rejects_bad_arguments(lib):
    assert fw(lib, q=NULL) == -1
    assert fw(lib, bt=NULL) == -1
    assert fw(lib, Hq=30) == -2          # not a multiple of Hkv
    assert fw(lib, S=0) == -2            # tokens without sequences
    assert fw(lib, MB=0) == -2
    assert fw(lib, D=96) == -3
    assert fw(lib, bs=8) == -3
    assert fw(lib, Hq=12, Hkv=4) == -3   # group of 3 is not built
    assert fw(lib, scale=float("nan")) == -2
    assert fw(lib, out=FAKE + 2) == -4
    assert fw(lib, ws=NULL) == -5
    assert fw(lib, wsb=16) == -5
    assert "workspace" in pa.last_error()
    assert fw(lib, T=0) == 0              # empty batch: no launch
    # unknown option flags are rejected before anything else happens
    assert lib.pa_forward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, 8, 2, 32, 4, 64, 16,
                             4, 64, 0, 0, FAKE, 1 << 30, 16, None) == -3
    assert "unknown flags" in pa.last_error()
    # PA_FORWARD_SERIAL (8) is a known flag: an empty batch with it succeeds
    assert lib.pa_forward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, 0, 2, 32, 4, 64, 16,
                             4, 64, 0, 0, FAKE, 1 << 30, 8 | 1, None) == 0
    # both decode schedules at once
    assert lib.pa_forward_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, 8, 2, 32, 4, 64, 16,
                             4, 64, 0, 0, FAKE, 1 << 30, 6, None) == -3
    assert "schedule" in pa.last_error()


def test_validate_rejects_null_before_touching_the_device(lib):
    assert lib.pa_validate_inputs(None, FAKE, FAKE, None, 4, 2, 4, 64, 16, 0, 0, 0, None) == -1
    assert lib.pa_validate_inputs(FAKE, FAKE, FAKE, None, 4, 2, 4, 64, 16, 3, 0, 0, None) == -1
    assert lib.pa_validate_inputs(FAKE, FAKE, FAKE, None, 4, 2, 4, 64, 8, 0, 0, 0, None) == -3


def test_read_probe_rejects_bad_arguments(lib):
    def probe(**kw):
        a = dict(kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, S=2, Hkv=4, D=64, MB=4, NB=64, W=8, C=16,
                 sink=FAKE)
        a.update(kw)
        return lib.pa_probe_block_read(a["kc"], a["vc"], a["bt"], a["sl"], a["S"], a["Hkv"],
                                       a["D"], a["MB"], a["NB"], a["W"], a["C"], a["sink"], None)
    assert probe(kc=NULL) == -1
    assert probe(sink=NULL) == -1
    assert probe(S=0) == -2
    assert probe(W=0) == -2 and probe(W=17) == -2
    assert probe(C=0) == -2
    assert probe(MB=1 << 20, C=1) == -2   # grid y past 65535
    assert probe(D=3, Hkv=1) == -3
    assert probe(vc=FAKE + 8) == -4


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_workspace_sizes_for_the_named_workloads(lib, i):
    s = wl.config(i)
    n = pa.forward_workspace_bytes(s.num_tokens, s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                   s.head_size, s.max_blocks_per_seq)
    # the counter region, then (when rows may be split) decode partials
    assert n > pa.WORKSPACE_COUNTER_BYTES
    assert n % 256 == 0
    assert n < 512 << 20
    # a tighter max_seq_len hint never needs more
    n2 = pa.forward_workspace_bytes(s.num_tokens, s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                    s.head_size, s.max_blocks_per_seq, max(s.seq_lens))
    assert n2 <= n


def test_workspace_for_multi_token_decode_rows(lib):
    # a hint of 4 query tokens per row at 4 query heads per KV head plans the
    # decode partials per query token (up to 4x); a hint past 16 / G does not
    args = (1024, 256, 32, 8, 128, 512)
    n1 = pa.forward_workspace_bytes(*args, 8192, max_query_len=1)
    n4 = pa.forward_workspace_bytes(*args, 8192, max_query_len=4)
    n5 = pa.forward_workspace_bytes(*args, 8192, max_query_len=5)
    assert n1 < n4 <= 4 * n1 and n5 <= n4


def test_shared_prefix_workspace(lib):
    s = wl.config(5)
    n = lib.pa_shared_prefix_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                             s.head_size, s.max_blocks_per_seq,
                                             s.shared_prefix_blocks, max(s.seq_lens))
    # partials: at least one chunk and the row's own blocks per row and head
    assert n >= s.num_seqs * 2 * s.num_q_heads * (s.head_size + 2) * 4
    assert n % 256 == 0
    # the prefix must leave keys for every row, and be at least one block
    assert lib.pa_shared_prefix_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                                s.head_size, s.max_blocks_per_seq, 0, 0) == 0
    assert lib.pa_shared_prefix_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads,
                                                s.head_size, s.max_blocks_per_seq,
                                                s.max_blocks_per_seq, 0) == 0


def test_table_width_past_the_int32_token_range_is_rejected(lib):
    """max_blocks_per_seq * 16 must stay within int32 tokens: wider tables
    plan no workspace and the calls fail before launching."""
    for mb in (1 << 27, (1 << 31) - 1):
        assert lib.pa_forward_workspace_bytes(8, 2, 32, 4, 64, mb, 0, 100) == 0
        assert lib.pa_shared_prefix_workspace_bytes(2, 32, 4, 64, mb, 1, 100) == 0
        assert fw(lib, MB=mb) == -2
    assert lib.pa_forward_workspace_bytes(8, 2, 32, 4, 64, (1 << 27) - 1, 0, 100) > 0


def test_shared_prefix_calls_reject_bad_arguments(lib):
    """Both shared-prefix entry points check their host arguments alike (the
    write-and-forward one also its k / v / slot_mapping) and launch nothing
    on an error or an empty batch."""
    def sp(write, **kw):
        a = dict(k=FAKE, v=FAKE, slot=FAKE, q=FAKE, S=8, Hq=32, Hkv=8, D=128, bs=16, MB=20,
                 NB=1000, pb=4, msl=0, ws=FAKE, wsb=1 << 30, flags=0)
        a.update(kw)
        tail = (a["q"], FAKE, FAKE, FAKE, 0.125, FAKE, a["S"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                a["MB"], a["NB"], a["pb"], a["msl"], a["ws"], a["wsb"], a["flags"], None)
        if write:
            return lib.pa_write_and_forward_shared_prefix(a["k"], a["v"], a["slot"], FAKE, FAKE,
                                                          *tail)
        return lib.pa_forward_shared_prefix(tail[0], FAKE, FAKE, *tail[1:])
    for write in (False, True):
        name = "pa_write_and_forward_shared_prefix" if write else "pa_forward_shared_prefix"
        assert sp(write, q=NULL) == -1
        assert sp(write, Hq=30) == -2
        assert sp(write, D=96) == -3
        assert sp(write, bs=8) == -3
        assert sp(write, pb=0) == -2
        assert sp(write, pb=20) == -2         # no key left past the prefix
        assert sp(write, flags=2) == -3       # only PA_FORWARD_SHARED_BLOCKS
        assert sp(write, ws=NULL) == -5
        assert sp(write, wsb=16) == -5
        assert pa.last_error().startswith(name), pa.last_error()
        assert sp(write, S=0) == 0            # empty batch: no launch
    assert sp(True, k=NULL) == -1
    assert sp(True, slot=NULL) == -1
    assert sp(True, v=FAKE + 8) == -4
    assert sp(True, k=NULL, S=0) == 0         # nothing to write


def test_validate_shared_prefix_rejects_bad_arguments_before_touching_the_device(lib):
    v = lib.pa_validate_shared_prefix
    assert v(None, FAKE, None, 4, 8, 2, None) == -1
    assert v(FAKE, None, None, 4, 8, 2, None) == -1
    assert v(FAKE, FAKE, None, 4, 8, 0, None) == -2     # no prefix
    assert v(FAKE, FAKE, None, 4, 8, 8, None) == -2     # prefix covers the table
    assert v(FAKE, FAKE, None, -1, 8, 2, None) == -2
    assert v(FAKE, FAKE, None, 4, 1 << 27, 2, None) == -2
    assert v(FAKE, FAKE, None, 0, 8, 2, None) == 0       # no rows: nothing to check


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define PA_BLOCK_SIZE (\d+)", text).group(1)) == pa.BLOCK_SIZE
    for name in ("SHARED_BLOCKS", "DECODE_EVEN_SHARES", "DECODE_PARTITIONED", "SERIAL"):
        assert int(re.search(rf"#define PA_FORWARD_{name} (\d+)u", text).group(1)) == \
            getattr(pa, "FORWARD_" + name)
    # kernel classes of the timing interface: the binding names every one
    classes = {int(v): k.lower() for k, v in re.findall(r"#define PA_KERNEL_(\w+) (\d+)", text)
               if k != "CLASSES"}
    assert classes == pa.KERNEL_CLASSES
    n = int(re.search(r"#define PA_KERNEL_CLASSES (\d+)", text).group(1))
    assert max(classes) < n
    m = re.search(r"#define PA_WORKSPACE_COUNTER_BYTES \((\d+)u \* (\d+)u\)", text)
    assert int(m.group(1)) * int(m.group(2)) == pa.WORKSPACE_COUNTER_BYTES


def test_workspace_starts_with_the_counter_region(lib):
    # any shape needs at least the counter region, 256-byte aligned sizes
    for args in ((64, 64, 32, 4, 64, 128, 0), (8192, 260, 32, 8, 128, 512, 0), (1, 1, 8, 8, 128, 1, 0)):
        n = pa.forward_workspace_bytes(*args)
        assert n > pa.WORKSPACE_COUNTER_BYTES and n % 256 == 0


def test_profile_with_no_launches_is_empty(lib):
    # begin/end with nothing launched in between touches no HIP call
    pa.profile_begin()
    assert pa.profile_end() == {}


def test_noalloc_rejects_sizes_past_its_scratch_before_launching(lib):
    """Sizes that need more workspace than the fixed scratch array: a
    PA_ERR_WORKSPACE error naming both sizes, with nothing launched (no
    device is touched: the check is host arithmetic)."""
    S, Hq, Hkv, D, MB = 4000, 64, 8, 128, 2048
    need = pa.forward_workspace_bytes(S, S, Hq, Hkv, D, MB)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    rc = lib.pa_write_and_forward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          0.1, FAKE, S, S, Hq, Hkv, D, 16, MB, 1 << 20, 1, 0, 0,
                                          None)
    assert rc == -5
    msg = pa.last_error()
    assert str(need) in msg and str(pa.NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_reports_argument_errors_like_the_workspace_call(lib):
    args = [FAKE] * 9 + [0.1, FAKE, 8, 2, 32, 4, 64, 16, 4, 64, 0, 0, 0, None]
    bad_block = list(args)
    bad_block[16] = 32  # block_size
    assert lib.pa_write_and_forward_noalloc(*bad_block) == -3
    bad_group = list(args)
    bad_group[13] = 3   # 32 q heads over 3 kv heads
    assert lib.pa_write_and_forward_noalloc(*bad_group) == -2
    empty = list(args)
    empty[11] = 0       # no tokens: nothing to do, nothing launched
    assert lib.pa_write_and_forward_noalloc(*empty) == 0


def test_build_rejects_a_library_with_its_own_symbols_undefined(tmp_path):
    """The build's last check: a library that references one of its own
    (namespace pa) symbols without defining it, as when the compiler drops a
    kernel's host launch stub, is refused and removed."""
    import shutil
    import subprocess
    from paged_attention_kv_amd import build
    gxx = shutil.which("g++")
    if not gxx or not shutil.which("nm"):
        pytest.skip("g++ and nm are needed")
    src = tmp_path / "u.cpp"
    src.write_text("namespace pa { void missing(); }\nvoid use() { pa::missing(); }\n")
    lib = tmp_path / "libu.so"
    subprocess.run([gxx, "-shared", "-fPIC", str(src), "-o", str(lib)], check=True)
    with pytest.raises(RuntimeError, match="undefined"):
        build.check_symbols(str(lib))
    assert not lib.exists()
    # the library built in-tree passes the same check
    build.check_symbols(pa.library_path())
