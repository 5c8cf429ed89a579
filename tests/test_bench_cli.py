"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this path runs on one GPU), and the HBM counter record's key
ignores comments in the decode sources."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_code_hash_ignores_comments(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "paged_attention_kv_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = {f: open(os.path.join(ROOT, "paged_attention_kv_amd", "csrc", f)).read()
           for f in ("decode.hip", "common.h")}
    for f, t in src.items():
        (csrc / f).write_text(t)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.decode_source_hash()
    (csrc / "decode.hip").write_text("// a new comment\n" + src["decode.hip"] + "\n/* and another */\n")
    assert bench.decode_source_hash() == h0
    (csrc / "decode.hip").write_text(src["decode.hip"].replace("kLazy = 8.0f", "kLazy = 7.0f"))
    assert bench.decode_source_hash() != h0
