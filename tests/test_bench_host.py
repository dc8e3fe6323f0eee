"""Host-side checks of bench.py that need no GPU: the one-GPU guard and the source key that
decides whether the stored HBM-traffic figure still describes the attention kernel."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_sources(tmp_path):
    for f in bench.ATTN_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)


def test_source_key_ignores_comments_not_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    key = bench.attn_source_hash()
    main = tmp_path / bench.ATTN_SOURCES[0]
    text = main.read_text()
    # comments, trailing comments and blank lines leave the key alone
    main.write_text("// a note\n\n/* a block\n   comment */\n" + text.replace("\n", "  // tail\n", 3) + "\n\n")
    assert bench.attn_source_hash() == key
    # a string literal that looks like a comment is code
    main.write_text(text + '\nstatic const char* k = "// not a comment";\n')
    assert bench.attn_source_hash() != key
    # any code change changes the key
    main.write_text(text + "\nstatic int unused_probe;\n")
    assert bench.attn_source_hash() != key


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
