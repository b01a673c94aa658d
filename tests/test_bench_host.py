"""Host logic of bench.py that needs no GPU: the comment-insensitive source hash that keys
the committed counter runs, and the --gpus guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_strip_comments_removes_comments_only():
    src = (
        '// header\n'
        '#include "a.h"  // trailing\n'
        'const char* s = "not // a comment /* either */";\n'
        "char c = '/';  /* block\n spanning */ int x = 1;\n"
        '\n'
        'int y = 2;   \n'
    )
    got = bench.strip_comments(src).split("\n")
    assert got == [
        '#include "a.h"',
        'const char* s = "not // a comment /* either */";',
        "char c = '/';    int x = 1;",
        'int y = 2;',
    ]


def test_strip_comments_keeps_escaped_quotes():
    src = 'auto s = "a \\" // b"; // gone\n'
    assert bench.strip_comments(src) == 'auto s = "a \\" // b";'


def test_hash_ignores_comment_edits_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "rwkv_linear_attention_libwkv_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f.write_text("// v1\nint f() { return 1; }\n")
    h1 = bench.kernel_source_hash(("k.hip",))
    f.write_text("// v2, reworded\n\nint f() { return 1; }  // same code\n")
    assert bench.kernel_source_hash(("k.hip",)) == h1
    f.write_text("// v1\nint f() { return 2; }\n")
    assert bench.kernel_source_hash(("k.hip",)) != h1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
