"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_source_hash_ignores_comments_and_blank_space(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n    return x + 1;   // one more\n}\n")
    b.write_text("// a header comment\nint f(int x)\n{\n\n    /* the sum */ return x + 1;\n}\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench._src_hash(str(a)) == bench._src_hash(str(b))
    assert bench._src_hash(str(a)) != bench._src_hash(str(c))
