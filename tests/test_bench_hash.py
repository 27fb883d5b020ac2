"""bench.py's source hash for the committed HBM-traffic record (CPU only):
comments and layout do not change it, code does."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_strip_comments_keeps_code_and_literals():
    src = ('int a = 1; // one\n/* two\n lines */ const char* s = "x // y /* z */";\n'
           "char q = '\"'; const char* t = \"esc \\\" // kept\"; // gone\n")
    out = bench.strip_comments(src)
    assert "one" not in out and "two" not in out and "gone" not in out
    assert '"x // y /* z */"' in out and "'\"'" in out and '"esc \\" // kept"' in out
    assert out.startswith("int a = 1;")


def test_comment_and_layout_edits_keep_the_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n")
    h0 = bench.source_hash(["k.hip"])
    (tmp_path / "k.hip").write_text("// the kernel\n__global__ void k(int* p)\n{\n    p[0] = 1;\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    (tmp_path / "k.hip").write_text("__global__ void k(int* p) {\n  p[0] = 2;\n}\n")
    assert bench.source_hash(["k.hip"]) != h0
