"""Host logic of bench.py (CPU only): the HBM counter records are keyed by a
hash of the kernel sources' code, which a comment edit leaves alone and a code
edit changes."""
import bench


def test_code_only_ignores_comments_and_blank_lines():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* a block\n   comment */\nint f(int x) {\n\n  return x + 1;\n}  // trailing\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)

