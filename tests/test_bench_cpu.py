"""bench.py host logic on the CPU: the kernel-code digest that gates the stored HBM counters."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_only_drops_comments_keeps_strings():
    src = 'int a;  // note "x"\n/* block\n comment */ char* s = "// kept"; c = \'/\'; y = a / b;'
    assert bench._code_only(src) == 'int a; char* s = "// kept"; c = \'/\'; y = a / b;'


def test_digest_ignores_comment_edits_only():
    a = "__global__ void k(float* p) { p[0] = 1.0f; }"
    b = "// a comment\n__global__  void k(float* p) {\n    p[0] = 1.0f;  /* set */\n}\n"
    c = "__global__ void k(float* p) { p[0] = 2.0f; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)

