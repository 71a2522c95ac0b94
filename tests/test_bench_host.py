"""Host-side logic of bench.py that needs no GPU: the kernel-source key under
which the committed HBM counters are stored."""
import bench


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {\n  // doubles x\n  return 2 * x;  /* fast */\n}\n"
    b = "int f(int x) { /* a different\n comment */ return 2 * x; }"
    assert bench._code_tokens(a) == bench._code_tokens(b)


def test_code_tokens_see_code_changes():
    a = "int f(int x) { return 2 * x; }"
    b = "int f(int x) { return 3 * x; }"
    assert bench._code_tokens(a) != bench._code_tokens(b)

