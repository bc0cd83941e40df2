"""The source hash that guards the committed byte counters: it follows the
code, not the comments (bench.strip_comments)."""

import bench


def test_comments_and_spacing_do_not_count():
    a = "int f(int x) {  // first\n    return x + 1; /* two\n lines */ }\n"
    b = "/* header */\nint f(int x) {\n  return x + 1;  }  // trailing\n"
    assert bench.strip_comments(a) == bench.strip_comments(b) == "int f(int x) { return x + 1; }"


def test_code_changes_count():
    assert bench.strip_comments("x = a + b;") != bench.strip_comments("x = a - b;")


def test_literals_keep_comment_markers():
    s = 'const char* p = "// not a comment"; char q = \'/\'; char e = \'\\\'\'; // gone'
    assert bench.strip_comments(s) == 'const char* p = "// not a comment"; char q = \'/\'; char e = \'\\\'\';'


def test_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16
