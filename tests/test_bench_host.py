"""Host-side pieces of bench.py (CPU only): the source stamp that decides
whether committed HBM-traffic counters still describe the built kernels."""
import bench


def test_code_only_drops_comments_and_layout_keeps_literals():
    a = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x /*y*/"; char c = \'"\';'
    b = 'int a = 1;\n\n   const char* s = "//x /*y*/";   char c = \'"\'; // other note'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) == 'int a = 1; const char* s = "//x /*y*/"; char c = \'"\';'
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_source_digest_is_stable():
    assert bench.source_digest() == bench.source_digest()
    assert len(bench.source_digest()) == 64
