"""Host-side logic of bench.py: the counter-traffic lookup keyed by a digest
of the kernel's code (CPU only)."""
import bench


def test_code_text_ignores_comments_not_code():
    a = "int x = 1;  // one\n/* block\n comment */ int y = 2;\n\n"
    b = "int x = 1;  // changed wording\n/* other\n text */ int y = 2;\n"
    c = "int x = 2;  // one\n/* block\n comment */ int y = 2;\n"
    assert bench._code_text(a) == bench._code_text(b)
    assert bench._code_text(a) != bench._code_text(c)


def test_counter_traffic_needs_matching_digest(monkeypatch):
    k = "fwd_sp_kernel<256,1>"
    good = {(k, "w"): {"source_sha256": bench.source_digest(k), "fetch_bytes": "10",
                       "write_bytes": "5"}}
    monkeypatch.setattr(bench, "_traffic_lines", lambda: good)
    assert bench.counter_traffic("w", k) == 15
    assert bench.counter_traffic("other", k) is None
    stale = {(k, "w"): dict(good[(k, "w")], source_sha256="0" * 16)}
    monkeypatch.setattr(bench, "_traffic_lines", lambda: stale)
    assert bench.counter_traffic("w", k) is None
