"""Host logic of bench.py that needs no GPU: the traffic record is keyed to
the decode kernels' code (comments and whitespace aside), and a record taken
on other code is not reported."""
import bench


def _write(path, text):
    path.write_text(text, encoding="utf-8")
    return str(path)


def test_kernel_sha_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    code = "int f(int a)\n{\n    return a + 1;\n}\n"
    a = _write(tmp_path / "a.hip", code)
    b = _write(tmp_path / "b.hip", "// a comment\nint  f(int a) /* and\nanother */ {\n\treturn a + 1;  // end\n}\n")
    c = _write(tmp_path / "c.hip", code.replace("+ 1", "+ 2"))
    h = _write(tmp_path / "h.h", "#define X 1\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", [a, h])
    sha_a = bench.kernel_source_sha()
    monkeypatch.setattr(bench, "KERNEL_SRC", [b, h])
    assert bench.kernel_source_sha() == sha_a
    monkeypatch.setattr(bench, "KERNEL_SRC", [c, h])
    assert bench.kernel_source_sha() != sha_a
    # the header is part of the key too
    h2 = _write(tmp_path / "h2.h", "#define X 2\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", [a, h2])
    assert bench.kernel_source_sha() != sha_a


def test_recorded_traffic_only_for_the_same_code(tmp_path, monkeypatch):
    src = _write(tmp_path / "k.hip", "int g() { return 3; }\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", [src])
    sha = bench.kernel_source_sha()
    rec = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic() is None  # no record
    _write(rec, f"traffic_bytes_per_launch: 123456\nkernel_source_sha256: {sha}\n")
    assert bench.recorded_traffic() == 123456
    _write(rec, f"traffic_bytes_per_launch: 123456\nkernel_source_sha256: {'0' * 64}\n")
    assert bench.recorded_traffic() is None  # taken on other code
    _write(rec, f"kernel_source_sha256: {sha}\n")
    assert bench.recorded_traffic() is None  # no figure


def test_committed_record_is_well_formed():
    text = open(bench.TRAFFIC_FILE, encoding="utf-8").read()
    assert "traffic_bytes_per_launch:" in text and "kernel_source_sha256:" in text
