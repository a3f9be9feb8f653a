"""Host-side rules of bench.py that need no GPU: the kernel-source hash that ties the stored
HBM-traffic figures to the kernel they were measured on, and the lookup that honours it."""
import os

import pytest

import bench


@pytest.fixture
def fake_kernel(tmp_path, monkeypatch):
    """A one-file kernel entry in bench.KERNELS whose source and traffic summary live in tmp_path."""
    src = tmp_path / "k_fake.hip"
    src.write_text("// header comment\nint f(int a) {\n  return a + 1;  // add one\n}\n")
    monkeypatch.setitem(bench.KERNELS, "fake", ("fake kernel", [str(src)]))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "traffic_file", lambda path: str(tmp_path / f"{path}_traffic.md"))
    return src


def test_hash_ignores_comments_and_blank_lines(fake_kernel):
    h0 = bench.kernel_source_hash("fake")
    fake_kernel.write_text("// another header\n\nint f(int a) {\n  return a + 1;\n}\n// trailer\n")
    assert bench.kernel_source_hash("fake") == h0


def test_hash_follows_code(fake_kernel):
    h0 = bench.kernel_source_hash("fake")
    fake_kernel.write_text("// header comment\nint f(int a) {\n  return a + 2;  // add one\n}\n")
    assert bench.kernel_source_hash("fake") != h0


def test_stored_traffic_needs_the_matching_hash(fake_kernel):
    assert bench.stored_traffic("fake") is None            # no summary yet
    summary = os.path.join(bench.ROOT, "fake_traffic.md")
    with open(summary, "w") as f:
        f.write(f"hbm_bytes_per_launch: 12345\nkernel_source_sha256: {bench.kernel_source_hash('fake')}\n")
    assert bench.stored_traffic("fake") == 12345.0
    fake_kernel.write_text("int f(int a) { return a; }\n")    # the code changed since
    assert bench.stored_traffic("fake") is None


def test_every_listed_kernel_source_exists():
    for path, (_, files) in bench.KERNELS.items():
        for rel in files:
            assert os.path.exists(os.path.join(bench.ROOT, rel)), (path, rel)


def test_stored_trace_needs_the_path_and_the_matching_hash(fake_kernel, tmp_path, monkeypatch):
    summary = tmp_path / "trace.md"
    monkeypatch.setattr(bench, "trace_file", lambda path: str(summary))
    assert bench.stored_trace_ns("fake") is None            # no summary yet
    h = bench.kernel_source_hash("fake")
    summary.write_text(f"dominant_path: slab\ndominant_kernel_trace_mean_ns: 900\nkernel_source_sha256: {h}\n")
    assert bench.stored_trace_ns("fake") is None            # another path's figure
    summary.write_text(f"dominant_path: fake\ndominant_kernel_trace_mean_ns: 900\nkernel_source_sha256: {h}\n")
    assert bench.stored_trace_ns("fake") == 900.0
    fake_kernel.write_text("int f(int a) { return a; }\n")  # the code changed since
    assert bench.stored_trace_ns("fake") is None


def test_committed_trace_summary_matches_the_slab_sources():
    # the committed summary names the slab kernel; its figure is used only while the sources match
    ns = bench.stored_trace_ns("slab")
    assert ns is None or 50e3 < ns < 200e3
