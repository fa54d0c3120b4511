"""Host logic of bench.py (no GPU): the kernel-source hash that decides
whether the committed HBM counter summary still describes the kernels."""
import os

import bench


def test_strip_comments_keeps_code_and_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "// kept /* too */";\nchar c = \'"\';  int  b =\n 2;'
    assert bench.strip_comments(src) == 'int a = 1; const char* s = "// kept /* too */"; char c = \'"\'; int b = 2;'


def test_escaped_quotes_inside_literals():
    src = r'const char* s = "a\"b // not a comment"; // gone'
    assert bench.strip_comments(src) == r'const char* s = "a\"b // not a comment";'


def test_comment_edits_keep_the_hash_and_code_edits_change_it(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": (str(f),)})
    f.write_text("// header\n__global__ void k(float* x) { x[0] = 1.0f; }\n")
    h0 = bench.kernel_source_sha("k")
    f.write_text("/* another header */\n__global__ void k(float* x) {\n  x[0] = 1.0f;  // one\n}\n")
    assert bench.kernel_source_sha("k") == h0
    f.write_text("__global__ void k(float* x) { x[0] = 2.0f; }\n")
    assert bench.kernel_source_sha("k") != h0


def test_a_kernel_hash_covers_its_own_sources_only(tmp_path, monkeypatch):
    """An edit of another kernel's file leaves a kernel's hash (and so its
    counters) alone; an edit of a shared header changes both."""
    fa, fb, hdr = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "common.h"
    for f, body in ((fa, "void a() {}"), (fb, "void b() {}"), (hdr, "#define X 1")):
        f.write_text(body + "\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"a": (str(fa), str(hdr)), "b": (str(fb), str(hdr))})
    ha, hb = bench.kernel_source_sha("a"), bench.kernel_source_sha("b")
    fb.write_text("void b() { int x = 1; }\n")
    assert bench.kernel_source_sha("a") == ha and bench.kernel_source_sha("b") != hb
    hdr.write_text("#define X 2\n")
    assert bench.kernel_source_sha("a") != ha


def test_every_measured_kernel_has_sources():
    for kernel, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert os.path.exists(os.path.join(bench.ROOT, "gated_delta_rule_23_amd", "csrc", n)), (kernel, n)


def test_committed_traffic_lines_parse():
    """Every kernel line of the committed summary names a kernel, a hash and
    a byte count; bench.py uses a line only while the hash matches."""
    path = bench.PROFILE_TRAFFIC
    assert os.path.exists(path)
    lines = [ln for ln in open(path) if ln.startswith("kernel=")]
    assert {dict(t.split("=", 1) for t in ln.split())["kernel"] for ln in lines} >= {bench.PREFILL_KERNEL,
                                                                                     "decode_kernel"}
    for ln in lines:
        fields = dict(t.split("=", 1) for t in ln.split())
        assert len(fields["kernel_source_sha"]) == 16 and float(fields["hbm_bytes_per_launch"]) > 0
