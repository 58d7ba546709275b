"""bench.py's host helpers (CPU only): the kernel source hash covers code only,
so that a comment edit keeps committed counter summaries matched to the kernels
they measured, while any code change does not."""
import bench


def test_code_text_drops_comments_and_space_keeps_strings():
    src = 'int a = 1;  // note\n/* block\n comment */ const char* s = "//x /*y*/";\tchar c = \'/\';'
    assert bench.code_text(src) == 'int a = 1; const char* s = "//x /*y*/"; char c = \'/\';'


def test_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    base = tmp_path / "context_varlen_attention_amd" / "csrc" / "kernels"
    base.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": ["kernels/a.hip"]})
    monkeypatch.setattr(bench, "COMMON_SOURCES", [])
    f = base / "a.hip"
    f.write_text("int f() { return 1; }\n")
    h0 = bench.kernel_source_hash("k")
    f.write_text("// header\nint f() {\n  return 1;  /* same */\n}\n")
    assert bench.kernel_source_hash("k") == h0
    f.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash("k") != h0
