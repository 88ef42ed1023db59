"""CPU checks of bench.py's bookkeeping (no GPU): the kernel-source hash that ties a recorded
HBM-traffic summary to the code it was taken on ignores comments and blank lines but not code,
every kernel's sources exist, and the committed traffic summaries parse."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _fake_tree(tmp_path):
    for name in bench.KERNEL_SOURCES["verify_attn"]:
        path = tmp_path / name
        path.parent.mkdir(parents=True, exist_ok=True)
        path.write_text("int unchanged;\n")
    return tmp_path / "tree_verify_mla_02_amd" / "csrc"


def test_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = _fake_tree(tmp_path)
    (csrc / "verify_attn.hip").write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    (csrc / "kdt_internal.h").write_text("/* header */\n#pragma once\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("verify_attn")
    (csrc / "verify_attn.hip").write_text("// a new comment\nint f(int x) {\n\n  return x + 1;  // two\n}\n")
    assert bench.kernel_source_hash("verify_attn") == h0
    (csrc / "kdt_internal.h").write_text("/* another\n   header */\n#pragma once\n")
    assert bench.kernel_source_hash("verify_attn") == h0
    (csrc / "verify_attn.hip").write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash("verify_attn") != h0


def test_hash_covers_launch_geometry_and_flags(tmp_path, monkeypatch):
    """The split policy lives in the C-ABI layer: a change there (or to the build flags) must
    void a recorded traffic figure too."""
    csrc = _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("verify_attn")
    (csrc / "api.cpp").write_text("int chunk = 512;\n")
    h1 = bench.kernel_source_hash("verify_attn")
    assert h1 != h0
    from tree_verify_mla_02_amd import build as kbuild
    monkeypatch.setattr(kbuild, "FLAGS", kbuild.FLAGS + ["-DKDT_MIN_CHUNK=128"])
    assert bench.kernel_source_hash("verify_attn") != h1


def test_every_kernel_source_exists():
    for kernel, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert os.path.exists(os.path.join(ROOT, n)), (kernel, n)
        assert len(bench.kernel_source_hash(kernel)) == 16


def test_committed_traffic_summaries_parse():
    prof = os.path.join(ROOT, "profiles")
    found = 0
    for name in sorted(os.listdir(prof)):
        if not name.endswith("_hbm_traffic.md"):
            continue
        found += 1
        fields = {}
        for line in open(os.path.join(prof, name)):
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
        total = int(fields["hbm_bytes_per_launch"])
        parts = int(fields["hbm_read_bytes_per_launch"]) + int(fields["hbm_write_bytes_per_launch"])
        assert abs(total - parts) <= 2          # each figure rounded on its own
        assert len(fields["kernel_source_hash"]) == 16
    assert found >= 1
