"""Host-side checks of bench.py's bookkeeping (no GPU): the fused-kernel code
hash that keys the committed traffic summaries ignores comments and blank
lines but not code, and a summary is used only while its hash matches."""
import os
import shutil

import bench


def _copy_sources(tmp_path):
    csrc = tmp_path / "chunkwise_gated_recurrence_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(bench.ROOT, "chunkwise_gated_recurrence_amd", "csrc")
    for f in bench.FUSED_SOURCES:
        shutil.copy(os.path.join(src, f), csrc / f)
    return csrc


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_hash()
    f = csrc / bench.FUSED_SOURCES[-1]
    text = f.read_text(encoding="utf-8")
    f.write_text("// a new comment line\n\n" + text.replace("{\n", "{   // trailing note\n", 1),
                 encoding="utf-8")
    assert bench.kernel_hash() == h0
    f.write_text(text.replace("kPollSleep = 2", "kPollSleep = 3", 1), encoding="utf-8")
    assert bench.kernel_hash() != h0


def test_traffic_summary_only_for_matching_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    h = bench.kernel_hash()
    (tmp_path / "traffic_w.txt").write_text(f"# x\nbytes_per_launch: 1234\nkernel_hash: {h}\n")
    assert bench.measured_traffic("w") == 1234.0
    (tmp_path / "traffic_w.txt").write_text("bytes_per_launch: 1234\nkernel_hash: 0000\n")
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("missing") is None
