"""Host-side checks of bench.py's bookkeeping (no GPU): the fused-kernel code
hash that keys the committed traffic summaries ignores comments and blank
lines but not code, a summary is used only while its hash matches, and the
Spatial SwiGLU / low-rank summary's hash covers those kernels' sources."""
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


def test_rotation_spans_512_mib_for_any_step_count():
    import gla_synth
    for name in ("img640", "img1024", "batched640", "long2048"):
        w = gla_synth.WORKLOADS[name]
        per_call = bench.alg_bytes(w)
        groups = bench.rotation_groups(per_call, True)
        assert groups * len(bench.DIRS) * per_call >= bench.ROTATE_BYTES, name
        assert (groups - 1) * len(bench.DIRS) * per_call < bench.ROTATE_BYTES, name
    assert bench.rotation_groups(10 ** 6, False) == 1


def test_replay_plan_runs_exactly_the_requested_steps():
    for n_groups in (1, 3, 22, 87):
        for steps in (0, 1, 5, 20, 21, 200, 201):
            full, rem = bench.replay_plan(steps, n_groups)
            assert full * n_groups + rem == steps and 0 <= rem < n_groups


def test_host_cpu_fields():
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and 1 <= h["affinity"] <= h["nproc"]
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)


def test_mixer_hash_covers_the_mixer_sources():
    src = os.path.join(bench.ROOT, "chunkwise_gated_recurrence_amd", "csrc")
    for f in bench.MIXER_SOURCES:
        assert os.path.exists(os.path.join(src, f)), f
    assert "sswiglu.hip" in bench.MIXER_SOURCES and "gla_gate.hip" in bench.MIXER_SOURCES
    assert bench.kernel_hash(bench.MIXER_SOURCES) != bench.kernel_hash()
    # the committed summary names the hash it was taken at
    with open(os.path.join(bench.ROOT, "profiles", "mixer_and_lowrank_kernels.txt")) as fh:
        assert "kernel_hash(MIXER_SOURCES)" in fh.read()
