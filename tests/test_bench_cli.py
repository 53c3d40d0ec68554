"""CPU checks of bench.py's host logic: more than one GPU is refused with a message and a non-zero
status before anything touches a device, --help prints the options, and the attention kernel's HBM
traffic is reported only while the kernel sources are the ones the committed counter summary was taken
on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)


def test_help_lists_the_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    for opt in ("--gpus", "--steps", "--warmup", "--config", "--keep", "--kv-block", "--extra", "--ablation"):
        assert opt in r.stdout


def test_live_clock_is_none_without_a_gpu():
    # no GPU in this container: the AMD SMI sampler gives up without raising and without launching
    sys.path.insert(0, ROOT)
    import bench
    launched = []
    assert bench.live_gfx_clock_ghz(lambda: launched.append(1), 3) is None
    assert not launched


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.attend_source_digest()
    assert len(digest) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = tmp_path / "block_sparse_attention_34_amd" / "csrc"
    src.mkdir(parents=True)
    for name in ("absa_attend_tiles.h", "absa_attend.hip", "absa_attend_pp.hip"):
        (src / name).write_bytes(open(os.path.join(ROOT, "block_sparse_attention_34_amd", "csrc", name), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = prof / "attend_kernel_t_traffic.md"
    f.write_text(f"traffic_bytes_per_launch: 123\nattend_source_sha256_16: {digest}\n")
    assert bench.measured_traffic("t") == 123
    f.write_text("traffic_bytes_per_launch: 123\nattend_source_sha256_16: 0000000000000000\n")
    assert bench.measured_traffic("t") is None           # the kernel changed since the counters were taken
    (src / "absa_attend_pp.hip").write_bytes(b"// edited\n")
    f.write_text(f"traffic_bytes_per_launch: 123\nattend_source_sha256_16: {digest}\n")
    assert bench.measured_traffic("t") is None
    assert bench.measured_traffic("missing") is None


def test_workload_tags_name_the_committed_profiles():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.workload_tag(3, 16, 0.095) == "wan14b_720p"
    assert bench.workload_tag(3, 16, 0.08) == "wan14b_720p_keep8"
    assert bench.workload_tag(3, 16, 0.11) == "wan14b_720p_keep11"
    assert bench.workload_tag(2, 16, 0.10) == "wan13b_480p_keep10"
    assert bench.workload_tag(4, 32, 0.08) == "hunyuan_720p_bk32_keep8"
    # a summary under the combined selection + attention name is found as well
    tag = bench.workload_tag(4, 16, 0.08)
    assert tag == "hunyuan_720p_keep8"
    path = os.path.join(ROOT, "profiles", f"attend_select_kernels_{tag}_traffic.md")
    if os.path.exists(path):
        v = bench.measured_traffic(tag)
        assert v is None or v > 0
