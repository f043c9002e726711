"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the stored counter record
that supplies roofline.traffic."""
import hashlib
import json
import os
import subprocess
import sys

from dual_ar_codec_amd import metrics, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "drives one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """The stored HBM bytes are reported only while the kernel source is the one they were taken on."""
    sys.path.insert(0, ROOT)
    import bench

    (tmp_path / "profiles").mkdir()
    (tmp_path / "dual_ar_codec_amd" / "csrc").mkdir(parents=True)
    src = tmp_path / "dual_ar_codec_amd" / "csrc" / "kernels.hip"
    rec_path = tmp_path / "profiles" / "gate_up_hbm_traffic.json"
    src.write_bytes(b"// one kernel source\n")
    rec_path.write_text(json.dumps({"kernels_hip_sha256": hashlib.sha256(src.read_bytes()).hexdigest(),
                                    "traffic_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == 123
    src.write_bytes(b"// an edited kernel source\n")
    assert bench.measured_traffic() is None
    rec_path.write_text("{")
    assert bench.measured_traffic() is None
    rec_path.unlink()
    assert bench.measured_traffic() is None


def test_stored_traffic_record_is_consistent():
    """Each counter is scaled so that the copy probe reads exactly its size, the launch's bytes are
    the two scaled counters summed, and the algorithmic bytes are the gate/up launch's byte model."""
    with open(os.path.join(ROOT, "profiles", "gate_up_hbm_traffic.json")) as f:
        rec = json.load(f)
    cp = rec["copy_probe"]
    sf = cp["bytes_each_way"] / 1024 / cp["fetch_kib"]
    sw = cp["bytes_each_way"] / 1024 / cp["write_kib"]
    assert abs(sf - rec["scale_fetch"]) < 1e-5 and abs(sw - rec["scale_write"]) < 1e-5
    traffic = (rec["fetch_kib_per_launch"] * sf + rec["write_kib_per_launch"] * sw) * 1024
    assert abs(traffic - rec["traffic_bytes_per_launch"]) <= 1
    assert rec["algorithmic_bytes_per_launch"] == metrics.gate_up_launch_bytes(synth.config("full"))
    # the counters see the weights once: within 1% of the byte model
    assert 1.0 <= rec["traffic_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.01
