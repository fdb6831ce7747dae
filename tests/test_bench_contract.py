"""Host-side parts of bench.py: the one-GPU guard and the kernel-source hash
that decides whether the committed HBM counters still describe the kernels."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc")
    copy = tmp_path / "combine_ep_get_layout_amd" / "csrc"
    shutil.copytree(src, copy)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = copy / "ep_combine.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* trailing */\n")
    assert bench.kernel_source_hash() == h0
    f.write_text(text.replace("kRowsInFlight = 4", "kRowsInFlight = 2", 1))
    assert bench.kernel_source_hash() != h0
    (copy / "ep_api.hip").write_text("// host layer, not hashed\n")
    f.write_text(text)
    assert bench.kernel_source_hash() == h0
