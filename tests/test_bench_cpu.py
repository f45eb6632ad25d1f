"""Host-side parts of bench.py (no GPU): the kernel-source hash that keys the
committed counter traffic, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_hash_follows_code_not_text(tmp_path):
    base = "__global__ void k(int* p) {\n  p[0] = 1;  // one\n}\n"
    variants = {
        "same": base,
        "comments": "/* a kernel */\n__global__ void k(int* p) {\n  p[0] = 1;  // the first\n}\n",
        "spacing": "__global__   void k(int* p)\n{ p[0] = 1; }\n",
        "code": "__global__ void k(int* p) {\n  p[0] = 2;  // one\n}\n",
    }
    h = {}
    for name, text in variants.items():
        f = tmp_path / (name + ".hip")
        f.write_text(text)
        h[name] = bench.source_hash([str(f)])
    assert h["same"] == h["comments"] == h["spacing"]
    assert h["code"] != h["same"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
