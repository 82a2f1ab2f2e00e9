"""CONVROT_LOG=1: one stderr line per call that enqueues work, naming the
entry point, its sizes and format arguments and the kernels enqueued; no line
without it. The setting is read once per process, so each case runs a small
child process (one quantize call and one GEMM call on the GPU)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
import torch
import w4a8_rotated_quantized_amd as cr
x = torch.randn((64, 512), device="cuda:0").to(torch.bfloat16)
w = (torch.randn((256, 512), device="cuda:0") * 0.02).to(torch.bfloat16)
xc, xs, _, _ = cr.convrot_rotate_quantize(x, 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
wc, ws, _, _ = cr.convrot_rotate_quantize(w, 256, cr.Q.SYM_INT8, cr.GRAN.TENSOR)
y = cr.int8_tensorwise_gemm(xc, xs, wc, ws, 64, 256, 512)
torch.cuda.synchronize()
print("child done", flush=True)
"""


def _run(log):
    env = dict(os.environ)
    env.pop("CONVROT_LOG", None)
    if log:
        env["CONVROT_LOG"] = "1"
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "child done" in r.stdout, r.stderr[-2000:]
    return [ln for ln in r.stderr.splitlines() if ln.startswith("[convrot]")]


def test_log_one_line_per_enqueuing_call():
    lines = _run(True)
    assert len(lines) == 3, lines
    assert lines[0].startswith("[convrot] convrot_rotate_quantize sizes 64 512 256 formats 1 0 0:"), lines[0]
    assert lines[1].startswith("[convrot] convrot_rotate_quantize sizes 256 512 256 formats 1 0 0:"), lines[1]
    assert lines[2].startswith("[convrot] int8_tensorwise_gemm sizes 64 256 512 formats 0 0 0: 1 kernel(s)"), lines[2]
    assert all(ln.endswith("enqueued") for ln in lines), lines


def test_log_silent_by_default():
    assert _run(False) == []
