"""The XCD-local split-K paths after the hardware's round robin has moved.

Workgroups are dealt to the eight XCDs in round-robin order, but which XCD
takes workgroup 0 is not fixed: after graph replays it moved in probes on
MI355X.  The library's once-per-device placement probe must accept any
starting XCD (the kernels only rely on ids equal modulo 8 sharing an XCD),
so a process whose first GEMM follows graph replays must still choose the
XCD-local kernels, and their results must stay exact.  A child process
gives the probe a fresh start."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_xcd_paths_after_graph_replay():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = {k: v for k, v in os.environ.items() if not k.startswith("MGEMM_")}
    print("  child: graph replays, then 16x4096x2048 and split-tail 1024x4096x264", flush=True)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "xcd_after_graph_child.py")],
                          env=env, capture_output=True, text=True, timeout=110)
    assert proc.returncode == 0, proc.stderr[-3000:]
    line = [l for l in proc.stdout.splitlines() if l.startswith("{")][-1]
    out = json.loads(line)
    assert out["replays_ok"], out
    assert out["skinny"] == "skinny_bf16_splitk_xcd", out
    assert out["pp"] == "bf16_pp_256x256x32_splitk_xcd", out
    assert out["skinny_exact"] and out["pp_exact"], out
