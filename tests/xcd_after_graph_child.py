"""Child process of test_gpu_xcd_probe: replays a captured graph of small
library launches first (which moves the XCD that takes workgroup 0 of later
launches), then makes this process's first decode-shaped and split-tail
GEMM calls, which run the once-per-device placement probe.  Prints one JSON
line: the kernels chosen and whether each output matched the oracle exactly
(integer inputs)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from gpu_helpers import to_device  # noqa: E402
from roofline_driven_optimisation_amd import binding  # noqa: E402
from roofline_driven_optimisation_amd.inputs import make_case  # noqa: E402


def main():
    A = torch.zeros(1, 0, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(0, 8, dtype=torch.bfloat16, device="cuda")
    C = torch.ones(1, 8, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.gemm(A, B, C, 1.0, 0.0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(203):
            binding.gemm(A, B, C, 1.0, 0.0)
    replays_ok = True
    for _ in range(3):
        C.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        replays_ok = replays_ok and bool(torch.all(C == 0.0))
    out = {"replays_ok": replays_ok}
    for key, shape, env in (("skinny", (16, 4096, 2048), {}),
                            ("pp", (1024, 4096, 264), {"MGEMM_BF16_TILE": "bf16_pp_256x256x32",
                                                       "MGEMM_DISABLE_SKINNY": "1"})):
        os.environ.update(env)
        case = make_case(*shape, "bf16", 1.0, 0.5, "i:4", "i:4", "i:4", seed=70)
        dA, dB, dC = to_device(case)
        binding.gemm(dA, dB, dC, 1.0, 0.5)
        name = binding.last_kernel()
        torch.cuda.synchronize()
        ref, _ = oracle.gemm(case.A, case.B, case.C, 1.0, 0.5, bf16=True)
        out[key] = name
        out[key + "_exact"] = bool(np.array_equal(dC.cpu().numpy().astype(np.float64), ref))
        for k in env:
            del os.environ[k]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
