"""Child process of test_gpu_workspace.test_workspace_cap_in_child: runs one
decode-shaped bf16 GEMM (8 x 4096 x 4096, integer inputs) on each of twenty
fresh streams and prints, as one JSON line, the kernel each call launched
and whether its result equals the oracle's exactly."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))


def main():
    import torch
    import oracle
    from gpu_helpers import to_device
    from roofline_driven_optimisation_amd import binding
    from roofline_driven_optimisation_amd.inputs import make_case

    torch.cuda.set_device(0)
    oracle.build(force=False)
    case = make_case(8, 4096, 4096, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=43)
    ref, _ = oracle.gemm(case.A, case.B, case.C, 1.5, 0.5, bf16=True)
    streams = [torch.cuda.Stream() for _ in range(20)]
    handles = {s.cuda_stream for s in streams}
    if len(handles) != 20 or 0 in handles:
        print("streams are not distinct", file=sys.stderr)
        sys.exit(3)
    names, exact = [], []
    for i, s in enumerate(streams):
        print("child: stream %d" % i, file=sys.stderr, flush=True)
        A, B, C = to_device(case)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            binding.gemm(A, B, C, 1.5, 0.5, stream=s)
        names.append(binding.last_kernel())
        s.synchronize()
        exact.append(bool(np.array_equal(C.cpu().numpy().astype(np.float64), ref)))
    print(json.dumps({"names": names, "exact": exact}), flush=True)


if __name__ == "__main__":
    main()
