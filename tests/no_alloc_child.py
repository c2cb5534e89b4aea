"""Child process of the no-allocation entry point's test: in a fresh
process, gemm_bf16_noalloc on several shapes (the first call sets the
scratch up and runs the XCD probe itself), three rounds, the C copies with
beta != 0 restored between rounds; prints one JSON line with the kernels,
exactness against the oracle and the device's free memory before and after
the second and third rounds (the first round also launches each kernel for
the first time in the process, which the runtime may back with memory of
its own)."""
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
    shapes = [(16, 11008, 4096), (8, 4096, 4096), (1, 4096, 11008), (4, 2048, 1024),
              (300, 520, 256)]
    cases = [make_case(*sh, "bf16", 1.5, 0.5, "i:4", "i:4", "i:4", seed=70 + i)
             for i, sh in enumerate(shapes)]
    dev = [to_device(c) for c in cases]  # every tensor exists before the first call
    staged = [torch.from_numpy(c.C).cuda() for c in cases]  # copies of C for later rounds
    torch.cuda.synchronize()
    kernels, exact, free = [], [], []
    for rnd in range(3):
        for i, (case, (A, B, C)) in enumerate(zip(cases, dev)):
            print("child: round %d call %d %s" % (rnd, i, shapes[i]), file=sys.stderr, flush=True)
            if rnd > 0 and case.C is not None:
                C.copy_(staged[i])
                torch.cuda.synchronize()
            if rnd == 1 and i == 0:
                free.append(torch.cuda.mem_get_info()[0])  # after every kernel's first launch
            binding.gemm_bf16_noalloc(A, B, C, 1.5, 0.5)
            torch.cuda.synchronize()
            if rnd == 0:
                kernels.append(binding.last_kernel())
                print("child: free after call %d: %d" % (i, torch.cuda.mem_get_info()[0]),
                      file=sys.stderr, flush=True)
            ref, _ = oracle.gemm(case.A, case.B, case.C, 1.5, 0.5, bf16=True)
            exact.append(bool(np.array_equal(C.cpu().numpy().astype(np.float64), ref)))
    free.append(torch.cuda.mem_get_info()[0])
    print(json.dumps({"kernels": kernels, "exact": exact, "free_before_later_rounds": free[0],
                      "free_after_later_rounds": free[1]}), flush=True)


if __name__ == "__main__":
    main()
