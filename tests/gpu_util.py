"""Shared helpers of the GPU parity tests (not a test module)."""
import math

import torch

# Tolerances: max-abs error of O, and of LSE, against the fp64 oracle.
TOL_O = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 2e-2}
TOL_LSE = 1e-3

DEV = torch.device("cuda:0")


def report(name, o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    """Print and return (max|dO|, max|dLSE|); -inf must match -inf exactly."""
    do = (o_gpu.detach().double().cpu() - o_ref.double()).abs().max().item() if o_ref.numel() else 0.0
    dl = 0.0
    if lse_gpu is not None:
        lg, lr = lse_gpu.detach().double().cpu(), lse_ref.double()
        inf_g, inf_r = torch.isinf(lg), torch.isinf(lr)
        assert torch.equal(inf_g, inf_r), f"{name}: -inf pattern of LSE differs"
        fin = ~inf_r
        dl = (lg[fin] - lr[fin]).abs().max().item() if fin.any() else 0.0
    print(f"{name}: max|dO|={do:.3e} max|dLSE|={dl:.3e}", flush=True)
    return do, dl


def check(name, o_gpu, o_ref, lse_gpu, lse_ref, dtype):
    do, dl = report(name, o_gpu, o_ref, lse_gpu, lse_ref)
    assert math.isfinite(do) and do <= TOL_O[dtype], f"{name}: max|dO| {do} > {TOL_O[dtype]}"
    assert dl <= TOL_LSE, f"{name}: max|dLSE| {dl} > {TOL_LSE}"
