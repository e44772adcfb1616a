"""Shared helpers of the GPU parity tests: host<->device conversion and the
tolerance checks.  Tolerances: float32 path max |gpu - oracle| <= 1e-5;
bfloat16 path per element |gpu - oracle| <= 3e-2 + 2e-2*|oracle| and
||gpu - oracle||_2 / ||oracle||_2 <= 2e-2 (both sides see the same
bf16-rounded inputs; the oracle computes in float64)."""
import sys

import numpy as np

import wsp_inputs as I

F32_MAX_ABS = 1e-5
BF16_ATOL, BF16_RTOL, BF16_REL_L2 = 3e-2, 2e-2, 2e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(values, bits, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).cuda()


def from_dev(t):
    """Device tensor -> float64 numpy (exact widening of bf16)."""
    import torch
    if t.dtype == torch.bfloat16:
        b = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(b).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def dev_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_f32(gpu, ref, what=""):
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    log(f"  {what}: max|err| = {err:.3e} (bar {F32_MAX_ABS:.0e})")
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert err <= F32_MAX_ABS, f"{what}: max abs error {err}"


def check_bf16(gpu, ref, what=""):
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    diff = np.abs(gpu - ref)
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    worst = float(np.max(diff / bound)) if gpu.size else 0.0
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"  {what}: max|err| = {float(diff.max()):.3e}, rel-L2 = {rel:.3e} (bar {BF16_REL_L2})")
    assert worst <= 1.0, f"{what}: element error exceeds 3e-2 + 2e-2*|ref| (ratio {worst})"
    assert rel <= BF16_REL_L2, f"{what}: relative L2 error {rel}"
