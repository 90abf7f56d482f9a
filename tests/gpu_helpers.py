"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device,
reading results back as float64, and the parity bars.

Bars (fixed for this library): bf16 -- max-abs <= 2e-2 and relative L2 <=
5e-3 against the float64 oracle; fp32 -- max-abs <= 1e-5.
"""
import sys

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5


def dev(a, dtype):
    """numpy (float32, or uint16 bf16 bits) -> contiguous device tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda").contiguous()


def host64(t):
    """device tensor (bf16 or fp32) -> float64 numpy, exact."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(got, ref):
    d = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(d.max()) if d.size else 0.0, rel


def check(got, ref, dtype, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, rel = errors(got, ref)
    print(f"[parity] {what} dtype={dtype} max_abs={mx:.3e} rel_l2={rel:.3e}", flush=True)
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, f"{what}: max_abs {mx:.3e}, rel_l2 {rel:.3e}"
    else:
        assert mx <= FP32_MAX_ABS, f"{what}: max_abs {mx:.3e}"


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()
