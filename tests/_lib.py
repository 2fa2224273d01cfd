"""Shared helpers for the library tests: build-if-missing, device upload, metrics."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_paged_decode_03_amd", "libmla_decode.so")


def ensure_built():
    """Build the HIP library if it is not there yet (hipcc cross-compiles without a GPU)."""
    if not os.path.exists(LIB):
        subprocess.check_call([sys.executable, "-m", "mla_paged_decode_03_amd.build"], cwd=ROOT)
    return LIB


def bf16_dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def u8_dev(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn).to(device)


def bf16_host(t):
    """bf16 device tensor -> float64 numpy."""
    import torch
    return t.float().cpu().numpy().astype(np.float64)


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel_l2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
    return max_abs, rel_l2


# Tolerances for bf16 outputs against the fp64 oracle (fp8 caches are compared against
# the oracle fed the identically dequantised values) and for the LSE.
O_MAX_ABS, O_REL_L2, LSE_MAX_ABS = 1e-2, 5e-3, 1e-3
