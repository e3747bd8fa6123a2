"""Shared helpers of the GPU parity tests: host <-> device copies and the tolerances."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")

# Final GEMM outputs: |gpu - oracle| <= ABS + REL * |oracle| per element (bfloat16 outputs use the
# stated rel 1e-2 / abs 1e-3; fp32 outputs are held ten times tighter).
BF16_ABS, BF16_REL = 1e-3, 1e-2
F32_ABS, F32_REL = 1e-4, 1e-3


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def cu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def bf16_dev(bits):
    return cu(np.ascontiguousarray(bits).view(np.int16), torch.bfloat16)


def weights_dev(w):
    """(codes u8 [N/16][G][1024], meta i32 [N/16][G][16]) on the device."""
    return cu(w["codes"]), cu(np.ascontiguousarray(w["meta"]).view(np.int32))


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close(got: np.ndarray, ref: np.ndarray, bf16: bool, what: str = ""):
    a, r = (BF16_ABS, BF16_REL) if bf16 else (F32_ABS, F32_REL)
    err = np.abs(got - ref)
    bad = err > a + r * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} oracle {ref[tuple(i)]!r}")
