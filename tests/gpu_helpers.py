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


# ---- guard regions around device outputs ----------------------------------------------------

GUARD_BYTES = 4096          # keeps the inner tensor 256-byte aligned
GUARD_FILL = 0xA5


class Guarded:
    """A device output tensor with GUARD_BYTES of a known byte pattern on either side, in one
    allocation; check() asserts that no kernel wrote outside the tensor."""

    def __init__(self, shape, dtype, fill=None):
        itemsize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * itemsize
        self.raw = torch.full((GUARD_BYTES * 2 + self.nbytes,), GUARD_FILL, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(tuple(shape))
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what: str = ""):
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.nbytes:]
        bad = int((head != GUARD_FILL).sum()) + int((tail != GUARD_FILL).sum())
        assert bad == 0, f"{what}: {bad} guard bytes overwritten around the output"


# ---- sampled output tiles of full-size layers ----------------------------------------------

def sample_tiles(T: int, count: int, seed: int) -> np.ndarray:
    """Column tiles (16 columns each) to check on a full-size layer: the first and last two,
    both sides of every workgroup boundary that falls on an XCD-range edge for each workgroup
    width the kernels use (1, 2, 4, 8, 16 tiles; ranges of about 1/8 of the blocks each), and
    seeded random tiles up to `count`."""
    s = {0, 1, T - 2, T - 1}
    for w in (1, 2, 4, 8, 16):
        blocks = -(-T // w)
        for x in range(1, 8):
            for b in {x * blocks // 8, -(-x * blocks // 8)}:
                for t in (b * w - 1, b * w):
                    if 0 <= t < T:
                        s.add(t)
        s.add(min(T - 1, (blocks - 1) * w))               # first tile of the last block
    r = np.random.Generator(np.random.PCG64(seed))
    while len(s) < min(count, T):
        s.add(int(r.integers(0, T)))
    return np.array(sorted(s), dtype=np.int64)
