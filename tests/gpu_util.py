"""Helpers shared by the GPU tests: device upload of the seeded bf16 bit patterns and the
parity bars.  No arithmetic of the method lives here."""
import numpy as np
import torch

# Parity bars for floating point: max |err| <= 2e-2 and mean |err| <= 2e-3 against the fp64
# oracle, for out_lat and for lse.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on cuda:0 (bitwise)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.mean())


def assert_close(out, lse, ref_out, ref_lse, what=""):
    assert np.isfinite(out).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    mo, ao = errors(out, ref_out)
    ml, al = errors(lse, ref_lse)
    assert mo <= MAX_ABS and ao <= MEAN_ABS, f"{what}: out max {mo:.3e} mean {ao:.3e}"
    assert ml <= MAX_ABS and al <= MEAN_ABS, f"{what}: lse max {ml:.3e} mean {al:.3e}"
    return mo, ao, ml, al


# Guard bands: a device tensor placed between two bands of canary bytes, so that a test can
# check that a call wrote nothing outside the tensor it was given.
GUARD_BYTES = 4096
CANARY = 0xA5


class Guarded:
    """``t``: a contiguous device tensor of ``shape`` / ``dtype`` with GUARD_BYTES of CANARY bytes
    right before and right after it in one allocation (``t`` stays 256-byte aligned)."""

    def __init__(self, shape, dtype, fill=None):
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(shape)) * itemsize
        self.buf = torch.full((2 * GUARD_BYTES + self.nbytes,), CANARY, dtype=torch.uint8, device="cuda:0")
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill if isinstance(fill, torch.Tensor) else torch.as_tensor(fill))

    def intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool((b[:GUARD_BYTES] == CANARY).all() and (b[GUARD_BYTES + self.nbytes:] == CANARY).all())


def guarded_bf16(bits: np.ndarray) -> Guarded:
    """uint16 bf16 bit patterns -> a guarded torch.bfloat16 device tensor (bitwise)."""
    g = Guarded(bits.shape, torch.bfloat16)
    g.t.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)))
    return g


def guarded_i32(a: np.ndarray) -> Guarded:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return Guarded(a.shape, torch.int32, fill=torch.from_numpy(a))
