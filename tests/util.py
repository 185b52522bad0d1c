"""Shared helpers for the GPU parity tests: host<->device transfer of raw
bit patterns and ulp distances. No optimizer arithmetic here."""

import numpy as np
import torch

TORCH_16 = {"fp16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a, dtype):
    """numpy array (uint16 bit patterns for 16-bit dtypes, float32 for fp32)
    -> contiguous device tensor of the named dtype with the same bytes."""
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(TORCH_16[dtype])


def to_host(t):
    """Device tensor -> numpy: uint16 bit patterns for 16-bit, float32 else."""
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def ordered(bits, width):
    """Map IEEE bit patterns to integers ordered like the values (+0 == -0)."""
    b = bits.astype(np.int64)
    sign = np.int64(1) << (width - 1)
    mag = b & (sign - 1)
    return np.where(b & sign, -mag, mag)


def ulp_diff32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    assert not np.isnan(a).any() and not np.isnan(b).any(), "NaN in fp32 state"
    return np.abs(ordered(a.view(np.uint32), 32) - ordered(b.view(np.uint32), 32))


def ulp_diff16(a, b):
    return np.abs(ordered(np.asarray(a, np.uint16), 16) - ordered(np.asarray(b, np.uint16), 16))


def assert_state_close(name, got, want, max_ulp):
    d = ulp_diff32(got, want)
    if d.size and d.max() > max_ulp:
        i = int(np.argmax(d))
        raise AssertionError("%s: %d elements over %d ulp, worst %d ulp at %d (got %r want %r)"
                             % (name, int((d > max_ulp).sum()), max_ulp, int(d.max()), i,
                                float(got[i]), float(want[i])))
    return int(d.max()) if d.size else 0


def assert_p16_close(name, got, want, max_ulp=1):
    d = ulp_diff16(got, want)
    if d.size and d.max() > max_ulp:
        i = int(np.argmax(d))
        raise AssertionError("%s: %d elements over %d ulp, worst %d at %d (got %04x want %04x)"
                             % (name, int((d > max_ulp).sum()), max_ulp, int(d.max()), i,
                                int(got[i]), int(want[i])))
    return int(d.max()) if d.size else 0
