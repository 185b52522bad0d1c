"""The allocation-free overflow / norm entry point against the one with a
caller workspace: the same kernels, so the same scalars bit for bit, on two
calls in a row (the second with a smaller input, so the fixed array holds
the first call's partials when it starts), both dtypes, a ragged length and
an overflow; the size limit is rejected on the host."""

import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from zero_sharded_mixed_tensor_amd import zds  # noqa: E402

LIMIT = 1_073_217_536


def _scalars_bytes(t):
    torch.cuda.synchronize()
    return bytes(t.cpu().numpy().tobytes())


def test_noalloc_norm_matches_the_workspace_entry_point():
    state = zds.new_state()
    zds.zds_step_state_init(state, zds.scaler_config(initial_scale_power=12))
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    cases = [("bf16", 50_000_003), ("fp16", 1_234_567), ("fp32", 7_000_001), ("bf16", 4099)]
    for k, (dt, n) in enumerate(cases):
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dt]
        x = torch.empty(n, dtype=tdt, device="cuda").normal_(0.0, 1e-3 * 4096, generator=g)
        if k == 2:
            x[n // 3] = float("inf")
        want = zds.new_scalars()
        zds.zds_overflow_and_norm(x, 4, 1.0, state, want, zds.new_workspace(n))
        got = zds.new_scalars()
        zds.zds_overflow_and_norm_noalloc(x, 4, 1.0, state, got)
        assert _scalars_bytes(got) == _scalars_bytes(want), (dt, n)
        sc = zds.read_scalars(got)
        assert sc.overflow == (1 if k == 2 else 0)
    # n = 0: the scalars of an empty shard
    want, got = zds.new_scalars(), zds.new_scalars()
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    zds.zds_overflow_and_norm(e, 1, 1.0, state, want, zds.new_workspace(0))
    zds.zds_overflow_and_norm_noalloc(e, 1, 1.0, state, got)
    assert _scalars_bytes(got) == _scalars_bytes(want)


def test_noalloc_norm_size_limit():
    state = zds.new_state()
    sc = zds.new_scalars()
    lib = zds.lib
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    # sizes are checked before any launch: a pointer to 16 elements with a
    # larger n is never read when the call is rejected
    assert zds.zds_workspace_bytes(LIMIT) <= 4 << 20 < zds.zds_workspace_bytes(LIMIT + 1)
    rc = lib.zds_overflow_and_norm_noalloc(ctypes.c_void_p(x.data_ptr()), zds.ZDS_FP32, LIMIT + 1, 1,
                                           ctypes.c_float(1.0), ctypes.c_void_p(state.data_ptr()),
                                           ctypes.c_void_p(sc.data_ptr()), None)
    assert rc == zds.ZDS_EINVAL and b"fixed array" in zds.lib.zds_last_error()
