"""The offloaded (host) optimizer shard against the oracle, on the CPU: the
library's zds_cpu_adam_step must reproduce the oracle's AdamW + cast bit for
bit on every dtype pair, size, thread count and step count, and leave
everything untouched on an overflow step."""

import numpy as np
import pytest

import oracle as O
from workloads import draw_grads, draw_master, draw_prior_moments

zds = pytest.importorskip("zero_sharded_mixed_tensor_amd.zds", reason="libzds.so not built")

CODE = {"fp16": zds.ZDS_FP16, "bf16": zds.ZDS_BF16, "fp32": zds.ZDS_FP32}


def _host_state(t0):
    s = zds.zds_step_state_init_host(zds.scaler_config(initial_scale_power=12), t0,
                                     float(np.float32(0.9)) ** t0, float(np.float32(0.999)) ** t0)
    return s


@pytest.mark.parametrize("n", [1, 7, 1023, 1024, 1025, 100003])
@pytest.mark.parametrize("gdt,pdt", [("fp16", "fp16"), ("bf16", "bf16"), ("fp32", "fp16"), ("fp16", "bf16")])
@pytest.mark.parametrize("threads", [1, 3, 0])
def test_cpu_adam_matches_oracle(n, gdt, pdt, threads):
    seed = n + threads * 101 + len(gdt)
    g = draw_grads(n, gdt, 1e-3, 2.0 ** 12, seed, 96, 1)
    p = draw_master(n, 0.02, seed, 96)
    m, v = draw_prior_moments(n, 1e-3, seed, 96)
    t0 = 0 if n % 2 else 3
    if t0 == 0:
        m[:] = 0
        v[:] = 0
    hp = O.AdamW()
    st = O.scaler_init(initial_scale_power=12, t=t0, beta1_pow=float(np.float32(0.9)) ** t0,
                       beta2_pow=float(np.float32(0.999)) ** t0)
    oP, oM, oV, o16, ost, osc = O.optimizer_step(g, gdt, p.copy(), m.copy(), v.copy(), st, hp, 1.0, 1, pdt)
    sc = zds.zds_clip_scalars_host(osc["sumsq"], 2.0 ** 12, 1, 1.0)
    assert sc.grad_scale == osc["grad_scale"]
    P, M, V = p.copy(), m.copy(), v.copy()
    out = np.zeros(n, np.uint16)
    zds.zds_cpu_adam_step(zds.hparams(), g, P, M, V, out, sc, _host_state(t0), num_threads=threads,
                          grad_dtype=CODE[gdt], param_dtype=CODE[pdt])
    assert (P.view(np.uint32) == oP.view(np.uint32)).all()
    assert (M.view(np.uint32) == oM.view(np.uint32)).all()
    assert (V.view(np.uint32) == oV.view(np.uint32)).all()
    assert (out == o16).all()


def test_cpu_adam_overflow_skip_and_multi_step():
    n = 50000
    g = draw_grads(n, "fp16", 1e-3, 2.0 ** 12, 3, 97, 1)
    p = draw_master(n, 0.02, 3, 97)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    P, M, V = p.copy(), m.copy(), v.copy()
    skip = zds.StepScalars(overflow=1, grad_scale=1.0)
    zds.zds_cpu_adam_step(zds.hparams(), g, P, M, V, None, skip, _host_state(0), grad_dtype=zds.ZDS_FP16)
    assert (P == p).all() and (M == 0).all() and (V == 0).all()
    # five steps with the host scaler twin advancing the state, against the oracle
    hs = _host_state(0)
    ost = O.scaler_init(initial_scale_power=12)
    oP, oM, oV = p.copy(), m.copy(), v.copy()
    for k in range(5):
        gk = draw_grads(n, "fp16", 1e-3, ost.scale, 3, 97, k + 2)
        oP, oM, oV, o16, ost, osc = O.optimizer_step(gk, "fp16", oP, oM, oV, ost, O.AdamW(), 1.0, 1, "fp16")
        sc = zds.zds_clip_scalars_host(osc["sumsq"], hs.scale, 1, 1.0)
        out = np.zeros(n, np.uint16)
        zds.zds_cpu_adam_step(zds.hparams(), gk, P, M, V, out, sc, hs, grad_dtype=zds.ZDS_FP16,
                              param_dtype=zds.ZDS_FP16)
        zds.zds_loss_scaler_update_host(hs, sc.overflow, zds.hparams())
        assert (P.view(np.uint32) == oP.view(np.uint32)).all() and (out == o16).all()
        assert hs.t == ost.t


def test_cpu_adam_argument_errors():
    lib = zds.lib
    hp = zds.hparams()
    sc = zds.StepScalars()
    st = zds.StepState()
    import ctypes
    assert lib.zds_cpu_adam_step(None, None, 0, None, None, None, None, 0, 10, None, None, 0) == zds.ZDS_EINVAL
    assert lib.zds_cpu_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, 10, ctypes.byref(sc),
                                 ctypes.byref(st), -1) == zds.ZDS_EINVAL
    assert lib.zds_cpu_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, 10, ctypes.byref(sc),
                                 ctypes.byref(st), 0) == zds.ZDS_EINVAL
    assert lib.zds_cpu_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, 0, ctypes.byref(sc),
                                 ctypes.byref(st), 0) == zds.ZDS_OK
