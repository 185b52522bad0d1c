"""CPU checks of the C-ABI library: it loads, exports every function the
header declares, and its host-side logic (geometry, scaler twin, step
constants, clip arithmetic, argument checks) agrees with the oracle. No
kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from workloads import llama_7b_tensors, llama_65b_tensors, tiny_shard_sizes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
zds = pytest.importorskip("zero_sharded_mixed_tensor_amd.zds", reason="libzds.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "zds.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zds_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 20
    lib = ctypes.CDLL(zds.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(zds._SIGS), set(names) ^ set(zds._SIGS)
    assert zds.zds_abi_version() == 3


def test_struct_layouts():
    assert ctypes.sizeof(zds.StepState) == 64
    assert zds.StepState.t.offset == 32 and zds.StepState.beta1_pow.offset == 40
    assert ctypes.sizeof(zds.StepScalars) == 64 and zds.StepScalars.sumsq.offset == 8
    assert zds.StepScalars.inv_bc2_sqrt.offset == 32 and zds.StepScalars.step_size.offset == 40
    assert zds.StepScalars.eps.offset == 60


@pytest.mark.parametrize("seed", range(20))
def test_geometry_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    numels = [int(x) for x in rng.integers(0, 5000, int(rng.integers(1, 40)))]
    align = int(rng.choice([1, 2, 8, 64, 256]))
    offs, total = zds.zds_flat_layout(numels, align)
    o_offs, o_total = O.flat_layout(numels, align)
    assert offs == o_offs and total == o_total
    world = int(rng.integers(1, 9))
    for r in range(world):
        lo, hi = zds.zds_shard_range(total, world, r, align)
        assert (lo, hi) == O.shard_range(total, world, r, align)
        assert zds.zds_shard_entries(numels, align, lo, hi) == O.shard_entries(numels, align, lo, hi)
    # arbitrary ranges too
    for _ in range(5):
        a, b = sorted(int(x) for x in rng.integers(0, total + 1, 2))
        assert zds.zds_shard_entries(numels, align, a, b) == O.shard_entries(numels, align, a, b)


def test_geometry_workloads():
    for tensors, world in ((llama_7b_tensors(), 8), (llama_65b_tensors(), 8), (tiny_shard_sizes(), 3)):
        numels = [n for _, n in tensors]
        _, total = zds.zds_flat_layout(numels, 64)
        for r in (0, world - 1):
            lo, hi = zds.zds_shard_range(total, world, r, 64)
            assert zds.zds_shard_entries(numels, 64, lo, hi) == O.shard_entries(numels, 64, lo, hi)


def _state_eq(s, o):
    assert s.scale == np.float32(o.scale)
    assert (s.good_steps, s.hyst_left, s.t, s.last_skip) == (o.good_steps, o.hyst_left, o.t, o.last_skip)
    assert s.beta1_pow == o.beta1_pow and s.beta2_pow == o.beta2_pow


@pytest.mark.parametrize("seed", range(10))
def test_scaler_host_twin_matches_oracle(seed):
    rng = np.random.default_rng(200 + seed)
    W = int(rng.integers(1, 5))
    H = int(rng.integers(1, 4))
    dyn = bool(seed % 5)
    p = int(rng.integers(0, 20))
    cfg = zds.scaler_config(dynamic=dyn, initial_scale_power=p, window=W, hysteresis=H,
                            min_scale=float(2.0 ** int(rng.integers(0, 3))), static_scale=1.0)
    hp = zds.hparams()
    s = zds.zds_step_state_init_host(cfg)
    o = O.scaler_init(dynamic=dyn, initial_scale_power=p, window=W, hysteresis=H,
                      min_scale=cfg.min_scale, static_scale=1.0)
    _state_eq(s, o)
    for f in rng.random(200) < 0.3:
        zds.zds_loss_scaler_update_host(s, int(f), hp)
        o = O.scaler_update(o, int(f), 0.9, 0.999)
        _state_eq(s, o)


def test_adam_constants_host_match_oracle():
    for hpv in (dict(), dict(lr=2e-5, weight_decay=0.0), dict(lr=0.1, beta1=0.5, beta2=0.95, eps=1e-6,
                                                               weight_decay=0.1)):
        hp = zds.hparams(**hpv)
        ohp = O.AdamW(**hpv)
        cfg = zds.scaler_config()
        s = zds.zds_step_state_init_host(cfg)
        o = O.scaler_init()
        for t in range(3000):
            c = zds.zds_adam_constants_host(hp, s)
            oc = O.adamw_constants(ohp, o.beta1_pow, o.beta2_pow)
            for k in ("step_size", "bc2_sqrt", "decay", "omb1", "omb2"):
                assert np.float32(c[k]) == oc[k], (t, k)
            zds.zds_loss_scaler_update_host(s, 0, hp)
            o = O.scaler_update(o, 0, ohp.beta1, ohp.beta2)


def test_clip_scalars_host_match_oracle():
    rng = np.random.default_rng(7)
    for _ in range(2000):
        sumsq = float(10.0 ** rng.uniform(-12, 20))
        S = float(2.0 ** int(rng.integers(0, 24)))
        K = int(rng.integers(1, 33))
        mx = float(np.float32(rng.choice([0.0, 1.0, 0.5, 3.0])))
        s = zds.zds_clip_scalars_host(sumsq, S, K, mx)
        norm, coef, gs = O.clip_scalars(sumsq, S, K, mx)
        assert s.overflow == 0
        assert s.grad_scale == gs and s.norm == np.float32(norm) and s.clip_coef == np.float32(coef)
    for bad in (float("inf"), float("nan")):
        s = zds.zds_clip_scalars_host(bad, 1.0, 1, 1.0)
        assert s.overflow == 1 and s.grad_scale == 0.0


def test_argument_errors():
    lib = zds.lib
    hp = zds.hparams()
    assert lib.zds_adam_step(None, None, 0, None, None, None, None, 0, 10, None, None, None) == zds.ZDS_EINVAL
    assert "hparams" in zds.zds_last_error()
    # bad dtype, negative n, betas out of range: rejected before any launch
    assert lib.zds_adam_step(ctypes.byref(hp), None, 7, None, None, None, None, 0, 10, None, None, None) == zds.ZDS_EINVAL
    assert lib.zds_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, -1, None, None, None) == zds.ZDS_EINVAL
    # n at or past 2^40 (the kernels' tile indices are 32-bit)
    assert lib.zds_adam_step(ctypes.byref(hp), 16, 0, 32, 48, 64, None, 0, 1 << 40, 128, 192, None) == zds.ZDS_EINVAL
    assert "2^40" in zds.zds_last_error()
    bad = zds.hparams(beta1=1.0)
    assert lib.zds_adam_step(ctypes.byref(bad), None, 0, None, None, None, None, 0, 10, None, None, None) == zds.ZDS_EINVAL
    # zero length is a no-op
    assert lib.zds_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, 0, None, None, None) == zds.ZDS_OK
    # null pointers with n > 0
    assert lib.zds_adam_step(ctypes.byref(hp), None, 0, None, None, None, None, 0, 8, None, None, None) == zds.ZDS_EINVAL
    # misaligned fp32 pointer
    assert lib.zds_adam_step(ctypes.byref(hp), 16, 0, 18, 32, 48, None, 0, 8, 64, 128, None) == zds.ZDS_EALIGN
    assert lib.zds_overflow_and_norm(None, 0, 10, 0, 1.0, 64, 128, 256, 4096, None) == zds.ZDS_EINVAL
    assert lib.zds_overflow_and_norm(None, 0, 10, 1, 1.0, 64, 128, 256, 0, None) == zds.ZDS_EINVAL
    assert lib.zds_overflow_and_norm(3, 0, 10, 1, 1.0, 64, 128, 256, 4096, None) == zds.ZDS_EALIGN
    cfg = zds.scaler_config(window=0)
    assert lib.zds_step_state_init_host(ctypes.byref(zds.StepState()), ctypes.byref(cfg), 0, 1.0, 1.0) == zds.ZDS_EINVAL
    assert lib.zds_grad_accumulate(None, None, 0, None, 0, 0, None) == zds.ZDS_EINVAL
    with pytest.raises(zds.ZdsError):
        zds.zds_shard_range(100, 0, 0, 8)
    with pytest.raises(zds.ZdsError):
        zds.zds_flat_layout([10, -1], 8)
    assert zds.lib.zds_workspace_bytes(0) >= 8
    # one float64 partial per 2048-element unit (plus their fold levels), so
    # about 0.4 % of the bytes of n fp32 grads, constant past the grid cap
    for n in (1, 2047, 2048, 2049, 842301440, 1 << 33):
        units = -(-n // 2048)
        assert units * 8 <= zds.lib.zds_workspace_bytes(n) <= units * 8 * 1.001 + 64, n
    assert zds.lib.zds_workspace_bytes(1 << 35) == zds.lib.zds_workspace_bytes(1 << 36)


def test_reciprocal_product_gives_the_correctly_rounded_quotient():
    """The AdamW kernels divide sqrt(v) by the per-step fp32 constant
    bc2 = sqrt(1 - beta2^t) as fp32(float64(a) * (1 / float64(bc2))); the
    claim is that this is the IEEE fp32 quotient for every a. Checked here for
    every fp32 significand in one binade and a million random a over all
    exponents a square root can have, against numpy's IEEE fp32 division, for
    bc2 of the first 8 steps of two beta2 values (the step constants the
    library derives) and random values in (0, 1]."""
    rng = np.random.default_rng(11)
    bs = []
    for b2 in (0.999, 0.95):
        hp = zds.hparams(beta2=b2)
        s = zds.zds_step_state_init_host(zds.scaler_config())
        for _ in range(8):
            bs.append(np.float32(zds.zds_adam_constants_host(hp, s)["bc2_sqrt"]))
            zds.zds_loss_scaler_update_host(s, 0, hp)
    bs += [np.float32(x) for x in rng.uniform(1e-3, 1.0, 8)]
    binade = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32)
    # sqrt(v) of an fp32 v: 0 or at least 2^-74.5, below 2^64
    rnd = np.sqrt(rng.uniform(0, 1, 1 << 20).astype(np.float32) *
                  np.exp2(rng.integers(-149, 128, 1 << 20)).astype(np.float32)).astype(np.float32)
    edge = np.array([0.0, np.sqrt(np.float32(1.4e-45)), 1.0, np.inf, np.nan], np.float32)
    for b in bs:
        r = 1.0 / np.float64(b)
        for a in (binade, rnd, edge):
            got = (a.astype(np.float64) * r).astype(np.float32)
            want = a / b
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)) or \
                np.array_equal(got, want, equal_nan=True), float(b)
