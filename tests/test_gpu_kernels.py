"""GPU parity of each hot-path kernel against the CPU oracle, through the C ABI.

Sizes span several launch tiles plus ragged tails; edge cases: empty and
one-element inputs, misaligned (element-aligned only) buffers, non-finite
values at the head, tail and inside a vector group, all 16-bit bit patterns.
Bars: flags, skips and scale trajectories equal; fp32 master/m/v within 2 ulp;
16-bit params within 1 ulp; norm within 1e-6 relative."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from tests.util import (assert_p16_close, assert_state_close, to_dev, to_host)
from workloads import draw_grads, draw_master, draw_prior_moments

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from zero_sharded_mixed_tensor_amd import zds  # noqa: E402
from zero_sharded_mixed_tensor_amd.step import ShardStep  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# The AdamW kernel works in 1024-element tiles of two 512-element halves,
# the first n & ~7 elements, then n % 8 element-wise: sizes below cover a
# lone partial tile, whole tiles, and partial last tiles that end inside the
# first half, exactly at the halves' edge, and inside the second half.
SIZES = [1, 7, 8, 9, 255, 4099, 3 * 2048 + 5, 65536 * 3 + 13, (1 << 20) + 3,
         1024 + 523, 3 * 1024 + 512, 5 * 1024 + 709]


def _inputs(n, gdt, seed, scale=2.0 ** 12, sigma=1e-3, prior=True):
    g = draw_grads(n, gdt, sigma, scale, seed, 90, 1)
    p = draw_master(n, 0.02, seed, 90)
    if prior:
        m, v = draw_prior_moments(n, sigma, seed, 90)
    else:
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    return g, p, m, v


def _run_step(g, p, m, v, gdt, pdt, scale_pow, t0, max_norm, hp, offset=0, accum=1, dynamic=True, offset16=0):
    """One step on the GPU. offset > 0 places every buffer `offset` elements
    into a larger allocation (element-aligned, not 16-byte aligned); offset16
    does the same for the 16-bit buffers only (grads when 16-bit, params out)."""
    n = p.shape[0]
    og = offset + (offset16 if gdt != "fp32" else 0)
    oo = offset + offset16
    dg = to_dev(np.concatenate([np.zeros(og, g.dtype), g]), gdt)[og:]
    dp = to_dev(np.concatenate([np.zeros(offset, np.float32), p]), "fp32")[offset:]
    dm = to_dev(np.concatenate([np.zeros(offset, np.float32), m]), "fp32")[offset:]
    dv = to_dev(np.concatenate([np.zeros(offset, np.float32), v]), "fp32")[offset:]
    dout = to_dev(np.concatenate([np.zeros(oo, np.uint16), np.full(n, 0x7E00, np.uint16)]), pdt)[oo:]
    b1p = float(np.float32(hp.beta1)) ** t0
    b2p = float(np.float32(hp.beta2)) ** t0
    cfg = zds.scaler_config(dynamic=dynamic, initial_scale_power=scale_pow, window=1000, hysteresis=1,
                            static_scale=1.0)
    st = ShardStep(n, zds.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay), cfg,
                   max_norm=max_norm, accum_steps=accum, t0=t0, beta1_pow0=b1p, beta2_pow0=b2p)
    st.step(dg, dp, dm, dv, dout)
    torch.cuda.synchronize()
    return (to_host(dp), to_host(dm), to_host(dv), to_host(dout), st.read_scalars(), st.read_state(),
            (b1p, b2p))


def _oracle_step(g, p, m, v, gdt, pdt, scale, t0, pows, max_norm, hp, accum=1, dynamic=True):
    st = O.scaler_init(dynamic=dynamic, initial_scale_power=int(np.log2(scale)) if dynamic else 0,
                       window=1000, hysteresis=1, static_scale=1.0, t=t0, beta1_pow=pows[0],
                       beta2_pow=pows[1])
    return O.optimizer_step(g, gdt, p.copy(), m.copy(), v.copy(), st, hp, max_norm, accum, pdt)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("gdt,pdt", [("fp16", "fp16"), ("bf16", "bf16"), ("fp32", "fp16"), ("fp16", "bf16")])
def test_adam_step_parity(n, gdt, pdt):
    say("adam parity n=%d grads=%s params=%s" % (n, gdt, pdt))
    hp = O.AdamW()
    seed = n * 7 + len(gdt)
    g, p, m, v = _inputs(n, gdt, seed)
    t0 = 1 if n % 2 else 0
    if t0 == 0:
        m[:] = 0
        v[:] = 0
    max_norm = 1.0 if n % 3 else 0.0
    P, M, V, OUT, sc, st, pows = _run_step(g, p, m, v, gdt, pdt, 12, t0, max_norm, hp)
    oP, oM, oV, oOUT, ost, osc = _oracle_step(g, p, m, v, gdt, pdt, 2.0 ** 12, t0, pows, max_norm, hp)
    assert sc.overflow == osc["overflow"] == 0
    assert abs(sc.sumsq - osc["sumsq"]) <= 1e-12 * osc["sumsq"]
    assert abs(float(sc.norm) - float(osc["norm"])) <= 1e-6 * float(osc["norm"])
    assert sc.grad_scale == osc["grad_scale"], (sc.grad_scale, osc["grad_scale"])
    assert_state_close("master", P, oP, 2)
    assert_state_close("exp_avg", M, oM, 2)
    assert_state_close("exp_avg_sq", V, oV, 2)
    assert_p16_close("params_out", OUT, oOUT, 1)
    assert st.t == ost.t and st.beta1_pow == ost.beta1_pow and st.last_skip == 0


@pytest.mark.parametrize("n", [9, 4099, 3 * 1024 + 512, 65536 * 3 + 13])
@pytest.mark.parametrize("gdt,pdt", [("fp16", "fp16"), ("fp16", "bf16"), ("bf16", "fp16"), ("bf16", "bf16"),
                                     ("fp32", "fp16"), ("fp32", "bf16")])
def test_adam_step_bit_exact(n, gdt, pdt):
    """Every dtype pair: the kernel performs the oracle's fp32 operations in
    its order with correctly rounded divide and sqrt, so master/m/v and the
    16-bit params agree bit for bit (the stated bound elsewhere is 2 ulp /
    1 ulp; this is the stronger property the kernel has)."""
    say("adam bit-exact n=%d grads=%s params=%s" % (n, gdt, pdt))
    hp = O.AdamW()
    g, p, m, v = _inputs(n, gdt, 3 * n + len(gdt) + 7 * len(pdt))
    P, M, V, OUT, sc, st, pows = _run_step(g, p, m, v, gdt, pdt, 12, 2, 1.0, hp)
    oP, oM, oV, oOUT, ost, osc = _oracle_step(g, p, m, v, gdt, pdt, 2.0 ** 12, 2, pows, 1.0, hp)
    assert sc.grad_scale == osc["grad_scale"]
    for name, a, b in (("master", P, oP), ("exp_avg", M, oM), ("exp_avg_sq", V, oV)):
        assert (a.view(np.uint32) == b.view(np.uint32)).all(), (name, assert_state_close(name, a, b, 2))
    assert (OUT == oOUT).all(), assert_p16_close("params_out", OUT, oOUT, 1)


@pytest.mark.parametrize("n", [1, 9, 4099, 3 * 1024 + 512, 65536 * 3 + 13])
@pytest.mark.parametrize("gdt", ["fp16", "bf16", "fp32"])
def test_adam_step_without_params_out(n, gdt):
    """params_out NULL skips the cast (the kernel's no-output form):
    master/m/v bit for bit against the oracle's update."""
    say("adam without params_out n=%d grads=%s" % (n, gdt))
    hp = O.AdamW()
    g, p, m, v = _inputs(n, gdt, 11 * n + len(gdt))
    dg, dp, dm, dv = to_dev(g, gdt), to_dev(p, "fp32"), to_dev(m, "fp32"), to_dev(v, "fp32")
    b1p, b2p = float(np.float32(hp.beta1)), float(np.float32(hp.beta2))
    cfg = zds.scaler_config(dynamic=True, initial_scale_power=12, window=1000, hysteresis=1, static_scale=1.0)
    st = ShardStep(n, zds.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay), cfg,
                   max_norm=1.0, accum_steps=1, t0=1, beta1_pow0=b1p, beta2_pow0=b2p)
    st.step(dg, dp, dm, dv, None)
    torch.cuda.synchronize()
    oP, oM, oV, _, _, osc = _oracle_step(g, p, m, v, gdt, "bf16", 2.0 ** 12, 1, (b1p, b2p), 1.0, hp)
    assert st.read_scalars().grad_scale == osc["grad_scale"]
    for name, a, b in (("master", to_host(dp), oP), ("exp_avg", to_host(dm), oM), ("exp_avg_sq", to_host(dv), oV)):
        assert (a.view(np.uint32) == b.view(np.uint32)).all(), name
    assert st.read_state().t == 2


def test_empty_shard_step():
    """n = 0: the step launches and returns, the scalars are those of an
    empty sum (no overflow, norm 0, no clipping) and the scaler commits the
    step like the oracle's."""
    say("empty shard step")
    hp = O.AdamW()
    e32 = torch.empty(0, dtype=torch.float32, device="cuda")
    g = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    cfg = zds.scaler_config(dynamic=True, initial_scale_power=12, window=2, hysteresis=1, static_scale=1.0)
    st = ShardStep(0, zds.hparams(), cfg, max_norm=1.0, accum_steps=1, t0=0)
    ost = O.scaler_init(dynamic=True, initial_scale_power=12, window=2, hysteresis=1)
    for _ in range(3):
        st.step(g, e32, e32.clone(), e32.clone(), out)
        ost = O.optimizer_step(np.zeros(0, np.uint16), O.BF16, np.zeros(0, np.float32), np.zeros(0, np.float32),
                               np.zeros(0, np.float32), ost, hp, 1.0, 1, O.BF16)[4]
    torch.cuda.synchronize()
    sc, dst = st.read_scalars(), st.read_state()
    assert sc.overflow == 0 and sc.sumsq == 0.0 and float(sc.norm) == 0.0 and float(sc.clip_coef) == 1.0
    assert dst.t == ost.t == 3 and float(dst.scale) == ost.scale == 2.0 ** 13 and dst.good_steps == ost.good_steps
    assert dst.beta1_pow == ost.beta1_pow and dst.beta2_pow == ost.beta2_pow


@pytest.mark.parametrize("n", [1, 9, 4099, 65536 + 3])
@pytest.mark.parametrize("gdt", ["fp16", "bf16", "fp32"])
def test_adam_step_misaligned_buffers(n, gdt):
    say("adam misaligned n=%d grads=%s" % (n, gdt))
    hp = O.AdamW()
    g, p, m, v = _inputs(n, gdt, 31 + n)
    P, M, V, OUT, sc, st, pows = _run_step(g, p, m, v, gdt, "bf16", 12, 1, 1.0, hp, offset=1)
    oP, oM, oV, oOUT, ost, osc = _oracle_step(g, p, m, v, gdt, "bf16", 2.0 ** 12, 1, pows, 1.0, hp)
    assert sc.grad_scale == osc["grad_scale"]
    assert_state_close("master", P, oP, 2)
    assert_state_close("exp_avg", M, oM, 2)
    assert_state_close("exp_avg_sq", V, oV, 2)
    assert_p16_close("params_out", OUT, oOUT, 1)


@pytest.mark.parametrize("n", [1, 9, 4099, 512 * 37 + 13, 65536 + 3])
@pytest.mark.parametrize("gdt,pdt", [("fp16", "fp16"), ("bf16", "bf16"), ("fp32", "bf16")])
def test_adam_step_8_byte_aligned_16bit_buffers(n, gdt, pdt):
    """16-bit buffers 8- but not 16-byte aligned (fp32 arrays 16-byte aligned):
    the AdamW kernel's 8-byte form of its 16-bit accesses."""
    say("adam 16-bit buffers at 8-byte alignment n=%d grads=%s params=%s" % (n, gdt, pdt))
    hp = O.AdamW()
    g, p, m, v = _inputs(n, gdt, 57 + n)
    P, M, V, OUT, sc, st, pows = _run_step(g, p, m, v, gdt, pdt, 12, 1, 1.0, hp, offset16=4)
    oP, oM, oV, oOUT, ost, osc = _oracle_step(g, p, m, v, gdt, pdt, 2.0 ** 12, 1, pows, 1.0, hp)
    assert sc.grad_scale == osc["grad_scale"]
    assert_state_close("master", P, oP, 2)
    assert_state_close("exp_avg", M, oM, 2)
    assert_state_close("exp_avg_sq", V, oV, 2)
    assert_p16_close("params_out", OUT, oOUT, 1)


@pytest.mark.parametrize("where", ["head", "tail", "mid_group", "last_vector"])
@pytest.mark.parametrize("gdt,bad", [("fp16", np.inf), ("fp16", np.nan), ("bf16", -np.inf), ("fp32", np.nan)])
def test_overflow_skips_step(where, gdt, bad):
    say("overflow skip where=%s grads=%s value=%r" % (where, gdt, bad))
    n = 4096 * 5 + 3
    hp = O.AdamW()
    g, p, m, v = _inputs(n, gdt, 77)
    pos = {"head": 0, "tail": n - 1, "mid_group": 8 * 37 + 5, "last_vector": (n // 8) * 8 - 1}[where]
    if gdt == "fp32":
        g[pos] = bad
    elif gdt == "fp16":
        g[pos] = np.array([bad], np.float16).view(np.uint16)[0]
    else:
        g[pos] = (np.array([bad], np.float32).view(np.uint32)[0] >> 16)
    P, M, V, OUT, sc, st, _ = _run_step(g, p, m, v, gdt, "fp16", 14, 3, 1.0, hp)
    assert sc.overflow == 1
    assert (P.view(np.uint32) == p.view(np.uint32)).all()
    assert (M.view(np.uint32) == m.view(np.uint32)).all()
    assert (V.view(np.uint32) == v.view(np.uint32)).all()
    assert (OUT == 0x7E00).all()  # params untouched
    assert st.scale == 2.0 ** 13 and st.t == 3 and st.last_skip == 1 and st.steps_skipped == 1


def _norm(x_dev, n=None, accum=1, max_norm=1.0, scale_pow=0):
    n = x_dev.numel() if n is None else n
    st = ShardStep(max(n, 1), zds.hparams(), zds.scaler_config(initial_scale_power=scale_pow),
                   max_norm=max_norm, accum_steps=accum)
    st.n = n
    st.norm(x_dev)
    torch.cuda.synchronize()
    return st.read_scalars()


def test_norm_all_fp16_and_bf16_patterns():
    say("norm: all finite 16-bit patterns, then each non-finite pattern")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt, mask in (("fp16", 0x7C00), ("bf16", 0x7F80)):
        finite = bits[(bits & mask) != mask]
        sc = _norm(to_dev(finite, dt))
        want = O.sum_of_squares(finite, dt)
        assert sc.overflow == 0 and abs(sc.sumsq - want) <= 1e-13 * want
        bad = bits[(bits & mask) == mask]
        # each non-finite pattern alone inside a finite array, at a rotating position
        base = finite[:1000].copy()
        scal = []
        for i, b in enumerate(bad):
            x = base.copy()
            x[(i * 37) % 1000] = b
            st = ShardStep(1000, zds.hparams(), zds.scaler_config(initial_scale_power=0), max_norm=1.0)
            st.norm(to_dev(x, dt))
            scal.append(st)
        torch.cuda.synchronize()
        flags = [s.read_scalars().overflow for s in scal]
        assert flags == [1] * len(bad), dt


@pytest.mark.parametrize("n", [0, 1, 8, 1000, 2048 * 4 * 256 + 77, 3_000_001])
@pytest.mark.parametrize("dt", ["fp16", "bf16", "fp32"])
def test_norm_parity_and_determinism(n, dt):
    say("norm parity n=%d dtype=%s" % (n, dt))
    x = draw_grads(n, dt, 1e-3, 2.0 ** 10, 5, 91, 2) if n else np.zeros(0, np.uint16 if dt != "fp32" else np.float32)
    d = to_dev(x, dt) if n else torch.zeros(8, dtype=torch.float16 if dt != "fp32" else torch.float32, device="cuda")
    s1 = _norm(d, n=n, accum=4, max_norm=0.5, scale_pow=10)
    s2 = _norm(d, n=n, accum=4, max_norm=0.5, scale_pow=10)
    assert s1.sumsq == s2.sumsq and s1.grad_scale == s2.grad_scale  # run-to-run identical
    r = O.overflow_and_norm(x, dt, 2.0 ** 10, 4, 0.5)
    assert s1.overflow == 0
    if n == 0:
        assert s1.sumsq == 0.0 and s1.norm == 0.0 and s1.grad_scale == np.float32(1.0 / 4096)
        return
    assert abs(s1.sumsq - r["sumsq"]) <= 1e-12 * r["sumsq"]
    assert abs(float(s1.norm) - float(r["norm"])) <= 1e-6 * float(r["norm"])
    assert s1.grad_scale == r["grad_scale"]
    # misaligned start (element aligned): scalar path
    if n > 1:
        s3 = _norm(d[1:], n=n - 1, accum=4, max_norm=0.5, scale_pow=10)
        r3 = O.overflow_and_norm(x[1:], dt, 2.0 ** 10, 4, 0.5)
        assert abs(s3.sumsq - r3["sumsq"]) <= 1e-12 * r3["sumsq"]


def test_scaler_device_trajectories():
    say("scaler device trajectories")
    rng = np.random.default_rng(3)
    hp = zds.hparams()
    for W, H, dyn in ((1, 1, True), (2, 1, True), (3, 2, True), (1000, 1, True), (5, 3, True), (1, 1, False)):
        cfg = zds.scaler_config(dynamic=dyn, initial_scale_power=6, window=W, hysteresis=H,
                                min_scale=1.0, static_scale=1.0)
        state = zds.new_state()
        zds.zds_step_state_init(state, cfg)
        o = O.scaler_init(dynamic=dyn, initial_scale_power=6, window=W, hysteresis=H, min_scale=1.0,
                          static_scale=1.0)
        flags = (rng.random(60) < 0.35).astype(int)
        sc_bufs = []
        for f in flags:
            sc = zds.new_scalars()
            zds.write_scalars(sc, zds.StepScalars(overflow=int(f)))
            sc_bufs.append(sc)
        traj = []
        for sc in sc_bufs:
            zds.zds_loss_scaler_update(state, sc, hp)
            traj.append(state.clone())
        torch.cuda.synchronize()
        for f, s in zip(flags, traj):
            o = O.scaler_update(o, int(f), 0.9, 0.999)
            g = zds.read_state(s)
            assert (g.scale, g.good_steps, g.hyst_left, g.t, g.last_skip) == \
                (np.float32(o.scale), o.good_steps, o.hyst_left, o.t, o.last_skip), (W, H, dyn)
            assert g.beta1_pow == o.beta1_pow and g.beta2_pow == o.beta2_pow


def _make_table(rng, T, dtype, misalign=False):
    """misalign: every third source starts 1 element (True) or `misalign`
    elements (an int: 4 gives 8-byte but not 16-byte aligned 16-bit
    sources) past an aligned address."""
    numels = [int(x) for x in rng.integers(1, 40000, T)]
    numels[0] = 5  # a tiny tensor
    if T > 2:
        numels[1] = 16384 * 2 + 1  # crosses chunk edges with a ragged end
    srcs_np, srcs_dev = [], []
    for i, n in enumerate(numels):
        a = draw_grads(n, dtype, 1e-3, 2.0 ** 12, 9, 92, i)
        srcs_np.append(a)
        if misalign and i % 3 == 1:
            k = 1 if misalign is True else int(misalign)
            d = to_dev(np.concatenate([a[:k], a]), dtype)[k:]
        else:
            d = to_dev(a, dtype)
        srcs_dev.append(d)
    return numels, srcs_np, srcs_dev


@pytest.mark.parametrize("T,align,world,misalign", [(1, 64, 1, False), (7, 64, 3, False), (33, 8, 4, True),
                                                    (100, 64, 8, False), (300, 1, 5, True), (40, 64, 4, 4)])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_accumulate_parity(T, align, world, misalign, dtype):
    say("accumulate T=%d align=%d world=%d misalign=%s dtype=%s" % (T, align, world, misalign, dtype))
    rng = np.random.default_rng(T * 13 + align)
    numels, srcs_np, srcs_dev = _make_table(rng, T, dtype, misalign)
    _, total = O.flat_layout(numels, align)
    for rank in sorted({0, world - 1, world // 2}):
        lo, hi = O.shard_range(total, world, rank, align)
        ent = O.shard_entries(numels, align, lo, hi)
        plan = zds.zds_plan_create(numels, align, lo, hi)
        assert plan.entries() == ent
        L = hi - lo
        # copy mode into a 16-bit bucket (padding left at its sentinel)
        bucket = to_dev(np.full(L, 0x1234, np.uint16), dtype)
        zds.zds_grad_accumulate(plan, srcs_dev, bucket, zds.ZDS_COPY)
        want = O.flatten_copy(srcs_np, ent, np.full(L, 0x1234, np.uint16))
        # overwrite then two accumulates into fp32
        acc = to_dev(np.full(L, 7.0, np.float32), "fp32")
        zds.zds_grad_accumulate(plan, srcs_dev, acc, zds.ZDS_OVERWRITE)
        zds.zds_grad_accumulate(plan, srcs_dev, acc, zds.ZDS_ACCUMULATE)
        zds.zds_grad_accumulate(plan, srcs_dev, acc, zds.ZDS_ACCUMULATE)
        torch.cuda.synchronize()
        wacc = np.full(L, 7.0, np.float32)
        O.flatten_accumulate(srcs_np, dtype, ent, wacc, overwrite=True)
        O.flatten_accumulate(srcs_np, dtype, ent, wacc, overwrite=False)
        O.flatten_accumulate(srcs_np, dtype, ent, wacc, overwrite=False)
        assert (to_host(bucket) == want).all()
        assert (to_host(acc).view(np.uint32) == wacc.view(np.uint32)).all()
        plan.close()


def test_accumulate_many_calls_reuse_staging():
    """More calls than staging slots, with different source sets per call."""
    say("accumulate: 20 calls over 4 source sets")
    rng = np.random.default_rng(44)
    sets = [_make_table(np.random.default_rng(s), 12, "fp16") for s in range(4)]
    numels = sets[0][0]
    sets = [(numels, [draw_grads(n, "fp16", 1e-3, 64.0, 9, 93 + s, i) for i, n in enumerate(numels)])
            for s in range(4)]
    devs = [[to_dev(a, "fp16") for a in st[1]] for st in sets]
    _, total = O.flat_layout(numels, 64)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    ent = O.shard_entries(numels, 64, 0, total)
    acc = torch.zeros(total, dtype=torch.float32, device="cuda")
    wacc = np.zeros(total, np.float32)
    order = rng.integers(0, 4, 20)
    for k, s in enumerate(order):
        zds.zds_grad_accumulate(plan, devs[s], acc, zds.ZDS_OVERWRITE if k == 0 else zds.ZDS_ACCUMULATE)
        O.flatten_accumulate(sets[s][1], "fp16", ent, wacc, overwrite=(k == 0))
    torch.cuda.synchronize()
    assert (to_host(acc).view(np.uint32) == wacc.view(np.uint32)).all()


def test_binding_refuses_short_buffers_before_launch():
    """A source shorter than its plan entries, or a dst shorter than the
    plan's range, is refused by the binding; the plan stays usable and the
    next full-length call matches the oracle."""
    say("binding: short source and dst refused with a real plan")
    numels = [1000, 77, 4096]
    _, total = O.flat_layout(numels, 64)
    lo, hi = O.shard_range(total, 2, 1, 64)
    plan = zds.zds_plan_create(numels, 64, lo, hi)
    ent = O.shard_entries(numels, 64, lo, hi)
    host = [draw_grads(n, "bf16", 1e-3, 1.0, 3, 5, i) for i, n in enumerate(numels)]
    devs = [to_dev(a, "bf16") for a in host]
    dst = torch.zeros(hi - lo, dtype=torch.bfloat16, device="cuda")
    t_last = ent[-1][0]
    short = list(devs)
    short[t_last] = devs[t_last][:-1]
    with pytest.raises(zds.ZdsError, match="source %d holds" % t_last):
        zds.zds_grad_accumulate(plan, short, dst, zds.ZDS_COPY)
    with pytest.raises(zds.ZdsError, match="dst holds"):
        zds.zds_grad_accumulate(plan, devs, dst[:-1], zds.ZDS_COPY)
    zds.zds_grad_accumulate(plan, devs, dst, zds.ZDS_COPY)
    want = np.zeros(hi - lo, np.uint16)
    O.flatten_copy(host, ent, want)
    torch.cuda.synchronize()
    assert (to_host(dst).view(np.uint16) == want).all()
    plan.close()


def test_accumulate_reused_upload_on_another_stream():
    """A call that reuses the previous call's pointer upload on another stream
    must not run before that upload: stream A is kept busy, the call on A
    uploads the pointers, the next call (same pointers, its own destination,
    no data dependency) runs on stream B."""
    say("accumulate: reused pointer upload across streams")
    numels, srcs_np, srcs = _make_table(np.random.default_rng(46), 9, "bf16")
    _, total = O.flat_layout(numels, 64)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    ent = O.shard_entries(numels, 64, 0, total)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    busy = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    outs = [torch.full((total,), 3.0, dtype=torch.float32, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    for k in range(4):
        with torch.cuda.stream(a):
            for _ in range(20):
                busy.mul_(1.0)
            zds.zds_grad_accumulate(plan, srcs, outs[2 * k], zds.ZDS_OVERWRITE)
        with torch.cuda.stream(b):
            zds.zds_grad_accumulate(plan, srcs, outs[2 * k + 1], zds.ZDS_OVERWRITE)
    torch.cuda.synchronize()
    want = np.full(total, 3.0, np.float32)
    O.flatten_accumulate(srcs_np, "bf16", ent, want, overwrite=True)
    for o in outs:
        assert (to_host(o).view(np.uint32) == want.view(np.uint32)).all()
    plan.close()


def test_sharded_updates_concatenate_to_unsharded():
    """Stage-1 invariant on the GPU: N shard updates with the global scalars
    equal the unsharded update bit for bit."""
    say("stage-1 concat invariant on GPU")
    n = 8 * 4096 * 3 + 40  # divisible by 8 * 64 after padding below
    hp = O.AdamW()
    g, p, m, v = _inputs(n, "fp16", 55)
    full = _run_step(g, p, m, v, "fp16", "fp16", 12, 1, 1.0, hp)
    for N in (2, 3, 8):
        padded = O.align_up(n, N * 64)
        gp = np.concatenate([g, np.zeros(padded - n, np.uint16)])
        pp = np.concatenate([p, np.zeros(padded - n, np.float32)])
        mp = np.concatenate([m, np.zeros(padded - n, np.float32)])
        vp = np.concatenate([v, np.zeros(padded - n, np.float32)])
        dg, dp, dm, dv = to_dev(gp, "fp16"), to_dev(pp, "fp32"), to_dev(mp, "fp32"), to_dev(vp, "fp32")
        out = torch.zeros(padded, dtype=torch.float16, device="cuda")
        # global scalars from the whole buffer, then one adam launch per shard
        st = ShardStep(padded, zds.hparams(), zds.scaler_config(initial_scale_power=12), max_norm=1.0,
                       t0=1, beta1_pow0=full[6][0], beta2_pow0=full[6][1])
        st.norm(dg)
        for r in range(N):
            lo, hi = O.shard_range(n, N, r, 64)
            zds.zds_adam_step(st.hp, dg[lo:hi], dp[lo:hi], dm[lo:hi], dv[lo:hi], out[lo:hi], st.scalars,
                              st.state)
        torch.cuda.synchronize()
        assert (to_host(dp)[:n].view(np.uint32) == full[0].view(np.uint32)).all()
        assert (to_host(dm)[:n].view(np.uint32) == full[1].view(np.uint32)).all()
        assert (to_host(dv)[:n].view(np.uint32) == full[2].view(np.uint32)).all()
        assert (to_host(out)[:n] == full[3]).all()
        assert (to_host(dp)[n:] == 0).all()


def test_cast_all_fp32_exponents():
    """With lr = 0 and zero grads the master passes through unchanged, so the
    16-bit output is exactly the cast: check it on a sweep of fp32 patterns
    covering every exponent, ties and overflow."""
    say("cast sweep through the adam kernel")
    rng = np.random.default_rng(8)
    his = np.arange(0, 65536, dtype=np.uint32)
    his = his[(his & 0x7F80) != 0x7F80]  # finite only
    los = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1000, 0x2000], np.uint32)
    pats = ((his[:, None] << 16) | los[None, :]).reshape(-1)
    pats = np.concatenate([pats, rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)])
    p = pats.view(np.float32)
    p = p[np.isfinite(p)].copy()
    n = p.shape[0]
    hp = O.AdamW(lr=0.0, weight_decay=0.0)
    z16 = np.zeros(n, np.uint16)
    zf = np.zeros(n, np.float32)
    for pdt in ("bf16", "fp16"):
        P, M, V, OUT, sc, st, pows = _run_step(z16, p, zf, zf, "fp16", pdt, 0, 0, 0.0, hp)
        assert (P.view(np.uint32) == p.view(np.uint32)).all()
        want = O.narrow(p, pdt)
        assert (OUT == want).all(), pdt


@pytest.mark.parametrize("mode", ["copy", "overwrite", "accumulate"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("T,align,world,misalign", [(7, 64, 3, False), (33, 8, 4, True), (200, 64, 8, False)])
def test_accumulate_norm_fused_parity(mode, dtype, T, align, world, misalign):
    """zds_grad_accumulate_norm: the stored values equal the oracle's
    flatten/accumulate, and the scalars equal the oracle's overflow and norm
    of that flat buffer (padding zero)."""
    say("fused accumulate+norm mode=%s dtype=%s T=%d" % (mode, dtype, T))
    rng = np.random.default_rng(T * 7 + align + world)
    numels, srcs_np, srcs_dev = _make_table(rng, T, dtype, misalign)
    _, total = O.flat_layout(numels, align)
    for rank in sorted({0, world - 1}):
        lo, hi = O.shard_range(total, world, rank, align)
        ent = O.shard_entries(numels, align, lo, hi)
        L = hi - lo
        plan = zds.zds_plan_create(numels, align, lo, hi)
        st = ShardStep(max(L, 1), zds.hparams(), zds.scaler_config(initial_scale_power=12), max_norm=1.0,
                       accum_steps=2)
        ws = zds.new_plan_workspace(plan)
        if mode == "copy":
            dst = to_dev(np.zeros(L, np.uint16), dtype)
            zds.zds_grad_accumulate_norm(plan, srcs_dev, dst, zds.ZDS_COPY, 2, 1.0, st.state, st.scalars, ws)
            want = O.flatten_copy(srcs_np, ent, np.zeros(L, np.uint16))
            wdt = dtype
        else:
            dst = torch.zeros(L, dtype=torch.float32, device="cuda")
            want = np.zeros(L, np.float32)
            if mode == "accumulate":
                zds.zds_grad_accumulate(plan, srcs_dev, dst, zds.ZDS_OVERWRITE)
                O.flatten_accumulate(srcs_np, dtype, ent, want, overwrite=True)
            m = zds.ZDS_OVERWRITE if mode == "overwrite" else zds.ZDS_ACCUMULATE
            zds.zds_grad_accumulate_norm(plan, srcs_dev, dst, m, 2, 1.0, st.state, st.scalars, ws)
            O.flatten_accumulate(srcs_np, dtype, ent, want, overwrite=(mode == "overwrite"))
            wdt = "fp32"
        torch.cuda.synchronize()
        got = to_host(dst)
        assert (got.view(np.uint32 if wdt == "fp32" else np.uint16) ==
                want.view(np.uint32 if wdt == "fp32" else np.uint16)).all()
        sc = st.read_scalars()
        r = O.overflow_and_norm(want, wdt, 2.0 ** 12, 2, 1.0)
        assert sc.overflow == r["overflow"] == 0
        if L:
            assert abs(sc.sumsq - r["sumsq"]) <= 1e-12 * max(r["sumsq"], 1e-300)
            assert sc.grad_scale == r["grad_scale"]
        plan.close()


@pytest.mark.parametrize("bad", [np.inf, np.nan])
def test_accumulate_norm_fused_overflow(bad):
    say("fused accumulate+norm overflow %r" % bad)
    rng = np.random.default_rng(5)
    numels, srcs_np, srcs_dev = _make_table(rng, 9, "fp16")
    t = 4
    srcs_np[t][numels[t] // 2] = np.array([bad], np.float16).view(np.uint16)[0]
    srcs_dev[t] = to_dev(srcs_np[t], "fp16")
    _, total = O.flat_layout(numels, 64)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    st = ShardStep(total, zds.hparams(), zds.scaler_config(initial_scale_power=12), max_norm=1.0)
    ws = zds.new_plan_workspace(plan)
    dst = torch.zeros(total, dtype=torch.float16, device="cuda")
    zds.zds_grad_accumulate_norm(plan, srcs_dev, dst, zds.ZDS_COPY, 1, 1.0, st.state, st.scalars, ws)
    torch.cuda.synchronize()
    assert st.read_scalars().overflow == 1
    # an empty range (all padding) still writes the scalars of an empty shard
    plan0 = zds.zds_plan_create([5], 64, 32, 64)
    assert plan0.num_entries == 0
    st0 = ShardStep(32, zds.hparams(), zds.scaler_config(initial_scale_power=0), max_norm=1.0)
    zds.zds_grad_accumulate_norm(plan0, [srcs_dev[0]], torch.zeros(32, dtype=torch.float16, device="cuda"),
                                 zds.ZDS_COPY, 1, 1.0, st0.state, st0.scalars, zds.new_plan_workspace(plan0))
    torch.cuda.synchronize()
    s0 = st0.read_scalars()
    assert s0.overflow == 0 and s0.sumsq == 0.0 and s0.grad_scale == 1.0


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 11, 12, 16])
@pytest.mark.parametrize("sdt,ddt", [("bf16", "fp32"), ("fp16", "fp32"), ("bf16", "bf16"), ("fp16", "fp16")])
def test_reduce_peer_slices_parity(N, sdt, ddt):
    say("reduce peers N=%d %s -> %s" % (N, sdt, ddt))
    for n, offset in ((1, 0), (7, 0), (513, 0), (512 * 37 + 13, 0), (100003, 0), (4099, 1)):
        peers = [draw_grads(n, sdt, 1e-2, 1.0, 40 + k, 94, n) for k in range(N)]
        dpeers = [to_dev(np.concatenate([np.zeros(offset, np.uint16), p]), sdt)[offset:] for p in peers]
        for acc in (False, True):
            if ddt == "fp32":
                base = draw_master(n, 0.5, 7, 95)
                dst = to_dev(np.concatenate([np.zeros(offset, np.float32), base]), "fp32")[offset:]
            else:
                base = draw_grads(n, ddt, 0.5, 1.0, 8, 95, 0)
                dst = to_dev(np.concatenate([np.zeros(offset, np.uint16), base]), ddt)[offset:]
            zds.zds_reduce_peer_slices(dpeers, dst, zds.ZDS_ACCUMULATE if acc else zds.ZDS_OVERWRITE)
            torch.cuda.synchronize()
            want = O.reduce_peer_slices(peers, sdt, base.copy(), ddt, accumulate=acc)
            got = to_host(dst)
            if ddt == "fp32":
                assert (got.view(np.uint32) == want.view(np.uint32)).all(), (n, acc)
            else:
                assert (got == want).all(), (n, acc)


@pytest.mark.parametrize("N", [1, 3, 8, 11, 16])
@pytest.mark.parametrize("sdt,ddt", [("bf16", "fp32"), ("fp16", "fp32"), ("bf16", "bf16"), ("fp16", "fp16")])
def test_reduce_peer_slices_norm_parity(N, sdt, ddt):
    """zds_reduce_peer_slices_norm: the stored values equal the oracle's
    intake, and the scalars equal the oracle's overflow and norm of them."""
    say("reduce peers + norm N=%d %s -> %s" % (N, sdt, ddt))
    for n, offset in ((0, 0), (1, 0), (7, 0), (513, 0), (512 * 37 + 13, 0), (1024 * 2049 + 5, 0), (4099, 1)):
        peers = [draw_grads(n, sdt, 1e-2, 1.0, 60 + k, 96, n) for k in range(N)]
        dpeers = [to_dev(np.concatenate([np.zeros(offset, np.uint16), p]), sdt)[offset:] for p in peers]
        for acc in (False, True):
            if ddt == "fp32":
                base = draw_master(n, 0.5, 9, 97)
                dst = to_dev(np.concatenate([np.zeros(offset, np.float32), base]), "fp32")[offset:]
            else:
                base = draw_grads(n, ddt, 0.5, 1.0, 10, 97, 0)
                dst = to_dev(np.concatenate([np.zeros(offset, np.uint16), base]), ddt)[offset:]
            st = ShardStep(max(n, 1), zds.hparams(), zds.scaler_config(initial_scale_power=3), max_norm=1.0,
                           accum_steps=N)
            ws = zds.new_reduce_workspace(n)
            zds.zds_reduce_peer_slices_norm(dpeers, dst, zds.ZDS_ACCUMULATE if acc else zds.ZDS_OVERWRITE, N, 1.0,
                                            st.state, st.scalars, ws)
            torch.cuda.synchronize()
            want = O.reduce_peer_slices(peers, sdt, base.copy(), ddt, accumulate=acc)
            got = to_host(dst)
            if ddt == "fp32":
                assert (got.view(np.uint32) == want.view(np.uint32)).all(), (n, acc)
            else:
                assert (got == want).all(), (n, acc)
            sc = st.read_scalars()
            r = O.overflow_and_norm(want, ddt, 2.0 ** 3, N, 1.0)
            assert sc.overflow == r["overflow"] == 0, (n, acc)
            assert abs(sc.sumsq - r["sumsq"]) <= 1e-12 * max(r["sumsq"], 1e-300), (n, acc)
            assert sc.grad_scale == r["grad_scale"], (n, acc)
            if n == 0:
                assert sc.sumsq == 0.0 and sc.grad_scale == np.float32(1.0 / (8.0 * N))


@pytest.mark.parametrize("ddt", ["fp32", "bf16"])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_reduce_peer_slices_norm_overflow(ddt, bad):
    """A non-finite element in one peer's slice sets the overflow flag."""
    say("reduce peers + norm overflow %s %r" % (ddt, bad))
    n, N = 512 * 300 + 3, 4
    peers = [draw_grads(n, "bf16", 1e-2, 1.0, 70 + k, 98, 0) for k in range(N)]
    for where in (0, n // 2, n - 1):
        ps = [p.copy() for p in peers]
        ps[2][where] = (np.array([bad], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
        dst = torch.zeros(n, dtype=torch.float32 if ddt == "fp32" else torch.bfloat16, device="cuda")
        st = ShardStep(n, zds.hparams(), zds.scaler_config(initial_scale_power=3), max_norm=1.0, accum_steps=N)
        zds.zds_reduce_peer_slices_norm([to_dev(p, "bf16") for p in ps], dst, zds.ZDS_OVERWRITE, N, 1.0, st.state,
                                        st.scalars, zds.new_reduce_workspace(n))
        torch.cuda.synchronize()
        want = O.reduce_peer_slices(ps, "bf16", np.zeros(n, np.float32 if ddt == "fp32" else np.uint16), ddt,
                                    accumulate=False)
        assert O.overflow_and_norm(want, ddt, 8.0, N, 1.0)["overflow"] == 1
        assert st.read_scalars().overflow == 1, where


def test_accumulate_with_bound_source_set():
    """A SourceSet (pointers marshalled once) gives the same result as the
    list, call after call, and is refused for a plan of another size."""
    say("accumulate: bound source set")
    numels, srcs_np, srcs = _make_table(np.random.default_rng(47), 12, "fp16")
    _, total = O.flat_layout(numels, 64)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    ent = O.shard_entries(numels, 64, 0, total)
    bound = zds.SourceSet(plan, srcs)
    acc = torch.zeros(total, dtype=torch.float32, device="cuda")
    want = np.zeros(total, np.float32)
    for k in range(3):
        zds.zds_grad_accumulate(plan, bound, acc, zds.ZDS_OVERWRITE if k == 0 else zds.ZDS_ACCUMULATE)
        O.flatten_accumulate(srcs_np, "fp16", ent, want, overwrite=(k == 0))
    torch.cuda.synchronize()
    assert (to_host(acc).view(np.uint32) == want.view(np.uint32)).all()
    other = zds.zds_plan_create(numels[:-1], 64, 0, O.flat_layout(numels[:-1], 64)[1])
    with pytest.raises(zds.ZdsError):
        zds.zds_grad_accumulate(other, bound, acc, zds.ZDS_OVERWRITE)
    other.close()
    plan.close()
