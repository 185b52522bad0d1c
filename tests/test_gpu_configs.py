"""Whole-step GPU runs of the workload shapes against the free-running oracle:
the tiny 64-tensor shard over 5 steps with an overflow at step 3, gradient
accumulation over 16 micro-batches, a 1,024-tensor table over 20 steps with a
seeded overflow schedule, and a bf16 Stage-1 shard with prior moments. The
large shapes run at reduced size here; full-size runs are in
test_gpu_fullsize.py."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from tests.util import assert_p16_close, assert_state_close, to_dev, to_host
from workloads import draw_grads, draw_master, draw_prior_moments, tiny_shard_sizes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from zero_sharded_mixed_tensor_amd import zds  # noqa: E402
from zero_sharded_mixed_tensor_amd.step import ShardStep  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _flat_master(numels, align, seed, cfg):
    offs, total = O.flat_layout(numels, align)
    full = draw_master(total, 0.02, seed, cfg)
    master = np.zeros(total, np.float32)
    for o, n in zip(offs, numels):
        master[o:o + n] = full[o:o + n]
    return offs, total, master


def _compare(tag, got, want_state, want_sc, osc, ost, st):
    P, M, V, OUT = got
    oP, oM, oV, oOUT = want_state
    assert st.last_skip == ost.last_skip and st.t == ost.t, tag
    assert st.scale == np.float32(ost.scale), tag
    assert want_sc.overflow == osc["overflow"], tag
    if not osc["overflow"]:
        assert want_sc.grad_scale == osc["grad_scale"], tag
        assert abs(float(want_sc.norm) - float(osc["norm"])) <= 1e-6 * float(osc["norm"]), tag
    assert_state_close(tag + " master", P, oP, 2)
    assert_state_close(tag + " exp_avg", M, oM, 2)
    assert_state_close(tag + " exp_avg_sq", V, oV, 2)
    if OUT is not None and oOUT is not None:
        assert_p16_close(tag + " params", OUT, oOUT, 1)


@pytest.mark.parametrize("inf_at", ["seeded", "first", "last"])
def test_tiny_shard_five_steps(inf_at):
    """64 tensors (log-uniform sizes, seed 0), fp16 grads N(0, 1e-3) x scale,
    AdamW lr 1e-3, clip 1.0, dynamic scale from 2^16 with hysteresis 1; +inf
    in step 3's grads skips that step and halves the scale."""
    say("tiny shard 5 steps, inf at", inf_at)
    numels = [n for _, n in tiny_shard_sizes()]
    offs, total, master = _flat_master(numels, 64, 0, 1)
    hp = O.AdamW()
    plan = zds.zds_plan_create(numels, 64, 0, total)
    ent = O.shard_entries(numels, 64, 0, total)
    st = ShardStep(total, zds.hparams(), zds.scaler_config(initial_scale_power=16, window=1000,
                                                          hysteresis=1), max_norm=1.0)
    dP = to_dev(master, "fp32")
    dM = torch.zeros(total, dtype=torch.float32, device="cuda")
    dV = torch.zeros(total, dtype=torch.float32, device="cuda")
    dOUT = to_dev(O.narrow(master, "fp16"), "fp16")
    bucket = torch.zeros(total, dtype=torch.float16, device="cuda")
    oP, oM, oV = master.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32)
    oOUT = O.narrow(master, "fp16")
    ost = O.scaler_init(initial_scale_power=16, window=1000, hysteresis=1)
    scales, applied = [], []
    for k in range(1, 6):
        S = ost.scale
        scales.append(S)
        srcs = [draw_grads(n, "fp16", 1e-3, S, 0, 1, k, offset=o) for o, n in zip(offs, numels)]
        if k == 3:
            t = {"seeded": int(np.random.default_rng(3).integers(0, 64)), "first": 0, "last": 63}[inf_at]
            pos = {"seeded": int(np.random.default_rng(4).integers(0, numels[t])), "first": 0,
                   "last": numels[63] - 1}[inf_at]
            srcs[t][pos] = 0x7C00
        zds.zds_grad_accumulate(plan, [to_dev(s, "fp16") for s in srcs], bucket, zds.ZDS_COPY)
        st.step(bucket, dP, dM, dV, dOUT)
        torch.cuda.synchronize()
        flat = O.flatten_copy(srcs, ent, np.zeros(total, np.uint16))
        assert (to_host(bucket) == flat).all()
        oP, oM, oV, out16, ost, osc = O.optimizer_step(flat, "fp16", oP, oM, oV, ost, hp, 1.0, 1, "fp16")
        if out16 is not None:
            oOUT = out16
        applied.append(None if ost.last_skip else ost.t)
        _compare("step %d" % k, (to_host(dP), to_host(dM), to_host(dV), to_host(dOUT)),
                 (oP, oM, oV, oOUT), st.read_scalars(), osc, ost, st.read_state())
    assert scales == [2.0 ** 16] * 3 + [2.0 ** 15] * 2
    assert applied == [1, 2, None, 3, 4]
    plan.close()


def test_tiny_shard_from_ds_config():
    """The tiny shard stepped with the settings of a DeepSpeed-style JSON
    block (the tutorial's fp16 block: dynamic scale from 2^16, window 1000,
    hysteresis 2; AdamW lr 2e-5; clip 1.0) through ShardStep.from_config,
    against the oracle with the same settings: overflows at steps 2 and 3
    skip both, and only the second halves the scale."""
    from zero_sharded_mixed_tensor_amd.config import from_ds_config
    say("tiny shard from a JSON config")
    cfg = from_ds_config({"fp16": {"enabled": True, "loss_scale": 0, "loss_scale_window": 1000,
                                   "initial_scale_power": 16, "hysteresis": 2, "min_loss_scale": 1},
                          "optimizer": {"type": "AdamW", "params": {"lr": 2e-5, "betas": [0.9, 0.999],
                                                                   "eps": 1e-8, "weight_decay": 0.01}},
                          "gradient_clipping": 1.0})
    numels = [n for _, n in tiny_shard_sizes()]
    offs, total, master = _flat_master(numels, 64, 0, 1)
    hp = O.AdamW(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    ent = O.shard_entries(numels, 64, 0, total)
    st = ShardStep.from_config(total, cfg)
    dP = to_dev(master, "fp32")
    dM = torch.zeros(total, dtype=torch.float32, device="cuda")
    dV = torch.zeros(total, dtype=torch.float32, device="cuda")
    dOUT = to_dev(O.narrow(master, "fp16"), "fp16")
    bucket = torch.zeros(total, dtype=torch.float16, device="cuda")
    oP, oM, oV = master.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32)
    oOUT = O.narrow(master, "fp16")
    ost = O.scaler_init(initial_scale_power=16, window=1000, hysteresis=2, min_scale=1.0)
    scales, applied = [], []
    for k in range(1, 6):
        S = ost.scale
        scales.append(S)
        srcs = [draw_grads(n, "fp16", 1e-3, S, 0, 1, k, offset=o) for o, n in zip(offs, numels)]
        if k in (2, 3):
            srcs[7 * k][k] = 0xFC00  # -inf
        zds.zds_grad_accumulate(plan, [to_dev(s, "fp16") for s in srcs], bucket, zds.ZDS_COPY)
        st.step(bucket, dP, dM, dV, dOUT)
        torch.cuda.synchronize()
        flat = O.flatten_copy(srcs, ent, np.zeros(total, np.uint16))
        oP, oM, oV, out16, ost, osc = O.optimizer_step(flat, "fp16", oP, oM, oV, ost, hp, cfg.max_norm,
                                                       cfg.accum_steps, "fp16")
        if out16 is not None:
            oOUT = out16
        applied.append(None if ost.last_skip else ost.t)
        _compare("config step %d" % k, (to_host(dP), to_host(dM), to_host(dV), to_host(dOUT)),
                 (oP, oM, oV, oOUT), st.read_scalars(), osc, ost, st.read_state())
    assert scales == [2.0 ** 16] * 3 + [2.0 ** 15] * 2
    assert applied == [1, None, None, 2, 3]
    plan.close()


def test_gradient_accumulation_sixteen_microbatches():
    """16 micro-batches of fp16 grads N(0, 1e-3) x 2^14 accumulated in fp32,
    then overflow check, clip at 1.0 and AdamW (t = 2, prior moments), on a
    reduced Stage-1 shard of 10 tensors."""
    say("accumulation K=16")
    rng = np.random.default_rng(21)
    numels = [int(x) for x in rng.integers(1000, 60000, 10)]
    _, total = O.flat_layout(numels, 64)
    lo, hi = O.shard_range(total, 3, 1, 64)
    ent = O.shard_entries(numels, 64, lo, hi)
    L = hi - lo
    plan = zds.zds_plan_create(numels, 64, lo, hi)
    offs, _ = O.flat_layout(numels, 64)
    acc = torch.empty(L, dtype=torch.float32, device="cuda")
    wacc = np.zeros(L, np.float32)
    for k in range(16):
        srcs = [draw_grads(n, "fp16", 1e-3, 2.0 ** 14, 2, 3, k, offset=o) for o, n in zip(offs, numels)]
        zds.zds_grad_accumulate(plan, [to_dev(s, "fp16") for s in srcs], acc,
                                zds.ZDS_OVERWRITE if k == 0 else zds.ZDS_ACCUMULATE)
        O.flatten_accumulate(srcs, "fp16", ent, wacc, overwrite=(k == 0))
    # padding inside the range is never written by the accumulate: zero it as
    # the caller must (the oracle's buffer starts at zero)
    pad = np.ones(L, bool)
    for t, s, n, d in ent:
        pad[d:d + n] = False
    acc[torch.from_numpy(pad).cuda()] = 0.0
    master = draw_master(L, 0.02, 2, 3)
    m, v = draw_prior_moments(L, 1e-3, 2, 3)
    master[pad] = 0
    m[pad] = 0
    v[pad] = 0
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    # at this reduced size the averaged grads have norm ~0.08, so the clip
    # threshold is lowered to keep the clip path active
    max_norm = 0.0625
    st = ShardStep(L, zds.hparams(), zds.scaler_config(initial_scale_power=14), max_norm=max_norm,
                   accum_steps=16, t0=1, beta1_pow0=b1, beta2_pow0=b2)
    dP, dM, dV = to_dev(master, "fp32"), to_dev(m, "fp32"), to_dev(v, "fp32")
    dOUT = torch.zeros(L, dtype=torch.float16, device="cuda")
    st.step(acc, dP, dM, dV, dOUT)
    torch.cuda.synchronize()
    assert (to_host(acc).view(np.uint32) == wacc.view(np.uint32)).all()
    ost = O.scaler_init(initial_scale_power=14, t=1, beta1_pow=b1, beta2_pow=b2)
    oP, oM, oV, oOUT, ost, osc = O.optimizer_step(wacc, "fp32", master, m, v, ost, O.AdamW(), max_norm, 16,
                                                  "fp16")
    assert osc["coef"] < 1.0  # the clip is active
    _compare("accum", (to_host(dP), to_host(dM), to_host(dV), to_host(dOUT)), (oP, oM, oV, oOUT),
             st.read_scalars(), osc, ost, st.read_state())
    plan.close()


def test_thousand_tensor_table_twenty_steps():
    """1,024 tensors (reduced sizes, norms-like 4096-element pieces among
    them), fp16 grads, copy into a flat bucket, 20 steps with a seeded
    overflow schedule: Bernoulli(0.001) per step plus one forced overflow at a
    seeded step in [2, 19], inf and NaN alternately."""
    say("1024-tensor table, 20 steps")
    rng = np.random.default_rng(1024)
    numels = [4096 if i % 15 == 14 else int(rng.integers(64, 3000)) for i in range(1024)]
    offs, total, master = _flat_master(numels, 64, 4, 4)
    plan = zds.zds_plan_create(numels, 64, 0, total)
    assert plan.num_entries == 1024
    ent = O.shard_entries(numels, 64, 0, total)
    sched = np.random.default_rng(17)
    forced = int(sched.integers(2, 20))
    over = [(k == forced) or (sched.random() < 0.001) for k in range(1, 21)]
    st = ShardStep(total, zds.hparams(), zds.scaler_config(initial_scale_power=16, window=1000), max_norm=1.0)
    dP = to_dev(master, "fp32")
    dM = torch.zeros(total, dtype=torch.float32, device="cuda")
    dV = torch.zeros(total, dtype=torch.float32, device="cuda")
    dOUT = torch.zeros(total, dtype=torch.float16, device="cuda")
    bucket = torch.zeros(total, dtype=torch.float16, device="cuda")
    oP, oM, oV = master.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32)
    oOUT = np.zeros(total, np.uint16)
    ost = O.scaler_init(initial_scale_power=16, window=1000)
    nov = 0
    traj = []
    for k in range(1, 21):
        # one draw over the flat range per step; tensor t is its slice (the
        # same values a per-tensor draw at the tensor's flat offset gives)
        flat_src = draw_grads(total, "fp16", 1e-3, ost.scale, 4, 4, k)
        srcs = [flat_src[o:o + n] for o, n in zip(offs, numels)]
        if over[k - 1]:
            t = int(sched.integers(0, 1024))
            srcs[t][int(sched.integers(0, numels[t]))] = 0x7C00 if nov % 2 == 0 else 0x7E00
            nov += 1
        dsrc = to_dev(flat_src, "fp16")
        zds.zds_grad_accumulate(plan, [dsrc[o:o + n] for o, n in zip(offs, numels)], bucket, zds.ZDS_COPY)
        st.step(bucket, dP, dM, dV, dOUT)
        flat = O.flatten_copy(srcs, ent, np.zeros(total, np.uint16))
        oP, oM, oV, out16, ost, osc = O.optimizer_step(flat, "fp16", oP, oM, oV, ost, O.AdamW(), 1.0, 1, "fp16")
        if out16 is not None:
            oOUT = out16
        torch.cuda.synchronize()
        gst = st.read_state()
        traj.append(gst.scale)
        _compare("step %d" % k, (to_host(dP), to_host(dM), to_host(dV), to_host(dOUT)),
                 (oP, oM, oV, oOUT), st.read_scalars(), osc, ost, gst)
    assert min(traj) < 2.0 ** 16  # the trajectory contains a halving
    plan.close()


def test_bf16_stage1_shard_prior_moments():
    """Reduced Llama-like shard: bf16 grads N(0, 2e-3), static scale 1, clip
    active, m and v from a prior step (t = 1 -> 2), bf16 params out."""
    say("bf16 stage-1 shard, one step")
    numels = [4096 * 40, 4096 * 12, 4096 * 12, 4096, 4096 * 30, 4096 * 30]
    _, total = O.flat_layout(numels, 64)
    lo, hi = O.shard_range(total, 8, 5, 64)
    L = hi - lo
    g = draw_grads(L, "bf16", 2e-3, 1.0, 6, 2, 0)
    master = draw_master(L, 0.02, 6, 2)
    m, v = draw_prior_moments(L, 2e-3, 6, 2)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    # the reduced shard's grad norm is ~0.5, so the clip threshold is lowered
    # to keep the clip path active
    max_norm = 0.25
    st = ShardStep(L, zds.hparams(), zds.scaler_config(dynamic=False, static_scale=1.0), max_norm=max_norm,
                   t0=1, beta1_pow0=b1, beta2_pow0=b2)
    dP, dM, dV = to_dev(master, "fp32"), to_dev(m, "fp32"), to_dev(v, "fp32")
    dOUT = torch.zeros(L, dtype=torch.bfloat16, device="cuda")
    st.step(to_dev(g, "bf16"), dP, dM, dV, dOUT)
    torch.cuda.synchronize()
    ost = O.scaler_init(dynamic=False, static_scale=1.0, t=1, beta1_pow=b1, beta2_pow=b2)
    oP, oM, oV, oOUT, ost, osc = O.optimizer_step(g, "bf16", master, m, v, ost, O.AdamW(), max_norm, 1, "bf16")
    assert osc["coef"] < 1.0
    _compare("bf16 shard", (to_host(dP), to_host(dM), to_host(dV), to_host(dOUT)), (oP, oM, oV, oOUT),
             st.read_scalars(), osc, ost, st.read_state())


def test_offloaded_optimizer_shard_steps():
    """Optimizer shard in pinned host memory: device norm, chunked download,
    host AdamW, upload of the 16-bit params, device scaler; 4 steps with an
    overflow at step 2, against the oracle."""
    say("offload: 4 steps, overflow at step 2")
    from zero_sharded_mixed_tensor_amd.step import OffloadStep
    n = 300_001
    master = draw_master(n, 0.02, 8, 9)
    hm = torch.from_numpy(master.copy()).pin_memory()
    hmm = torch.zeros(n, dtype=torch.float32).pin_memory()
    hv = torch.zeros(n, dtype=torch.float32).pin_memory()
    off = OffloadStep(n, hm, hmm, hv, torch.float16, torch.float16, zds.hparams(),
                      zds.scaler_config(initial_scale_power=12), max_norm=1.0, chunk=65536, threads=3)
    out = torch.zeros(n, dtype=torch.float16, device="cuda")
    oP, oM, oV = master.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    o16 = np.zeros(n, np.uint16)
    ost = O.scaler_init(initial_scale_power=12)
    for k in range(1, 5):
        g = draw_grads(n, "fp16", 1e-3, ost.scale, 8, 9, k)
        if k == 2:
            g[n // 3] = 0x7C00
        sc = off.step(to_dev(g, "fp16"), out)
        torch.cuda.synchronize()
        oP, oM, oV, r16, ost, osc = O.optimizer_step(g, "fp16", oP, oM, oV, ost, O.AdamW(), 1.0, 1, "fp16")
        if r16 is not None:
            o16 = r16
        assert sc.overflow == osc["overflow"]
        if not sc.overflow:
            assert sc.grad_scale == osc["grad_scale"]
        assert (hm.numpy().view(np.uint32) == oP.view(np.uint32)).all(), k
        assert (hmm.numpy().view(np.uint32) == oM.view(np.uint32)).all(), k
        assert (hv.numpy().view(np.uint32) == oV.view(np.uint32)).all(), k
        assert (to_host(out) == o16).all(), k
        s = off.dev.read_state()
        assert (s.scale, s.t) == (np.float32(ost.scale), ost.t), k


def test_tiny_shard_graph_replays():
    """The tiny shard's step captured once into a HIP graph and replayed for
    5 steps (grads refilled in place between replays, an overflow at step 3),
    with eager work on the same plan between replays that cycles through more
    source sets than the plan has staging slots. Every replay must equal the
    eagerly run step bit for bit: state, params, step state and scalars."""
    say("tiny shard: graph replays vs eager steps")
    numels = [n for _, n in tiny_shard_sizes()]
    offs, total, master = _flat_master(numels, 64, 0, 1)
    cfg = dict(initial_scale_power=16, window=2, hysteresis=1)

    def setup():
        st = ShardStep(total, zds.hparams(), zds.scaler_config(**cfg), max_norm=1.0)
        bufs = [to_dev(master, "fp32"), torch.zeros(total, dtype=torch.float32, device="cuda"),
                torch.zeros(total, dtype=torch.float32, device="cuda"),
                to_dev(O.narrow(master, "fp16"), "fp16")]
        srcs = [torch.empty(n, dtype=torch.float16, device="cuda") for n in numels]
        bucket = torch.zeros(total, dtype=torch.float16, device="cuda")
        return st, bufs, srcs, bucket

    def fill(srcs, k, scale):
        for t, (o, n) in enumerate(zip(offs, numels)):
            g = draw_grads(n, "fp16", 1e-3, scale, 0, 1, k, offset=o)
            if k == 3 and t == 7:
                g[5] = 0x7C00
            srcs[t].copy_(to_dev(g, "fp16"))

    plan_a = zds.zds_plan_create(numels, 64, 0, total)
    plan_b = zds.zds_plan_create(numels, 64, 0, total)
    ea, ba, sa, bka = setup()
    eb, bb, sb, bkb = setup()
    wsa, wsb = zds.new_plan_workspace(plan_a), zds.new_plan_workspace(plan_b)
    graph = eb.capture(plan_b, sb, bkb, zds.ZDS_COPY, wsb, *bb)
    others = [[torch.zeros(n, dtype=torch.float16, device="cuda") for n in numels] for _ in range(10)]
    junk = torch.empty(total, dtype=torch.float16, device="cuda")
    for k in range(1, 6):
        scale = ea.read_state().scale
        fill(sa, k, scale)
        ea.accumulate_norm(plan_a, sa, bka, zds.ZDS_COPY, wsa)
        ea.adam(bka, *ba)
        ea.scaler()
        fill(sb, k, eb.read_state().scale)
        graph.replay()
        for o in others:  # eager calls with other pointers between replays
            zds.zds_grad_accumulate(plan_b, o, junk, zds.ZDS_COPY)
        torch.cuda.synchronize()
        for x, y in zip(ba, bb):
            assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                               y.view(torch.int16 if y.element_size() == 2 else torch.int32)), k
        assert bytes(ea.read_state()) == bytes(eb.read_state()), k
        assert bytes(ea.read_scalars()) == bytes(eb.read_scalars()), k
    assert eb.read_state().last_skip == 0 and ea.read_state().t == 4
    plan_a.close()
    plan_b.close()


def test_stage2_step_graph_replays():
    """The Stage-2 step (the fused intake of 4 bf16 peers into the fp32 shard
    grad, AdamW, the scaler) captured once into a HIP graph and replayed for
    5 steps, the peers' slices refilled in place (an inf in one of them at
    step 3) and eager intake work between replays. Every replay must equal
    the same step run eagerly, bit for bit: shard grad, state, params, step
    state and scalars."""
    say("stage-2 step: graph replays vs eager steps")
    n, N = 100003, 4
    master = draw_master(n, 0.02, 3, 11)
    cfg = dict(initial_scale_power=10, window=2, hysteresis=1)

    def setup():
        st = ShardStep(n, zds.hparams(), zds.scaler_config(**cfg), max_norm=1.0, accum_steps=N)
        bufs = [to_dev(master, "fp32"), torch.zeros(n, dtype=torch.float32, device="cuda"),
                torch.zeros(n, dtype=torch.float32, device="cuda"),
                torch.zeros(n, dtype=torch.bfloat16, device="cuda")]
        peers = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
        return st, bufs, peers, torch.zeros(n, dtype=torch.float32, device="cuda"), zds.new_reduce_workspace(n)

    def fill(peers, k, scale):
        for i, p in enumerate(peers):
            g = draw_grads(n, "bf16", 1e-3, scale, 5 + i, 2, k)
            if k == 3 and i == 1:
                g[777] = 0x7F80  # +inf
            p.copy_(to_dev(g, "bf16"))

    sa, ba, pa, acc_a, wsa = setup()
    sb, bb, pb, acc_b, wsb = setup()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sb.intake_norm(pb, acc_b, zds.ZDS_OVERWRITE, wsb)
        sb.adam(acc_b, *bb)
        sb.scaler()
    junk = torch.empty(n, dtype=torch.float32, device="cuda")
    for k in range(1, 6):
        fill(pa, k, sa.read_state().scale)
        sa.intake_norm(pa, acc_a, zds.ZDS_OVERWRITE, wsa)
        sa.adam(acc_a, *ba)
        sa.scaler()
        fill(pb, k, sb.read_state().scale)
        graph.replay()
        zds.zds_reduce_peer_slices(pa, junk, zds.ZDS_OVERWRITE)  # eager work between replays
        torch.cuda.synchronize()
        for x, y in zip(ba + [acc_a], bb + [acc_b]):
            assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                               y.view(torch.int16 if y.element_size() == 2 else torch.int32)), k
        assert bytes(sa.read_state()) == bytes(sb.read_state()), k
        assert bytes(sa.read_scalars()) == bytes(sb.read_scalars()), k
    st = sb.read_state()
    assert st.steps_skipped == 1 and st.t == 4
