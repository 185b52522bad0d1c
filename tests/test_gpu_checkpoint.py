"""Sharded checkpoint / resume on the GPU: a run that saves its shards after
k steps, reloads them into fresh buffers and runs j more steps ends
bit-identical to the run that went k + j steps straight; the consolidated
fp32 state of the saved shards is the oracle's merge of the same device
shards bit for bit, and within the step tolerance of the free-running
oracle after the same k steps."""

import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from tests.util import assert_state_close, to_dev, to_host
from workloads import draw_grads, draw_master, tiny_shard_sizes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from zero_sharded_mixed_tensor_amd import zds  # noqa: E402
from zero_sharded_mixed_tensor_amd.step import ShardStep  # noqa: E402

ALIGN = 64
WORLD = 4
SCALER = dict(initial_scale_power=16, window=2, hysteresis=2)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Run:
    """One rank-set's device state: the whole flat buffer, padded to WORLD
    shards; rank r's shard is the slice [lo_r, hi_r)."""

    def __init__(self, numels, master0):
        self.numels = numels
        self.offs, total = O.flat_layout(numels, ALIGN)
        self.ranges = [O.shard_range(total, WORLD, r, ALIGN) for r in range(WORLD)]
        self.n = self.ranges[-1][1]
        self.P = to_dev(master0, "fp32")
        self.M = torch.zeros(self.n, dtype=torch.float32, device="cuda")
        self.V = torch.zeros(self.n, dtype=torch.float32, device="cuda")
        self.OUT = self.P.to(torch.float16)  # the model's 16-bit weights at the start
        self.bucket = torch.zeros(self.n, dtype=torch.float16, device="cuda")
        self.plan = zds.zds_plan_create(numels, ALIGN, 0, self.n)
        self.st = ShardStep(self.n, zds.hparams(), zds.scaler_config(**SCALER), max_norm=1.0)

    def grads(self, k, scale):
        srcs = [draw_grads(n, "fp16", 1e-3, scale, 0, 7, k, offset=o) for o, n in zip(self.offs, self.numels)]
        if k == 2:
            srcs[5][17] = 0x7C00  # +inf: step 2 is skipped
        return srcs

    def step(self, k):
        scale = self.st.read_state().scale
        srcs = self.grads(k, scale)
        zds.zds_grad_accumulate(self.plan, [to_dev(s, "fp16") for s in srcs], self.bucket, zds.ZDS_COPY)
        self.st.step(self.bucket, self.P, self.M, self.V, self.OUT)
        torch.cuda.synchronize()
        return srcs

    def meta(self, r):
        return zds.checkpoint_meta(self.numels, WORLD, r, ALIGN, stage=1)

    def save(self, d):
        paths = []
        for r, (lo, hi) in enumerate(self.ranges):
            p = os.path.join(d, "zero_rank%d.zckpt" % r)
            zds.zds_checkpoint_save(p, self.meta(r), self.numels, self.P[lo:hi], self.M[lo:hi], self.V[lo:hi],
                                    self.st.state)
            paths.append(p)
        return paths

    def load(self, paths):
        for r, (lo, hi) in enumerate(self.ranges):
            zds.zds_checkpoint_load(paths[r], self.meta(r), self.numels, self.P[lo:hi], self.M[lo:hi],
                                    self.V[lo:hi], self.st.state)


def _numels():
    return [n for _, n in tiny_shard_sizes()]


def _master(numels):
    offs, total = O.flat_layout(numels, ALIGN)
    padded = O.shard_range(total, WORLD, WORLD - 1, ALIGN)[1]
    full = draw_master(padded, 0.02, 0, 7)
    master = np.zeros(padded, np.float32)
    for o, n in zip(offs, numels):
        master[o:o + n] = full[o:o + n]
    return master


def _same(a, b):
    return torch.equal(a.view(torch.int32 if a.element_size() == 4 else torch.int16),
                       b.view(torch.int32 if b.element_size() == 4 else torch.int16))


@pytest.mark.parametrize("k,j", [(3, 3), (1, 4), (2, 1)])
def test_resume_is_bit_identical(k, j, tmp_path):
    say("resume after", k, "steps, then", j)
    numels = _numels()
    master0 = _master(numels)
    a = Run(numels, master0)
    for s in range(1, k + j + 1):
        a.step(s)
    b = Run(numels, master0)
    for s in range(1, k + 1):
        b.step(s)
    paths = b.save(str(tmp_path))
    out16 = to_host(b.OUT)  # the model's own checkpoint holds its 16-bit weights
    del b
    torch.cuda.synchronize()
    c = Run(numels, np.full(master0.shape, np.nan, np.float32))
    c.M.fill_(float("nan"))
    c.V.fill_(-1.0)
    zds.zds_step_state_init(c.st.state, zds.scaler_config(initial_scale_power=3), 99, 0.5, 0.5)
    c.OUT.copy_(to_dev(out16, "fp16"))
    c.load(paths)
    for s in range(k + 1, k + j + 1):
        c.step(s)
    for name in ("P", "M", "V", "OUT"):
        assert _same(getattr(a, name), getattr(c, name)), name
    assert bytes(a.st.read_state()) == bytes(c.st.read_state())
    assert bytes(a.st.read_scalars()) == bytes(c.st.read_scalars())


def test_consolidated_state_matches_oracle(tmp_path):
    say("consolidation of 4 device shards after 3 steps")
    numels = _numels()
    master0 = _master(numels)
    r = Run(numels, master0)
    hp = O.AdamW()
    oP, oM, oV = master0.copy(), np.zeros(r.n, np.float32), np.zeros(r.n, np.float32)
    ost = O.scaler_init(**SCALER)
    ent = O.shard_entries(numels, ALIGN, 0, r.n)
    for s in range(1, 4):
        srcs = r.step(s)
        flat = O.flatten_copy(srcs, ent, np.zeros(r.n, np.uint16))
        oP, oM, oV, _, ost, _ = O.optimizer_step(flat, "fp16", oP, oM, oV, ost, hp, 1.0, 1, "fp16")
    paths = r.save(str(tmp_path))
    meta, st, table = zds.zds_checkpoint_read_meta(paths[2])
    assert table == numels and meta.rank == 2 and meta.world == WORLD
    assert st.t == ost.t == 2 and st.scale == np.float32(ost.scale)
    dev = [to_host(x) for x in (r.P, r.M, r.V)]
    for section, want in enumerate((oP, oM, oV)):
        got = zds.zds_consolidate_fp32(paths[::-1], section)
        # the partition map, bit for bit: the oracle's merge of the same device shards
        mine = O.consolidate([(lo, hi, dev[section][lo:hi]) for lo, hi in r.ranges], numels, ALIGN)
        assert (got.view(np.uint32) == np.concatenate(mine).view(np.uint32)).all()
        # the state itself: the oracle's own run, merged the same way
        theirs = O.consolidate([(lo, hi, want[lo:hi]) for lo, hi in r.ranges], numels, ALIGN)
        assert_state_close("section %d" % section, got, np.concatenate(theirs), 2)


def test_load_refuses_mismatch_on_device(tmp_path):
    numels = _numels()
    r = Run(numels, _master(numels))
    r.step(1)
    paths = r.save(str(tmp_path))
    lo, hi = r.ranges[1]
    with pytest.raises(zds.ZdsError) as e:
        zds.zds_checkpoint_load(paths[0], r.meta(1), numels, r.P[lo:hi], r.M[lo:hi], r.V[lo:hi], r.st.state)
    assert e.value.status == zds.ZDS_EINVAL
    before = to_host(r.P)
    with open(paths[1], "r+b") as f:
        f.seek(256 + 8 * len(numels) + 4 * (hi - lo) + 8)
        f.write(b"\x00\x01\x02\x03")
    with pytest.raises(zds.ZdsError) as e:
        zds.zds_checkpoint_load(paths[1], r.meta(1), numels, r.P[lo:hi], r.M[lo:hi], r.V[lo:hi], r.st.state)
    assert e.value.status == zds.ZDS_EIO
    # master had been restored before the corrupt exp_avg section was found: same bytes as saved
    assert (to_host(r.P) == before).all()
