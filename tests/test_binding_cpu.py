"""CPU checks of the Python binding's buffer-length checks. The library takes
plain pointers and sizes, so a tensor shorter than what a call reads or
writes would be accessed past its end; the binding refuses such a call before
it touches the device. Each case gives one buffer that is too short and
expects the length error; the same call with every buffer long enough (but on
the host, where a device tensor is expected) gets past the length checks and
fails on the device check instead."""

import types

import numpy as np
import pytest
import torch

zds = pytest.importorskip("zero_sharded_mixed_tensor_amd.zds", reason="libzds.so not built")


def _f32(n):
    return torch.zeros(n, dtype=torch.float32)


def _bf16(n):
    return torch.zeros(n, dtype=torch.bfloat16)


def _raises(fn, text):
    with pytest.raises(zds.ZdsError) as e:
        fn()
    assert text in str(e.value), str(e.value)


def test_adam_step_lengths():
    hp = zds.hparams()
    st, sc = torch.zeros(64, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
    n = 1000
    ok = dict(grads=_bf16(n), master=_f32(n), exp_avg=_f32(n), exp_avg_sq=_f32(n), params_out=_bf16(n))
    for name in ok:
        args = dict(ok)
        args[name] = (_bf16 if name in ("grads", "params_out") else _f32)(n - 1)
        _raises(lambda: zds.zds_adam_step(hp, args["grads"], args["master"], args["exp_avg"], args["exp_avg_sq"],
                                          args["params_out"], sc, st, n=n), "%s holds %d" % (name, n - 1))
    # an explicit n beyond every buffer names master first
    _raises(lambda: zds.zds_adam_step(hp, ok["grads"], ok["master"], ok["exp_avg"], ok["exp_avg_sq"],
                                      ok["params_out"], sc, st, n=n + 1), "master holds %d" % n)
    _raises(lambda: zds.zds_adam_step(hp, ok["grads"], ok["master"], ok["exp_avg"], ok["exp_avg_sq"],
                                      ok["params_out"], sc, st), "must be a device tensor")


def test_norm_and_reduce_lengths():
    st, sc = torch.zeros(64, dtype=torch.uint8), torch.zeros(64, dtype=torch.uint8)
    ws = torch.zeros(8, dtype=torch.float64)
    _raises(lambda: zds.zds_overflow_and_norm(_bf16(10), 1, 1.0, st, sc, ws, n=11), "grads holds 10")
    peers = [_bf16(100), _bf16(100)]
    _raises(lambda: zds.zds_reduce_peer_slices(peers, _f32(99), zds.ZDS_OVERWRITE, n=100), "dst holds 99")
    _raises(lambda: zds.zds_reduce_peer_slices([_bf16(100), _bf16(99)], _f32(100), zds.ZDS_OVERWRITE),
            "too short")
    _raises(lambda: zds.zds_reduce_peer_slices(peers, _f32(100), zds.ZDS_OVERWRITE), "must be a device tensor")


@pytest.mark.parametrize("n,chunk", [(1, 1024), (256, 2048), (257, 1024), (5000, 4096)])
def test_onebit_payload_lengths(n, chunk):
    words, scales = zds.onebit_payload(n, chunk, device="cpu")
    assert words.numel() * 4 == 256 * ((n + 2047) // 2048) and scales.numel() == (n + chunk - 1) // chunk
    x, err = _f32(n), _f32(n)
    _raises(lambda: zds.zds_onebit_compress(x, err, chunk, words[:-1], scales), "words holds")
    _raises(lambda: zds.zds_onebit_compress(x, err, chunk, words, scales[:-1]), "scales holds")
    _raises(lambda: zds.zds_onebit_compress(x, _f32(n - 1), chunk, words, scales), "error holds %d" % (n - 1))
    _raises(lambda: zds.zds_onebit_compress(x, err, chunk, words, scales, n=n + 256), "x holds %d" % n)
    _raises(lambda: zds.zds_onebit_compress(x, err, chunk, words, scales), "must be a device tensor")
    dst = _f32(n)
    _raises(lambda: zds.zds_onebit_decompress([(words, scales), (words[:-1], scales)], chunk, dst), "words holds")
    _raises(lambda: zds.zds_onebit_decompress([(words, scales)], chunk, dst, n=n + 1), "dst holds %d" % n)
    _raises(lambda: zds.zds_onebit_decompress([(words, scales)], chunk, dst), "must be a device tensor")


def _fake_plan():
    # entries (tensor, start, length, flat offset): tensor 0 from 5, 10
    # elements; tensor 2 whole, 7 elements at offset 64; tensor 1 unused
    ents = [(0, 5, 10, 0), (2, 0, 7, 64)]
    p = types.SimpleNamespace(num_tensors=3, handle=None)
    p.src_need = {0: 15, 2: 7}
    p.span = 71
    p.entries = lambda: ents
    return p


def test_accumulate_lengths():
    plan = _fake_plan()
    srcs = [_bf16(15), None, _bf16(7)]
    dst = _bf16(71)
    _raises(lambda: zds.zds_grad_accumulate(plan, [_bf16(14), None, _bf16(7)], dst, zds.ZDS_COPY),
            "source 0 holds 14")
    _raises(lambda: zds.zds_grad_accumulate(plan, [_bf16(15), None, None], dst, zds.ZDS_COPY), "source 2 is None")
    _raises(lambda: zds.zds_grad_accumulate(plan, srcs[:2], dst, zds.ZDS_COPY), "need 3 source tensors")
    _raises(lambda: zds.zds_grad_accumulate(plan, srcs, _bf16(70), zds.ZDS_COPY), "dst holds 70")
    _raises(lambda: zds.SourceSet(plan, [_bf16(15), None, _bf16(6)]), "source 2 holds 6")
    # long enough: the device check is next
    _raises(lambda: zds.zds_grad_accumulate(plan, srcs, dst, zds.ZDS_COPY), "must be a device tensor")


def test_checkpoint_lengths(tmp_path):
    numels = [100, 37]
    meta = zds.checkpoint_meta(numels, world=2, rank=1, flat_align=64)
    n = meta.hi - meta.lo
    st = zds.zds_step_state_init_host(zds.scaler_config())
    m = [np.zeros(n, np.float32) for _ in range(3)]
    path = str(tmp_path / "r1.zds")
    for i, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
        bufs = list(m)
        bufs[i] = np.zeros(n - 1, np.float32)
        _raises(lambda: zds.zds_checkpoint_save(path, meta, numels, *bufs, st), "%s holds %d" % (name, n - 1))
        _raises(lambda: zds.zds_checkpoint_load(path, meta, numels, *bufs, st), "%s holds %d" % (name, n - 1))
    # the host path with full-length buffers saves and loads
    rng = np.random.default_rng(3)
    for a in m:
        a[:] = rng.standard_normal(n).astype(np.float32)
    zds.zds_checkpoint_save(path, meta, numels, *m, st)
    back = [np.zeros(n, np.float32) for _ in range(3)]
    zds.zds_checkpoint_load(path, meta, numels, *back, zds.StepState())
    for a, b in zip(m, back):
        assert np.array_equal(a, b)


def test_cpu_adam_lengths():
    hp = zds.hparams()
    n = 64
    st = zds.zds_step_state_init_host(zds.scaler_config(dynamic=False))
    sc = zds.zds_clip_scalars_host(0.0, 1.0, 1, 1.0)
    g = np.zeros(n, np.float16)
    full = [np.zeros(n, np.float32) for _ in range(3)]
    _raises(lambda: zds.zds_cpu_adam_step(hp, g[:-1], *full, None, sc, st), "grads holds %d" % (n - 1))
    _raises(lambda: zds.zds_cpu_adam_step(hp, g, full[0], full[1][:-1], full[2], None, sc, st),
            "exp_avg holds %d" % (n - 1))
    _raises(lambda: zds.zds_cpu_adam_step(hp, g, *full, np.zeros(n - 1, np.float16), sc, st),
            "params_out holds %d" % (n - 1))


def test_device_structs_sizes():
    cfg = zds.scaler_config()
    _raises(lambda: zds.zds_step_state_init(torch.zeros(63, dtype=torch.uint8), cfg), "state holds 63 bytes")
    _raises(lambda: zds.zds_loss_scaler_update(torch.zeros(64, dtype=torch.uint8), torch.zeros(32, dtype=torch.uint8),
                                               zds.hparams()), "scalars holds 32 bytes")
