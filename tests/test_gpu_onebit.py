"""1-bit codec on the GPU against the oracle: encode (signs, per-chunk RMS
scales, error feedback) and the N-peer decode, at sizes spanning many chunks
with ragged tails, over several error-feedback rounds, and at the Llama-7B
Stage-1 shard size on sampled chunks.

Tolerance, from the arithmetic: the signs depend only on c = x + error (one
fp32 add on both sides), so they are bit-exact. The scale is
fp32(sqrt(sumsq / len)); the library sums the float64 squares in a block-tree
order, the oracle exactly, so the two sums differ by at most a few float64
ulps and the fp32 scales can differ by 1 ulp, rarely. The new error is then
bit-exact wherever the scale is, and within one ulp of the scale elsewhere.
The decode is a fixed-order fp32 sum and is bit-exact given the same
payloads."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from tests.util import to_host, ulp_diff32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from zero_sharded_mixed_tensor_amd import zds  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _words_host(t):
    return t.cpu().numpy().view(np.uint32)


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 2, n)).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    x[rng.integers(0, n, max(1, n // 500))] = 0.0
    return x, e


def _check_encode(tag, n, chunk, words, scales, err, o_words, o_scales, o_err, err_given=True):
    assert (words == o_words).all(), "%s: sign words differ" % tag
    du = ulp_diff32(scales, o_scales)
    assert du.max() <= 1, "%s: scale off by %d ulp" % (tag, int(du.max()))
    assert (du > 0).sum() <= max(1, scales.size // 1000), "%s: %d scales differ" % (tag, int((du > 0).sum()))
    if not err_given:
        return
    same = np.repeat(du == 0, chunk)[:n]
    assert (err[same].view(np.uint32) == o_err[same].view(np.uint32)).all(), "%s: error differs" % tag
    if (~same).any():
        tol = np.spacing(np.repeat(np.maximum(scales, o_scales), chunk)[:n])
        assert (np.abs(err[~same] - o_err[~same]) <= tol[~same]).all(), tag


@pytest.mark.parametrize("chunk", [1024, 2048, 16384])
@pytest.mark.parametrize("n", [1, 31, 1000, 1024, 5 * 1024 + 7, 70001])
def test_encode_matches_oracle(n, chunk):
    say("encode n", n, "chunk", chunk)
    x, e = _inputs(n, n + chunk)
    o_words, o_scales, o_err = O.onebit_compress(x, e, chunk)
    dx, de = _dev(x), _dev(e)
    words, scales = zds.onebit_payload(n, chunk)
    zds.zds_onebit_compress(dx, de, chunk, words, scales)
    torch.cuda.synchronize()
    _check_encode("n=%d chunk=%d" % (n, chunk), n, chunk, _words_host(words), to_host(scales), to_host(de),
                  o_words, o_scales, o_err)
    assert (to_host(dx) == x).all()  # x is read only


@pytest.mark.parametrize("chunk", [1024, 2048, 4096])
@pytest.mark.parametrize("n", [500, 2048 * 3 + 500, 2048 * 3 + 1500, 2048 * 4])
def test_encode_overwrites_stale_words(n, chunk):
    """Every word of the payload is written, bits past n as 0, whatever the
    buffer held before (here all bits set)."""
    say("encode into a stale payload n", n, "chunk", chunk)
    x, e = _inputs(n, n + 3 * chunk)
    o_words, o_scales, _ = O.onebit_compress(x, e, chunk)
    words, scales = zds.onebit_payload(n, chunk)
    words.fill_(-1)
    scales.fill_(float("nan"))
    zds.zds_onebit_compress(_dev(x), _dev(e), chunk, words, scales)
    torch.cuda.synchronize()
    assert (_words_host(words) == o_words).all()
    assert ulp_diff32(to_host(scales), o_scales).max() <= 1


def test_encode_without_error_buffer():
    n, chunk = 9000, 2048
    x, _ = _inputs(n, 5)
    x[7] = -0.0
    o_words, o_scales, _ = O.onebit_compress(x, np.zeros(n, np.float32), chunk)
    words, scales = zds.onebit_payload(n, chunk)
    zds.zds_onebit_compress(_dev(x), None, chunk, words, scales)
    torch.cuda.synchronize()
    _check_encode("no error", n, chunk, _words_host(words), to_host(scales), None, o_words, o_scales, None,
                  err_given=False)


def test_error_feedback_rounds():
    """Both sides run their own error buffers. A chunk whose scale once came
    out 1 ulp apart carries a slightly different error from then on; such
    chunks are only held to the scale tolerance afterwards."""
    say("error feedback, 6 rounds")
    n, chunk = 300_000 + 13, 4096
    nch = -(-n // chunk)
    rng = np.random.default_rng(9)
    e = np.zeros(n, np.float32)
    de = _dev(e)
    words, scales = zds.onebit_payload(n, chunk)
    apart = np.zeros(nch, bool)
    for r in range(6):
        x = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        o_words, o_scales, e = O.onebit_compress(x, e, chunk)
        zds.zds_onebit_compress(_dev(x), de, chunk, words, scales)
        torch.cuda.synchronize()
        w, sc, ge = _words_host(words), to_host(scales), to_host(de)
        du = ulp_diff32(sc, o_scales)
        keep = ~apart
        el = np.repeat(keep, chunk)[:n]
        wl = np.repeat(keep, chunk // 32)[:w.size]  # 64 words per 2048 elements
        assert (w[wl] == o_words[wl]).all(), r
        assert du[keep].max() <= 1 and (du > 0).sum() <= 2, r
        same = el & np.repeat(du == 0, chunk)[:n]
        assert (ge[same].view(np.uint32) == e[same].view(np.uint32)).all(), r
        assert (np.abs(sc[apart] - o_scales[apart]) <= 1e-5 * np.abs(o_scales[apart])).all(), r
        apart |= du > 0
    assert apart.sum() <= 2


@pytest.mark.parametrize("peers", list(range(1, 17)))
@pytest.mark.parametrize("mode", ["overwrite", "accumulate"])
def test_decode_matches_oracle(peers, mode):
    """Every peer count is its own kernel instance (1-2: the quarter-unit
    kernel; 3-8: the unit kernel with one store in flight per wave; 9-16: the
    unit kernel with the peers past the table added per element)."""
    _decode_case(peers, mode, 3 * 2048 + 1001, 2048)


@pytest.mark.parametrize("peers", [2, 5, 8, 12])
def test_decode_matches_oracle_1024_chunks(peers):
    """1024-element chunks: a 2048-element unit spans two chunks (two tables)."""
    _decode_case(peers, "accumulate", 5 * 2048 + 777, 1024)


def _decode_case(peers, mode, n, chunk):
    say("decode peers", peers, mode, "n", n, "chunk", chunk)
    payloads, dev_payloads = [], []
    for k in range(peers):
        x, e = _inputs(n, 100 + k)
        w, s, _ = O.onebit_compress(x, e, chunk)
        payloads.append((w, s))
        dev_payloads.append((torch.from_numpy(w.view(np.int32)).cuda(), _dev(s)))
    base = np.random.default_rng(7).standard_normal(n).astype(np.float32)
    acc = mode == "accumulate"
    want = O.onebit_decompress(payloads, n, chunk, base.copy(), acc)
    dst = _dev(base)
    zds.zds_onebit_decompress(dev_payloads, chunk, dst, zds.ZDS_ACCUMULATE if acc else zds.ZDS_OVERWRITE)
    torch.cuda.synchronize()
    assert (to_host(dst).view(np.uint32) == want.view(np.uint32)).all()


def test_round_trip_and_edges():
    n, chunk = 50_000, 1024
    x, e = _inputs(n, 3)
    words, scales = zds.onebit_payload(n, chunk)
    de = _dev(e)
    zds.zds_onebit_compress(_dev(x), de, chunk, words, scales)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    zds.zds_onebit_decompress([(words, scales)], chunk, out)
    torch.cuda.synchronize()
    d, c = to_host(out), x + e
    assert ((d > 0) == (c >= 0)).all()
    resid = np.abs(d.astype(np.float64) + to_host(de).astype(np.float64) - c.astype(np.float64))
    assert (resid <= np.spacing(np.abs(to_host(de))) / 2).all()
    # empty input launches nothing; bad chunk, peers or alignment are refused
    zds.zds_onebit_compress(_dev(x[:0]), None, chunk, words, scales, n=0)
    for bad in (512, 3072, 32768):
        with pytest.raises(zds.ZdsError) as ex:
            zds.zds_onebit_compress(_dev(x), None, bad, words, scales)
        assert ex.value.status == zds.ZDS_EINVAL
    with pytest.raises(zds.ZdsError) as ex:
        zds.zds_onebit_compress(_dev(x)[1:], None, chunk, words, scales)
    assert ex.value.status == zds.ZDS_EALIGN
    with pytest.raises(zds.ZdsError) as ex:
        zds.zds_onebit_decompress([(words, scales)] * 17, chunk, out)
    assert ex.value.status == zds.ZDS_EINVAL
    # a NaN makes its chunk's scale NaN
    x2 = x.copy()
    x2[5000] = np.nan
    zds.zds_onebit_compress(_dev(x2), None, chunk, words, scales)
    s = to_host(scales)
    assert np.isnan(s[5000 // chunk]) and np.isfinite(np.delete(s, 5000 // chunk)).all()
