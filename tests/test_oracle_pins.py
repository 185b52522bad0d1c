"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (the pages' printed numbers, closed forms, exact rational or
high-precision decimal arithmetic, brute-force enumeration, format
definitions), chosen so that a dropped term, a wrong sign or index or a
swapped operand in the oracle fails at least one of them."""

import decimal
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import llama_7b_tensors, llama_65b_tensors, llama_7b_split_1024, tiny_shard_sizes

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))

PSI_7B = 6_738_411_520
PSI_65B = 65_285_652_480


# ---------------------------------------------------------------- accounting

def test_accounting_pages_numbers():
    g = GOLDEN["bytes_per_param_mixed_adam"]
    assert O.state_bytes_ddp(1) == g["total"] == g["fp16_param"] + g["fp16_grad"] + 12
    s = GOLDEN["seven_b_static_bytes"]
    assert O.state_bytes_ddp(s["psi"]) == s["bytes"]


def test_accounting_brute_force_bytes():
    """Materialise each stage's per-rank buffers as real arrays and count."""
    for psi in (96, 840):
        for n in (1, 2, 3, 4, 8):
            if psi % n:
                continue
            sh = psi // n
            full16 = np.zeros(psi, np.float16).nbytes
            shard16 = np.zeros(sh, np.float16).nbytes
            shard32x3 = 3 * np.zeros(sh, np.float32).nbytes
            full32x3 = 3 * np.zeros(psi, np.float32).nbytes
            assert O.state_bytes_ddp(psi) == 2 * full16 + full32x3
            assert O.state_bytes_stage1(psi, n) == 2 * full16 + shard32x3
            assert O.state_bytes_stage2(psi, n) == full16 + shard16 + shard32x3
            assert O.state_bytes_stage3(psi, n) == 2 * shard16 + shard32x3


def test_accounting_limits_and_n1():
    r = GOLDEN["memory_reduction_approx"]
    big = 10 ** 12
    psi = 7 * 10 ** 9
    assert abs(float(O.state_bytes_ddp(psi) / O.state_bytes_stage1(psi, big)) - r["stage1"]) < 1e-6
    assert abs(float(O.state_bytes_ddp(psi) / O.state_bytes_stage2(psi, big)) - r["stage2"]) < 1e-6
    for f in (O.state_bytes_stage1, O.state_bytes_stage2, O.state_bytes_stage3):
        assert f(psi, 1) == 16 * psi
    # at N = 8 the reduction is well short of the limits
    assert round(float(Fraction(16) / Fraction(O.state_bytes_stage1(1, 8))), 2) == 2.91
    assert round(float(Fraction(16) / Fraction(O.state_bytes_stage2(1, 8))), 2) == 4.27


def test_accounting_workload_footprints():
    assert sum(n for _, n in llama_7b_tensors()) == PSI_7B
    assert sum(n for _, n in llama_65b_tensors()) == PSI_65B
    assert O.state_bytes_ddp(PSI_7B) == 107_814_584_320          # whole 7B, ~108 GB
    assert O.state_bytes_stage3(PSI_65B, 8) == 130_571_304_960    # 65B 1/8 shard, ~130 GB


def test_accumulation_example():
    g = GOLDEN["grad_accumulation_example"]
    assert g["global_batch"] // (g["gpus"] * g["micro_batch"]) == g["accumulation_steps"]


# ---------------------------------------------------------------- layout

def _brute_flat(numels, align):
    """Flat buffer of (tensor id, index) labels, -1 for padding, built
    element by element."""
    lab_t, lab_i = [], []
    for t, n in enumerate(numels):
        while len(lab_t) % align:
            lab_t.append(-1)
            lab_i.append(-1)
        lab_t.extend([t] * n)
        lab_i.extend(range(n))
    while len(lab_t) % align:
        lab_t.append(-1)
        lab_i.append(-1)
    return np.array(lab_t), np.array(lab_i)


@pytest.mark.parametrize("seed", range(12))
def test_shard_entries_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(1, 300, T)]
    align = int(rng.choice([1, 4, 8, 64]))
    world = int(rng.integers(1, 9))
    lab_t, lab_i = _brute_flat(numels, align)
    _, total = O.flat_layout(numels, align)
    assert total == len(lab_t)
    padded = total
    while padded % (world * align):
        padded += 1
    lab_t = np.concatenate([lab_t, -np.ones(padded - total, int)])
    lab_i = np.concatenate([lab_i, -np.ones(padded - total, int)])
    per = padded // world
    seen = np.zeros(padded, bool)
    for r in range(world):
        lo, hi = O.shard_range(total, world, r, align)
        assert (lo, hi) == (r * per, (r + 1) * per)
        for t, s, n, d in O.shard_entries(numels, align, lo, hi):
            seg_t = lab_t[lo + d: lo + d + n]
            seg_i = lab_i[lo + d: lo + d + n]
            assert (seg_t == t).all()
            assert (seg_i == np.arange(s, s + n)).all()
            assert not seen[lo + d: lo + d + n].any()
            seen[lo + d: lo + d + n] = True
    assert (seen == (lab_t >= 0)).all()


def test_shard_entries_llama():
    t7 = llama_7b_tensors()
    n7 = [n for _, n in t7]
    lo, hi = O.shard_range(PSI_7B, 8, 0, 64)
    assert hi - lo == 842_301_440
    e0 = O.shard_entries(n7, 64, lo, hi)
    assert len(e0) == 33
    assert t7[e0[-1][0]][0] == "gate3" and e0[-1][1] == 0 and e0[-1][2] == 36_970_496
    lo, hi = O.shard_range(PSI_7B, 8, 7, 64)
    e7 = O.shard_entries(n7, 64, lo, hi)
    assert len(e7) == 33
    assert t7[e7[0][0]][0] == "gate28" and e7[0][1] == 31_195_136 and e7[0][2] == 13_893_632
    t65 = llama_65b_tensors()
    lo, hi = O.shard_range(PSI_65B, 8, 0, 64)
    e = O.shard_entries([n for _, n in t65], 64, lo, hi)
    assert hi - lo == 8_160_706_560 and len(e) == 88
    assert t65[e[-1][0]][0] == "up9" and e[-1][1] == 0 and e[-1][2] == 164_118_528
    s1024 = llama_7b_split_1024()
    assert len(s1024) == 1024 and sum(n for _, n in s1024) == PSI_7B
    tiny = tiny_shard_sizes()
    assert sum(n for _, n in tiny) == 733_953


def test_round_robin_demo_partition():
    d = GOLDEN["zero1_demo"]
    names = ["w%d" % i for i in range(len(d["sizes"]))]
    assert O.round_robin_owners(names, d["world_size"]) == [["w0"], ["w1"], ["w2"], []]


# ---------------------------------------------------------------- formats

def _fp16_by_definition(h):
    s = -1.0 if h >> 15 else 1.0
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 0x1F:
        return s * math.inf if f == 0 else math.nan
    if e == 0:
        return s * math.ldexp(f, -24)
    return s * math.ldexp(1024 + f, e - 25)


def test_widen_fp16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        w = O.widen(bits, O.FP16).astype(np.float64)
    ref = np.array([_fp16_by_definition(int(h)) for h in range(65536)])
    same = (w == ref) | (np.isnan(w) & np.isnan(ref))
    assert same.all()


def test_widen_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = O.widen(bits, O.BF16)
    ref = [struct.unpack(">f", struct.pack(">HH", h, 0))[0] for h in range(65536)]
    for a, b in zip(w.tolist(), ref):
        assert (a == b and math.copysign(1, a) == math.copysign(1, b)) or (math.isnan(a) and math.isnan(b))


def _bf16_value(pat):
    return Fraction(struct.unpack("<f", struct.pack("<I", pat << 16))[0])


def _bf16_rne_exact(u32):
    """Nearest-even bf16 pattern of the fp32 pattern u32, chosen by exact
    rational distances to the two neighbouring bf16 values; None for NaN."""
    x = struct.unpack("<f", struct.pack("<I", u32))[0]
    if math.isnan(x):
        return None
    lo_pat = u32 >> 16           # same sign, magnitude truncated
    if math.isinf(x):
        return lo_pat
    up_pat = lo_pat + 1          # next magnitude away from zero
    ax = abs(Fraction(x))
    if (up_pat & 0x7F80) == 0x7F80:
        # above the largest finite bf16 (2^128 - 2^120): overflow to inf at
        # half an ulp past it, the tie going to the even (infinite) side
        return up_pat if ax >= Fraction(2) ** 128 - Fraction(2) ** 119 else lo_pat
    dlo = ax - abs(_bf16_value(lo_pat))
    dup = abs(_bf16_value(up_pat)) - ax
    if dlo != dup:
        return lo_pat if dlo < dup else up_pat
    return lo_pat if (lo_pat & 1) == 0 else up_pat


def test_narrow_bf16_exact_rounding():
    rng = np.random.default_rng(5)
    his = rng.integers(0, 65536, 3000)
    los = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF])
    pats = [(int(h) << 16) | int(l) for h in his for l in los]
    pats += [int(x) for x in rng.integers(0, 2 ** 32, 4000, dtype=np.uint64)]
    pats += [0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0xFF7F8000, 0x00008000, 0x00018000]
    # NaNs whose payload lies only in the dropped half, or fills it: a
    # conversion of a NaN is a NaN (rounding them like numbers gives inf or -0)
    pats += [0x7F800001, 0xFF800001, 0x7F807FFF, 0x7F80FFFF, 0x7FBFFFFF, 0x7FFFFFFF, 0xFFFFFFFF]
    arr = np.array(pats, dtype=np.uint32)
    got = O.narrow(arr.view(np.float32), O.BF16)
    for p, g in zip(pats, got):
        want = _bf16_rne_exact(p)
        if want is None:
            assert (int(g) & 0x7F80) == 0x7F80 and (int(g) & 0x7F) != 0
        else:
            assert int(g) == want, hex(p)


def _fp16_rne_exact(x32):
    """Nearest-even fp16 pattern of an fp32 value from the binary16 grid: the
    quantum is 2^-24 below 2^-14 and 2^(e-10) in binade [2^e, 2^(e+1));
    magnitudes from 65504 + 16 up overflow to inf."""
    x = float(x32)
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(Fraction(x))
    if a >= Fraction(65520):
        return sign | 0x7C00
    if a < Fraction(1, 2 ** 14):
        q = Fraction(1, 2 ** 24)
    else:
        e = 0
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        q = Fraction(2) ** (e - 10)
    k = a / q
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign | int(np.float16(float(fl * q)).view(np.uint16))


def test_narrow_fp16_exact_rounding():
    rng = np.random.default_rng(6)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
        np.array([65504.0, 65519.99, 65520.0, 6.1035156e-05, 5.96e-08, 2.98e-08, 2.99e-08,
                  -0.0, 0.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11]),
    ]).astype(np.float32)
    got = O.narrow(vals, O.FP16)
    for x, g in zip(vals, got):
        want = _fp16_rne_exact(x)
        assert int(g) == want, (float(x), hex(int(g)), hex(want))


def test_nonfinite_detection_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    m16 = O.nonfinite_mask(bits, O.FP16)
    assert (m16 == ~np.isfinite(bits.view(np.float16))).all() and m16.sum() == 2048
    mb = O.nonfinite_mask(bits, O.BF16)
    ref = np.array([not math.isfinite(struct.unpack(">f", struct.pack(">HH", h, 0))[0])
                    for h in range(65536)])
    assert (mb == ref).all() and mb.sum() == 256
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    u[:4] = [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F7FFFFF]
    assert (O.nonfinite_mask(u.view(np.float32), O.FP32) == ~np.isfinite(u.view(np.float32))).all()


# ---------------------------------------------------------------- norm and clip

@pytest.mark.parametrize("dtype", [O.FP16, O.BF16, O.FP32])
def test_sum_of_squares_exact(dtype):
    rng = np.random.default_rng(7)
    for n in (1, 5, 333, 4096):
        x64 = rng.standard_normal(n) * 10.0 ** rng.integers(-3, 3, n)
        if dtype == O.FP16:
            x = x64.astype(np.float16).view(np.uint16)
        elif dtype == O.BF16:
            x = (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        else:
            x = x64.astype(np.float32)
        vals = O.widen(x, dtype)
        exact = sum((Fraction(float(v)) ** 2 for v in vals), Fraction(0))
        got = O.sum_of_squares(x, dtype)
        assert abs(Fraction(got) - exact) <= exact * Fraction(n + 1, 2 ** 53)


def test_norm_special_cases():
    z = np.zeros(1000, np.float32)
    assert O.sum_of_squares(z, O.FP32) == 0.0
    x = np.zeros(999, np.float16)
    x[417] = np.float16(-3.5)
    bits = x.view(np.uint16)
    s = O.sum_of_squares(bits, O.FP16)
    assert s == 12.25
    norm, coef, gs = O.clip_scalars(s, 2.0 ** 10, 4, 0.0)
    assert norm == 3.5 / (2 ** 10 * 4) and coef == 1.0 and gs == np.float32(1.0 / 4096)
    rng = np.random.default_rng(3)
    y = rng.standard_normal(5000).astype(np.float32)
    a = O.sum_of_squares(y, O.FP32)
    b = O.sum_of_squares(y[rng.permutation(5000)], O.FP32)
    assert abs(a - b) <= 1e-15 * a


def test_clip_brings_norm_to_max():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * 0.05 * 1024).astype(np.float16).view(np.uint16)
    S, K, mx = 1024.0, 2, 1.0
    s = O.sum_of_squares(x, O.FP16)
    norm, coef, gs = O.clip_scalars(s, S, K, mx)
    assert norm > mx and coef < 1.0
    g = O.widen(x, O.FP16).astype(np.float64) * float(gs)
    assert abs(math.sqrt(float(np.sum(g * g))) - mx) < 1e-6
    # below the threshold nothing is clipped
    _, coef2, gs2 = O.clip_scalars(s, S, K, 10 * norm)
    assert coef2 == 1.0 and gs2 == np.float32(1.0 / (S * K))


def test_clip_matches_the_library_global_norm_clip():
    """The conventional global-norm clip as PyTorch implements it
    (torch.nn.utils.clip_grad_norm_ multiplies the grads by
    min(1, max_norm / (norm + 1e-6))) against clip_scalars: the norm and the
    coefficient agree, the 1e-6 included, away from the 1e-6-wide band just
    below max_norm where the two readings differ (clip_scalars leaves grads
    whose norm is at most max_norm unscaled)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    S, K = 2.0 ** 12, 4
    for max_norm in (0.3, 1.0, 5.0):
        for ratio in (0.25, 0.9, 0.9995, 1.01, 1.5, 2.0, 10.0, 1000.0):
            base = rng.standard_normal(3000)
            g = base / np.linalg.norm(base) * max_norm * ratio
            x = (g * S * K).astype(np.float32)  # the raw grads the step sees
            norm, coef, gs = O.clip_scalars(O.sum_of_squares(x, O.FP32), S, K, max_norm)
            gt = torch.from_numpy(x.astype(np.float64) / (S * K))
            p = torch.zeros_like(gt, requires_grad=True)
            p.grad = gt.clone()
            total = float(torch.nn.utils.clip_grad_norm_([p], max_norm))
            nz = gt != 0
            factor = float((p.grad[nz] / gt[nz]).mean())
            assert abs(total - norm) <= 1e-12 * norm, (max_norm, ratio)
            assert abs(coef - factor) <= 1e-12 * factor, (max_norm, ratio, coef, factor)
            assert gs == np.float32(coef / (S * K))


def test_overflow_and_norm_flags():
    x = np.ones(100, np.float16)
    x[37] = np.inf
    r = O.overflow_and_norm(x.view(np.uint16), O.FP16, 1.0, 1, 1.0)
    assert r["overflow"] == 1
    x[37] = np.nan
    assert O.overflow_and_norm(x.view(np.uint16), O.FP16, 1.0, 1, 1.0)["overflow"] == 1
    x[37] = 65504
    assert O.overflow_and_norm(x.view(np.uint16), O.FP16, 1.0, 1, 1.0)["overflow"] == 0
    # an overflowing step is skipped: it reports an infinite norm, no
    # clipping and a grad factor of 0 (nothing may be applied)
    x[37] = -np.inf
    r = O.overflow_and_norm(x.view(np.uint16), O.FP16, 1.0, 1, 1.0)
    assert r["norm"] == np.inf and r["coef"] == 1.0 and r["grad_scale"] == 0.0


# ---------------------------------------------------------------- accumulation

def test_accumulate_identical_microbatches():
    rng = np.random.default_rng(8)
    numels = [37, 1000, 5]
    src = [(rng.standard_normal(n) * 1e-3 * 2 ** 14).astype(np.float16).view(np.uint16)
           for n in numels]
    ent = O.shard_entries(numels, 8, 0, O.flat_layout(numels, 8)[1])
    for K in (1, 2, 4, 16):
        acc = np.full(O.flat_layout(numels, 8)[1], np.float32(np.nan))
        O.flatten_accumulate(src, O.FP16, ent, acc, overwrite=True)
        for _ in range(K - 1):
            O.flatten_accumulate(src, O.FP16, ent, acc, overwrite=False)
        for t, s, n, d in ent:
            assert (acc[d:d + n] / np.float32(K) == O.widen(src[t], O.FP16)).all()
    bucket = np.zeros(O.flat_layout(numels, 8)[1], np.uint16)
    O.flatten_copy(src, ent, bucket)
    assert (bucket[ent[1][3]:ent[1][3] + 1000] == src[1]).all()


def _labelled_flat(numels, align, world, label):
    """The flat buffer written out element by element from its definition:
    tensor i starts at the next multiple of `align` after tensor i-1 ends, the
    buffer is padded to a multiple of world * align; padding holds None."""
    flat = []
    for t, n in enumerate(numels):
        while len(flat) % align:
            flat.append(None)
        flat.extend(label(t, i) for i in range(n))
    while len(flat) % (world * align):
        flat.append(None)
    return flat


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flatten_at_shard_edges_labelled(seed):
    """Stage-1 slices cut tensors mid-way ([csdn] §2.4 each rank updates its own
    part; §3.2 contiguous_gradients), so a rank's first and last entries start
    or end inside a tensor. Every source element carries a label that names
    its tensor and its index inside the tensor; each rank's flatten (copy,
    overwrite and += modes) must put exactly the labels the definition of the
    flat buffer puts at each of its positions, and leave padding alone."""
    rng = np.random.default_rng(700 + seed)
    for world in (2, 3, 8):
        numels = [int(x) for x in rng.integers(1, 400, size=int(rng.integers(1, 9)))]
        align = int(rng.choice([1, 8, 64]))
        # copy mode moves bit patterns: any 16-bit label will do
        lab16 = lambda t, i: (t * 40503 + i * 2654435761 + 17) & 0xFFFF  # noqa: E731
        # fp32 modes: small integers, exact in fp16 and bf16 and in their sums
        labint = {O.FP16: lambda t, i: (t * 7 + i) % 2039 - 1000,
                  O.BF16: lambda t, i: (t * 7 + i) % 251 - 125}
        srcs16 = [np.array([lab16(t, i) for i in range(n)], np.uint16) for t, n in enumerate(numels)]
        flat16 = _labelled_flat(numels, align, world, lab16)
        per = len(flat16) // world
        for rank in range(world):
            lo, hi = rank * per, (rank + 1) * per
            ent = O.shard_entries(numels, align, lo, hi)
            sentinel = 0xABCD
            bucket = O.flatten_copy(srcs16, ent, np.full(hi - lo, sentinel, np.uint16))
            want = [sentinel if x is None else x for x in flat16[lo:hi]]
            assert bucket.tolist() == want, (world, rank)
            for dt, lab in labint.items():
                srcs = [np.array([lab(t, i) for i in range(n)], np.float32) for t, n in enumerate(numels)]
                srcs = [O.narrow(s, dt) for s in srcs]
                flat = _labelled_flat(numels, align, world, lab)[lo:hi]
                init = rng.integers(-3000, 3000, size=hi - lo).astype(np.float32)
                acc = O.flatten_accumulate(srcs, dt, ent, init.copy(), overwrite=True)
                assert acc.tolist() == [float(i) if x is None else float(x) for x, i in zip(flat, init)]
                acc = O.flatten_accumulate(srcs, dt, ent, init.copy(), overwrite=False)
                assert acc.tolist() == [float(i) if x is None else float(i) + x for x, i in zip(flat, init)]


def test_flatten_llama_rank7_starts_inside_gate28():
    """The 7B shard of rank 7 of 8 starts 31,195,136 elements into the 28th
    layer's gate projection; its first bucket element is that tensor's element
    at that index (checked on a labelled stand-in of the tensor's tail)."""
    numels = [n for _, n in llama_7b_tensors()]
    _, total = O.flat_layout(numels, 64)
    lo, hi = O.shard_range(total, 8, 7, 64)
    ent = O.shard_entries(numels, 64, lo, hi)
    t0, s0, n0, d0 = ent[0]
    assert (s0, n0, d0) == (31_195_136, 13_893_632, 0)
    srcs = {t0: np.arange(numels[t0], dtype=np.int64).astype(np.uint16)}
    bucket = O.flatten_copy(srcs, [ent[0]], np.zeros(n0, np.uint16))
    assert bucket[0] == 31_195_136 & 0xFFFF and bucket[-1] == (31_195_136 + n0 - 1) & 0xFFFF
    assert (np.diff(bucket.astype(np.int64)) % 65536 == 1).all()


def test_accumulated_step_equals_single_step():
    """K identical micro-batches with the mean folded into grad_scale give the
    same update, bit for bit, as one micro-batch."""
    rng = np.random.default_rng(9)
    n = 3000
    x = (rng.standard_normal(n) * 1e-3 * 2 ** 14).astype(np.float16).view(np.uint16)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hp = O.AdamW()
    st = O.scaler_init(initial_scale_power=14)
    r1 = O.optimizer_step(x, O.FP16, master, m, v, st, hp, 1.0, 1, O.FP16)
    acc = O.widen(x, O.FP16).copy()
    for _ in range(15):
        acc = acc + O.widen(x, O.FP16)
    r16 = O.optimizer_step(acc, O.FP32, master, m, v, st, hp, 1.0, 16, O.FP16)
    for a, b in zip(r1[:4], r16[:4]):
        assert (a.view(np.uint32 if a.dtype == np.float32 else np.uint16) ==
                b.view(np.uint32 if b.dtype == np.float32 else np.uint16)).all()


# ---------------------------------------------------------------- loss scaler

def test_scaler_tiny_config_trajectory():
    """Five steps, +inf in step 3's grads, dynamic scaler from 2^16 with
    hysteresis 1: the scales in force are 2^16, 2^16, 2^16, 2^15, 2^15 and Adam
    steps 1, 2, (skipped), 3, 4 are applied."""
    st = O.scaler_init(initial_scale_power=16, window=1000, hysteresis=1)
    scales, ts = [], []
    for k in range(1, 6):
        scales.append(st.scale)
        st = O.scaler_update(st, 1 if k == 3 else 0, 0.9, 0.999)
        ts.append(None if st.last_skip else st.t)
    assert scales == [2.0 ** 16] * 3 + [2.0 ** 15] * 2
    assert ts == [1, 2, None, 3, 4]


def _scale_by_runs(seq, init, W, H, mn):
    """Independent statement of the scaler: walk maximal runs of equal flags.
    A clean run of length L grows the scale floor((g0 + L) / W) times, where g0
    is the clean count carried in (0 after any overflow). An overflow run of
    length R halves the scale once per H overflows in it, floored at min."""
    scale = init
    carried = 0
    i = 0
    while i < len(seq):
        j = i
        while j < len(seq) and seq[j] == seq[i]:
            j += 1
        L = j - i
        if seq[i] == 0:
            total = carried + L
            scale *= 2.0 ** (total // W)
            carried = total % W
        else:
            for _ in range(L // H):
                scale = max(scale / 2.0, mn)
            carried = 0
        i = j
    return scale


def test_scaler_brute_force_all_sequences():
    import itertools
    for W in (1, 2, 3):
        for H in (1, 2):
            for L in range(0, 11):
                for seq in itertools.product((0, 1), repeat=L):
                    st = O.scaler_init(initial_scale_power=4, window=W, hysteresis=H, min_scale=1.0)
                    for f in seq:
                        st = O.scaler_update(st, f, 0.9, 0.999)
                    assert st.scale == _scale_by_runs(seq, 16.0, W, H, 1.0), (W, H, seq)
                    assert st.t == len(seq) - sum(seq)


def test_scaler_hysteresis1_matches_the_library_amp_scaler():
    """With hysteresis 1 the dynamic scaler is the one PyTorch's AMP grad
    scaler runs (torch._amp_update_scale_: halve on an overflow and reset the
    clean-step count; double after `window` clean steps): scale and count
    agree on random overflow sequences, the floor kept out of reach."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    # (window, overflow probability) pairs whose random walks stay between
    # the floor and the 2^127 cap
    for W, p_ovf in ((1, 0.4), (1, 0.5), (1, 0.6), (2, 0.2), (2, 0.35), (5, 0.05), (5, 0.12), (13, 0.02),
                     (13, 0.06)):
        st = O.scaler_init(initial_scale_power=16, window=W, hysteresis=1, min_scale=2.0 ** -100)
        scale = torch.tensor([2.0 ** 16])
        tracker = torch.tensor([0], dtype=torch.int32)
        found = torch.tensor([0.0])
        for f in (rng.random(200) < p_ovf).astype(int):
            st = O.scaler_update(st, int(f), 0.9, 0.999)
            assert st.min_scale < st.scale < 2.0 ** 127  # neither bound binds here
            found.fill_(float(f))
            torch._amp_update_scale_(scale, tracker, found, 2.0, 0.5, W)
            assert st.scale == float(scale) and st.good_steps == int(tracker), (W, p_ovf)


def test_scaler_static_and_floor():
    st = O.scaler_init(dynamic=False, static_scale=1.0)
    for f in (1, 0, 1, 1, 0):
        st = O.scaler_update(st, f, 0.9, 0.999)
        assert st.scale == 1.0 and st.last_skip == f
    assert st.t == 2
    st = O.scaler_init(initial_scale_power=2, hysteresis=1, min_scale=1.0)
    for _ in range(6):
        st = O.scaler_update(st, 1, 0.9, 0.999)
        assert st.last_skip == 1
    assert st.scale == 1.0 and st.t == 0


def test_scaler_growth_saturates_at_2_127():
    # the scale is an fp32 power of two, so growth stops at the largest one
    st = O.scaler_init(initial_scale_power=126, window=1)
    for k in range(3):
        st = O.scaler_update(st, 0, 0.9, 0.999)
        assert st.scale == 2.0 ** 127 and st.good_steps == 0
    assert st.t == 3


def test_beta_powers():
    st = O.scaler_init()
    for _ in range(50):
        st = O.scaler_update(st, 0, 0.9, 0.999)
    b1 = Fraction(float(np.float32(0.9)))
    b2 = Fraction(float(np.float32(0.999)))
    assert abs(Fraction(st.beta1_pow) - b1 ** 50) <= b1 ** 50 * Fraction(60, 2 ** 53)
    assert abs(Fraction(st.beta2_pow) - b2 ** 50) <= b2 ** 50 * Fraction(60, 2 ** 53)


# ---------------------------------------------------------------- AdamW

def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(np.maximum(x, np.float32(1.1754944e-38))).astype(np.float64)


@pytest.mark.parametrize("sigma", [1e-8, 1e-6, 1e-3, 1.0])
def test_adamw_first_step_closed_form(sigma):
    """With zero moments at t = 0 the bias-corrected first update is
    lr * g / (|g| + eps)."""
    rng = np.random.default_rng(11)
    n = 100000
    g = (rng.standard_normal(n) * sigma).astype(np.float32)
    hp = O.AdamW(lr=1e-3, weight_decay=0.01)
    c = O.adamw_constants(hp, 1.0, 1.0)
    p, m, v = O.adamw_update(g, O.FP32, np.float32(1.0), np.zeros(n, np.float32),
                             np.zeros(n, np.float32), np.zeros(n, np.float32), c)
    g64 = g.astype(np.float64)
    closed = -1e-3 * g64 / (np.abs(g64) + 1e-8)
    err = np.abs(p.astype(np.float64) - closed) / _ulp32(np.float32(1e-3))
    assert err.max() <= 4.0


def test_bias_correction_cancels_at_t1():
    c = O.adamw_constants(O.AdamW(), 1.0, 1.0)
    assert np.float32(1.0 - float(np.float32(0.9))) == c["omb1"]
    assert np.float32(1.0 - float(np.float32(0.999))) == c["omb2"]


def _adamw_decimal(g, p, m, v, lr, b1, b2, eps, wd, b1pow, b2pow):
    """Real-number AdamW (decoupled decay, bias correction) in 60-digit
    decimal arithmetic from the exact values of the fp32 inputs."""
    D = decimal.Decimal
    g, p, m, v = D(float(g)), D(float(p)), D(float(m)), D(float(v))
    lr, b1, b2, eps, wd = (D(float(np.float32(t))) for t in (lr, b1, b2, eps, wd))
    bp1 = D(b1pow) * b1
    bp2 = D(b2pow) * b2
    m1 = b1 * m + (1 - b1) * g
    v1 = b2 * v + (1 - b2) * g * g
    upd = (lr / (1 - bp1)) * m1 / (v1.sqrt() / (1 - bp2).sqrt() + eps)
    return p * (1 - lr * wd) - upd, m1, v1, abs(upd), abs(p * (1 - lr * wd))


def test_adamw_against_high_precision():
    decimal.getcontext().prec = 60
    rng = np.random.default_rng(12)
    n = 2048
    hp = O.AdamW(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    for t_prev, gsig in ((0, 1e-3), (1, 2e-3), (7, 1.0), (100, 1e-7)):
        b1p = float(np.float32(0.9)) ** t_prev
        b2p = float(np.float32(0.999)) ** t_prev
        g = (rng.standard_normal(n) * gsig).astype(np.float32)
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * gsig * 0.1).astype(np.float32) if t_prev else np.zeros(n, np.float32)
        v = ((rng.standard_normal(n) * gsig) ** 2 * 1e-3).astype(np.float32) if t_prev else np.zeros(n, np.float32)
        c = O.adamw_constants(hp, b1p, b2p)
        P, M, V = O.adamw_update(g, O.FP32, np.float32(1.0), p, m, v, c)
        for i in range(n):
            pe, me, ve, au, ap = _adamw_decimal(g[i], p[i], m[i], v[i], hp.lr, hp.beta1, hp.beta2,
                                                hp.eps, hp.weight_decay, b1p, b2p)
            # m: three roundings; the sum may cancel, so bound by its operands
            bm = _ulp32(np.float32(0.9) * m[i]) + _ulp32(np.float32(0.1) * g[i]) + _ulp32(M[i])
            assert abs(decimal.Decimal(float(M[i])) - me) <= decimal.Decimal(float(bm))
            # v: all terms non-negative, a few roundings relative to the result
            assert abs(decimal.Decimal(float(V[i])) - ve) <= decimal.Decimal(2.5 * _ulp32(V[i]))
            # p: error bounded by a few ulp of the larger operand of the last subtraction
            bound = 6.0 * max(_ulp32(np.float32(float(au))), _ulp32(np.float32(float(ap)))) + _ulp32(P[i])
            assert abs(decimal.Decimal(float(P[i])) - pe) <= decimal.Decimal(float(bound)), (t_prev, i)


def test_adamw_special_cases():
    hp = O.AdamW()
    c = O.adamw_constants(hp, 0.9, 0.999)
    p0 = np.array([0.5, -0.25, 0.0, 1e-20], np.float32)
    m0 = np.array([1e-3, 0.0, -2e-4, 0.0], np.float32)
    v0 = np.array([1e-6, 0.0, 1e-8, 0.0], np.float32)
    P, M, V = O.adamw_update(np.zeros(4, np.float32), O.FP32, np.float32(1.0), p0, m0, v0, c)
    assert (M == c["b1"] * m0).all() and (V == c["b2"] * v0).all()
    assert P[1] == p0[1] * c["decay"] and P[3] == p0[3] * c["decay"]
    # large |g|: the Adam term has magnitude close to lr
    g = np.array([3.0, -5.0], np.float32)
    cc = O.adamw_constants(hp, 1.0, 1.0)
    P, _, _ = O.adamw_update(g, O.FP32, np.float32(1.0), np.array([0.1, 0.1], np.float32),
                             np.zeros(2, np.float32), np.zeros(2, np.float32), cc)
    d = P - np.float32(0.1) * cc["decay"]
    assert np.allclose(d, [-1e-3, 1e-3], rtol=1e-5)


def test_zero1_demo_update():
    """Demo variant: no bias correction, no decay, lr 0.01, every grad 1/4.
    Each element moves down by lr*0.1*g / (sqrt(0.001)*g + 1e-8)."""
    d = GOLDEN["zero1_demo"]
    hp = O.AdamW(lr=d["lr"], beta1=d["beta1"], beta2=d["beta2"], eps=d["eps"], weight_decay=0.0)
    c = O.adamw_constants(hp, 1.0, 1.0, bias_correction=False)
    n = sum(d["sizes"])
    g = np.full(n, 1.0 / d["world_size"], np.float32)
    p0 = np.random.default_rng(0).standard_normal(n).astype(np.float32)
    P, _, _ = O.adamw_update(g, O.FP32, np.float32(1.0), p0, np.zeros(n, np.float32),
                             np.zeros(n, np.float32), c)
    decimal.getcontext().prec = 40
    D = decimal.Decimal
    gg = D(1) / D(4)
    closed = D("0.01") * D("0.1") * gg / (D("0.001").sqrt() * gg + D("1e-8"))
    assert abs(float(closed) - 0.0316227366) < 1e-10
    drop = p0.astype(np.float64) - P.astype(np.float64)
    assert np.max(np.abs(drop - float(closed))) <= 2 * np.max(_ulp32(p0)) + 1e-9


# ---------------------------------------------------------------- whole step

def test_stage1_concat_invariant():
    rng = np.random.default_rng(13)
    numels = [int(s) for s in rng.integers(1, 5000, 9)]
    _, total = O.flat_layout(numels, 64)
    x = np.zeros(total, np.uint16)
    off, _ = O.flat_layout(numels, 64)
    for o, n in zip(off, numels):
        x[o:o + n] = (rng.standard_normal(n) * 1e-3 * 2 ** 16).astype(np.float16).view(np.uint16)
    master = np.zeros(total, np.float32)
    for o, n in zip(off, numels):
        master[o:o + n] = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = O.AdamW()
    st = O.scaler_init()
    full = O.optimizer_step(x, O.FP16, master, np.zeros(total, np.float32),
                            np.zeros(total, np.float32), st, hp, 1.0, 1, O.FP16)
    for N in (1, 2, 3, 4, 7, 8):
        padded = O.align_up(total, N * 64)
        xp = np.concatenate([x, np.zeros(padded - total, np.uint16)])
        mp = np.concatenate([master, np.zeros(padded - total, np.float32)])
        ssq = 0.0
        pieces = []
        for r in range(N):
            lo, hi = O.shard_range(total, N, r, 64)
            ssq += O.sum_of_squares(xp[lo:hi], O.FP16)
            pieces.append((lo, hi))
        assert abs(ssq - full[5]["sumsq"]) <= 1e-12 * full[5]["sumsq"]
        norm, coef, gs = O.clip_scalars(full[5]["sumsq"], st.scale, 1, 1.0)
        c = O.adamw_constants(hp, st.beta1_pow, st.beta2_pow)
        outs = [O.adamw_update(xp[lo:hi], O.FP16, gs, mp[lo:hi], np.zeros(hi - lo, np.float32),
                               np.zeros(hi - lo, np.float32), c) for lo, hi in pieces]
        for k in range(3):
            cat = np.concatenate([o[k] for o in outs])[:total]
            assert (cat.view(np.uint32) == full[k].view(np.uint32)).all()
        # padding stays exactly zero
        assert (np.concatenate([o[0] for o in outs])[total:] == 0).all()


def test_step_params_are_the_cast_of_the_new_master():
    # the 16-bit params written by a step are the round-to-nearest cast of the
    # master values it returns, element for element (checked on enough
    # elements that some lie within an fp32 ulp of a 16-bit rounding tie)
    rng = np.random.default_rng(16)
    n = 400000
    for gdt, pdt in ((O.FP16, O.FP16), (O.BF16, O.BF16), (O.FP32, O.BF16)):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        x = g if gdt == O.FP32 else O.narrow(g, gdt)
        master = (rng.standard_normal(n) * 0.05).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (rng.standard_normal(n) ** 2 * 1e-7).astype(np.float32)
        st = O.scaler_init(dynamic=False, t=3, beta1_pow=0.9 ** 3, beta2_pow=0.999 ** 3)
        r = O.optimizer_step(x, gdt, master, m, v, st, O.AdamW(), 1.0, 1, pdt)
        p = r[0].view(np.uint32).astype(np.uint64)
        if pdt == O.FP16:
            want = r[0].astype(np.float16).view(np.uint16)
        else:  # nearest bf16, ties to even, from the exact fp32 bits (no NaN here)
            lo = p & np.uint64(0xFFFF)
            hi = p >> np.uint64(16)
            up = (lo > np.uint64(0x8000)) | ((lo == np.uint64(0x8000)) & ((hi & np.uint64(1)) == np.uint64(1)))
            want = (hi + up.astype(np.uint64)).astype(np.uint16)
        assert (r[3] == want).all(), (gdt, pdt)


def test_overflow_step_leaves_state():
    rng = np.random.default_rng(14)
    n = 777
    x = (rng.standard_normal(n) * 1e-3 * 2 ** 16).astype(np.float16)
    x[n - 1] = np.inf
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.standard_normal(n) ** 2 * 1e-7).astype(np.float32)
    st = O.scaler_init(t=5, beta1_pow=0.9 ** 5, beta2_pow=0.999 ** 5)
    r = O.optimizer_step(x.view(np.uint16), O.FP16, master.copy(), m.copy(), v.copy(), st,
                         O.AdamW(), 1.0, 1, O.FP16)
    assert r[3] is None
    assert (r[0] == master).all() and (r[1] == m).all() and (r[2] == v).all()
    assert r[4].scale == st.scale / 2 and r[4].t == 5 and r[4].last_skip == 1
    assert r[4].beta1_pow == st.beta1_pow


# ---------------------------------------------------------------- Stage-2 intake

def test_reduce_peers_single_and_identical():
    rng = np.random.default_rng(30)
    x = (rng.standard_normal(5000) * 3).astype(np.float16).view(np.uint16)
    one = O.reduce_peer_slices([x], O.FP16, None, O.FP32, accumulate=False)
    assert (one.view(np.uint32) == O.widen(x, O.FP16).view(np.uint32)).all()
    for N in (2, 3, 7, 8, 16):
        s = O.reduce_peer_slices([x] * N, O.FP16, None, O.FP32, accumulate=False)
        # k * x needs at most 11 + log2(k) significand bits: every partial sum is exact
        assert (s == O.widen(x, O.FP16) * np.float32(N)).all()


def test_reduce_peers_exact_rational_bound():
    rng = np.random.default_rng(31)
    for N in (2, 5, 8):
        sl = [(rng.standard_normal(400) * 10.0 ** rng.integers(-3, 3, 400)).astype(np.float16).view(np.uint16)
              for _ in range(N)]
        got = O.reduce_peer_slices(sl, O.FP16, None, O.FP32, accumulate=False)
        for j in range(400):
            vals = [Fraction(float(O.widen(s[j:j + 1], O.FP16)[0])) for s in sl]
            exact = sum(vals, Fraction(0))
            mag = sum(abs(v) for v in vals)
            assert abs(Fraction(float(got[j])) - exact) <= mag * Fraction(N, 2 ** 24)


def test_reduce_peers_accumulate_and_16bit_destination():
    rng = np.random.default_rng(32)
    sl = [(rng.standard_normal(3000)).astype(np.float32) for _ in range(4)]
    bits = [(s.view(np.uint32) >> 16).astype(np.uint16) for s in sl]
    base = rng.standard_normal(3000).astype(np.float32)
    acc = O.reduce_peer_slices(bits, O.BF16, base.copy(), O.FP32, accumulate=True)
    plain = O.reduce_peer_slices(bits, O.BF16, None, O.FP32, accumulate=False)
    assert (acc == base + plain).all()
    # 16-bit destination: the fp32 sum rounded once, to nearest even
    out16 = O.reduce_peer_slices(bits, O.BF16, None, O.BF16, accumulate=False)
    for j in range(0, 3000, 7):
        assert int(out16[j]) == _bf16_rne_exact(int(plain[j:j + 1].view(np.uint32)[0]))


# ---------------------------------------------------------------- consolidation

def test_consolidate_hand_example():
    # tensors of 3 and 2 elements, align 4: t0 at 0, t1 at 4, total 8; two
    # ranks of 4 elements each (rank 0 = t0 + 1 pad, rank 1 = t1 + 2 pad)
    r0 = np.array([1, 2, 3, -7], np.float32)
    r1 = np.array([4, 5, -8, -9], np.float32)
    t = O.consolidate([(4, 8, r1), (0, 4, r0)], [3, 2], 4)
    assert [list(x) for x in t] == [[1, 2, 3], [4, 5]]
    # one rank per element, align 1
    t = O.consolidate([(i, i + 1, np.array([10 + i], np.float32)) for i in range(5)], [2, 0, 3], 1)
    assert [list(x) for x in t] == [[10, 11], [], [12, 13, 14]]


@pytest.mark.parametrize("seed", range(12))
def test_consolidate_inverts_the_partition(seed):
    # Brute force: place every tensor element at its flat index by hand, cut
    # the buffer into the world's equal slices, shuffle them, merge back.
    rng = np.random.default_rng(400 + seed)
    numels = [int(x) for x in rng.integers(0, 300, int(rng.integers(1, 12)))]
    align = int(rng.choice([1, 4, 16, 64]))
    world = int(rng.integers(1, 9))
    tensors = [rng.standard_normal(n).astype(np.float32) for n in numels]
    pos, flat_index = 0, []
    for n in numels:
        flat_index.append(list(range(pos, pos + n)))
        pos = -(-(pos + n) // align) * align
    padded = -(-pos // (world * align)) * (world * align)
    flat = np.full(padded, np.nan, np.float32)  # padding must never reach the output
    for t, idx in zip(tensors, flat_index):
        for v, i in zip(t, idx):
            flat[i] = v
    per = padded // world
    shards = [(r * per, (r + 1) * per, flat[r * per:(r + 1) * per]) for r in range(world)]
    assert all(O.shard_range(pos, world, r, align) == shards[r][:2] for r in range(world))
    order = rng.permutation(world)
    got = O.consolidate([shards[i] for i in order], numels, align)
    assert len(got) == len(tensors)
    for a, b in zip(got, tensors):
        assert a.dtype == np.float32 and (a.view(np.uint32) == b.view(np.uint32)).all()


def test_consolidate_rejects_gaps_and_overlaps():
    a = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        O.consolidate([(0, 4, a), (5, 9, a)], [8], 1)      # gap
    with pytest.raises(ValueError):
        O.consolidate([(0, 4, a), (3, 7, a)], [7], 1)      # overlap
    with pytest.raises(ValueError):
        O.consolidate([(0, 4, a)], [6], 1)                 # too short


# ---------------------------------------------------------------- 1-bit codec

def _f32_sqrt_of_fraction(q):
    """fp32 nearest to sqrt(q) for a rational q, from 60-digit decimal
    arithmetic (far from any rounding tie for the values used here)."""
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        r = (decimal.Decimal(q.numerator) / decimal.Decimal(q.denominator)).sqrt()
    return np.float32(float(r))


def test_onebit_hand_example():
    x = np.array([1, -2, 3, -4, 0, -0.0], np.float32)
    words, scales, err = O.onebit_compress(x, np.zeros(6, np.float32), 4)
    # signs + - + - (+0) (-0 counts as +); in the first unit and group,
    # element e sits in word e // 4 at bit e % 4
    assert words.dtype == np.uint32 and words.size == 64
    assert words[:2].tolist() == [0b0101, 0b11] and not words[2:].any()
    s = _f32_sqrt_of_fraction(Fraction(1 + 4 + 9 + 16, 4))
    assert scales[0] == s and scales[1] == 0.0
    assert err[:4].tolist() == [np.float32(1) - s, np.float32(-2) + s, np.float32(3) - s, np.float32(-4) + s]
    assert err[4] == 0.0 and err[5] == 0.0
    d = O.onebit_decompress([(words, scales)], 6, 4, None, accumulate=False)
    assert d.tolist() == [s, -s, s, -s, 0.0, 0.0]


def test_onebit_bit_layout():
    # element 2048u + 256r + 4l + i is bit 4r + i of word 64u + l
    n = 4700
    for i, (word, bit) in {0: (0, 0), 1: (0, 1), 3: (0, 3), 4: (1, 0), 255: (63, 3), 256: (0, 4), 259: (0, 7),
                           511: (63, 7), 1792: (0, 28), 2047: (63, 31), 2048: (64, 0), 2300: (127, 0),
                           4699: (150, 11)}.items():
        x = -np.ones(n, np.float32)
        x[i] = 1.0
        words, _, _ = O.onebit_compress(x, np.zeros(n, np.float32), 1024)
        want = np.zeros(192, np.uint32)
        want[word] = np.uint32(1) << np.uint32(bit)
        assert (words == want).all(), i
        assert O.onebit_signs(words, n).tolist() == [1.0 if j == i else -1.0 for j in range(n)]
    # NaN encodes as 0, and bits past the end stay 0: 40 elements fill the
    # low nibble of words 0..9
    x = np.ones(40, np.float32)
    x[3] = np.nan
    words, scales, err = O.onebit_compress(x, np.zeros(40, np.float32), 1024)
    assert words[:10].tolist() == [0x7] + [0xF] * 9 and not words[10:].any()
    assert np.isnan(scales[0]) and np.isnan(err).all()


@pytest.mark.parametrize("k", [-20, -3, 0, 5])
def test_onebit_equal_magnitudes_are_exact(k):
    rng = np.random.default_rng(50 + k)
    a = np.float32(2.0 ** k * 1.375)
    n = 3 * 256 + 17
    c = np.where(rng.random(n) < 0.5, a, -a).astype(np.float32)
    words, scales, err = O.onebit_compress(c, np.zeros(n, np.float32), 256)
    assert (scales == a).all() and (err == 0).all()
    assert (O.onebit_decompress([(words, scales)], n, 256, None, False) == c).all()
    # the error buffer is added before encoding: x + err with err = -x encodes zeros
    _, s0, e0 = O.onebit_compress(c, -c, 256)
    assert (s0 == 0).all() and (e0 == 0).all()


def test_onebit_partial_last_chunk_uses_its_length():
    n = 1024 + 3
    x = np.full(n, 0.5, np.float32)
    x[-3:] = np.float32(-3.0)
    _, scales, _ = O.onebit_compress(x, np.zeros(n, np.float32), 1024)
    assert scales.tolist() == [0.5, 3.0]


@pytest.mark.parametrize("seed", range(4))
def test_onebit_keeps_norm_and_loses_only_rounding(seed):
    rng = np.random.default_rng(60 + seed)
    n, chunk = 5000, 512
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-4, 2, n)).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    words, scales, err = O.onebit_compress(x, e, chunk)
    c = x + e
    for j in range(scales.size):
        a, b = j * chunk, min(n, (j + 1) * chunk)
        exact = sum((Fraction(float(v)) ** 2 for v in c[a:b]), Fraction(0))
        got = Fraction(float(scales[j])) ** 2 * (b - a)
        assert abs(got - exact) <= exact * Fraction(1, 2 ** 22)        # one fp32 rounding of the RMS
    d = O.onebit_decompress([(words, scales)], n, chunk, None, False)
    assert ((d > 0) == (c >= 0)).all()
    # decoded + new error == encoded input, up to the one rounding of the error
    resid = np.abs(d.astype(np.float64) + err.astype(np.float64) - c.astype(np.float64))
    assert (resid <= np.spacing(np.abs(err)).astype(np.float64) / 2 + 0.0).all()


def test_onebit_error_feedback_telescopes():
    # sum over T steps of what was sent + the final error == T * x + e0: the
    # compression loses nothing over time but rounding
    rng = np.random.default_rng(70)
    n, chunk, T = 3000, 256, 40
    x = rng.standard_normal(n).astype(np.float32)
    e = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    bound = np.zeros(n, np.float64)
    for _ in range(T):
        words, scales, e_new = O.onebit_compress(x, e, chunk)
        sent += O.onebit_decompress([(words, scales)], n, chunk, None, False)
        bound += np.spacing(np.abs(x + e)).astype(np.float64) + np.spacing(np.abs(e_new)).astype(np.float64)
        e = e_new
    assert (np.abs(sent + e - T * x.astype(np.float64)) <= bound).all()
    assert np.abs(sent / T - x).max() < np.abs(e).max() / T + 1e-5


def test_onebit_decompress_adds_peers_in_order():
    # 1 + 2^-24 is a tie that rounds to 1 (even), so adding the two small
    # scales one at a time after the large one leaves 1, while adding the
    # small ones first gives 1 + 2^-23
    n = chunk = 4
    words = np.zeros(64, np.uint32)
    words[0] = 0xF  # elements 0..3: bits 0..3 of word 0, all positive
    small = np.float32(2.0 ** -24)
    pay = [(words, np.array([1.0], np.float32)), (words, np.array([small])), (words, np.array([small]))]
    assert (O.onebit_decompress(pay, n, chunk, None, False) == np.float32(1.0)).all()
    assert (O.onebit_decompress(pay[::-1], n, chunk, None, False) == np.float32(1.0 + 2.0 ** -23)).all()


def test_onebit_scale_is_the_correctly_rounded_rms():
    # the scale is sqrt(S / len) for the exact sum of squares S; summing
    # rounded fp32 squares in fp32 gives another scale on some of these
    # chunks, which the last assertion makes sure of
    rng = np.random.default_rng(90)
    chunk, differ = 1024, 0
    for _ in range(48):
        c = (rng.standard_normal(chunk) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        _, scales, _ = O.onebit_compress(c, np.zeros(chunk, np.float32), chunk)
        S = sum(Fraction(float(v)) ** 2 for v in c)
        want = _f32_sqrt_of_fraction(S / chunk)
        assert scales[0] == want
        differ += np.float32(math.sqrt(float(np.sum(c * c)) / chunk)) != want
    assert differ >= 2, differ


def test_onebit_decompress_sums_peers_exactly():
    # power-of-two magnitudes: every partial sum is exact, so the peer sum is
    # the integer sum of the signed scales
    rng = np.random.default_rng(80)
    n, chunk, N = 2000, 128, 6
    payloads, ints = [], []
    for k in range(N):
        exps = rng.integers(-3, 4, -(-n // chunk))
        sgn = np.where(rng.random(n) < 0.5, 1, -1)
        mag = (2.0 ** exps[np.arange(n) // chunk]).astype(np.float32)
        words, scales, _ = O.onebit_compress((sgn * mag).astype(np.float32), np.zeros(n, np.float32), chunk)
        assert (scales == 2.0 ** exps).all()
        payloads.append((words, scales))
        ints.append(sgn * (2.0 ** (exps[np.arange(n) // chunk] + 3)))  # scaled by 8: integers
    want = np.sum(ints, axis=0) / 8.0
    got = O.onebit_decompress(payloads, n, chunk, None, False)
    assert (got == want).all()
    base = rng.standard_normal(n).astype(np.float32)
    assert (O.onebit_decompress(payloads, n, chunk, base.copy(), True) == base + got).all()
