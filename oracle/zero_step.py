"""CPU oracle: one data-parallel rank's share of the ZeRO mixed-precision
AdamW step, written out plainly in NumPy.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously-correct
definition the HIP library is checked against. Only the test suite, the
smoke check and the bench's CPU-baseline leg may import it. It shares no
code with the library and imports nothing from it.

Pages the definitions follow (cited by title and section below):
  [algomooc]  algomooc.com interview answer on the DeepSpeed framework
  [aidhplus]  aidhplus.com, "DeepSpeed" overview
  [csdn]      devpress.csdn.net DeepSpeed distributed-training tutorial
  [aiqz]      aiqz.cc, "DeepSpeed ZeRO引擎深入"
  [ch01]      jwzheng96.github.io llm-train-tutorials, DeepSpeed chapter 1

Arrays: 16-bit values (fp16, bf16) travel as their raw bit patterns
(np.uint16); fp32 arrays are np.float32. NumPy's float32 array arithmetic is
IEEE round-to-nearest-even, one rounding per operation and never fused, and
its float32 sqrt and divide are correctly rounded; the step below relies on
exactly that.

Pin status: every function here is pinned by a CPU test against closed
forms, exact rational arithmetic, brute force or the pages' printed numbers.
Two constants have no page behind them and are readings, not pins: the 1e-6
added to the norm in the clip coefficient, and the hysteresis rule for H > 1.
"""

from dataclasses import dataclass, replace
from fractions import Fraction
import math

import numpy as np

FP16, BF16, FP32 = "fp16", "bf16", "fp32"


# ---------------------------------------------------------------------------
# Byte accounting of mixed-precision Adam state.
# [csdn] §2.1 ZeRO: per parameter, 2 B fp16 param + 2 B fp16 grad + 12 B of
# fp32 master/momentum/variance, i.e. 16 B; [aiqz] 显存四巨头 gives the same
# split. Per-stage per-GPU formulas: [ch01] §1.2 and [aiqz] ZeRO三阶段.
# ---------------------------------------------------------------------------

def state_bytes_ddp(psi):
    """Every data-parallel replica holds all 16 bytes per parameter."""
    return 2 * psi + 2 * psi + 12 * psi


def state_bytes_stage1(psi, n):
    """Optimizer state (12 B/param) split over n ranks; params and grads whole."""
    return Fraction(4 * psi) + Fraction(12 * psi, n)


def state_bytes_stage2(psi, n):
    """Optimizer state and grads (14 B/param) split; params whole."""
    return Fraction(2 * psi) + Fraction(14 * psi, n)


def state_bytes_stage3(psi, n):
    """All 16 B/param split over n ranks."""
    return Fraction(16 * psi, n)


# ---------------------------------------------------------------------------
# Flat buffer layout and the Stage-1 contiguous shard.
# [csdn] §3.2: contiguous_gradients keeps the grads in one contiguous buffer;
# [aiqz] 通信优化: many small grad tensors are packed into buckets.
# [csdn] §2.1 and §2.4: under Stage 1 each rank holds and updates only its own
# part of the optimizer state. The part is a contiguous 1/N slice of the flat
# buffer (reading: equal slices, the buffer padded with zeros to a multiple of
# N * align).
# ---------------------------------------------------------------------------

def align_up(x, a):
    return ((x + a - 1) // a) * a


def flat_layout(numels, align):
    """Each tensor starts at the next multiple of `align` elements after the
    previous one ends. Returns (offsets, padded_total)."""
    offsets = []
    pos = 0
    for n in numels:
        offsets.append(pos)
        pos = align_up(pos + n, align)
    return offsets, pos


def shard_range(flat_total, world, rank, align):
    """[lo, hi) of rank `rank` out of `world` equal contiguous slices of the
    flat buffer padded to a multiple of world * align."""
    padded = align_up(flat_total, world * align)
    per = padded // world
    return rank * per, (rank + 1) * per


def shard_entries(numels, align, lo, hi):
    """Pieces of tensors that fall inside flat range [lo, hi).

    Returns a list of (tensor_index, start_in_tensor, length, dst_offset) where
    dst_offset is relative to lo."""
    offsets, _ = flat_layout(numels, align)
    out = []
    for t, (o, n) in enumerate(zip(offsets, numels)):
        a = max(o, lo)
        b = min(o + n, hi)
        if a < b:
            out.append((t, a - o, b - a, a - lo))
    return out


def round_robin_owners(names, world):
    """The partition of the [aiqz] Python 演示: whole tensors dealt to ranks in
    turn, rank r owning names[r], names[r + world], ..."""
    return [list(names[r::world]) for r in range(world)]


# ---------------------------------------------------------------------------
# 16-bit <-> fp32 element conversions.
# ---------------------------------------------------------------------------

def widen(x, dtype):
    """Exact conversion of fp16/bf16 bit patterns (or fp32 values) to fp32."""
    if dtype == FP16:
        return x.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == FP32:
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def narrow(p, dtype):
    """fp32 -> 16-bit bit patterns, round to nearest, ties to even.

    fp16: NumPy's IEEE conversion (overflow to inf, subnormals kept).
    bf16: keep the upper 16 bits of the fp32 pattern after adding half of the
    dropped range plus the tie-to-even bit; NaN stays a quiet NaN."""
    p = np.asarray(p, dtype=np.float32)
    if dtype == FP16:
        return p.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = p.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
        nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
        r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
        return r.astype(np.uint16)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Row a1: flatten / accumulate gradients into the flat bucket.
# [csdn] §2.3: micro-batch grads are summed in memory and one update is made
# at the end; [csdn] §3.2 contiguous_gradients; [aiqz] 通信优化 buckets.
# ---------------------------------------------------------------------------

COPY, OVERWRITE, ACCUMULATE = 0, 1, 2


def flatten_copy(srcs, entries, bucket):
    """COPY: bucket[d + j] = src_t[s + j] (16-bit to 16-bit)."""
    for t, s, n, d in entries:
        bucket[d:d + n] = srcs[t][s:s + n]
    return bucket


def flatten_accumulate(srcs, src_dtype, entries, acc, overwrite):
    """OVERWRITE: acc[d + j] = fp32(src); ACCUMULATE: acc[d + j] += fp32(src)
    with one fp32 round-to-nearest add per element."""
    for t, s, n, d in entries:
        x = widen(srcs[t][s:s + n], src_dtype)
        if overwrite:
            acc[d:d + n] = x
        else:
            acc[d:d + n] = acc[d:d + n] + x
    return acc


# ---------------------------------------------------------------------------
# Row a2: overflow check, L2 norm, clip coefficient.
# [csdn] §2.2: grads overflowing to inf under the loss scale are detected and
# the scale is lowered; §4.4 a NaN loss points at the fp16 setup. Clipping by
# the global norm is not on the pages: it is the conventional
# coef = max_norm / (norm + 1e-6), applied only when norm > max_norm (reading;
# pinned to a library's global-norm clip, which agrees except within 1e-6
# below max_norm, where it scales by slightly less than 1 and this leaves
# the grads alone). Accumulated grads are averaged over the K
# micro-batches ([csdn] §2.3: the accumulated grad stands for the big batch).
# ---------------------------------------------------------------------------

_EXP_MASK = {FP16: 0x7C00, BF16: 0x7F80, FP32: 0x7F800000}


def nonfinite_mask(x, dtype):
    """Element is inf or NaN: its exponent field is all ones."""
    if dtype == FP32:
        bits = np.asarray(x, dtype=np.float32).view(np.uint32)
    else:
        bits = x
    m = bits.dtype.type(_EXP_MASK[dtype])
    return (bits & m) == m


def overflow_flag(x, dtype):
    return int(bool(np.any(nonfinite_mask(x, dtype))))


def sum_of_squares(x, dtype, chunk=1 << 22):
    """Sum over elements of float64(x)^2, chunk partials added in order."""
    total = 0.0
    for a in range(0, x.shape[0], chunk):
        xc = widen(x[a:a + chunk], dtype).astype(np.float64)
        total += float(np.sum(xc * xc))
    return total


def clip_scalars(sumsq, scale, accum_steps, max_norm):
    """From the raw (loss-scaled, summed over K micro-batches) sum of squares:
    the true norm, the clip coefficient and the single fp32 factor the Adam
    pass multiplies every raw grad element by. All in float64, rounded once."""
    sk = float(scale) * float(accum_steps)
    norm = math.sqrt(sumsq) / sk
    coef = 1.0
    if max_norm > 0.0 and norm > max_norm:
        coef = float(max_norm) / (norm + 1e-6)
    grad_scale = np.float32(coef / sk)
    return norm, coef, grad_scale


def overflow_and_norm(x, dtype, scale, accum_steps, max_norm):
    ovf = overflow_flag(x, dtype)
    sumsq = sum_of_squares(x, dtype)
    if ovf:
        return dict(overflow=1, sumsq=sumsq, norm=np.float32(np.inf),
                    coef=1.0, grad_scale=np.float32(0.0))
    norm, coef, gs = clip_scalars(sumsq, scale, accum_steps, max_norm)
    return dict(overflow=0, sumsq=sumsq, norm=np.float32(norm), coef=coef, grad_scale=gs)


# ---------------------------------------------------------------------------
# Row a3: dynamic loss-scale state machine.
# [csdn] §2.2: multiply the loss so fp16 grads do not underflow, unscale
# before the update, lower the scale when an overflow is detected and try to
# raise it again once training is stable. [csdn] §3.2 fp16 block: loss_scale 0
# selects the dynamic mode; loss_scale_window, initial_scale_power, hysteresis
# and min_loss_scale. [aidhplus] feature list: dynamic loss scaling.
# Readings: factor 2 both ways; grow after `window` consecutive clean steps;
# halve when `hysteresis` overflows have come in a row (clean steps reset the
# count); never below min_scale; an overflow always skips the step, which
# leaves the Adam step counter and beta powers untouched. The scale is kept as
# an fp32 power of two, so growth stops at 2^127 (no cap is stated; this only
# keeps it finite).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ScalerState:
    scale: float
    good_steps: int
    hyst_left: int
    window: int
    hysteresis: int
    min_scale: float
    dynamic: bool
    t: int            # Adam steps applied so far
    beta1_pow: float  # beta1^t in float64
    beta2_pow: float  # beta2^t in float64
    last_skip: int


def scaler_init(dynamic=True, initial_scale_power=16, window=1000, hysteresis=1,
                min_scale=1.0, static_scale=1.0, t=0, beta1_pow=1.0, beta2_pow=1.0):
    scale = float(2.0 ** initial_scale_power) if dynamic else float(static_scale)
    return ScalerState(scale=scale, good_steps=0, hyst_left=hysteresis, window=window,
                       hysteresis=hysteresis, min_scale=float(min_scale), dynamic=bool(dynamic),
                       t=t, beta1_pow=beta1_pow, beta2_pow=beta2_pow, last_skip=0)


def scaler_update(st, overflow, beta1, beta2):
    """State after a step whose grads had the given overflow flag. beta1 and
    beta2 are the fp32 hyperparameters; the powers advance in float64."""
    if overflow:
        if not st.dynamic:
            return replace(st, last_skip=1)
        if st.hyst_left <= 1:
            return replace(st, scale=max(st.scale / 2.0, st.min_scale),
                           hyst_left=st.hysteresis, good_steps=0, last_skip=1)
        return replace(st, hyst_left=st.hyst_left - 1, good_steps=0, last_skip=1)
    b1 = float(np.float32(beta1))
    b2 = float(np.float32(beta2))
    st = replace(st, t=st.t + 1, beta1_pow=st.beta1_pow * b1, beta2_pow=st.beta2_pow * b2,
                 last_skip=0)
    if not st.dynamic:
        return st
    good = st.good_steps + 1
    if good == st.window:
        # the scale is an fp32 power of two: it saturates at 2^127
        return replace(st, scale=min(st.scale * 2.0, 2.0 ** 127), good_steps=0,
                       hyst_left=st.hysteresis)
    return replace(st, good_steps=good, hyst_left=st.hysteresis)


# ---------------------------------------------------------------------------
# Row a4: AdamW on the fp32 master shard, then the cast back to 16 bits.
# [csdn] §2.2 and [aiqz] 混合精度: forward/backward in 16 bits, the update on
# the fp32 master copy. [csdn] §3.2 optimizer block: AdamW, betas, eps,
# weight_decay. [csdn] §2.4: each rank updates only its slice. [aiqz] Python
# 演示: the two moment recurrences and p -= lr * m / (sqrt(v) + eps).
# Readings: bias correction on (off reproduces the demo); eps added after
# dividing sqrt(v) by sqrt(1 - beta2^t); decoupled decay p *= 1 - lr * wd
# applied before the Adam term; hyperparameters rounded to fp32 first; the
# per-step scalars derived in float64 and rounded once to fp32; every
# element operation in fp32 in the order written below.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_constants(hp, beta1_pow, beta2_pow, bias_correction=True):
    """fp32 scalars for the step that raises t by one. beta?_pow are the
    float64 powers before the step."""
    lr = np.float32(hp.lr)
    b1 = np.float32(hp.beta1)
    b2 = np.float32(hp.beta2)
    eps = np.float32(hp.eps)
    wd = np.float32(hp.weight_decay)
    c = dict(b1=b1, b2=b2, eps=eps,
             omb1=np.float32(np.float32(1.0) - b1),
             omb2=np.float32(np.float32(1.0) - b2))
    if bias_correction:
        p1 = beta1_pow * float(b1)
        p2 = beta2_pow * float(b2)
        c["step_size"] = np.float32(float(lr) / (1.0 - p1))
        c["bc2_sqrt"] = np.float32(math.sqrt(1.0 - p2))
    else:
        c["step_size"] = lr
        c["bc2_sqrt"] = np.float32(1.0)
    c["decay"] = np.float32(1.0 - float(lr) * float(wd))
    return c


def adamw_update(x, dtype, grad_scale, master, m, v, c):
    """New (master, m, v) for raw grads x, with grad_scale folding the loss
    unscale, the 1/K mean and the clip coefficient into one fp32 factor."""
    g = widen(x, dtype) * np.float32(grad_scale)
    m = c["b1"] * m + c["omb1"] * g
    v = c["b2"] * v + c["omb2"] * (g * g)
    denom = np.sqrt(v) / c["bc2_sqrt"] + c["eps"]
    p = master * c["decay"]
    p = p - c["step_size"] * (m / denom)
    return p, m, v


# ---------------------------------------------------------------------------
# One whole optimizer step on the rank's shard, in the engine's order
# ([csdn] §3.3: backward per micro-batch, then one step that handles
# accumulation, mixed precision and the optimizer).
# ---------------------------------------------------------------------------

def optimizer_step(x, gdtype, master, m, v, state, hp, max_norm, accum_steps, pdtype):
    """Returns (master, m, v, p16 or None, new_state, scalars). On overflow the
    state arrays are returned unchanged and p16 is None (not written)."""
    sc = overflow_and_norm(x, gdtype, state.scale, accum_steps, max_norm)
    if sc["overflow"]:
        return master, m, v, None, scaler_update(state, 1, hp.beta1, hp.beta2), sc
    c = adamw_constants(hp, state.beta1_pow, state.beta2_pow)
    master, m, v = adamw_update(x, gdtype, sc["grad_scale"], master, m, v, c)
    p16 = narrow(master, pdtype)
    return master, m, v, p16, scaler_update(state, 0, hp.beta1, hp.beta2), sc


# ---------------------------------------------------------------------------
# Next row: Stage-2 reduce-scatter intake on one rank.
# [aidhplus] ZeRO-2 section and [ch01] §1.2 table: under Stage 2 the grads are
# reduce-scattered instead of all-reduced, each rank keeping only the grads of
# its own slice. The rank's part of that collective is the sum, over the N
# peers, of the peers' copies of its slice. Reading: the sum is formed in fp32
# in peer order (one round-to-nearest add per peer), then stored in the
# destination dtype (16-bit: one rounding at the end). The mean over peers is
# not taken here: the step divides by accum_steps, so passing K * N there
# averages over micro-batches and peers at once.
# ---------------------------------------------------------------------------

def reduce_peer_slices(slices, src_dtype, dst, dst_dtype, accumulate):
    """dst (+)= sum over peers k = 0..N-1 of fp32(slices[k]), in that order.
    dst is an fp32 array or 16-bit bit patterns; returned updated."""
    acc = widen(slices[0], src_dtype).copy()
    for sl in slices[1:]:
        acc = acc + widen(sl, src_dtype)
    if dst_dtype == FP32:
        return dst + acc if accumulate else acc
    if accumulate:
        acc = widen(dst, dst_dtype) + acc
    return narrow(acc, dst_dtype)


# ---------------------------------------------------------------------------
# Checkpoint consolidation. [algomooc] 训练与恢复边界 and the checkpoint
# paragraph of its spoken answer: every rank saves its own shard, and a
# separate export step merges the ZeRO shards into one full fp32 state dict.
# Reading: the rank shards, put side by side in rank order, are the flat
# buffer; the full state of tensor t is the flat range [offset_t,
# offset_t + numel_t) of it, and the padding between and after tensors is
# dropped.
# ---------------------------------------------------------------------------

def consolidate(shards, numels, align):
    """shards: (lo, hi, fp32 array of hi - lo elements) per rank, in any
    order, together covering [0, padded total) without gaps or overlaps.
    Returns the list of full per-tensor fp32 arrays."""
    shards = sorted(shards, key=lambda s: s[0])
    pos = 0
    for lo, hi, a in shards:
        if lo != pos or hi < lo or len(a) != hi - lo:
            raise ValueError("shards do not tile the flat buffer at %d" % pos)
        pos = hi
    offsets, total = flat_layout(numels, align)
    if pos < total:
        raise ValueError("shards end at %d, the layout needs %d" % (pos, total))
    flat = np.concatenate([np.asarray(a, dtype=np.float32) for _, _, a in shards]) if shards else \
        np.zeros(0, np.float32)
    return [flat[o:o + n].copy() for o, n in zip(offsets, numels)]


# ---------------------------------------------------------------------------
# 1-bit compression with error compensation (a next row). [csdn] §4.2
# 通信压缩: 1-bit Adam sends only the sign of each gradient element and
# compensates the compression error afterwards, on the receiving side.
# Readings (the page gives no more detail):
#  - the magnitude travels as one fp32 scale per chunk of `chunk` consecutive
#    elements (the last chunk may be shorter): the chunk's root mean square,
#    so that the decoded chunk keeps the L2 norm of what was encoded;
#  - error compensation is error feedback: whatever the encoding lost is kept
#    in an fp32 error buffer and added to the next input before it is
#    encoded. Every end that encodes (the sender, and the receiver when it
#    sends the combined result on) keeps its own buffer;
#  - a sign bit is 1 for c >= 0 (so -0 encodes as +) and 0 otherwise (NaN
#    included). The signs travel in 32-bit words, 64 per unit of 2048
#    elements: bit 4r + i of word 64u + l is element 2048u + 256r + 4l + i
#    (r < 8, l < 64, i < 4), so that word l of a unit holds the signs of the
#    l-th quad of each of the unit's eight groups of 256 elements; bits past
#    the end are 0. (The pages fix one sign bit per element; this order is
#    the library's wire format.);
#  - the receiver's decode of N peers' payloads is their sum, formed in fp32
#    in peer order; the mean over peers is left to the caller (as for the
#    Stage-2 intake above).
# ---------------------------------------------------------------------------

def onebit_compress(x, err, chunk):
    """Encode c = x + err (fp32). Returns (words uint32[64 * ceil(n/2048)],
    scales float32[ceil(n/chunk)], new_err float32[n]) with, per chunk j,
    s_j = fp32(sqrt(sum(c_i^2) / len_j)) (exact squares, correctly rounded sum,
    float64 divide and sqrt) and new_err_i = c_i - s_j * sign_i (one fp32
    rounding)."""
    x = np.asarray(x, np.float32)
    c = x + np.asarray(err, np.float32)
    n = c.size
    pos = c >= np.float32(0.0)
    scales = np.zeros(-(-n // chunk), np.float32)
    new_err = np.empty(n, np.float32)
    for j in range(scales.size):
        a, b = j * chunk, min(n, (j + 1) * chunk)
        sumsq = math.fsum(float(v) * float(v) for v in c[a:b])
        s = np.float32(math.sqrt(sumsq / (b - a)))
        scales[j] = s
        new_err[a:b] = np.where(pos[a:b], c[a:b] - s, c[a:b] + s)
    words = np.zeros(64 * -(-n // 2048), np.uint32)
    for i in np.nonzero(pos)[0]:
        u, rem = divmod(int(i), 2048)
        r, q = divmod(rem, 256)
        lane, k = divmod(q, 4)
        words[64 * u + lane] |= np.uint32(1) << np.uint32(4 * r + k)
    return words, scales, new_err


def onebit_signs(words, n):
    """+1 / -1 (fp32) of elements 0 .. n-1 of a packed sign stream."""
    i = np.arange(n)
    word = 64 * (i // 2048) + (i % 256) // 4
    pos = 4 * ((i % 2048) // 256) + i % 4
    bit = (np.asarray(words, np.uint32)[word] >> pos.astype(np.uint32)) & np.uint32(1)
    return np.where(bit == 1, np.float32(1.0), np.float32(-1.0))


def onebit_decompress(payloads, n, chunk, dst, accumulate):
    """payloads: [(words, scales)] of N peers. Returns the fp32 sum over
    peers k = 0..N-1, in that order, of s_{k, chunk(i)} * sign_{k, i}; with
    accumulate, dst + that sum."""
    j = np.arange(n) // chunk
    acc = None
    for words, scales in payloads:
        d = np.asarray(scales, np.float32)[j] * onebit_signs(words, n)
        acc = d if acc is None else acc + d
    return dst + acc if accumulate else acc
