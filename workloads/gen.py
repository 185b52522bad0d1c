"""Seeded host-side draws.

Every array is produced in CHUNK-element pieces. Piece c of array a at step k
comes from numpy's PCG64 seeded with [seed, cfg, a, k, c], so any piece can be
regenerated on its own and in parallel. Values are float64 normal draws times
sigma (times a loss scale where one applies), then rounded to the storage
dtype by the rules in round_to().

16-bit arrays are returned as their raw bit patterns (np.uint16) so that fp16
and bf16 travel the same way; fp32 arrays are np.float32.
"""

import numpy as np

CHUNK = 1 << 24

# array ids
A_MASTER, A_GRAD, A_PRIOR_M, A_PRIOR_V = 0, 1, 2, 3


def chunk_rng(seed, cfg, array, step, chunk):
    return np.random.default_rng([int(seed), int(cfg), int(array), int(step), int(chunk)])


def normal_draw(n, seed, cfg, array, step, offset=0):
    """float64 standard normal values for elements [offset, offset + n) of the
    array, assembled from the CHUNK-sized seeded pieces that cover them."""
    out = np.empty(n, dtype=np.float64)
    pos = 0
    while pos < n:
        g = offset + pos
        c, within = divmod(g, CHUNK)
        take = min(CHUNK - within, n - pos)
        # A prefix of a PCG64 normal stream does not depend on how many
        # values are requested, so draw only up to the last one needed.
        piece = chunk_rng(seed, cfg, array, step, c).standard_normal(within + take)
        out[pos:pos + take] = piece[within:within + take]
        pos += take
    return out


def round_to(x64, dtype):
    """Round a float64 draw to the storage dtype.

    fp16: numpy's float64 -> float16 conversion. bf16: the upper 16 bits of the
    float32 value (truncation). fp32: numpy's float64 -> float32 conversion.
    16-bit results are bit patterns (np.uint16)."""
    if dtype == "fp16":
        return x64.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if dtype == "fp32":
        return x64.astype(np.float32)
    raise ValueError(dtype)


def f16_bits_to_f32(bits):
    return bits.view(np.float16).astype(np.float32)


def bf16_bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw_grads(n, dtype, sigma, scale, seed, cfg, step, offset=0):
    """Gradient draw: round(N(0, sigma) * scale) in the gradient dtype."""
    return round_to(normal_draw(n, seed, cfg, A_GRAD, step, offset) * (sigma * scale), dtype)


def draw_master(n, sigma, seed, cfg, offset=0):
    """fp32 master weights ~ N(0, sigma)."""
    return round_to(normal_draw(n, seed, cfg, A_MASTER, 0, offset) * sigma, "fp32")


def draw_prior_moments(n, sigma, seed, cfg, offset=0):
    """Moment buffers shaped like the state one optimizer step leaves behind:
    m ~ 0.1 * N(0, sigma) and v ~ 0.001 * N(0, sigma)^2, both fp32."""
    m = round_to(normal_draw(n, seed, cfg, A_PRIOR_M, 0, offset) * (0.1 * sigma), "fp32")
    z = normal_draw(n, seed, cfg, A_PRIOR_V, 0, offset) * sigma
    v = round_to(z * z * 0.001, "fp32")
    return m, v
