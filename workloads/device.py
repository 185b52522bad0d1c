"""Seeded device-side draws for the full-size workloads (hundreds of millions
to billions of elements), using torch's device generator. Same distributions
as the host draws in gen.py; used by the bench and the full-size tests, which
gather the values they check back to the host."""

import torch


def fill_normal_(t, sigma, seed):
    """t ~ N(0, sigma) from torch's device generator seeded with `seed`
    (drawn in fp32, rounded to t's dtype)."""
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    t.normal_(0.0, float(sigma), generator=g)
    return t


def draw_master_(t, seed):
    return fill_normal_(t, 0.02, seed)


def draw_prior_moments_(m, v, sigma, seed):
    """m ~ 0.1 * N(0, sigma); v ~ 0.001 * N(0, sigma)^2 (state after one step)."""
    fill_normal_(m, 0.1 * sigma, seed)
    fill_normal_(v, sigma, seed + 1)
    v.mul_(v).mul_(0.001)
    return m, v


def draw_sources_(srcs, sigma, scale, seed, step):
    """Per-tensor gradient draws of one micro-batch / step: tensor t of the
    list gets N(0, sigma * scale) seeded by (seed, step, t); None entries are
    skipped."""
    for t, s in enumerate(srcs):
        if s is not None:
            fill_normal_(s, sigma * scale, (int(seed) * 1_000_003 + int(step) * 4099 + t) & 0x7FFFFFFFFFFF)
    return srcs


def draw_payload_(words, scales, sigma, seed):
    """A random 1-bit message: uniformly random sign words (any integer
    storage; filled as 32-bit halves) and per-chunk scales |N(0, sigma)|,
    from torch's device generator."""
    g = torch.Generator(device=words.device)
    g.manual_seed(int(seed))
    words.view(torch.int32).random_(-(1 << 31), 1 << 31, generator=g)
    scales.normal_(0.0, float(sigma), generator=g).abs_()
    return words, scales
