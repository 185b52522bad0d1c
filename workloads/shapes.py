"""Tensor shapes of the synthetic workloads.

Each function returns a list of (name, numel) in the order the tensors are
laid out in the flat buffer. Shapes follow the Llama decoder: a token
embedding, then per layer the q/k/v/o attention projections, the gate/up/down
MLP projections and two RMSNorm weight vectors, then the LM head.
"""

import numpy as np


def llama_tensors(hidden, inter, layers, vocab):
    """Flat order: embed; per layer q, k, v, o, gate, up, down, norm_in,
    norm_post; head. No final norm vector."""
    out = [("embed", vocab * hidden)]
    for i in range(layers):
        for p in ("q", "k", "v", "o"):
            out.append((f"{p}{i}", hidden * hidden))
        for p in ("gate", "up", "down"):
            out.append((f"{p}{i}", hidden * inter))
        out.append((f"norm_in{i}", hidden))
        out.append((f"norm_post{i}", hidden))
    out.append(("head", vocab * hidden))
    return out


def llama_7b_tensors():
    """Llama-7B shape: 32 layers, hidden 4096, MLP 11008, vocab 32000."""
    return llama_tensors(4096, 11008, 32, 32000)


def llama_65b_tensors():
    """65B-class shape: 80 layers, hidden 8192, MLP 22016, vocab 32000."""
    return llama_tensors(8192, 22016, 80, 32000)


def llama_7b_split_1024():
    """The Llama-7B shape cut into 1,024 per-layer tensors: every projection
    in 4 row chunks, the norms whole, embed and head in 32 row chunks each.
    The total parameter count is unchanged."""
    out = []
    for c in range(32):
        out.append((f"embed.{c}", 1000 * 4096))
    for i in range(32):
        for p in ("q", "k", "v", "o"):
            for c in range(4):
                out.append((f"{p}{i}.{c}", 1024 * 4096))
        for p in ("gate", "up"):
            for c in range(4):
                out.append((f"{p}{i}.{c}", 2752 * 4096))
        for c in range(4):
            out.append((f"down{i}.{c}", 1024 * 11008))
        out.append((f"norm_in{i}", 4096))
        out.append((f"norm_post{i}", 4096))
    for c in range(32):
        out.append((f"head.{c}", 1000 * 4096))
    return out


def tiny_shard_sizes(seed=0, count=64, lo=256, hi=65536):
    """Sizes drawn log-uniform in [lo, hi] and rounded to the nearest integer."""
    rng = np.random.default_rng(seed)
    s = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), count)))
    return [(f"t{i}", int(n)) for i, n in enumerate(s)]
