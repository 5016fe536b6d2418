"""Seeded inputs for testing one entry point at a time (small shapes).

NumPy PCG64 streams keyed by a test seed; every float array is returned as
fp32 values exactly representable in the requested storage type, so the
same bits go to the GPU and to the oracle.  Computes nothing of the layer.
"""
import numpy as np

from .rng import round_to_dtype


def gen(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(seed, shape, std=1.0, dtype="bf16"):
    a = (gen(seed).standard_normal(shape) * std).astype(np.float32)
    return round_to_dtype(a, dtype)


def routing(seed, T, E, k, hot=None, hot_frac=0.0, dead=()):
    """topk_idx [T,k] int32: k distinct experts per token.

    hot/hot_frac: expert `hot` is in a token's set with probability hot_frac;
    dead: experts never chosen (zero-load segments).
    """
    g = gen(seed)
    live = np.array([e for e in range(E) if e not in set(dead)])
    assert len(live) >= k
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        if hot is not None and g.random() < hot_frac:
            rest = live[live != hot]
            pick = [hot] + list(g.choice(rest, size=k - 1, replace=False))
            g.shuffle(pick)
        else:
            pick = list(g.choice(live, size=k, replace=False))
        out[t] = pick
    return out


def counts_to_offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off
