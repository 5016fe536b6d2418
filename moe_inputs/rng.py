"""Seeded, counter-based input generator (host side, NumPy).

Every synthetic tensor element is a pure function of (seed, tensor id,
expert, element index), so any block of any tensor -- one expert of a 45 GB
weight set, a few token rows -- can be regenerated on the host without
materialising the rest, and the device twin in ``csrc/fill.hip`` produces
the very same bits.

Definition (both sides implement exactly this):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state_c = key + (c+1)*0x9E3779B97F4A7C15, output
  = the SplitMix64 finaliser (xor-shift 30, mul 0xBF58476D1CE4E5B9,
  xor-shift 27, mul 0x94D049BB133111EB, xor-shift 31), all mod 2^64.
* stream key of (seed, tensor, expert) = SplitMix64 output of state ``seed``
  at counter ``tensor * 65536 + expert``.
* normal deviate (Irwin-Hall with 12 terms, the sum of twelve uniforms
  minus 6): element c takes the SplitMix64 outputs at counters 3c, 3c+1 and
  3c+2, each cut into four 16-bit integers, twelve in all; D = sum(h) + 6 -
  393216 is the exact integer 65536*(sum of the twelve uniforms (h+1/2)/65536
  minus 6), and z = fl32(D) * 2^-16 is exact.  z has mean 0, variance 1,
  kurtosis 2.9 (a Gaussian's is 3) and tails out to +-6.
* value = fl32(z * scale), scale = fl32(std); bf16 tensors then round to
  nearest even.

Only correctly rounded IEEE operations on exactly representable operands
are used, so NumPy and the GPU agree bit for bit.  The twelve-term sum stands
in for a Gaussian (N(0, std) in the workload statement): it has the stated
mean and standard deviation, and only |z| > 6 (probability 2e-9 for a
Gaussian) never occurs.

Nothing here computes any part of the MoE layer.
"""
import numpy as np

from .configs import MoEConfig

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
NTERM = 12                         # uniforms per deviate (3 outputs x 4)
INV65536 = np.float32(1.0 / 65536.0)

# tensor ids of the stream keys
TID_X, TID_WG, TID_W1, TID_W3, TID_W2, TID_DY = 1, 2, 3, 4, 5, 6


def _finalise(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def splitmix64_at(key, counters: np.ndarray) -> np.ndarray:
    """SplitMix64 output number c+1 of a generator seeded with ``key``."""
    with np.errstate(over="ignore"):
        c = np.asarray(counters, dtype=np.uint64)
        z = np.uint64(key) + (c + np.uint64(1)) * GAMMA
        return _finalise(z)


def stream_key(seed: int, tensor: int, expert: int = 0) -> int:
    return int(splitmix64_at(np.uint64(seed),
                             np.array([tensor * 65536 + expert]))[0])


def _fill_chunk(out, key, start, lo, n, sc):
    mask = np.uint64(0xFFFF)
    c = np.arange(start + lo, start + lo + n, dtype=np.uint64) * np.uint64(3)
    s = np.zeros(n, dtype=np.uint64)
    for q in range(3):
        h = splitmix64_at(key, c + np.uint64(q))
        s += ((h & mask) + ((h >> np.uint64(16)) & mask)
              + ((h >> np.uint64(32)) & mask) + (h >> np.uint64(48)))
    dd = s.astype(np.int64) + NTERM // 2 - NTERM * 32768
    z = dd.astype(np.float32) * INV65536
    out[lo:lo + n] = z * sc


def _threads():
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 1


def normal_f32(key: int, start: int, count: int, scale: float,
               chunk: int = 1 << 20) -> np.ndarray:
    """``count`` deviates of stream ``key`` from element ``start`` on, fp32.

    Large requests are split into chunks filled by a thread pool (NumPy
    releases the GIL); every element depends only on its own counter, so
    the result does not depend on the chunking.
    """
    out = np.empty(count, dtype=np.float32)
    sc = np.float32(scale)
    starts = list(range(0, count, chunk))
    if len(starts) <= 2:
        for lo in starts:
            _fill_chunk(out, key, start, lo, min(chunk, count - lo), sc)
        return out
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda lo: _fill_chunk(out, key, start, lo,
                                           min(chunk, count - lo), sc), starts))
    return out


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def _round_inplace_bf16(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 values in place (chunked, threaded)."""
    flat = a.reshape(-1)
    step = 1 << 22

    def one(lo):
        seg = flat[lo:lo + step]
        seg[:] = bf16_bits_to_f32(bf16_round_bits(seg))
    if flat.size <= 2 * step:
        one(0) if flat.size <= step else (one(0), one(step))
        return a
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(0, flat.size, step)))
    return a


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values exactly representable in ``dtype``, held as fp32."""
    if dtype == "f32":
        return a
    if a.size > (1 << 23):
        return _round_inplace_bf16(np.ascontiguousarray(a, dtype=np.float32))
    return bf16_bits_to_f32(bf16_round_bits(a))


# ---------------------------------------------------------------- tensors

def tensor_spec(cfg: MoEConfig, name: str):
    """(tensor id, per-expert shape, std) of a named layer input."""
    d, f = cfg.d, cfg.f
    return {
        "x": (TID_X, (cfg.T, d), 1.0),
        "Wg": (TID_WG, (d, cfg.E), 1.0 / np.sqrt(d)),
        "W1": (TID_W1, (d, f), 1.0 / np.sqrt(d)),
        "W3": (TID_W3, (d, f), 1.0 / np.sqrt(d)),
        "W2": (TID_W2, (f, d), 1.0 / np.sqrt(f)),
        "dy": (TID_DY, (cfg.T, d), 1.0),
    }[name]


def gen_rows(cfg: MoEConfig, name: str, rows: np.ndarray,
             expert: int = 0) -> np.ndarray:
    """Selected rows of a 2-D tensor (of one expert), fp32 values of dtype."""
    tid, shape, std = tensor_spec(cfg, name)
    key = stream_key(cfg.seed, tid, expert)
    ncol = shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), ncol), dtype=np.float32)
    for i, r in enumerate(rows):
        out[i] = normal_f32(key, int(r) * ncol, ncol, std)
    return round_to_dtype(out, cfg.dtype)


def gen(cfg: MoEConfig, name: str, expert: int = 0) -> np.ndarray:
    """A whole 2-D tensor (one expert's slice for W1/W2/W3), fp32 values."""
    tid, shape, std = tensor_spec(cfg, name)
    key = stream_key(cfg.seed, tid, expert)
    a = normal_f32(key, 0, shape[0] * shape[1], std).reshape(shape)
    return round_to_dtype(a, cfg.dtype)


def gen_experts(cfg: MoEConfig, name: str, experts=None) -> np.ndarray:
    """Stacked per-expert weights [len(experts), ...]."""
    if experts is None:
        experts = range(cfg.E)
    return np.stack([gen(cfg, name, e) for e in experts])


def logit_bias(cfg: MoEConfig):
    """Per-expert routing bias b_e = -alpha*s*ln(rank_e), or None.

    rank is a seeded permutation of 1..E (NumPy PCG64 with the workload
    seed).  Returned as fp32 [E].
    """
    if cfg.zipf_s is None:
        return None
    rank = np.random.Generator(np.random.PCG64(cfg.seed)).permutation(cfg.E) + 1
    b = -cfg.alpha * cfg.zipf_s * np.log(rank.astype(np.float64))
    return b.astype(np.float32)


def seeded_experts(cfg: MoEConfig, n: int = 4) -> np.ndarray:
    """The experts whose FFN values large-workload tests compare in full."""
    g = np.random.Generator(np.random.PCG64(cfg.seed + 1))
    return np.sort(g.choice(cfg.E, size=min(n, cfg.E), replace=False))
