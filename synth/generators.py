"""Counter-based random streams and the synthetic tensors built from them.

Every value is a pure function of (seed, tensor name, flat index), so a tensor
can be regenerated in chunks, in any order, on any host, bit for bit.

* Mixer: SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom
  Number Generators", OOPSLA 2014): state advances by the golden-ratio
  increment and each output is the state passed through the published
  three-step xor-shift-multiply finaliser.  Here the state of draw j is
  ``key + (j + 1) * GOLDEN_GAMMA``, i.e. the generator is used in counter mode.
* Stream keys: FNV-1a 64-bit hash of the tensor name, mixed with the seed.
* Uniforms: the top 53 bits of a draw, centred in their cell, so 0 and 1 are
  never produced.
* Normals: Box-Muller on consecutive uniform pairs, in float64.
* Student-t with 3 degrees of freedom: Z / sqrt(V / 3), V a sum of three
  squared standard normals, all from independent sub-streams.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1

# Chunk size for streaming generation (elements); bounds temporary memory.
_CHUNK = 1 << 22


def fnv1a64(text: str) -> int:
    """FNV-1a 64-bit hash of a UTF-8 string (Fowler-Noll-Vo, variant 1a)."""
    h = _FNV_OFFSET
    for b in text.encode("utf-8"):
        h ^= b
        h = (h * _FNV_PRIME) & _MASK64
    return h


def splitmix64_mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser applied element-wise to uint64 states."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def _mix_int(x: int) -> int:
    return int(splitmix64_mix(np.array([x & _MASK64], dtype=np.uint64))[0])


def stream_key(seed: int, name: str) -> int:
    """64-bit key of the stream named ``name`` under ``seed``."""
    return _mix_int(_mix_int(seed & _MASK64) ^ fnv1a64(name))


def _raw(key: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of stream ``key`` as uint64."""
    j = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + j * GOLDEN_GAMMA
    return splitmix64_mix(state)


def uniform53(key: int, start: int, count: int) -> np.ndarray:
    """Uniforms in the open interval (0, 1), float64, from draws start.."""
    u = _raw(key, start, count) >> np.uint64(11)
    return (u.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def standard_normal(key: int, start: int, count: int) -> np.ndarray:
    """Standard normals start .. start+count-1 of stream ``key`` (float64).

    Normal 2p and 2p+1 come from uniform draws 2p and 2p+1 by Box-Muller
    (cosine and sine branch respectively).
    """
    out = np.empty(count, dtype=np.float64)
    pos = 0
    while pos < count:
        n = min(_CHUNK, count - pos)
        j0 = start + pos
        p0 = j0 // 2
        p1 = (j0 + n - 1) // 2
        npairs = p1 - p0 + 1
        u = uniform53(key, 2 * p0, 2 * npairs).reshape(npairs, 2)
        r = np.sqrt(-2.0 * np.log(u[:, 0]))
        theta = (2.0 * np.pi) * u[:, 1]
        z = np.empty((npairs, 2), dtype=np.float64)
        z[:, 0] = r * np.cos(theta)
        z[:, 1] = r * np.sin(theta)
        z = z.reshape(-1)
        off = j0 - 2 * p0
        out[pos:pos + n] = z[off:off + n]
        pos += n
    return out


def student_t3(key: int, start: int, count: int) -> np.ndarray:
    """Student-t (3 degrees of freedom) draws, float64."""
    z = standard_normal(_mix_int(key ^ 1), start, count)
    v = np.zeros(count, dtype=np.float64)
    for s in (2, 3, 4):
        g = standard_normal(_mix_int(key ^ s), start, count)
        v += g * g
    return z / np.sqrt(v / 3.0)


def _count_of(frac: Fraction, n: int) -> int:
    """round-half-up(frac * n) computed exactly."""
    x = Fraction(frac) * n
    return int((x + Fraction(1, 2)) // 1)


def outlier_channels(key: int, K: int, frac) -> np.ndarray:
    """Sorted channel indices picked by a seeded partial Fisher-Yates shuffle."""
    cnt = _count_of(Fraction(frac), K)
    perm = np.arange(K, dtype=np.int64)
    u = uniform53(key, 0, max(cnt, 1))
    for i in range(cnt):
        r = i + int(u[i] * (K - i))
        perm[i], perm[r] = perm[r], perm[i]
    return np.sort(perm[:cnt])


def make_weight(seed: int, name: str, N: int, K: int, sigma: float) -> np.ndarray:
    """Latent weight W [N][K], fp32, i.i.d. N(0, sigma^2) (sigma = std dev)."""
    key = stream_key(seed, name)
    out = np.empty(N * K, dtype=np.float32)
    pos = 0
    while pos < N * K:
        n = min(_CHUNK * 4, N * K - pos)
        out[pos:pos + n] = (standard_normal(key, pos, n) * sigma).astype(np.float32)
        pos += n
    return out.reshape(N, K)


def make_acts(seed: int, name: str, M: int, K: int, recipe: dict) -> np.ndarray:
    """Activations X [M][K], fp32, following a workload recipe.

    recipe keys:
      ``outlier_frac`` / ``outlier_scale``: a fixed set of channels (shared by
      every token) multiplied by the scale.
      ``t3_frac``: a fixed set of channels drawn from Student-t(3) instead of
      N(0, 1).
    """
    key = stream_key(seed, name)
    x = standard_normal(key, 0, M * K).reshape(M, K)
    if recipe.get("t3_frac"):
        ch = outlier_channels(stream_key(seed, name + "/t3-channels"), K, recipe["t3_frac"])
        if len(ch):
            t = student_t3(stream_key(seed, name + "/t3"), 0, M * len(ch))
            x[:, ch] = t.reshape(M, len(ch))
    if recipe.get("outlier_frac"):
        ch = outlier_channels(stream_key(seed, name + "/outlier-channels"), K,
                              recipe["outlier_frac"])
        x[:, ch] *= float(recipe["outlier_scale"])
    return x.astype(np.float32)
