"""Oracle of Gumbel-max sampling -- TEST INFRASTRUCTURE ONLY.

The devpress page ("Gumbel-Max采样") samples a category from softmax(logits / T)
in parallel: add independent Gumbel noise g = -ln(-ln u), u ~ U(0, 1), to
ln p_i and take the argmax; ln p_i differs from logits_i / T by a constant, so
the argmax of logits_i / T + g_i is the same draw.  T <= 0 is read as greedy
(plain argmax).  The MRV2 page (section 6) draws the noise inside the kernel
from seeded inputs with no stored state; the generator here is Philox4x32-10
as Salmon, Moraes, Dror and Shaw define it ("Parallel Random Numbers: As Easy
as 1, 2, 3", SC 2011), with key = the row's seed and counter = (index / 4,
the row's offset), word index % 4 giving u = ((x >> 9) + 0.5) * 2^-23.

The scores are formed in float32, the precision the GPU kernel decides in:
logits / T rounded to float32, g from float32 logarithms, their float32 sum,
then the first maximum.  numpy, vectorised over the vocabulary.
"""
from __future__ import annotations

import numpy as np

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of counters (uint32 values) and one key."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0, k1 = int(k0) & _MASK, int(k1) & _MASK
    for _ in range(10):
        p0 = c[0] * np.uint64(_M0)
        p1 = c[2] * np.uint64(_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return [x.astype(np.uint32) for x in c]


def random_words(seed: int, offset: int, V: int) -> np.ndarray:
    """The 32-bit word of each vocabulary index 0..V-1 for one (seed, offset)."""
    seed, offset = int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFFFFFFFFFF
    q = np.arange((V + 3) // 4, dtype=np.uint64)
    words = philox4x32_10(q, offset & _MASK, offset >> 32, 0, seed & _MASK, seed >> 32)
    return np.stack(words, axis=1).reshape(-1)[:V]


def uniforms(words: np.ndarray) -> np.ndarray:
    """u = ((x >> 9) + 0.5) * 2^-23, exact in float32 and inside (0, 1)."""
    return ((words >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel(u: np.ndarray) -> np.ndarray:
    """g = -ln(-ln u) in float32."""
    u = u.astype(np.float32)
    return -np.log(-np.log(u))


def scores(logits_row, temperature: float, seed: int, offset: int) -> np.ndarray:
    """float32 score of every index of one row."""
    x = np.asarray(logits_row, dtype=np.float32)
    T = np.float32(temperature)
    if not T > 0:
        return x
    g = gumbel(uniforms(random_words(seed, offset, x.shape[0])))
    return (x / T + g).astype(np.float32)


def sample(logits, temperatures, seeds, offsets=None):
    """Token of every row (first maximum of its scores); also the scores."""
    logits = np.asarray(logits, dtype=np.float32)
    B = logits.shape[0]
    temps = np.ones(B, np.float32) if temperatures is None else np.asarray(temperatures, np.float32)
    offs = np.zeros(B, np.int64) if offsets is None else np.asarray(offsets, np.int64)
    seeds = np.asarray(seeds, np.int64)
    toks = np.empty(B, np.int64)
    all_scores = []
    for b in range(B):
        s = scores(logits[b], float(temps[b]), int(seeds[b]), int(offs[b]))
        toks[b] = int(np.argmax(s))
        all_scores.append(s)
    return toks, all_scores
