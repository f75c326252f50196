"""Plain CPU oracle of sampled drafting (temperature > 0) and of lossless
verification of a sampled block.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module.

The pages report DFlash at temperature 0 (atlas summary, "Key results") and
call speculative decoding lossless (paper, Introduction: the drafted block is
verified by the target, so the output follows the target's distribution).
They do not spell out a sampled variant; this takes the standard one from the
speculative-sampling literature:

* a draft position samples its token from the drafter's distribution
  q = softmax(logits / T), here by the Gumbel-max rule: the index of the
  largest logits_v / T + G_v with G_v = -log(-log(U_v)) and U_v uniform;
* verification walks the block left to right; position i's draft x is kept
  when U_i * q_i(x) < p_i(x), with p_i = softmax(target logits_i / T);
  at the first rejection a token is drawn from the residual distribution
  proportional to max(0, p_i - q_i) and the block ends there; when every
  draft is kept, a bonus token is drawn from the target's distribution at
  the position after the block.  The emitted tokens then follow the target's
  distribution exactly, whatever q is.

Random numbers are inputs of the method, so both this oracle and the GPU
path compute them from one counter-based generator, Philox4x64-10 (Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
each from that published definition:

    U(seed, purpose, b, i, v) = (w >> 11 + 1/2) * 2^-53,
    w = word (i mod 4) of Philox4x64-10(counter (v, i div 4, b, 0),
                                        key (seed, purpose)),

with b the block (sequence) index within a call, i the position in the block
(1..B) and v the vocabulary index (0 where only one number is needed); one
generator block serves four consecutive positions of one index.
Purposes: 1 draft sampling, 2 acceptance tests, 3 residual and bonus samples.
Floating point is float64 throughout.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1

PURPOSE_DRAFT = 1
PURPOSE_ACCEPT = 2
PURPOSE_RESIDUAL = 3


def philox4x64_10(counter, key) -> Tuple[int, int, int, int]:
    """Philox4x64 with 10 rounds on Python integers: each round multiplies
    words 0 and 2 by the two round constants, forms the new words from the
    high and low halves of the 128-bit products, the other two words and the
    key, and then adds the Weyl constants to the key."""
    x0, x1, x2, x3 = (int(c) & _MASK64 for c in counter)
    k0, k1 = (int(k) & _MASK64 for k in key)
    for _ in range(10):
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0, p1 & _MASK64, (p0 >> 64) ^ x3 ^ k1, p0 & _MASK64)
        k0 = (k0 + PHILOX_W0) & _MASK64
        k1 = (k1 + PHILOX_W1) & _MASK64
    return x0, x1, x2, x3


def _mulhilo64(a: np.ndarray, m: int) -> Tuple[np.ndarray, np.ndarray]:
    """(high, low) 64-bit halves of a * m for uint64 arrays, by 32-bit limbs."""
    M32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a0, a1 = a & M32, a >> s32
    m0, m1 = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> s32) + (p01 & M32) + (p10 & M32)
    lo = (mid << s32) | (p00 & M32)
    hi = p11 + (p01 >> s32) + (p10 >> s32) + (mid >> s32)
    return hi, lo


def philox_words(c0, c1, c2, c3, k0: int, k1: int):
    """The four words of Philox4x64-10 for arrays of counters (numpy, wrapping uint64)."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    ka, kb = np.uint64(k0 & _MASK64), np.uint64(k1 & _MASK64)
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo64(x0, PHILOX_M0)
            hi1, lo1 = _mulhilo64(x2, PHILOX_M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
            ka = ka + np.uint64(PHILOX_W0)
            kb = kb + np.uint64(PHILOX_W1)
    return x0, x1, x2, x3


def uniforms(seed: int, purpose: int, b: int, i: int, v) -> np.ndarray:
    """U(seed, purpose, b, i, v) in (0, 1) for an array of vocabulary indices v."""
    w = philox_words(np.asarray(v, dtype=np.uint64), i // 4, b, 0, seed, purpose)[i % 4]
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def gumbel(u: np.ndarray) -> np.ndarray:
    return -np.log(-np.log(u))


def softmax_t(logits: np.ndarray, T: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def sample_scores(logits: np.ndarray, T: float, seed: int, b: int, i: int, purpose: int = PURPOSE_DRAFT):
    """logits_v / T + G_v over one row (the quantity whose argmax is the sample)."""
    V = logits.shape[-1]
    return np.asarray(logits, dtype=np.float64) / T + gumbel(uniforms(seed, purpose, b, i, np.arange(V)))


def sample_drafts(logits: np.ndarray, T: float, seed: int) -> np.ndarray:
    """Sampled drafts for block logits [n][B-1][V]: row i-1 of block b is
    position i (1..B-1).  Ties go to the lowest index."""
    n, bm1, _ = logits.shape
    out = np.empty((n, bm1), dtype=np.int64)
    for b in range(n):
        for i in range(1, bm1 + 1):
            out[b, i - 1] = int(np.argmax(sample_scores(logits[b, i - 1], T, seed, b, i)))
    return out


def verify_sampled(draft: np.ndarray, q_logits: np.ndarray, p_logits: np.ndarray, T: float,
                   seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """Lossless verification of sampled blocks.

    draft [n][B-1] (positions 1..B-1), q_logits [n][B-1][V] (the drafter's
    logits at those positions), p_logits [n][B][V] (the target's logits for
    positions 1..B; row B-1 is the position after the block).  Returns
    (accept, next_token): accept[b] = number of drafts kept (0..B-1) and
    next_token[b] = the residual sample at the first rejected position, or the
    bonus sample when all drafts are kept.
    """
    n, bm1 = draft.shape
    V = p_logits.shape[-1]
    acc = np.empty(n, dtype=np.int64)
    nxt = np.empty(n, dtype=np.int64)
    for b in range(n):
        acc[b], nxt[b] = bm1, -1
        for i in range(1, bm1 + 1):
            x = int(draft[b, i - 1])
            p = softmax_t(p_logits[b, i - 1], T)
            q = softmax_t(q_logits[b, i - 1], T)
            u = uniforms(seed, PURPOSE_ACCEPT, b, i, [0])[0]
            if u * q[x] < p[x]:
                continue
            r = np.maximum(p - q, 0.0)
            with np.errstate(divide="ignore"):
                sc = np.log(r) + gumbel(uniforms(seed, PURPOSE_RESIDUAL, b, i, np.arange(V)))
            acc[b], nxt[b] = i - 1, int(np.argmax(sc))
            break
        if nxt[b] < 0:
            nxt[b] = int(np.argmax(sample_scores(p_logits[b, bm1], T, seed, b, bm1 + 1, PURPOSE_RESIDUAL)))
    return acc, nxt


def accept_margins(draft, q_logits, p_logits, T, seed) -> np.ndarray:
    """|U_i q_i(x) - p_i(x)| relative to p_i(x), per draft: how close each
    acceptance decision is to its threshold (for tests that skip decisions a
    last-bit difference could flip)."""
    n, bm1 = draft.shape
    out = np.empty((n, bm1))
    for b in range(n):
        for i in range(1, bm1 + 1):
            x = int(draft[b, i - 1])
            p = softmax_t(p_logits[b, i - 1], T)[x]
            q = softmax_t(q_logits[b, i - 1], T)[x]
            u = uniforms(seed, PURPOSE_ACCEPT, b, i, [0])[0]
            out[b, i - 1] = abs(u * q - p) / max(p, 1e-300)
    return out
