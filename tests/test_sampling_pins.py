"""Pins of the sampling oracle: its Philox4x64-10 against numpy's own Philox
bit generator, the Gumbel-max rule against the softmax it samples, and the
verification rule against the target distribution it must reproduce (Monte
Carlo with fixed seeds, so every run is the same).  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import sampling as S

M64 = (1 << 64) - 1


def _np_philox_at(counter, key):
    """numpy's Philox bit generator steps its 256-bit counter before each
    block, so the block for counter c comes from state c - 1."""
    v = sum(int(c) << (64 * i) for i, c in enumerate(counter))
    v = (v - 1) % (1 << 256)
    prev = [(v >> (64 * i)) & M64 for i in range(4)]
    # set the state as exact uint64 arrays (the constructor takes big integers
    # through float64 and rounds them)
    bg = np.random.Philox()
    st = bg.state
    st["state"]["counter"] = np.array(prev, dtype=np.uint64)
    st["state"]["key"] = np.array([int(k) for k in key], dtype=np.uint64)
    st["buffer_pos"] = 4
    bg.state = st
    return tuple(int(w) for w in bg.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 2, 3, 4), (5, 6)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((151935, 15, 31, 0), (20260202, 1)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_matches_numpy_bit_generator(counter, key):
    assert S.philox4x64_10(counter, key) == _np_philox_at(counter, key)


def test_vectorized_philox_matches_scalar():
    rng = np.random.default_rng(0)
    c = rng.integers(0, 2 ** 63, size=(4, 64), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    k0, k1 = 0xFEDCBA9876543210, 3
    w = S.philox_words(c[0], c[1], c[2], c[3], k0, k1)
    for j in range(64):
        assert tuple(int(w[q][j]) for q in range(4)) == S.philox4x64_10([int(c[r, j]) for r in range(4)], (k0, k1))


def test_uniform_mapping_takes_one_word_per_position():
    """U(seed, purpose, b, i, v) is word i mod 4 of the block at counter (v, i div 4, b, 0)."""
    for i in (1, 2, 3, 4, 5, 15, 16):
        words = S.philox4x64_10((7, i // 4, 3, 0), (99, 2))
        u = S.uniforms(99, 2, 3, i, [7])[0]
        assert u == ((words[i % 4] >> 11) + 0.5) * 2.0 ** -53


def test_uniforms_are_in_the_open_unit_interval_and_uniform():
    u = S.uniforms(7, S.PURPOSE_DRAFT, 3, 5, np.arange(200_000))
    assert u.min() > 0.0 and u.max() < 1.0
    # Kolmogorov-Smirnov distance to U(0, 1); 1.63 / sqrt(n) is the 1% critical value
    us = np.sort(u)
    n = len(us)
    d = max(np.max(np.arange(1, n + 1) / n - us), np.max(us - np.arange(n) / n))
    assert d < 1.63 / np.sqrt(n)
    # distinct streams for distinct (purpose, b, i)
    assert not np.allclose(u[:100], S.uniforms(7, S.PURPOSE_DRAFT, 3, 6, np.arange(100)))
    assert not np.allclose(u[:100], S.uniforms(7, S.PURPOSE_ACCEPT, 3, 5, np.arange(100)))


def _chi2_ok(counts, probs, n):
    """Pearson chi-square below the 0.1% critical value for len(probs)-1
    degrees of freedom (Wilson-Hilferty approximation)."""
    k = len(probs) - 1
    exp = n * np.asarray(probs)
    chi2 = float(np.sum((counts - exp) ** 2 / exp))
    z = 3.09  # 0.1% upper quantile of N(0, 1)
    crit = k * (1 - 2 / (9 * k) + z * np.sqrt(2 / (9 * k))) ** 3
    return chi2, crit


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_gumbel_max_samples_the_tempered_softmax(T):
    logits = np.array([[[1.0, 0.2, -0.5, 2.0, 0.0, 1.3]]])
    n = 8000
    counts = np.zeros(6)
    for s in range(n):
        counts[S.sample_drafts(logits, T, seed=s)[0, 0]] += 1
    chi2, crit = _chi2_ok(counts, S.softmax_t(logits[0, 0], T), n)
    assert chi2 < crit, (chi2, crit)


def _lossless_case(seed0, n, q_row, p_rows, T):
    """n independent one-draft blocks (B = 2): draft from q, verify against p.
    Returns the first emitted token of each and the acceptance flags."""
    V = len(q_row)
    ql = np.tile(np.asarray(q_row, float), (n, 1, 1))
    pl = np.tile(np.asarray(p_rows, float), (n, 1, 1))
    drafts = S.sample_drafts(ql, T, seed0)
    acc, nxt = S.verify_sampled(drafts, ql, pl, T, seed0)
    first = np.where(acc >= 1, drafts[:, 0], nxt)
    return first, acc, drafts, nxt, V


def test_verification_reproduces_the_target_distribution():
    """The first emitted token follows p_1 whatever q is, and a draft is kept
    with probability sum_v min(p_1(v), q(v))."""
    q_row = [0.5, -1.0, 2.0, 0.3, 1.0]
    p_rows = [[1.5, 0.1, 0.2, -0.7, 1.1], [0.0, 0.0, 3.0, 0.0, 0.0]]
    T, n = 0.9, 8000
    first, acc, *_ = _lossless_case(11, n, q_row, p_rows, T)
    p1 = S.softmax_t(np.array(p_rows[0]), T)
    q = S.softmax_t(np.array(q_row), T)
    counts = np.bincount(first, minlength=5).astype(float)
    chi2, crit = _chi2_ok(counts, p1, n)
    assert chi2 < crit, (chi2, crit)
    rate, want = acc.mean(), np.minimum(p1, q).sum()
    assert abs(rate - want) < 4 * np.sqrt(want * (1 - want) / n)


def test_all_drafts_kept_when_draft_and_target_agree_and_bonus_follows_the_target():
    q_row = [0.4, 1.0, -0.3, 0.8]
    p_rows = [q_row, [2.0, -1.0, 0.5, 0.0]]
    T, n = 1.3, 5000
    first, acc, drafts, nxt, V = _lossless_case(5, n, q_row, p_rows, T)
    assert np.all(acc == 1)
    counts = np.bincount(nxt, minlength=V).astype(float)
    chi2, crit = _chi2_ok(counts, S.softmax_t(np.array(p_rows[1]), T), n)
    assert chi2 < crit


def test_draft_the_target_never_emits_is_always_rejected():
    V = 4
    ql = np.array([[[0.0, 9.0, 0.0, 0.0]]])
    pl = np.array([[[0.0, -800.0, 0.0, 1.0], [0.0, 0.0, 0.0, 0.0]]])  # p(1) underflows to 0
    for s in range(200):
        d = S.sample_drafts(ql, 1.0, s)
        acc, nxt = S.verify_sampled(d, ql, pl, 1.0, s)
        if d[0, 0] == 1:
            assert acc[0] == 0 and nxt[0] != 1


def test_rejection_stops_the_block():
    """A rejection at position i ends verification there: accept = i - 1."""
    ql = np.zeros((1, 3, 6))
    ql[0, :, 2] = 12.0
    pl = np.zeros((1, 4, 6))
    pl[0, 0] = ql[0, 0]   # position 1: target equals draft, always kept
    pl[0, 1, 2] = -900.0  # position 2 rejects token 2
    d = np.array([[2, 2, 2]])
    acc, nxt = S.verify_sampled(d, ql, pl, 1.0, 3)
    assert acc[0] == 1 and nxt[0] != 2
