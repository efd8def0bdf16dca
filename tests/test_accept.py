"""The acceptance rules themselves (tie band, attention and salience tolerances)."""
import numpy as np

import accept
import synthetic


def test_index_exact_and_invalid():
    s = np.array([5.0, 1.0, 4.0, 3.0, 2.0])
    assert accept.check_index_row([0, 2, 3], s, 3)[0]
    assert not accept.check_index_row([0, 2], s, 3)[0]          # wrong length
    assert not accept.check_index_row([2, 0, 3], s, 3)[0]       # not ascending
    assert not accept.check_index_row([0, 0, 3], s, 3)[0]       # duplicate
    assert not accept.check_index_row([0, 2, 5], s, 3)[0]       # out of range
    assert not accept.check_index_row([0, 2, 4], s, 3)[0]       # a real miss


def test_index_tie_band():
    s = np.array([10.0, 1.0, 5.0, 5.0 - 1e-6, 0.0])
    # swapping 2 and 3 straddles sigma_k = 5 by 1e-6 < 1e-5 * 5
    ok, n, _ = accept.check_index_row([0, 3], s, 2)
    assert ok and n == 1
    s2 = np.array([10.0, 1.0, 5.0, 5.0 - 1e-3, 0.0])
    assert not accept.check_index_row([0, 3], s2, 2)[0]
    # sigma_k ~ 0: the band falls back to the RMS of the scores
    s3 = np.array([3.0, 0.0, -1e-9, -3.0])
    assert accept.check_index_row([0, 2], s3, 2)[0]


def test_attention_and_salience_rules():
    r = np.ones((1, 2, 4))
    g = r.copy()
    g[0, 1, 0] += 1.9e-3
    assert accept.check_attention(g, r)[0]
    g[0, 1, 0] += 2e-4
    assert not accept.check_attention(g, r)[0]
    s = np.full((1, 4), 0.25)
    assert accept.check_salience(s * (1 + 5e-6), s)[0]
    bad = s.copy()
    bad[0, 0] *= 1 + 2e-4
    assert not accept.check_salience(bad, s)[0]


def test_multiturn_schedule():
    L = synthetic.multiturn_text_lengths()
    assert len(L) == 3 and all(len(r) == 128 for r in L)
    assert L[0][0] == 129 and L[0][-1] == 256
    assert max(max(r) for r in L) <= synthetic.DECODE["multiturn_128k"].Tmax
