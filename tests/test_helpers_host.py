"""The parity checkers of the GPU tests, pinned on the CPU: they accept the
oracle's own results and reject planted mistakes."""
import numpy as np
import pytest

from helpers import check_pool, check_topk
from oracle.csa2 import build_pool, topk


def test_check_pool_accepts_the_oracle_and_rejects_planted_mistakes():
    rng = np.random.default_rng(0)
    s = rng.standard_normal(5000)
    pool = build_pool(s, 64, 16, 4)
    assert check_pool(pool, s, 64, 16, 4) == 0
    # a block outside the best 16 whose maximum is far from the cut
    bmax = np.array([s[b * 64:(b + 1) * 64].max() for b in range(-(-5000 // 64))])
    worst = int(np.argmin(bmax))
    bad = np.sort(np.concatenate([pool[4:], worst * 64 + np.argsort(-s[worst * 64:(worst + 1) * 64])[:4]]))
    with pytest.raises(AssertionError):
        check_pool(bad, s, 64, 16, 4)
    # inside a chosen block, its worst entry instead of its 4th best
    b0 = pool[0] // 64
    seg = s[b0 * 64:(b0 + 1) * 64]
    swap = pool.copy()
    k = np.nonzero(swap // 64 == b0)[0]
    swap[k[-1]] = b0 * 64 + int(np.argmin(seg))
    with pytest.raises(AssertionError):
        check_pool(np.sort(swap), s, 64, 16, 4)
    # a near-tie at the block cut is exempt
    s2 = s.copy()
    order = np.argsort(-bmax)
    a, c = order[15], order[16]                    # 16th and 17th best blocks
    jc = c * 64 + int(np.argmax(s2[c * 64:(c + 1) * 64]))
    s2[jc] = bmax[a] * (1 - 1e-6)                  # block c now ties block a within 1e-6
    pool2 = build_pool(s2, 64, 16, 4)
    alt = pool2[pool2 // 64 != a]
    alt = np.sort(np.concatenate([alt, c * 64 + np.argsort(-s2[c * 64:(c + 1) * 64], kind="stable")[:4]]))
    assert check_pool(alt, s2, 64, 16, 4) > 0


def test_check_topk_rejects_a_far_index():
    rng = np.random.default_rng(1)
    s = rng.standard_normal(3000)
    sel = topk(s, 100)
    assert check_topk(sel, s, 100, rel=0.0) == 0
    bad = sel.copy()
    bad[0] = int(np.argmin(s))
    with pytest.raises(AssertionError):
        check_topk(np.sort(bad), s, 100)
