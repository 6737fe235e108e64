"""Pins of indexer scoring (R8), visibility (R3/R15), Top-K (R9), the candidate
pool (R10) and Reindex."""
import numpy as np
import pytest

from conftest import read_golden
from oracle.csa2 import build_pool, index_scores, reindex, topk, visible_count

rng = np.random.default_rng(9)


def test_score_unit_query_is_relu_of_channel():
    k = rng.standard_normal((50, 16))
    q = np.zeros((1, 16))
    q[0, 5] = 1.0
    assert np.array_equal(index_scores(q, [1.0], k), np.maximum(k[:, 5], 0))


def test_score_opposite_heads_give_abs():
    k = rng.standard_normal((40, 8))
    q0 = rng.standard_normal(8)
    q = np.stack([q0, -q0])
    s = index_scores(q, [0.5, 0.5], k)
    assert np.allclose(s, 0.5 * np.abs(k @ q0), atol=1e-14)


def test_score_weights_linear_and_relu_drops_negatives():
    k = rng.standard_normal((30, 8))
    q = rng.standard_normal((3, 8))
    w = np.array([0.2, 0.7, 0.0])
    s = index_scores(q, w, k)
    s2 = index_scores(q, 2 * w, k)
    assert np.allclose(s2, 2 * s, atol=1e-14)
    assert np.all(index_scores(q, [1, 1, 1], -np.abs(k) * 0) == 0)
    assert np.all(s >= 0)


def _brute_topk(s, K):
    order = sorted(range(len(s)), key=lambda j: (-s[j], j))[:K]
    out = sorted(order) + [-1] * (K - min(K, len(s)))
    return np.array(out)


@pytest.mark.parametrize("n,K", [(1, 1), (7, 3), (20, 20), (33, 50), (40, 8), (64, 17)])
def test_topk_bruteforce_with_ties(n, K):
    for _ in range(20):
        s = rng.integers(0, 5, n).astype(np.float64)  # many ties
        assert np.array_equal(topk(s, K), _brute_topk(s, K))


def test_topk_visible_prefix_and_all_selected():
    s = rng.standard_normal(100)
    assert np.array_equal(topk(s, 512)[:100], np.arange(100))
    assert np.all(topk(s, 512)[100:] == -1)
    s[60:] = 1e9  # invisible entries never enter
    assert np.array_equal(topk(s, 8, n_visible=60), _brute_topk(s[:60], 8))


def test_topk_tie_example():
    assert list(topk(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 2)) == [1, 2]


def test_visible_counts_prefill_chunk():
    # reading R3/R15 with m = 2: entry j sits at 2j+1; a chunk of 8,192 queries at positions
    # 24,576..32,767 sees 12,288..16,384 entries, 117,440,512 in total
    counts = [visible_count(t, 16384, 2) for t in range(24576, 32768)]
    assert counts[0] == 12288 and counts[-1] == 16384
    assert sum(counts) == 117440512
    assert visible_count(None, 16384, 2) == 16384
    assert visible_count(0, 100, 1) == 1 and visible_count(0, 100, 2) == 0


def test_pool_size_matches_pages():
    g = dict((r[0], r[1]) for r in read_golden("schedule_and_geometry.txt"))
    PB, PE = int(g["pool_blocks"]), int(g["pool_positions"])
    assert PB * PE == int(g["pool_size"])
    for nblk in (2048, 8192):
        s = rng.standard_normal(nblk * 128)
        pool = build_pool(s, 128, PB, PE)
        assert pool.shape[0] == int(g["pool_size"])
        assert np.all(np.diff(pool) > 0)


def _brute_pool(s, G, PB, PE):
    n = len(s)
    blocks = [list(range(b * G, min(n, (b + 1) * G))) for b in range(-(-n // G))]
    bmax = [max(s[j] for j in blk) for blk in blocks]
    chosen = sorted(range(len(blocks)), key=lambda b: (-bmax[b], b))[:PB]
    out = []
    for b in chosen:
        out += sorted(blocks[b], key=lambda j: (-s[j], j))[:PE]
    return np.array(sorted(out))


@pytest.mark.parametrize("n,G,PB,PE", [(50, 8, 3, 2), (64, 8, 8, 8), (29, 4, 5, 3), (100, 16, 2, 5)])
def test_pool_bruteforce(n, G, PB, PE):
    for _ in range(10):
        s = rng.integers(0, 6, n).astype(np.float64)
        assert np.array_equal(build_pool(s, G, PB, PE), _brute_pool(s, G, PB, PE))


def test_pool_covers_topk_blocks_and_reindex_equivalences():
    n, d_i, h = 8192, 16, 4
    k = rng.standard_normal((n, d_i))
    q = rng.standard_normal((h, d_i))
    w = rng.random(h)
    s = index_scores(q, w, k)
    K, G, PB, PE = 64, 32, 64, 8
    sel = topk(s, K)
    pool = build_pool(s, G, PB, PE)
    # every block holding a Full Top-K entry is in the pool (its maximum outranks >= PB - K blocks)
    assert set(sel // G) <= set(pool // G)
    # Reindex with the Full layer's own query returns the Full Top-K when no block holds > PE of it
    if np.bincount(sel // G).max() <= PE:
        assert np.array_equal(reindex(q, w, k, pool, K), sel)
    # Reindex over a pool that is every entry is the global Top-K
    assert np.array_equal(reindex(q, w, k, np.arange(n), K), sel)
