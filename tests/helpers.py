"""Shared helpers of the GPU parity tests (marshalling and comparison rules)."""
import numpy as np
import torch

from oracle.codecs import bf16_to_f64
from oracle.csa2 import topk as oracle_topk


def dev(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_bf16(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_topk(gpu_sel, ref_scores, K, n_vis=None, rel=1e-4, index_map=None):
    """Top-K parity: same size, ascending, -1 padded; a differing index is allowed only
    when its oracle score lies within `rel` (relative) of the oracle's K-th score.
    Returns the number of exempt differences."""
    gpu_sel = np.asarray(gpu_sel)
    s = np.asarray(ref_scores, dtype=np.float64)
    n = s.shape[0] if n_vis is None else int(n_vis)
    s = s[:n]
    k = min(K, n)
    g = gpu_sel[:k]
    assert np.all(gpu_sel[k:] == -1), "padding must be -1"
    assert np.all(g >= 0), "fewer than min(K, visible) entries selected"
    assert np.all(np.diff(g) > 0), "selection must be strictly ascending"
    ref = oracle_topk(s, K)[:k]
    if index_map is not None:
        ref = np.asarray(index_map)[ref]
    diff = set(g.tolist()) ^ set(ref.tolist())
    if diff:
        kth = np.sort(s)[::-1][k - 1]
        tol = rel * abs(kth)
        pos = {int(v): i for i, v in enumerate(index_map)} if index_map is not None else None
        for j in diff:
            jj = pos[j] if pos is not None else j
            assert abs(s[jj] - kth) <= tol, f"index {j}: score {s[jj]} vs K-th {kth}"
    return len(diff)


def score_tol(q, w, k):
    """fp32-accumulation bound of indexer scores: 2^-20 x sum_h w_h sum_c |q_hc k_jc|."""
    qa, ka = np.abs(bf16_to_f64(q)), np.abs(bf16_to_f64(k))
    return 2.0 ** -20 * ((ka @ qa.T) * np.asarray(w)[None, :]).sum(1) + 1e-30


def attn_close(out, ref):
    """Attention parity: max-abs error <= 2e-3 x RMS of the oracle output."""
    rms = np.sqrt(np.mean(np.asarray(ref) ** 2))
    assert np.max(np.abs(np.asarray(out) - ref)) <= 2e-3 * rms


def _near(v, cut, rel):
    return abs(v - cut) <= rel * abs(cut)


def check_pool(gpu_pool, ref_scores, G, PB, PE, rel=1e-4, n_vis=None):
    """Pool parity under the near-tie rule of the Top-K: the GPU pool (its valid
    prefix) is strictly ascending; it holds min(PB, blocks) blocks, which are the
    oracle's best blocks except where a differing block's maximum lies within
    `rel` (relative) of the cut (the PB-th best block maximum); inside each of its
    blocks it holds min(PE, block size) entries, the block's best ones except where
    a differing entry's score lies within `rel` of that block's PE-th score.
    Returns the number of exempt differences."""
    s = np.asarray(ref_scores, dtype=np.float64)
    n = s.shape[0] if n_vis is None else int(n_vis)
    s = s[:n]
    g = np.asarray(gpu_pool, dtype=np.int64)
    assert np.all(np.diff(g) > 0), "pool must be strictly ascending"
    assert g.size == 0 or (g[0] >= 0 and g[-1] < n), "pool entry outside the visible range"
    nblk = -(-n // G)
    bmax = np.array([s[b * G:min((b + 1) * G, n)].max() for b in range(nblk)])
    nb = min(PB, nblk)
    ref_blocks = np.lexsort((np.arange(nblk), -bmax))[:nb]
    gblocks = np.unique(g // G)
    assert gblocks.shape[0] == nb, f"{gblocks.shape[0]} blocks in the pool, expected {nb}"
    exempt = 0
    cut = np.sort(bmax)[::-1][nb - 1]
    for b in set(gblocks.tolist()) ^ set(ref_blocks.tolist()):
        assert _near(bmax[b], cut, rel), f"block {b}: max {bmax[b]} vs cut {cut}"
        exempt += 1
    for b in gblocks.tolist():
        lo, hi = b * G, min((b + 1) * G, n)
        ent = g[(g >= lo) & (g < hi)]
        cnt = min(PE, hi - lo)
        assert ent.shape[0] == cnt, f"block {b}: {ent.shape[0]} entries, expected {cnt}"
        seg = s[lo:hi]
        want = lo + np.lexsort((np.arange(hi - lo), -seg))[:cnt]
        bcut = np.sort(seg)[::-1][cnt - 1]
        for j in set(ent.tolist()) ^ set(want.tolist()):
            assert _near(s[j], bcut, rel), f"entry {j}: score {s[j]} vs block cut {bcut}"
            exempt += 1
    return exempt
