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
