"""Plain CPU reference of one CSA2 compressed-sparse-attention layer.

TEST INFRASTRUCTURE ONLY.  This module is the oracle the HIP library is checked
against.  Only ``tests/``, the smoke check (``__graft_entry__.smoke``) and the
CPU-baseline leg of ``bench.py`` may import it.  It shares no code with the
library: it reads seeded inputs (numpy arrays, bf16 as uint16 bit patterns,
FP8/FP4 as uint8 codes) and computes every step in float64 with numpy.

Sources (the pages; cited by title and section only)
----------------------------------------------------
[daily]     "每日技术报告｜2026-09-11：DeepSeek V4.1 Flash 将 KV 压缩推到模型架构层",
            blog.baizx.cool.  Section "核心机制": Full/Reindex/Reuse modes, the
            hierarchical indexer, FP4 E2M1 main KV with one E4M3 scale per 16
            channels.
[reading]   "DeepSeek-V4.1-Flash paper reading", inkeast.github.io (2026-09-19).
            §4.2: the mode table, and every layer keeps its own query and SWA KV.
[digest]    "DeepSeek V4.1 Flash 技术报告流出：死磕 KV cache 压缩", agihunt.info.
            Section "已确认": the indexer runs on the small KV and the selected
            entries are concatenated with the windowed KV before attention.
[deep-dive] "DeepSeek-V4.1-Flash deep dive", tanjunchen.github.io (2026-09-13).
            §2 (the projections C = H·W_KV, Z = H·W_Z), §3.1 (data flow, the
            non-overlapping compressor, m = 2 / m = 1), §3.2 (modes, layer
            schedule), §3.3 (hierarchical indexer, 2,048 blocks x 8 positions),
            §3.4 (FP4 after RoPE, SWA in FP8), §6.3 (dimensions).

Where the pages leave a step open, the reading taken is named R1..R15 in the
docstring of the function that implements it; the same labels are used in the
design notes of the repository.

Parity pins: each function below is checked by ``tests/test_oracle_*.py``
against closed forms, special cases, invariants, independent library routines
or brute force.  No function here is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .codecs import (bf16_to_f64, e2m1_decode, e2m1_encode, e4m3_decode,
                     e4m3_encode, f64_to_bf16)

# --------------------------------------------------------------------------
# a1: compressor  [deep-dive §2, §3.1]
# --------------------------------------------------------------------------


def project(H, W) -> np.ndarray:
    """C = H·W (or Z = H·W_Z) in float64 [deep-dive §2].

    ``H`` and ``W`` are float arrays (float32 inputs upcast exactly) or bf16
    bit patterns (uint16), which are decoded exactly first.
    """
    return _as_f64(H) @ _as_f64(W)


def fold(C, Z, m: int) -> np.ndarray:
    """Non-overlapping compression of each run of m tokens into one entry.

    [deep-dive §3.1]: every m consecutive tokens become one main-KV entry,
    windows do not overlap and no absolute position enters the compression;
    [deep-dive §2]: Z = H·W_Z are the "compression weights".

    R1 (the pages do not print the fold): per channel c, the weights are a
    softmax over the m tokens of the block,
        a[t, c] = exp(Z[t, c]) / sum_{t' in block} exp(Z[t', c]),
        entry[c] = sum_{t in block} a[t, c] * C[t, c].
    Z may have one column (a single weight per token, broadcast over channels).
    R2: only complete blocks fold; T mod m trailing tokens make no entry.
    """
    C = np.asarray(C, dtype=np.float64)
    Z = np.asarray(Z, dtype=np.float64)
    T, d = C.shape
    if Z.shape[0] != T or Z.shape[1] not in (1, d):
        raise ValueError("Z must be [T, 1] or [T, d]")
    n = T // m
    out = np.empty((n, d))
    for j in range(n):
        zb = Z[j * m:(j + 1) * m]
        a = np.exp(zb - zb.max(axis=0, keepdims=True))
        a = a / a.sum(axis=0, keepdims=True)
        out[j] = (a * C[j * m:(j + 1) * m]).sum(axis=0)
    return out


def entry_positions(n: int, m: int, pos0: int = 0) -> np.ndarray:
    """R3: an entry sits at the position of the last token it folds.

    Entry j of a stream whose first token has position pos0 covers tokens
    pos0 + j*m .. pos0 + j*m + m - 1, so p_j = pos0 + (j + 1)*m - 1.  With m = 1
    this is the token's own position.
    """
    return pos0 + (np.arange(n, dtype=np.int64) + 1) * m - 1


def rope(x, positions, rope_dim: int = 64, base: float = 10000.0) -> np.ndarray:
    """Rotary embedding of the last ``rope_dim`` channels [deep-dive §3.4: the
    main KV is rotated before it is quantised].

    R4 (the pages only say "after RoPE"): channel pairs (d-r+2i, d-r+2i+1),
    i = 0..r/2-1, are rotated by the angle p * base**(-2i/r), computed in
    float64:  (u, v) -> (u cos - v sin, u sin + v cos).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    n, d = x.shape
    r = rope_dim
    if r == 0:
        return x
    i = np.arange(r // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / r)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    u = x[:, d - r::2].copy()
    v = x[:, d - r + 1::2].copy()
    x[:, d - r::2] = u * c - v * s
    x[:, d - r + 1::2] = u * s + v * c
    return x


def compress(H, W_kv, W_z, m: int, pos0: int = 0, rope_dim: int = 64,
             base: float = 10000.0) -> np.ndarray:
    """Hidden states -> roped main-KV entries (float64) [deep-dive §2, §3.1, §3.4]."""
    C = project(H, W_kv)
    Z = project(H, W_z)
    kv = fold(C, Z, m)
    return rope(kv, entry_positions(kv.shape[0], m, pos0), rope_dim, base)


# --------------------------------------------------------------------------
# a2: FP4 quantisation and the indexer key  [daily 核心机制; deep-dive §3.1, §3.4]
# --------------------------------------------------------------------------

GROUP = 16  # channels per E4M3 scale [daily 核心机制; deep-dive §3.4]


@dataclass
class FP4Entries:
    codes: np.ndarray   # uint8 [n, d/2]; byte i = code[2i] | code[2i+1] << 4
    scales: np.ndarray  # uint8 [n, d/16]; E4M3FN


def quant_fp4(kv) -> FP4Entries:
    """FP4 E2M1 elements with one E4M3 scale per 16 channels.

    Input: the stored float32 entries [n, d].
    R5 (the pages name the formats only): absmax scaling onto the E2M1 maximum.
    Per group of 16 channels:
        amax = max |x|
        s32  = float32(amax / 6)           (one IEEE single division)
        S    = E4M3(s32)                   (nearest-even, saturating), s = value(S)
        code = E2M1(float32(x / s))        (nearest-even, saturating), sign of x kept
        code = sign(x)·0 when s == 0.
    Packing: low nibble = even channel.  Scales live in a separate plane.
    R6: E4M3 is the OCP "FN" variant (max 448).
    """
    x = np.asarray(kv)
    if x.dtype != np.float32:
        raise TypeError("quant_fp4 reads the stored float32 entries")
    n, d = x.shape
    if d % GROUP:
        raise ValueError("d must be a multiple of 16")
    g = x.reshape(n, d // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    s32 = (amax / np.float32(6.0)).astype(np.float32)
    S = e4m3_encode(s32.astype(np.float64))
    s = e4m3_decode(S).astype(np.float32)  # exact
    codes = np.zeros(g.shape, dtype=np.uint8)
    nz = s > 0
    sb = np.broadcast_to(s[:, :, None], g.shape)
    q = np.divide(g, sb, out=np.zeros_like(g), where=np.broadcast_to(nz[:, :, None], g.shape))
    codes[...] = e2m1_encode(q.astype(np.float64))
    # zero scale: every code is a signed zero
    zero_codes = np.where(np.signbit(g), np.uint8(8), np.uint8(0))
    codes = np.where(nz[:, :, None], codes, zero_codes).reshape(n, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return FP4Entries(packed, S.astype(np.uint8))


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n, h = p.shape
    out = np.empty((n, 2 * h), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequant_fp4(codes, scales) -> np.ndarray:
    """x̂ = E2M1(code) · E4M3(scale), exact in float64."""
    c = unpack_codes(codes)
    n, d = c.shape
    s = e4m3_decode(scales).reshape(n, d // GROUP, 1)
    return (e2m1_decode(c).reshape(n, d // GROUP, GROUP) * s).reshape(n, d)


def indexer_k(codes, scales, W_ik) -> np.ndarray:
    """Indexer key projected from the main KV [deep-dive §3.1: the indexer K is
    a projection of the main KV].

    R7: it is taken from the dequantised FP4 entry (only the FP4 global KV is
    persisted, [deep-dive §3.4], so the key must be re-derivable from it) and
    stored as bf16: k = bf16(x̂ · W_IK), accumulated in float64 and rounded once.
    Returns uint16 bf16 bit patterns [n, d_i].
    """
    return f64_to_bf16(dequant_fp4(codes, scales) @ _as_f64(W_ik))


# --------------------------------------------------------------------------
# a3/a9: indexer scores  [deep-dive §3.1, §3.2]
# --------------------------------------------------------------------------


def index_scores(q_idx, w, k_idx) -> np.ndarray:
    """Score of every key for one query: Indexer Q x Indexer K -> score.

    R8: s_j = sum_h w_h * max(0, q_h · k_j), float64.
    q_idx: [h_i, d_i] bf16 bits or floats; w: [h_i]; k_idx: [n, d_i].
    """
    q = _as_f64(q_idx)
    k = _as_f64(k_idx)
    dots = k @ q.T  # [n, h_i]
    return (np.maximum(dots, 0.0) * np.asarray(w, dtype=np.float64)[None, :]).sum(axis=1)


def visible_count(q_pos: Optional[int], n: int, m: int) -> int:
    """R15/R3: entry j is visible to a query at position t iff p_j <= t, i.e.
    j < floor((t + 1) / m) (entries counted from the start of the sequence).
    A decode query (q_pos None) sees every entry."""
    if q_pos is None:
        return n
    return int(min(n, max(0, (int(q_pos) + 1) // m)))


# --------------------------------------------------------------------------
# a5: Top-K  [deep-dive §3.3; K = 512 in §6.3]
# --------------------------------------------------------------------------


def topk(scores, K: int, n_visible: Optional[int] = None) -> np.ndarray:
    """The K best visible entries.

    R9: rank by (score descending, index ascending); take min(K, n_visible);
    return the indices ascending, padded with -1 to length K.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0] if n_visible is None else int(n_visible)
    s = s[:n]
    idx = np.arange(n)
    order = np.lexsort((idx, -s))  # primary: -s ascending; secondary: index ascending
    chosen = np.sort(order[:min(K, n)])
    out = np.full(K, -1, dtype=np.int64)
    out[:chosen.shape[0]] = chosen
    return out


# --------------------------------------------------------------------------
# a4: shared candidate pool  [deep-dive §3.3]
# --------------------------------------------------------------------------


def build_pool(scores, G: int = 128, PB: int = 2048, PE: int = 8,
               n_visible: Optional[int] = None) -> np.ndarray:
    """Candidate pool of the first Full indexer: PB blocks x PE positions.

    [deep-dive §3.3]: the first indexer scans the whole visible range and keeps
    the best positions of each block; 2,048 blocks x 8 positions = 16,384
    shared candidates.
    R10: a block is G = 128 consecutive entries; its score is its maximum; the
    PE best positions of a block rank by (score desc, index asc); the PB best
    blocks rank by (block max desc, block index asc).  The pool is the union,
    ascending (a block with fewer than PE visible entries gives all of them).
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0] if n_visible is None else int(n_visible)
    nblk = -(-n // G)
    bmax = np.array([s[b * G:min((b + 1) * G, n)].max() for b in range(nblk)])
    border = np.lexsort((np.arange(nblk), -bmax))[:PB]
    pool = []
    for b in border:
        lo, hi = b * G, min((b + 1) * G, n)
        seg = s[lo:hi]
        o = np.lexsort((np.arange(hi - lo), -seg))[:PE]
        pool.extend((lo + o).tolist())
    return np.sort(np.array(pool, dtype=np.int64))


def reindex(q_idx, w, k_idx, pool, K: int) -> np.ndarray:
    """Reindex layer: fresh scores over the pool only, then Top-K there.

    [deep-dive §3.2, §3.3; reading §4.2]: it reuses the shared main KV and
    indexer K, rescores with its own indexer query and picks a fresh Top-K
    inside the candidate pool.  Ties break to the lower entry index (the pool is
    ascending, so pool position order is entry order).
    """
    pool = np.asarray(pool, dtype=np.int64)
    s = index_scores(q_idx, w, _as_f64(k_idx)[pool])
    sel = topk(s, K)
    return np.where(sel >= 0, pool[np.maximum(sel, 0)], -1)


# --------------------------------------------------------------------------
# a8/a10: sparse attention  [deep-dive §3.1; digest 已确认; reading §4.2]
# --------------------------------------------------------------------------


def attention_keys(codes, scales, sel, swa_codes, swa_scale: float = 1.0,
                   swa_rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Selected main-KV entries (dequantised) followed by the layer's SWA tokens.

    R13: K = V = the whole dequantised entry.  R14: SWA tokens are E4M3 values
    times ``swa_scale``; ``swa_rows`` picks the visible window rows (all rows
    when None).
    """
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[sel >= 0]
    main = dequant_fp4(np.asarray(codes)[sel], np.asarray(scales)[sel])
    sw = np.asarray(swa_codes)
    if swa_rows is not None:
        sw = sw[np.asarray(swa_rows, dtype=np.int64)]
    swa = e4m3_decode(sw) * float(swa_scale)
    return np.concatenate([main, swa], axis=0)


def attend(q, keys, sm_scale: Optional[float] = None) -> np.ndarray:
    """Main-Q attention over the given keys, K = V (R13).

    o_h = sum_j softmax_j(q_h · key_j * sm_scale) key_j, one softmax over all
    keys (selected entries and window together, no de-duplication), default
    scale 1/sqrt(d).  No keys -> zeros.  float64 [H_q, d].
    """
    qf = _as_f64(q)
    k = np.asarray(keys, dtype=np.float64)
    d = qf.shape[-1]
    if k.shape[0] == 0:
        return np.zeros_like(qf)
    sc = 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)
    lg = qf @ k.T * sc
    lg = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(lg)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ k


def attend_lse(q, keys, sm_scale: Optional[float] = None) -> np.ndarray:
    """Natural-log normaliser of attend()'s softmax per head:
    log sum_j exp(q_h · key_j * sm_scale).  No keys -> -inf.  float64 [H_q]."""
    qf = _as_f64(q)
    k = np.asarray(keys, dtype=np.float64)
    if k.shape[0] == 0:
        return np.full(qf.shape[0], -np.inf)
    sc = 1.0 / np.sqrt(qf.shape[-1]) if sm_scale is None else float(sm_scale)
    lg = qf @ k.T * sc
    mx = lg.max(axis=1)
    return mx + np.log(np.exp(lg - mx[:, None]).sum(axis=1))


def swa_window_rows(q_pos: Optional[int], S: int, swa_pos0: int, n_win: int) -> np.ndarray:
    """R14: the window is the n_win most recent tokens including the query's
    own: positions (t - n_win, t].  A decode query (q_pos None) sees the whole
    window buffer.

    Buffer layout (reading R21): the buffer is a ring of S slots in which the
    token at position p >= swa_pos0 sits in slot (p - swa_pos0) mod S, so it
    holds at most the S most recent positions; a buffer filled in order from
    swa_pos0 that has not wrapped is the linear case (slot i = position
    swa_pos0 + i).  Returns the slots of the visible positions, oldest first:
    positions max(t - n_win + 1, swa_pos0, t - S + 1) .. t."""
    if q_pos is None:
        return np.arange(S)
    t = int(q_pos)
    lo = max(t - n_win + 1, swa_pos0, t - S + 1)
    pos = np.arange(lo, t + 1, dtype=np.int64)
    return (pos - swa_pos0) % S if S > 0 else pos[:0]


def sparse_attention(q, codes, scales, sel, swa_codes, swa_scale: float = 1.0,
                     q_pos: Optional[int] = None, swa_pos0: int = 0, n_win: int = 128,
                     sm_scale: Optional[float] = None) -> np.ndarray:
    """One query's CSA2 attention: selected FP4 entries ++ its SWA window."""
    rows = swa_window_rows(q_pos, np.asarray(swa_codes).shape[0], swa_pos0, n_win)
    keys = attention_keys(codes, scales, sel, swa_codes, swa_scale, rows)
    return attend(q, keys, sm_scale)


# --------------------------------------------------------------------------
# a11: layer schedule  [deep-dive §3.2; daily 核心机制]
# --------------------------------------------------------------------------

FULL, REINDEX, REUSE, SWA_ONLY = "F", "R", "U", "S"


def decoder_schedule() -> List[str]:
    """[deep-dive §3.2] decoder: group 1 = Full then 3 Reuse; groups 2-5 =
    Reindex then 3 Reuse (20 layers, ratio 1)."""
    return [FULL, REUSE, REUSE, REUSE] + [REINDEX, REUSE, REUSE, REUSE] * 4


def encoder_schedule() -> List[str]:
    """[deep-dive §3.2] encoder: layers 1-2 sliding window only, then three
    groups of Full then 5 Reuse (20 layers, ratio 2)."""
    return [SWA_ONLY, SWA_ONLY] + ([FULL] + [REUSE] * 5) * 3


@dataclass
class LayerInputs:
    q_main: np.ndarray                # [H_q, d] bf16 bits
    swa: np.ndarray                   # [S, d] E4M3 codes
    q_idx: Optional[np.ndarray] = None  # [h_i, d_i] bf16 bits (Full / Reindex)
    w: Optional[np.ndarray] = None      # [h_i]


@dataclass
class DecodeResult:
    sel: List[np.ndarray] = field(default_factory=list)   # per layer [K]
    out: List[np.ndarray] = field(default_factory=list)   # per layer [H_q, d]
    pool: Optional[np.ndarray] = None
    full_scores: Optional[np.ndarray] = None


def decode_step(schedule: Sequence[str], layers: Sequence[LayerInputs], codes, scales,
                k_idx, K: int = 512, G: int = 128, PB: int = 2048, PE: int = 8,
                swa_scale: float = 1.0, sm_scale: Optional[float] = None,
                need_pool: Optional[bool] = None) -> DecodeResult:
    """One decode query of one sequence through a layer schedule.

    [deep-dive §3.2, §3.3; reading §4.2]: Full scores every entry and makes a
    fresh Top-K (the first Full also builds the candidate pool); Reindex
    rescores the pool with its own indexer query; Reuse takes the most recent
    selection (R12) and runs no indexer; SWA-only layers attend to their window
    alone.  Every layer attends with its own query and its own window.
    R11: the Full layer's Top-K is global over the visible range.
    """
    if need_pool is None:
        need_pool = REINDEX in schedule
    res = DecodeResult()
    sel = None
    empty = np.full(K, -1, dtype=np.int64)
    for mode, li in zip(schedule, layers):
        if mode == FULL:
            s = index_scores(li.q_idx, li.w, k_idx)
            sel = topk(s, K)
            if need_pool and res.pool is None:
                res.pool = build_pool(s, G, PB, PE)
                res.full_scores = s
        elif mode == REINDEX:
            if res.pool is None:
                raise ValueError("Reindex before any Full layer")
            sel = reindex(li.q_idx, li.w, k_idx, res.pool, K)
        elif mode == REUSE:
            if sel is None:
                raise ValueError("Reuse before any Full/Reindex layer")
        elif mode == SWA_ONLY:
            pass
        else:
            raise ValueError(mode)
        cur = empty if mode == SWA_ONLY else sel
        res.sel.append(cur.copy())
        res.out.append(sparse_attention(li.q_main, codes, scales, cur, li.swa, swa_scale,
                                        sm_scale=sm_scale))
    return res


@dataclass
class PrefillLayerInputs:
    q_main: np.ndarray                  # [Tq, H_q, d] bf16 bits
    swa: np.ndarray                     # [S, d] E4M3 codes; row i is position swa_pos0 + i
    q_idx: Optional[np.ndarray] = None  # [Tq, h_i, d_i] bf16 bits (Full layers)
    w: Optional[np.ndarray] = None      # [Tq, h_i]


@dataclass
class PrefillResult:
    kv: np.ndarray                      # [n_new, d] float64: the chunk's compressed entries
    entries: FP4Entries                 # their FP4 form
    k_new: np.ndarray                   # [n_new, d_i] bf16 bits: their indexer keys
    rows: np.ndarray                    # query rows evaluated
    sel: List[np.ndarray] = field(default_factory=list)   # per layer [len(rows), K]
    out: List[np.ndarray] = field(default_factory=list)   # per layer [len(rows), H_q, d]


def prefill_chunk(schedule: Sequence[str], layers: Sequence[PrefillLayerInputs], H, W_kv, W_z,
                  m: int, pos0: int, codes_pre, scales_pre, k_pre, W_ik, K: int = 512,
                  swa_pos0: int = 0, n_win: int = 128, swa_scale: float = 1.0,
                  rows: Optional[Sequence[int]] = None, rope_dim: int = 64,
                  sm_scale: Optional[float] = None) -> PrefillResult:
    """One prefill chunk through an encoder layer schedule.

    [deep-dive §3.1, §3.2] the chunk's hidden states (tokens pos0 .. pos0+Tq-1)
    are compressed into new entries, which are quantised and given indexer keys
    and appended after the entries already cached (codes_pre etc., entry j at
    position (j+1)m-1, so pos0 must be a multiple of m).  Every chunk token is
    then a query at its own position t: a Full layer scores the entries visible
    to it (R3/R15: p_j <= t) and takes their Top-K; Reuse layers keep that
    selection (R12); SWA-only layers attend to the window alone; every layer
    attends over the selection and the window [t - n_win + 1, t] (R14).
    ``rows`` limits the evaluation to some query rows (all when None).
    """
    if pos0 % m:
        raise ValueError("pos0 must be a multiple of m")
    kv = compress(H, W_kv, W_z, m, pos0, rope_dim)
    q8 = quant_fp4(kv.astype(np.float32))  # the entries are stored as float32, then quantised
    k_new = indexer_k(q8.codes, q8.scales, W_ik)
    codes = np.concatenate([np.asarray(codes_pre), q8.codes], axis=0)
    scales = np.concatenate([np.asarray(scales_pre), q8.scales], axis=0)
    k_all = np.concatenate([np.asarray(k_pre), k_new], axis=0)
    n = codes.shape[0]
    Tq = np.asarray(H).shape[0]
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    res = PrefillResult(kv=kv, entries=q8, k_new=k_new, rows=rows)
    empty = np.full(K, -1, dtype=np.int64)
    sel = [None] * len(rows)
    for mode, li in zip(schedule, layers):
        if mode not in (FULL, REUSE, SWA_ONLY):
            raise ValueError(f"prefill layer mode {mode!r}")
        S_l, O_l = [], []
        for r, t in enumerate(rows):
            pos = pos0 + int(t)
            if mode == FULL:
                nvis = visible_count(pos, n, m)
                s = index_scores(li.q_idx[t], li.w[t], k_all[:nvis])
                sel[r] = topk(s, K, nvis)
            elif mode == REUSE and sel[r] is None:
                raise ValueError("Reuse before any Full layer")
            cur = empty if mode == SWA_ONLY else sel[r]
            S_l.append(cur.copy())
            O_l.append(sparse_attention(li.q_main[t], codes, scales, cur, li.swa, swa_scale,
                                        q_pos=pos, swa_pos0=swa_pos0, n_win=n_win,
                                        sm_scale=sm_scale))
        res.sel.append(np.stack(S_l) if S_l else np.zeros((0, K), dtype=np.int64))
        res.out.append(np.stack(O_l) if O_l else np.zeros((0,) + np.asarray(li.q_main).shape[1:]))
    return res


# --------------------------------------------------------------------------


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)
