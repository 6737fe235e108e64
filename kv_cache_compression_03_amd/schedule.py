"""Decode step and prefill chunk of a Full / Reindex / Reuse layer schedule on the
CSA2 library.

[deep-dive §3.2] every attention layer is statically Full (fresh indexer scores
and Top-K; the first Full layer of a step also builds the shared candidate pool,
§3.3), Reindex (fresh scores over the pool only) or Reuse (the most recent
selection, no indexer); every layer attends with its own main query and its own
window [reading §4.2].  The decoder schedule is Full + 3 Reuse, then four groups
of Reindex + 3 Reuse.

All buffers are allocated once, so a step can be captured into a HIP graph and
replayed.  Layers run in order on one stream (in a model, layer l+1's queries
depend on layer l's output, so layers are never fused).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as bd

FULL, REINDEX, REUSE, SWA_ONLY = "F", "R", "U", "S"


@dataclass
class LayerBuffers:
    """Per-layer inputs on the device: main query [B,1,H_q,d] bf16, window [B,S,d]
    E4M3 bytes and, for Full/Reindex layers, indexer query [B,1,h_i,d_i] bf16 and
    head weights [B,1,h_i] f32."""
    q_main: torch.Tensor
    swa: torch.Tensor
    q_idx: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None


class DecodeSchedule:
    def __init__(self, schedule: Sequence[str], B: int, N: int, d: int, h_i: int, d_i: int,
                 H_q: int, S: int, K: int = 512, G: int = 128, PB: int = 2048, PE: int = 8,
                 swa_scale: float = 1.0, device: str = "cuda", Tq: int = 1,
                 full_in_pool: bool = False):
        """Tq > 1: several queries per sequence in one step (a token and the positions
        drafted after it), each with its own Top-K from one shared scan of the keys.
        Reindex rescoring takes one query per sequence, so it needs Tq = 1.
        full_in_pool: a Full layer takes its Top-K inside the candidate pool built
        from its own scores rather than over every entry (the other reading of the
        Full layer's selection); one query per sequence."""
        self.layers: List[str] = list(schedule)
        if Tq < 1:
            raise ValueError("Tq must be >= 1")
        if Tq > 1 and (REINDEX in self.layers or full_in_pool):
            raise ValueError("Reindex and pool-restricted Full layers take one query per sequence (Tq = 1)")
        self.full_in_pool = full_in_pool
        for i, mode in enumerate(self.layers):
            if mode not in (FULL, REINDEX, REUSE, SWA_ONLY):
                raise ValueError(f"layer {i}: unknown mode {mode!r}")
            if mode in (REUSE,) and not any(x in (FULL, REINDEX) for x in self.layers[:i]):
                raise ValueError(f"layer {i}: Reuse before any Full/Reindex layer")
            if mode == REINDEX and FULL not in self.layers[:i]:
                raise ValueError(f"layer {i}: Reindex before any Full layer")
        self.B, self.Tq, self.N, self.d, self.h_i, self.d_i = B, Tq, N, d, h_i, d_i
        self.H_q, self.S, self.K, self.G, self.PB, self.PE = H_q, S, K, G, PB, PE
        self.swa_scale = swa_scale
        self.need_pool = REINDEX in self.layers or (full_in_pool and FULL in self.layers)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty(B, Tq, N, dtype=torch.float32, device=dev)
        self.sel: Dict[int, torch.Tensor] = {i: torch.empty(B, Tq, K, **i32)
                                             for i, m in enumerate(self.layers) if m in (FULL, REINDEX)}
        self.no_sel = torch.full((B, Tq, K), -1, **i32)
        self.pool = torch.empty(B, PB * PE, **i32) if self.need_pool else None
        self.pool_len = torch.empty(B, **i32) if self.need_pool else None
        self.out = [torch.empty(B, Tq, H_q, d, dtype=torch.float32, device=dev) for _ in self.layers]
        ws = max(bd.csa2_index_full_workspace(B, Tq, N, h_i, d_i, G if self.need_pool else 0,
                                              PB if self.need_pool else 0, PE,
                                              0 if full_in_pool else K),
                 bd.csa2_index_reindex_workspace(B, PB * PE, K) if self.need_pool else 0)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(max(bd.csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S), 256),
                                   dtype=torch.uint8, device=dev)

    def selection_of(self, layer: int) -> torch.Tensor:
        """The selection layer `layer` attends to (Reuse: the most recent Full/Reindex)."""
        if self.layers[layer] == SWA_ONLY:
            return self.no_sel
        for j in range(layer, -1, -1):
            if j in self.sel:
                return self.sel[j]
        raise ValueError("no selection")

    def step(self, codes: torch.Tensor, scales: torch.Tensor, k_idx: torch.Tensor,
             layers: Sequence[LayerBuffers], stream=None, q_pos=None, swa_pos0: int = 0,
             n_win: int = 128) -> List[torch.Tensor]:
        """Tq decode queries per sequence through every layer; returns the per-layer
        outputs.  q_pos [B, Tq] (optional) limits each query's window to the tokens
        at positions (t - n_win, t], window slot i holding position swa_pos0 + i."""
        B, K, R = self.B, self.K, self.B * self.Tq
        pool_built = False
        for i, (mode, lb) in enumerate(zip(self.layers, layers)):
            if mode == FULL:
                build = (self.need_pool and not pool_built) or self.full_in_pool
                # scores, the pool (first Full layer) and, unless it is taken inside
                # the pool, the layer's Top-K in one call
                bd.csa2_index_full(lb.q_idx, lb.w, k_idx, scores=self.scores,
                                   pool=self.pool if build else None,
                                   pool_len=self.pool_len if build else None,
                                   G=self.G, PB=self.PB, PE=self.PE,
                                   K=0 if self.full_in_pool else K,
                                   sel=None if self.full_in_pool else self.sel[i].view(R, K),
                                   ws=self.ws, stream=stream)
                pool_built = pool_built or build
                if self.full_in_pool:   # the Top-K inside the pool this layer just built
                    bd.csa2_index_reindex(lb.q_idx.view(B, self.h_i, self.d_i), lb.w.view(B, self.h_i),
                                          k_idx, self.pool, self.pool_len, K,
                                          sel=self.sel[i].view(B, K), ws=self.ws, stream=stream)
            elif mode == REINDEX:
                bd.csa2_index_reindex(lb.q_idx.view(B, self.h_i, self.d_i), lb.w.view(B, self.h_i),
                                      k_idx, self.pool, self.pool_len, K,
                                      sel=self.sel[i].view(B, K), ws=self.ws, stream=stream)
            bd.csa2_sparse_attn(lb.q_main, codes, scales, self.selection_of(i), lb.swa,
                                swa_scale=self.swa_scale, q_pos=q_pos, swa_pos0=swa_pos0,
                                n_win=n_win, out=self.out[i], ws=self.attn_ws, stream=stream)
        return self.out

    def capture(self, codes, scales, k_idx, layers, warmup: int = 1, **step_kw) -> torch.cuda.CUDAGraph:
        """Capture one step into a graph (after `warmup` eager steps on a side stream)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.step(codes, scales, k_idx, layers, **step_kw)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(codes, scales, k_idx, layers, **step_kw)
        return g


class PrefillChunk:
    """One prefill chunk of one sequence through an encoder schedule.

    [deep-dive §3.1, §3.2] the chunk's hidden states (tokens pos0 .. pos0+Tq-1)
    are compressed into Tq/m new entries, which are quantised to FP4 with their
    indexer keys and written after the n_pre entries already cached.  Every
    chunk token is then a query at its own position: a Full layer scores the
    entries visible to it (p_j <= t) and keeps its Top-K, Reuse layers keep that
    selection, SWA-only layers attend to the window alone, and every layer
    attends over the selection and the window [t - n_win + 1, t].

    The cache (codes [1, N, d/2], scales [1, N, d/16], k_idx [1, N, d_i]) is the
    caller's; this object owns the per-chunk buffers, allocated once.
    """

    def __init__(self, schedule: Sequence[str], N: int, n_pre: int, Tq: int, d: int, h_i: int,
                 d_i: int, H_q: int, S: int, K: int = 512, m: int = 2, pos0: int = 0,
                 swa_pos0: int = 0, n_win: int = 128, rope_dim: int = 64,
                 swa_scale: float = 1.0, device: str = "cuda"):
        self.layers: List[str] = list(schedule)
        for i, mode in enumerate(self.layers):
            if mode not in (FULL, REUSE, SWA_ONLY):
                raise ValueError(f"layer {i}: prefill layers are Full, Reuse or SWA-only, got {mode!r}")
            if mode == REUSE and FULL not in self.layers[:i]:
                raise ValueError(f"layer {i}: Reuse before any Full layer")
        if Tq % m or pos0 % m or n_pre != pos0 // m or n_pre + Tq // m > N:
            raise ValueError("chunk geometry: need Tq and pos0 multiples of m, n_pre = pos0/m, "
                             "n_pre + Tq/m <= N")
        self.N, self.n_pre, self.Tq, self.d, self.h_i, self.d_i = N, n_pre, Tq, d, h_i, d_i
        self.H_q, self.S, self.K, self.m, self.pos0 = H_q, S, K, m, pos0
        self.swa_pos0, self.n_win, self.rope_dim, self.swa_scale = swa_pos0, n_win, rope_dim, swa_scale
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.n_new = Tq // m
        self.kv_new = torch.empty(1, self.n_new, d, dtype=torch.float32, device=dev)
        self.q_pos = torch.arange(pos0, pos0 + Tq, **i32).view(1, Tq)
        self.scores = torch.empty(1, Tq, N, dtype=torch.float32, device=dev)
        self.sel: Dict[int, torch.Tensor] = {i: torch.empty(1, Tq, K, **i32)
                                             for i, mo in enumerate(self.layers) if mo == FULL}
        self.no_sel = torch.full((1, Tq, K), -1, **i32)
        self.out = [torch.empty(1, Tq, H_q, d, dtype=torch.float32, device=dev) for _ in self.layers]
        self.ws = torch.empty(max(bd.csa2_index_full_workspace(1, Tq, N, h_i, d_i, 0, 0, 8, K), 256),
                              dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(max(bd.csa2_sparse_attn_workspace(1, Tq, H_q, d, K, S), 256),
                                   dtype=torch.uint8, device=dev)

    def selection_of(self, layer: int) -> torch.Tensor:
        if self.layers[layer] == SWA_ONLY:
            return self.no_sel
        for j in range(layer, -1, -1):
            if j in self.sel:
                return self.sel[j]
        raise ValueError("no selection")

    def step(self, H: torch.Tensor, W_kv: torch.Tensor, W_z: torch.Tensor, W_ik: torch.Tensor,
             codes: torch.Tensor, scales: torch.Tensor, k_idx: torch.Tensor,
             layers: Sequence[LayerBuffers], stream=None) -> List[torch.Tensor]:
        """H [Tq, d_model] (bf16 or f32); layers[i]: q_main [1, Tq, H_q, d], swa [1, S, d] and,
        for Full layers, q_idx [1, Tq, h_i, d_i], w [1, Tq, h_i].  Returns per-layer outputs."""
        lo, hi = self.n_pre, self.n_pre + self.n_new
        bd.csa2_compress(H.view(1, self.Tq, -1), W_kv, W_z, self.m, pos0=self.pos0,
                         rope_dim=self.rope_dim, out=self.kv_new, stream=stream)
        bd.csa2_quant_fp4(self.kv_new[0], codes=codes[0, lo:hi], scales=scales[0, lo:hi], W_ik=W_ik,
                          k_idx=k_idx[0, lo:hi], stream=stream)
        for i, (mode, lb) in enumerate(zip(self.layers, layers)):
            if mode == FULL:
                # causal scores and each query's Top-K over the entries visible to it
                bd.csa2_index_full(lb.q_idx, lb.w, k_idx, q_pos=self.q_pos, m=self.m,
                                   scores=self.scores, K=self.K, sel=self.sel[i].view(self.Tq, self.K),
                                   ws=self.ws, stream=stream)
            bd.csa2_sparse_attn(lb.q_main, codes, scales, self.selection_of(i), lb.swa,
                                swa_scale=self.swa_scale, q_pos=self.q_pos, swa_pos0=self.swa_pos0,
                                n_win=self.n_win, out=self.out[i], ws=self.attn_ws, stream=stream)
        return self.out
