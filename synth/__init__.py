"""Seeded synthetic inputs for the CSA2 layer.

Shared by the tests, the benchmark and the smoke check.  This module only draws
random numbers and casts them to storage formats with library casts (torch's
bf16 and float8_e4m3fn conversions); it holds none of the method's arithmetic
(no compression, quantisation, scoring, selection or attention).

Every tensor of every sequence comes from its own stream,
``PCG64(SeedSequence([seed, tag, layer, b]))``, so any one sequence's inputs can
be regenerated alone (the oracle checks sampled sequences of large workloads
this way).

Workloads (synthetic stand-ins; no trained weights exist here):
  * hidden states H ~ N(0,1); W_KV, W_Z ~ N(0, 1/d_model);
  * decode main KV drawn directly as post-RoPE float32 N(0,1);
  * W_IK ~ N(0, 1/d) stored as bf16;
  * indexer queries N(0,1) bf16, head weights U(0,1) (or all ones);
  * main queries N(0,1) bf16; sliding-window tokens N(0,1) cast to E4M3;
  * planted keys: a fraction of entries gets beta * v added (v a seeded unit
    vector) and every indexer query head gets alpha * u, u = unit(v · W_IK),
    so that selection is not decided by noise alone.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import List, Optional

import numpy as np

TAG = {"kv": 1, "wik": 2, "qidx": 3, "w": 4, "qmain": 5, "swa": 6, "plant_pos": 7,
       "plant_dir": 8, "H": 9, "wkv": 10, "wz": 11, "qpos": 12, "winkv": 13, "Happ": 14}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # sequences
    N: int                 # main-KV entries per sequence
    d: int                 # main-KV / head dim
    h_i: int               # indexer heads
    d_i: int               # indexer dim
    H_q: int               # main query heads
    S: int = 128           # sliding-window tokens per layer
    K: int = 512           # Top-K
    m: int = 1             # compression ratio
    schedule: str = "F"    # F/R/U per layer
    seed: int = 0
    plant_frac: float = 0.0
    alpha: float = 8.0
    beta: float = 8.0
    equal_w: bool = False  # all head weights 1.0
    G: int = 128
    PB: int = 2048
    PE: int = 8
    # compressor (only for workloads that build the cache from hidden states)
    T: int = 0             # tokens of hidden state (0 = KV drawn directly)
    d_model: int = 0
    h_dtype: str = "f32"   # "f32" or "bf16"
    rope_dim: int = 64
    # prefill: the last `chunk` of T tokens are the queries; the entries of the
    # tokens before them are drawn directly (like decode KV), the chunk's own
    # entries come from its hidden states through the compressor
    chunk: int = 0
    n_win: int = 128
    # decode cache append: one new entry per sequence into row N-1 of an N-row
    # cache, and the token's window KV into every layer's window
    append: bool = False
    # decode with Tq queries per sequence (a token and the positions drafted after
    # it, the first at position N*m): one shared scan of the keys, a Top-K per
    # query; the window buffer holds n_win + Tq - 1 tokens ending at the last one
    Tq: int = 1

    @property
    def pos0(self) -> int:
        """Position of the first chunk token (prefill)."""
        return self.T - self.chunk

    @property
    def n_pre(self) -> int:
        """Entries that exist before the chunk (prefill)."""
        return self.pos0 // self.m

    @property
    def swa_pos0(self) -> int:
        """Position of the first window token a chunk query can see (prefill)."""
        return max(0, self.pos0 - (self.n_win - 1))

    @property
    def layers(self) -> List[str]:
        return self.schedule.split(",") if "," in self.schedule else list(self.schedule)

    @property
    def needs_pool(self) -> bool:
        return "R" in self.layers


WORKLOADS = {
    # single-layer Full decode, 4K context built from hidden states, m = 2
    "full_decode_4k": Workload("full_decode_4k", B=1, N=2048, d=256, h_i=4, d_i=64, H_q=16,
                               m=2, schedule="F", seed=0, equal_w=True, T=4096, d_model=1024),
    # batch 64 x 64K context, Full + 3 Reuse
    "decode_64k_b64": Workload("decode_64k_b64", B=64, N=65536, d=512, h_i=8, d_i=128, H_q=64,
                               schedule="FUUU", seed=1),
    # batch 32 x 256K, Full (pool) + 3 Reindex, 1% planted
    "reindex_256k_b32": Workload("reindex_256k_b32", B=32, N=262144, d=512, h_i=8, d_i=128,
                                 H_q=64, schedule="FRRR", seed=2, plant_frac=0.01),
    # batch 8 x 1M, the 20-layer decoder schedule, 0.5% planted
    "decode_1m_b8": Workload("decode_1m_b8", B=8, N=1 << 20, d=512, h_i=8, d_i=128, H_q=64,
                             schedule="FUUURUUURUUURUUURUUU", seed=4, plant_frac=0.005),
    # prefill chunk: the last 8,192 tokens of a 32,768-token sequence, m = 2
    # (16,384 entries, 12,288 before the chunk), d_model 5,120 bf16, Full + 5 Reuse
    "prefill_32k": Workload("prefill_32k", B=1, N=16384, d=512, h_i=8, d_i=128, H_q=64,
                            S=8192 + 127, m=2, schedule="FUUUUU", seed=3, T=32768,
                            chunk=8192, d_model=5120, h_dtype="bf16"),
    # decode_64k_b64 with 6 queries per sequence (1 + 5 drafted positions)
    "mtp_64k_b64": Workload("mtp_64k_b64", B=64, N=65536, d=512, h_i=8, d_i=128, H_q=64,
                            S=128 + 5, schedule="FUUU", seed=6, Tq=6),
    # decode cache append: 64 sequences, d = 512 entries with 128-dim keys, the
    # token's window KV for the 20 decoder layers (128-token windows); the entry
    # comes from hidden states of width 5,120 (bf16) through the compressor
    "append_b64": Workload("append_b64", B=64, N=65536, d=512, h_i=8, d_i=128, H_q=64,
                           schedule="FUUURUUURUUURUUURUUU", seed=5, d_model=5120, h_dtype="bf16",
                           append=True),
}


def workload(name: str, **over) -> Workload:
    return replace(WORKLOADS[name], **over)


# --------------------------------------------------------------------------


KV_CHUNK = 65536  # main-KV rows per random stream


def _rng(seed: int, tag: str, layer: int = 0, b: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAG[tag], layer, b, chunk])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), via torch's nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes (uint8), via torch's float8_e4m3fn cast (|x| < 448 here)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# --------------------------------------------------------------------------


def w_ik(wl: Workload) -> np.ndarray:
    """Indexer-key projection [d, d_i], bf16 bits, N(0, 1/d)."""
    r = _rng(wl.seed, "wik")
    return to_bf16_bits(r.standard_normal((wl.d, wl.d_i), dtype=np.float32) / np.float32(np.sqrt(wl.d)))


def plant_direction(wl: Workload):
    """(v, u): v a unit vector in main-KV space, u = unit(v · W_IK) in indexer space."""
    r = _rng(wl.seed, "plant_dir")
    v = r.standard_normal(wl.d)
    v /= np.linalg.norm(v)
    u = v @ bf16_bits_to_f32(w_ik(wl)).astype(np.float64)
    u /= np.linalg.norm(u)
    return v, u


def planted_positions(wl: Workload, b: int) -> np.ndarray:
    n = int(round(wl.plant_frac * wl.N))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(wl.seed, "plant_pos", 0, b)
    return np.sort(r.choice(wl.N, size=n, replace=False))


def main_kv(wl: Workload, b: int, lo: int = 0, hi: Optional[int] = None) -> np.ndarray:
    """Post-RoPE main KV of sequence b, float32 [N, d] (rows lo:hi)."""
    hi = wl.N if hi is None else hi
    x = np.empty((hi - lo, wl.d), dtype=np.float32)
    for c in range(lo // KV_CHUNK, -(-hi // KV_CHUNK)):
        c0, c1 = c * KV_CHUNK, min((c + 1) * KV_CHUNK, wl.N)
        blk = _rng(wl.seed, "kv", 0, b, c).standard_normal((c1 - c0, wl.d), dtype=np.float32)
        a, z = max(lo, c0), min(hi, c1)
        x[a - lo:z - lo] = blk[a - c0:z - c0]
    if wl.plant_frac > 0:
        pos = planted_positions(wl, b)
        v, _ = plant_direction(wl)
        pos = pos[(pos >= lo) & (pos < hi)] - lo
        x[pos] += (wl.beta * v).astype(np.float32)
    return x


Q_CHUNK = 256  # query rows per random stream


def _query_rows(wl: Workload, tag: str, layer: int, b: int, Tq: int, t0: int, shape, draw):
    """Rows t0 .. t0+Tq-1 of a per-query tensor; row t comes from the stream of
    query chunk t // Q_CHUNK, so any query range can be regenerated alone."""
    out = np.empty((Tq,) + tuple(shape), dtype=np.float32)
    t1 = t0 + Tq
    for c in range(t0 // Q_CHUNK, -(-t1 // Q_CHUNK)):
        c0 = c * Q_CHUNK
        a, z = max(t0, c0), min(t1, c0 + Q_CHUNK)
        blk = draw(_rng(wl.seed, tag, layer, b, c), (z - c0,) + tuple(shape))
        out[a - t0:z - t0] = blk[a - c0:]
    return out


def q_index(wl: Workload, layer: int, b: int, Tq: int = 1, t0: int = 0) -> np.ndarray:
    """Indexer query [Tq, h_i, d_i] bf16 bits (query rows t0 .. t0+Tq-1)."""
    q = _query_rows(wl, "qidx", layer, b, Tq, t0, (wl.h_i, wl.d_i),
                    lambda r, sh: r.standard_normal(sh, dtype=np.float32))
    if wl.plant_frac > 0:
        _, u = plant_direction(wl)
        q = q + (wl.alpha * u).astype(np.float32)[None, None, :]
    return to_bf16_bits(q)


def head_weights(wl: Workload, layer: int, b: int, Tq: int = 1, t0: int = 0) -> np.ndarray:
    if wl.equal_w:
        return np.ones((Tq, wl.h_i), dtype=np.float32)
    return _query_rows(wl, "w", layer, b, Tq, t0, (wl.h_i,),
                       lambda r, sh: r.random(sh, dtype=np.float32))


def q_main(wl: Workload, layer: int, b: int, Tq: int = 1, t0: int = 0) -> np.ndarray:
    """Main query [Tq, H_q, d] bf16 bits (query rows t0 .. t0+Tq-1)."""
    return to_bf16_bits(_query_rows(wl, "qmain", layer, b, Tq, t0, (wl.H_q, wl.d),
                                    lambda r, sh: r.standard_normal(sh, dtype=np.float32)))


def q_positions(wl: Workload) -> np.ndarray:
    """Positions of the chunk's queries (prefill): pos0 .. T-1, int32."""
    return np.arange(wl.pos0, wl.T, dtype=np.int32)


def new_token_window(wl: Workload) -> np.ndarray:
    """Window KV of one new token for every layer and sequence, float32 [L, B, d]."""
    return np.stack([np.stack([_rng(wl.seed, "winkv", li, b).standard_normal(wl.d, dtype=np.float32)
                               for b in range(wl.B)]) for li in range(len(wl.layers))])


def swa_tokens(wl: Workload, layer: int, b: int, S: Optional[int] = None) -> np.ndarray:
    r = _rng(wl.seed, "swa", layer, b)
    return to_e4m3_codes(r.standard_normal((wl.S if S is None else S, wl.d), dtype=np.float32))


def hidden(wl: Workload, b: int = 0) -> np.ndarray:
    """Hidden states of the tokens that go through the compressor: all T tokens,
    or the chunk's tokens in prefill.  [T or chunk, d_model] float32, or bf16
    bits when h_dtype == 'bf16'."""
    r = _rng(wl.seed, "H", 0, b)
    h = r.standard_normal((wl.chunk or wl.T, wl.d_model), dtype=np.float32)
    return to_bf16_bits(h) if wl.h_dtype == "bf16" else h


def append_hidden(wl: Workload) -> np.ndarray:
    """Hidden states of the block of m tokens that completes each sequence's new
    entry (decode cache append), bf16 bits [B, m, d_model]."""
    h = np.stack([_rng(wl.seed, "Happ", 0, b).standard_normal((wl.m, wl.d_model), dtype=np.float32)
                  for b in range(wl.B)])
    return to_bf16_bits(h)


def compressor_weights(wl: Workload, d_z: Optional[int] = None):
    """(W_KV, W_Z), N(0, 1/d_model); float32, or bf16 bits when h_dtype == 'bf16'."""
    d_z = wl.d if d_z is None else d_z
    sc = np.float32(1.0 / np.sqrt(wl.d_model))
    wkv = _rng(wl.seed, "wkv").standard_normal((wl.d_model, wl.d), dtype=np.float32) * sc
    wz = _rng(wl.seed, "wz").standard_normal((wl.d_model, d_z), dtype=np.float32) * sc
    if wl.h_dtype == "bf16":
        return to_bf16_bits(wkv), to_bf16_bits(wz)
    return wkv, wz
