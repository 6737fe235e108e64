"""Thin ctypes binding of libcsa2.so: the same six calls and helpers as
``include/csa2.h``.

Marshalling only: each function checks tensor device/dtype/contiguity, derives
sizes from shapes, allocates missing outputs/workspaces with torch (device
memory only) and calls the C entry point on the current (or given) stream.
Every step of the layer runs in the library's HIP kernels.  If the library has
not been built this module raises at first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

DTYPE_F32, DTYPE_BF16 = 0, 1

_c_p, _c_i, _c_ll, _c_f, _c_d, _c_sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong,
                                       ctypes.c_float, ctypes.c_double, ctypes.c_size_t)

_SIGS = {
    "csa2_version": ([], ctypes.c_char_p),
    "csa2_status_string": ([_c_i], ctypes.c_char_p),
    "csa2_last_error": ([], ctypes.c_char_p),
    "csa2_compress": ([_c_p, _c_i, _c_i, _c_i, _c_i, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_ll,
                       _c_i, _c_d, _c_p, _c_p], _c_i),
    "csa2_quant_fp4": ([_c_p, _c_ll, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_p], _c_i),
    "csa2_indexer_keys": ([_c_p, _c_p, _c_ll, _c_i, _c_p, _c_i, _c_p, _c_p], _c_i),
    "csa2_cache_append": ([_c_p, _c_i, _c_i, _c_ll, _c_ll, _c_p, _c_p, _c_p, _c_i, _c_p, _c_p, _c_i,
                           _c_i, _c_i, _c_f, _c_p, _c_p], _c_i),
    "csa2_index_full_workspace": ([_c_i, _c_i, _c_i, _c_i, _c_i, _c_i, _c_i, _c_i, _c_i], _c_sz),
    "csa2_index_full": ([_c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_i, _c_p, _c_i, _c_p, _c_p,
                         _c_p, _c_i, _c_i, _c_i, _c_i, _c_p, _c_p, _c_sz, _c_p], _c_i),
    "csa2_topk_workspace": ([_c_i, _c_i, _c_i], _c_sz),
    "csa2_topk": ([_c_p, _c_i, _c_i, _c_p, _c_p, _c_i, _c_p, _c_p, _c_sz, _c_p], _c_i),
    "csa2_topk_noalloc": ([_c_p, _c_i, _c_i, _c_p, _c_p, _c_i, _c_p, _c_p], _c_i),
    "csa2_index_reindex_workspace": ([_c_i, _c_i, _c_i], _c_sz),
    "csa2_index_reindex": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_i, _c_i, _c_i, _c_p,
                            _c_p, _c_sz, _c_p], _c_i),
    "csa2_sparse_attn_workspace": ([_c_i, _c_i, _c_i, _c_i, _c_i, _c_i], _c_sz),
    "csa2_sparse_attn": ([_c_p, _c_p, _c_p, _c_i, _c_p, _c_i, _c_p, _c_f, _c_i, _c_ll, _c_i, _c_p,
                          _c_i, _c_i, _c_i, _c_i, _c_f, _c_p, _c_p, _c_p, _c_sz, _c_p], _c_i),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_compression_03_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


class CSA2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        super().__init__(f"{fn}: {L.csa2_status_string(status).decode()}: "
                         f"{L.csa2_last_error().decode()}")
        self.status = status


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CSA2Error(name, st)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _chk(t, name: str, dtypes, shape=None, numel=None):
    """Type, dtype, full shape (or element count) and contiguity of one tensor
    argument.  The C ABI sees only pointers and the sizes derived from the primary
    inputs, so every buffer the caller hands in is checked against those sizes
    here: a smaller buffer would be read or written out of bounds on the device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if numel is not None and t.numel() != int(numel):
        raise ValueError(f"{name} has {t.numel()} elements, expected {int(numel)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(**tensors) -> None:
    """Every tensor handed to the library must be device memory."""
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")


BF16 = (torch.bfloat16, torch.int16, torch.uint16)
U8 = (torch.uint8, torch.float8_e4m3fn)
I32 = (torch.int32,)
F32 = (torch.float32,)


def _ws(nbytes: int, like: torch.Tensor, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
    return ws


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _ndim(t, name: str, n: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, has shape {tuple(t.shape)}")


# ------------------------------------------------------------------ helpers

def csa2_version() -> str:
    return lib().csa2_version().decode()


def csa2_index_full_workspace(B, Tq, N, h_i=8, d_i=128, G=128, PB=2048, PE=8, K=0) -> int:
    """Workspace of csa2_index_full (G or PB = 0: no pool; K = 0: no Top-K)."""
    return lib().csa2_index_full_workspace(B, Tq, N, h_i, d_i, G, PB, PE, K)


def csa2_topk_workspace(R, N, K) -> int:
    return lib().csa2_topk_workspace(R, N, K)


def csa2_index_reindex_workspace(B, P, K) -> int:
    return lib().csa2_index_reindex_workspace(B, P, K)


def csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S) -> int:
    return lib().csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S)


# ------------------------------------------------------------------ the calls

def csa2_compress(H, W_kv, W_z, m: int, pos0: int = 0, rope_dim: int = 64,
                  rope_theta: float = 10000.0, out=None, stream=None) -> torch.Tensor:
    """H [B, T, d_model] (f32 or bf16), W_kv [d_model, d], W_z [d_model, d or 1] -> [B, T//m, d] f32."""
    _ndim(H, "H", 3)
    _chk(H, "H", F32 + BF16)
    B, T, dm = H.shape
    _ndim(W_kv, "W_kv", 2)
    d = W_kv.shape[1]
    _chk(W_kv, "W_kv", F32 + BF16, (dm, d))
    _ndim(W_z, "W_z", 2)
    dz = W_z.shape[1]
    _chk(W_z, "W_z", F32 + BF16, (dm, dz))
    if m < 1:
        raise ValueError("m must be >= 1")
    dt = DTYPE_F32 if H.dtype == torch.float32 else DTYPE_BF16
    wdt = DTYPE_F32 if W_kv.dtype == torch.float32 else DTYPE_BF16
    if out is None:
        _on_device(H=H)
        out = torch.empty(B, T // m, d, dtype=torch.float32, device=H.device)
    _chk(out, "out", F32, (B, T // m, d))
    _on_device(H=H, W_kv=W_kv, W_z=W_z, out=out)
    _call("csa2_compress", _p(H), dt, B, T, dm, _p(W_kv), _p(W_z), wdt, d, dz, m, pos0, rope_dim,
          float(rope_theta), _p(out), _stream(stream))
    return out


def csa2_quant_fp4(kv, codes=None, scales=None, W_ik=None, k_idx=None, stream=None):
    """kv [..., d] f32 -> (codes [..., d/2] u8, scales [..., d/16] u8[, k_idx [..., d_i] bf16])."""
    _chk(kv, "kv", F32)
    d = kv.shape[-1]
    lead = tuple(kv.shape[:-1])
    n = kv.numel() // d if d else 0
    d_i = 0
    if W_ik is not None:
        _ndim(W_ik, "W_ik", 2)
        d_i = W_ik.shape[1]
        _chk(W_ik, "W_ik", BF16, (d, d_i))
    elif k_idx is not None:
        raise ValueError("k_idx needs W_ik")
    if codes is not None:
        _chk(codes, "codes", U8, lead + (d // 2,))
    if scales is not None:
        _chk(scales, "scales", U8, lead + (d // 16,))
    if k_idx is not None:
        _chk(k_idx, "k_idx", BF16, lead + (d_i,))
    _on_device(kv=kv)
    if codes is None:
        codes = torch.empty(*lead, d // 2, dtype=torch.uint8, device=kv.device)
    if scales is None:
        scales = torch.empty(*lead, d // 16, dtype=torch.uint8, device=kv.device)
    if W_ik is not None and k_idx is None:
        k_idx = torch.empty(*lead, d_i, dtype=torch.bfloat16, device=kv.device)
    _on_device(codes=codes, scales=scales, W_ik=W_ik, k_idx=k_idx)
    if n == 0:   # nothing to quantise (an empty tensor has no data pointer to pass)
        return (codes, scales) if W_ik is None else (codes, scales, k_idx)
    _call("csa2_quant_fp4", _p(kv), n, d, _p(codes), _p(scales), _p(W_ik), d_i, _p(k_idx),
          _stream(stream))
    return (codes, scales) if W_ik is None else (codes, scales, k_idx)


def csa2_indexer_keys(codes, scales, W_ik, k_idx=None, stream=None) -> torch.Tensor:
    """codes [..., d/2] u8, scales [..., d/16] u8, W_ik [d, d_i] bf16 -> k_idx [..., d_i] bf16
    (the keys of an existing FP4 cache, e.g. one reloaded from its codes and scales)."""
    _chk(codes, "codes", U8)
    d = codes.shape[-1] * 2
    lead = tuple(codes.shape[:-1])
    _chk(scales, "scales", U8, lead + (d // 16,))
    _ndim(W_ik, "W_ik", 2)
    d_i = W_ik.shape[1]
    _chk(W_ik, "W_ik", BF16, (d, d_i))
    n = codes.numel() // (d // 2) if d else 0
    if k_idx is not None:
        _chk(k_idx, "k_idx", BF16, lead + (d_i,))
    _on_device(codes=codes)
    if k_idx is None:
        k_idx = torch.empty(*lead, d_i, dtype=torch.bfloat16, device=codes.device)
    _on_device(codes=codes, scales=scales, W_ik=W_ik, k_idx=k_idx)
    _call("csa2_indexer_keys", _p(codes), _p(scales), n, d, _p(W_ik), d_i, _p(k_idx), _stream(stream))
    return k_idx


def csa2_cache_append(codes, scales, row: int, kv=None, W_ik=None, k_idx=None, win=None, swa=None,
                      slot: int = 0, swa_scale: float = 1.0, stream=None) -> None:
    """Decode cache append.  codes [B, cap, d/2], scales [B, cap, d/16] (and k_idx
    [B, cap, d_i] with W_ik [d, d_i]) receive kv [B, d] f32 in row `row`; swa
    [L, B, S, d] E4M3 bytes receive win [L, B, d] f32 in slot `slot` (the window
    is a ring: the token at position p goes to slot p mod S)."""
    _ndim(codes, "codes", 3)
    _chk(codes, "codes", U8)
    B, cap = codes.shape[0], codes.shape[1]
    d = codes.shape[2] * 2
    _chk(scales, "scales", U8, (B, cap, d // 16))
    if kv is not None:
        _chk(kv, "kv", F32, (B, d))
    d_i = 0
    if (W_ik is None) != (k_idx is None):
        raise ValueError("W_ik and k_idx must both be given or both be None")
    if W_ik is not None:
        _ndim(W_ik, "W_ik", 2)
        d_i = W_ik.shape[1]
        _chk(W_ik, "W_ik", BF16, (d, d_i))
        _chk(k_idx, "k_idx", BF16, (B, cap, d_i))
    L, S = 0, 1
    if (win is None) != (swa is None):
        raise ValueError("win and swa must both be given or both be None")
    if win is not None:
        _ndim(swa, "swa", 4)
        L, S = swa.shape[0], swa.shape[2]
        _chk(swa, "swa", U8, (L, B, S, d))
        _chk(win, "win", F32, (L, B, d))
    _on_device(codes=codes, scales=scales, kv=kv, W_ik=W_ik, k_idx=k_idx, win=win, swa=swa)
    _call("csa2_cache_append", _p(kv), B, d, cap, row, _p(codes), _p(scales), _p(W_ik), d_i,
          _p(k_idx), _p(win), L, S, slot, float(swa_scale), _p(swa), _stream(stream))


def csa2_index_full(q_idx, w, k_idx, q_pos=None, m: int = 1, scores=None, pool=None, pool_len=None,
                    G: int = 128, PB: int = 2048, PE: int = 8, with_pool: bool = False, K: int = 0,
                    sel=None, ws=None, stream=None):
    """q_idx [B, Tq, h_i, d_i] bf16, w [B, Tq, h_i] f32, k_idx [B, N, d_i] bf16 ->
    scores [B, Tq, N]; with a pool (with_pool, or pool given) also pool [B*Tq, PB*PE]
    and pool_len [B*Tq]; with K > 0 (or sel given) also the Full layer's Top-K
    sel [B*Tq, K].  Returns scores, or a tuple (scores, [pool, pool_len,] [sel])."""
    _ndim(q_idx, "q_idx", 4)
    _chk(q_idx, "q_idx", BF16)
    B, Tq, h_i, d_i = q_idx.shape
    _chk(w, "w", F32, (B, Tq, h_i))
    _ndim(k_idx, "k_idx", 3)
    N = k_idx.shape[1]
    _chk(k_idx, "k_idx", BF16, (B, N, d_i))
    if q_pos is not None:
        _chk(q_pos, "q_pos", I32, (B, Tq))
    if scores is not None:
        _chk(scores, "scores", F32, numel=B * Tq * N)
    want_pool = with_pool or pool is not None
    if pool is not None:
        _chk(pool, "pool", I32, numel=B * Tq * PB * PE)
    if pool_len is not None:
        _chk(pool_len, "pool_len", I32, numel=B * Tq)
    if sel is not None:
        if K <= 0:
            raise ValueError("sel needs K > 0")
        _chk(sel, "sel", I32, numel=B * Tq * K)
    want_sel = K > 0
    _on_device(q_idx=q_idx)
    if scores is None:
        scores = torch.empty(B, Tq, N, dtype=torch.float32, device=q_idx.device)
    if want_pool:
        if pool is None:
            pool = torch.empty(B * Tq, PB * PE, dtype=torch.int32, device=q_idx.device)
        if pool_len is None:
            pool_len = torch.empty(B * Tq, dtype=torch.int32, device=q_idx.device)
    if want_sel and sel is None:
        sel = torch.empty(B * Tq, K, dtype=torch.int32, device=q_idx.device)
    ws = _ws(csa2_index_full_workspace(B, Tq, N, h_i, d_i, G if want_pool else 0,
                                       PB if want_pool else 0, PE, K if want_sel else 0), q_idx, ws)
    _on_device(q_idx=q_idx, w=w, k_idx=k_idx, q_pos=q_pos, scores=scores, pool=pool,
               pool_len=pool_len, sel=sel, ws=ws)
    _call("csa2_index_full", _p(q_idx), _p(w), _p(k_idx), B, Tq, N, h_i, d_i, _p(q_pos), m,
          _p(scores), _p(pool), _p(pool_len), G, PB, PE, K if want_sel else 0, _p(sel), _p(ws),
          _nbytes(ws), _stream(stream))
    out = (scores,) + ((pool, pool_len) if want_pool else ()) + ((sel,) if want_sel else ())
    return out if len(out) > 1 else scores


def _topk_args(scores, K, valid_len, cand_map, out):
    _chk(scores, "scores", F32)
    N = scores.shape[-1] if scores.dim() else 0
    R = scores.numel() // N if N else 0
    if valid_len is not None:
        _chk(valid_len, "valid_len", I32, numel=R)
    if cand_map is not None:
        _chk(cand_map, "cand_map", I32, numel=R * N)
    if out is not None:
        _chk(out, "out", I32, numel=R * K)
    return R, N


def csa2_topk(scores, K: int, valid_len=None, cand_map=None, out=None, ws=None, stream=None):
    """scores [R, N] f32 -> [R, K] int32 ascending indices, -1 padded."""
    R, N = _topk_args(scores, K, valid_len, cand_map, out)
    _on_device(scores=scores)
    if out is None:
        out = torch.empty(R, K, dtype=torch.int32, device=scores.device)
    ws = _ws(csa2_topk_workspace(R, N, K), scores, ws)
    _on_device(scores=scores, valid_len=valid_len, cand_map=cand_map, out=out, ws=ws)
    _call("csa2_topk", _p(scores), R, N, _p(valid_len), _p(cand_map), K, _p(out), _p(ws),
          _nbytes(ws), _stream(stream))
    return out


def csa2_topk_noalloc(scores, K: int, out, valid_len=None, cand_map=None, stream=None):
    """csa2_topk with its scratch in the library's static device array: nothing is
    allocated, so `out` [R, K] int32 must be given."""
    if out is None:
        raise ValueError("out must be given (nothing is allocated)")
    R, N = _topk_args(scores, K, valid_len, cand_map, out)
    _on_device(scores=scores, valid_len=valid_len, cand_map=cand_map, out=out)
    _call("csa2_topk_noalloc", _p(scores), R, N, _p(valid_len), _p(cand_map), K, _p(out),
          _stream(stream))
    return out


def csa2_index_reindex(q_idx, w, k_idx, pool, pool_len, K: int = 512, sel=None, ws=None,
                       stream=None):
    """q_idx [B, h_i, d_i], w [B, h_i], k_idx [B, N, d_i], pool [B, P], pool_len [B] -> sel [B, K]."""
    _chk(q_idx, "q_idx", BF16)
    if q_idx.dim() < 3:
        raise ValueError(f"q_idx must be [B, h_i, d_i], has shape {tuple(q_idx.shape)}")
    B, h_i, d_i = q_idx.shape[0], q_idx.shape[-2], q_idx.shape[-1]
    if q_idx.numel() != B * h_i * d_i:
        raise ValueError(f"q_idx must hold one query per sequence, has shape {tuple(q_idx.shape)}")
    _chk(w, "w", F32, numel=B * h_i)
    _ndim(k_idx, "k_idx", 3)
    N = k_idx.shape[1]
    _chk(k_idx, "k_idx", BF16, (B, N, d_i))
    _ndim(pool, "pool", 2)
    P = pool.shape[-1]
    _chk(pool, "pool", I32, (B, P))
    _chk(pool_len, "pool_len", I32, numel=B)
    if sel is not None:
        _chk(sel, "sel", I32, numel=B * K)
    _on_device(q_idx=q_idx)
    if sel is None:
        sel = torch.empty(B, K, dtype=torch.int32, device=q_idx.device)
    ws = _ws(csa2_index_reindex_workspace(B, P, K), q_idx, ws)
    _on_device(q_idx=q_idx, w=w, k_idx=k_idx, pool=pool, pool_len=pool_len, sel=sel, ws=ws)
    _call("csa2_index_reindex", _p(q_idx), _p(w), _p(k_idx), _p(pool), _p(pool_len), B, P, N, h_i,
          d_i, K, _p(sel), _p(ws), _nbytes(ws), _stream(stream))
    return sel


def csa2_sparse_attn(q, codes, scales, sel, swa, swa_scale: float = 1.0, q_pos=None,
                     swa_pos0: int = 0, n_win: int = 128, sm_scale: float = 0.0, out=None, lse=None,
                     ws=None, stream=None):
    """q [B, Tq, H_q, d] bf16, codes [B, N, d/2], scales [B, N, d/16], sel [B, Tq, K],
    swa [B, S, d] E4M3 -> out [B, Tq, H_q, d] f32 (lse [B, Tq, H_q] f32 when given).
    The window is a ring: with positions, the token at position p >= swa_pos0 is in
    slot (p - swa_pos0) mod S."""
    _ndim(q, "q", 4)
    _chk(q, "q", BF16)
    B, Tq, H_q, d = q.shape
    _ndim(codes, "codes", 3)
    N = codes.shape[1]
    _chk(codes, "codes", U8, (B, N, d // 2))
    _chk(scales, "scales", U8, (B, N, d // 16))
    _ndim(sel, "sel", 3)
    K = sel.shape[-1]
    _chk(sel, "sel", I32, (B, Tq, K))
    _ndim(swa, "swa", 3)
    S = swa.shape[1]
    _chk(swa, "swa", U8, (B, S, d))
    if q_pos is not None:
        _chk(q_pos, "q_pos", I32, (B, Tq))
    if out is not None:
        _chk(out, "out", F32, (B, Tq, H_q, d))
    if lse is not None:
        _chk(lse, "lse", F32, numel=B * Tq * H_q)
    _on_device(q=q)
    if out is None:
        out = torch.empty(B, Tq, H_q, d, dtype=torch.float32, device=q.device)
    ws = _ws(csa2_sparse_attn_workspace(B, Tq, H_q, d, K, S), q, ws)
    _on_device(q=q, codes=codes, scales=scales, sel=sel, swa=swa, q_pos=q_pos, out=out, lse=lse, ws=ws)
    _call("csa2_sparse_attn", _p(q), _p(codes), _p(scales), N, _p(sel), K, _p(swa),
          float(swa_scale), S, swa_pos0, n_win, _p(q_pos), B, Tq, H_q, d, float(sm_scale), _p(out),
          _p(lse), _p(ws), _nbytes(ws), _stream(stream))
    return out
