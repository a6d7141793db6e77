"""numpy front end of the CPU oracle (oracle/cskv_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's
CPU-baseline leg.  The product package never imports this module.

The C library does the arithmetic; this module only marshals numpy arrays
and composes the per-layer CSA2 modes [P2 "CSA2：三种模式，40 层只存 4 份"]:
  full    - append the new token to the shared cache, score every entry with
            its own indexer query, keep the top-k, attend;
  reindex - score the shared indexer keys with its own indexer query, keep
            its own top-k, attend;
  reuse   - attend with the index list of the most recent full/reindex layer.
Every mode appends its own window row and uses its own query.
  P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

_lib = None

STATUS_OVERFLOW = 1
STATUS_ODD_ENTRY_APPEND = 2


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


def _p(a, ctype):
    return None if a is None else a.ctypes.data_as(C.POINTER(ctype))


class _Cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("capacity", C.c_int32), ("dim", C.c_int32),
                ("rope_dim", C.c_int32), ("k_group", C.c_int32), ("v_group", C.c_int32),
                ("idx_dim", C.c_int32),
                ("k_codes", C.POINTER(C.c_uint8)), ("k_scales", C.POINTER(C.c_float)),
                ("v_codes", C.POINTER(C.c_uint8)), ("v_scales", C.POINTER(C.c_float)),
                ("idx_keys", C.POINTER(C.c_uint16)), ("n_tokens", C.POINTER(C.c_int32)),
                ("pending", C.POINTER(C.c_float)), ("status", C.POINTER(C.c_int32)),
                ("idx_format", C.c_int32), ("idx_scales", C.POINTER(C.c_uint8)),
                ("swa_format", C.c_int32), ("k_format", C.c_int32), ("ratio", C.c_int32)]


def _declare(L):
    u64, i32, i64, f64 = C.c_uint64, C.c_int32, C.c_int64, C.c_double
    P = C.POINTER
    L.orc_kv_bytes.restype = u64
    L.orc_kv_bytes.argtypes = [u64] * 5
    L.orc_fp4_row_bytes.restype = f64
    L.orc_fp4_row_bytes.argtypes = [C.c_int, C.c_int, f64]
    L.orc_global_kv_per_token.restype = f64
    L.orc_global_kv_per_token.argtypes = [C.c_int, P(C.c_int), f64, f64]
    L.orc_e2m1_value.restype = f64
    L.orc_e2m1_value.argtypes = [C.c_uint]
    L.orc_e2m1_encode.restype = C.c_uint
    L.orc_e2m1_encode.argtypes = [C.c_float]
    L.orc_bf16_from_f32.restype = C.c_uint16
    L.orc_bf16_from_f32.argtypes = [C.c_float]
    L.orc_bf16_value.restype = f64
    L.orc_bf16_value.argtypes = [C.c_uint16]
    L.orc_e4m3_value.restype = f64
    L.orc_e4m3_value.argtypes = [C.c_uint8]
    L.orc_e4m3_encode.restype = C.c_uint8
    L.orc_e4m3_encode.argtypes = [C.c_float]
    L.orc_swa_append_fp8.restype = None
    L.orc_swa_append_fp8.argtypes = [P(C.c_uint8), C.c_int, C.c_int, C.c_int, P(C.c_float), P(i32), P(i32)]
    L.orc_e8m0_value.restype = f64
    L.orc_e8m0_value.argtypes = [C.c_uint8]
    L.orc_quantize_mx16.restype = None
    L.orc_quantize_mx16.argtypes = [P(C.c_uint16), C.c_int, P(C.c_uint8), P(C.c_uint8)]
    L.orc_quantize_mx16_f32.restype = None
    L.orc_quantize_mx16_f32.argtypes = [P(C.c_float), C.c_int, P(C.c_uint8), P(C.c_uint8)]
    L.orc_dequantize_mx16.restype = None
    L.orc_dequantize_mx16.argtypes = [P(C.c_uint8), P(C.c_uint8), C.c_int, P(f64)]
    L.orc_compress_pair.restype = None
    L.orc_compress_pair.argtypes = [P(C.c_float)] * 3 + [C.c_int, P(C.c_float)]
    L.orc_quantize_row.restype = None
    L.orc_quantize_row.argtypes = [P(C.c_float), C.c_int, C.c_int, P(C.c_uint8), P(C.c_float)]
    L.orc_dequantize_row.restype = None
    L.orc_dequantize_row.argtypes = [P(C.c_uint8), P(C.c_float), C.c_int, C.c_int, P(f64)]
    L.orc_kv_append.restype = None
    L.orc_ced_project.restype = None
    L.orc_ced_project.argtypes = [P(C.c_uint16), i64, C.c_int, P(C.c_uint16), C.c_int, P(C.c_float)]
    L.orc_kv_append.argtypes = [P(_Cache), P(C.c_float), P(i32), P(C.c_float), P(C.c_uint16)]
    L.orc_swa_append.restype = None
    L.orc_swa_append.argtypes = [P(C.c_uint16), C.c_int, C.c_int, C.c_int, P(C.c_float),
                                 P(i32), P(i32)]
    L.orc_indexer_scores.restype = None
    L.orc_indexer_scores.argtypes = [P(C.c_uint16), i64, C.c_int, P(C.c_uint16), C.c_int,
                                     P(C.c_float), P(f64)]
    L.orc_topk.restype = None
    L.orc_topk.argtypes = [P(f64), i64, C.c_int, P(i32)]
    L.orc_indexer_topk.restype = None
    L.orc_indexer_topk.argtypes = [P(_Cache), P(C.c_uint16), C.c_int, P(C.c_float), C.c_int,
                                   P(i32)]
    L.orc_pool_blocks.restype = None
    L.orc_pool_blocks.argtypes = [P(f64), i64, C.c_int, C.c_int, P(i32)]
    L.orc_topk_in_pool.restype = None
    L.orc_topk_in_pool.argtypes = [P(f64), i64, P(i32), C.c_int, C.c_int, C.c_int, P(i32)]
    L.orc_indexer_pool.restype = None
    L.orc_indexer_pool.argtypes = [P(_Cache), P(C.c_uint16), C.c_int, P(C.c_float), C.c_int,
                                   C.c_int, P(i32)]
    L.orc_indexer_topk_in_pool.restype = None
    L.orc_indexer_topk_in_pool.argtypes = [P(_Cache), P(C.c_uint16), C.c_int, P(C.c_float), P(i32),
                                           C.c_int, C.c_int, C.c_int, P(i32)]
    L.orc_sparse_attn.restype = None
    L.orc_sparse_attn.argtypes = [P(_Cache), P(C.c_float), C.c_int, P(i32), C.c_int,
                                  P(C.c_uint16), C.c_int, P(i32), f64, P(f64), P(f64)]


# ------------------------------------------------------------------ scalars

def kv_bytes(layers, tokens, heads, head_dim, elem_bytes) -> int:
    return int(lib().orc_kv_bytes(layers, tokens, heads, head_dim, elem_bytes))


def fp4_row_bytes(dims, group, scale_bytes) -> float:
    return float(lib().orc_fp4_row_bytes(dims, group, scale_bytes))


def global_kv_per_token(ratios, main_entry_bytes, idx_entry_bytes) -> float:
    r = (C.c_int * len(ratios))(*ratios)
    return float(lib().orc_global_kv_per_token(len(ratios), r, main_entry_bytes, idx_entry_bytes))


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(code))


def e2m1_encode(v: float) -> int:
    return int(lib().orc_e2m1_encode(v))


def bf16_from_f32(x: float) -> int:
    return int(lib().orc_bf16_from_f32(x))


def bf16_value(h: int) -> float:
    return float(lib().orc_bf16_value(h))


# ------------------------------------------------------------------ arrays

def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def compress_pair(W, x_even, x_odd) -> np.ndarray:
    W, xe, xo = _f32(W), _f32(x_even), _f32(x_odd)
    D = xe.shape[0]
    assert W.shape == (D, 2 * D)
    e = np.empty(D, np.float32)
    lib().orc_compress_pair(_p(W, C.c_float), _p(xe, C.c_float), _p(xo, C.c_float), D,
                            _p(e, C.c_float))
    return e


def quantize_row(x, group):
    x = _f32(x)
    n = x.shape[0]
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // group, np.float32)
    lib().orc_quantize_row(_p(x, C.c_float), n, group, _p(packed, C.c_uint8),
                           _p(scales, C.c_float))
    return packed, scales


def dequantize_row(packed, scales, n, group) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = _f32(scales)
    out = np.empty(n, np.float64)
    lib().orc_dequantize_row(_p(packed, C.c_uint8), _p(scales, C.c_float), n, group,
                             _p(out, C.c_double))
    return out


def indexer_scores(keys, q, head_w=None) -> np.ndarray:
    keys = np.ascontiguousarray(keys, np.uint16)
    q = np.ascontiguousarray(q, np.uint16)
    E, Di = keys.shape
    H = q.shape[0]
    hw = None if head_w is None else _f32(head_w)
    out = np.empty(E, np.float64)
    lib().orc_indexer_scores(_p(keys, C.c_uint16), E, Di, _p(q, C.c_uint16), H,
                             _p(hw, C.c_float), _p(out, C.c_double))
    return out


def topk(scores, k) -> np.ndarray:
    s = np.ascontiguousarray(scores, np.float64)
    out = np.empty(k, np.int32)
    lib().orc_topk(_p(s, C.c_double), s.shape[0], k, _p(out, C.c_int32))
    return out


def e8m0_value(s: int) -> float:
    return float(lib().orc_e8m0_value(s))


def quantize_mx16(x_bf16):
    """FP4 indexer key: E2M1 codes (low nibble first) and E8M0 scales per 16 dims."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    n = x.shape[0]
    codes = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    lib().orc_quantize_mx16(_p(x, C.c_uint16), n, _p(codes, C.c_uint8), _p(scales, C.c_uint8))
    return codes, scales


def quantize_mx16_f32(x):
    """Main-entry plane in the pages' form: E2M1 codes and E8M0 scales per 16 channels."""
    x = _f32(x)
    n = x.shape[0]
    codes = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    lib().orc_quantize_mx16_f32(_p(x, C.c_float), n, _p(codes, C.c_uint8), _p(scales, C.c_uint8))
    return codes, scales


def dequantize_mx16(codes, scales, n) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.empty(n, np.float64)
    lib().orc_dequantize_mx16(_p(codes, C.c_uint8), _p(scales, C.c_uint8), n, _p(out, C.c_double))
    return out


def pool_blocks(scores, block, nb) -> np.ndarray:
    """Candidate pool of the hierarchical indexer: the nb best blocks of
    `block` entries by block maximum (ties: lower block), ascending, -1 padded."""
    s = np.ascontiguousarray(scores, np.float64)
    out = np.empty(nb, np.int32)
    lib().orc_pool_blocks(_p(s, C.c_double), s.shape[0], block, nb, _p(out, C.c_int32))
    return out


def topk_in_pool(scores, pool, block, k) -> np.ndarray:
    """Exact top-k among the entries of the pooled blocks, ascending, -1 padded."""
    s = np.ascontiguousarray(scores, np.float64)
    pl = np.ascontiguousarray(pool, np.int32)
    out = np.empty(k, np.int32)
    lib().orc_topk_in_pool(_p(s, C.c_double), s.shape[0], _p(pl, C.c_int32), pl.shape[0], block, k,
                           _p(out, C.c_int32))
    return out


# ------------------------------------------------------------------ cache

@dataclass
class Cache:
    """Host mirror of the device cache planes."""
    batch: int
    capacity: int
    dim: int
    rope_dim: int
    k_group: int
    v_group: int
    idx_dim: int
    k_codes: np.ndarray
    k_scales: np.ndarray
    v_codes: Optional[np.ndarray]
    v_scales: Optional[np.ndarray]
    idx_keys: np.ndarray       # bf16 [B][cap][Di], or E2M1 codes u8 [B][cap][Di/2] (idx_format 1)
    n_tokens: np.ndarray
    pending: np.ndarray
    status: np.ndarray
    idx_format: int = 0
    idx_scales: Optional[np.ndarray] = None   # E8M0 u8 [B][cap][Di/16] (idx_format 1)
    swa_format: int = 0                        # window rings used with this cache: 0 bf16, 1 FP8 E4M3
    k_format: int = 0                          # 1: E8M0 byte scales per 16 channels (k_group 16)
    ratio: int = 2                             # tokens per entry: 2 (compressed pairs) or 1

    @classmethod
    def empty(cls, batch, capacity, dim=576, rope_dim=64, k_group=32, v_group=0, idx_dim=128,
              idx_format=0, swa_format=0, k_format=0, ratio=2):
        if ratio not in (1, 2):
            raise ValueError(f"ratio {ratio}: 1 or 2 tokens per entry")
        Dv = dim - rope_dim
        fp4 = idx_format == 1
        st = np.uint8 if k_format == 1 else np.float32
        return cls(batch, capacity, dim, rope_dim, k_group, v_group, idx_dim,
                   np.zeros((batch, capacity, dim // 2), np.uint8),
                   np.zeros((batch, capacity, dim // k_group), st),
                   np.zeros((batch, capacity, Dv // 2), np.uint8) if v_group else None,
                   np.zeros((batch, capacity, Dv // v_group), st) if v_group else None,
                   np.zeros((batch, capacity, idx_dim // 2), np.uint8) if fp4
                   else np.zeros((batch, capacity, idx_dim), np.uint16),
                   np.zeros(batch, np.int32), np.zeros((batch, dim), np.float32),
                   np.zeros(1, np.int32), idx_format,
                   np.zeros((batch, capacity, idx_dim // 16), np.uint8) if fp4 else None, swa_format,
                   k_format, ratio)

    def _c(self) -> _Cache:
        return _Cache(self.batch, self.capacity, self.dim, self.rope_dim, self.k_group,
                      self.v_group, self.idx_dim,
                      _p(self.k_codes, C.c_uint8), _p(self.k_scales, C.c_float),
                      _p(self.v_codes, C.c_uint8), _p(self.v_scales, C.c_float),
                      _p(self.idx_keys, C.c_uint16), _p(self.n_tokens, C.c_int32),
                      _p(self.pending, C.c_float), _p(self.status, C.c_int32),
                      self.idx_format, _p(self.idx_scales, C.c_uint8), self.swa_format, self.k_format,
                      self.ratio)

    def entries(self) -> np.ndarray:
        return np.clip(self.n_tokens // self.ratio, 0, self.capacity)


def kv_append(cache: Cache, tokens, cu_new, w_comp, idx_rows) -> None:
    tokens = _f32(tokens).reshape(-1, cache.dim)
    cu = np.ascontiguousarray(cu_new, np.int32)
    assert cu.shape == (cache.batch + 1,)
    irows = np.ascontiguousarray(idx_rows, np.uint16).reshape(-1, cache.idx_dim)
    W = None if w_comp is None else _f32(w_comp)
    if W is not None and cache.ratio != 2:
        raise ValueError("the 2->1 compressor needs a ratio-2 cache")
    c = cache._c()
    lib().orc_kv_append(C.byref(c), _p(tokens, C.c_float), _p(cu, C.c_int32),
                        _p(W, C.c_float), _p(irows, C.c_uint16))


def swa_append(ring, rows, cu_new, end_pos) -> None:
    """ring: bf16 bits (uint16) or FP8 E4M3 bytes (uint8) [B, W, dim], updated in place."""
    assert ring.dtype in (np.uint16, np.uint8) and ring.flags.c_contiguous
    B, W, D = ring.shape
    rows = _f32(rows).reshape(-1, D)
    cu = np.ascontiguousarray(cu_new, np.int32)
    ep = np.ascontiguousarray(end_pos, np.int32)
    if ring.dtype == np.uint8:
        lib().orc_swa_append_fp8(_p(ring, C.c_uint8), B, W, D, _p(rows, C.c_float), _p(cu, C.c_int32),
                                 _p(ep, C.c_int32))
    else:
        lib().orc_swa_append(_p(ring, C.c_uint16), B, W, D, _p(rows, C.c_float), _p(cu, C.c_int32),
                             _p(ep, C.c_int32))


def e4m3_value(v: int) -> float:
    return float(lib().orc_e4m3_value(v))


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def indexer_topk(cache: Cache, q_idx, k, head_w=None) -> np.ndarray:
    q = np.ascontiguousarray(q_idx, np.uint16)
    H = q.shape[1]
    hw = None if head_w is None else _f32(head_w)
    out = np.empty((cache.batch, k), np.int32)
    c = cache._c()
    lib().orc_indexer_topk(C.byref(c), _p(q, C.c_uint16), H, _p(hw, C.c_float), k,
                           _p(out, C.c_int32))
    return out


def indexer_pool(cache: Cache, q_idx, block, nb, head_w=None) -> np.ndarray:
    q = np.ascontiguousarray(q_idx, np.uint16)
    hw = None if head_w is None else _f32(head_w)
    out = np.empty((cache.batch, nb), np.int32)
    c = cache._c()
    lib().orc_indexer_pool(C.byref(c), _p(q, C.c_uint16), q.shape[1], _p(hw, C.c_float), block, nb,
                           _p(out, C.c_int32))
    return out


def indexer_topk_in_pool(cache: Cache, q_idx, pool, block, k, head_w=None) -> np.ndarray:
    q = np.ascontiguousarray(q_idx, np.uint16)
    hw = None if head_w is None else _f32(head_w)
    pl = np.ascontiguousarray(pool, np.int32)
    out = np.empty((cache.batch, k), np.int32)
    c = cache._c()
    lib().orc_indexer_topk_in_pool(C.byref(c), _p(q, C.c_uint16), q.shape[1], _p(hw, C.c_float),
                                   _p(pl, C.c_int32), pl.shape[1], block, k, _p(out, C.c_int32))
    return out


def sparse_attn(cache: Cache, q, idx, swa, scale, swa_len=None):
    q = _f32(q)
    B, H, D = q.shape
    idx = np.ascontiguousarray(idx, np.int32)
    k = idx.shape[1]
    swa = np.ascontiguousarray(swa, np.uint8 if cache.swa_format == 1 else np.uint16)
    W = swa.shape[1]
    sl = None if swa_len is None else np.ascontiguousarray(swa_len, np.int32)
    out = np.empty((B, H, cache.dim - cache.rope_dim), np.float64)
    lse = np.empty((B, H), np.float64)
    c = cache._c()
    lib().orc_sparse_attn(C.byref(c), _p(q, C.c_float), H, _p(idx, C.c_int32), k,
                          swa.ctypes.data_as(C.POINTER(C.c_uint16)), W, _p(sl, C.c_int32), float(scale),
                          _p(out, C.c_double), _p(lse, C.c_double))
    return out, lse


def layer_group_decode(cache: Cache, modes, new_token, new_idx_row, w_comp, q, q_idx,
                       swa_rings, swa_rows, k, scale, head_w=None, pool=None):
    """One CSA2 layer-group decode step over a shared cache.

    new_token fp32 [B, dim] (appended by the full layer, or None);
    q / q_idx / swa_rings / swa_rows: per-layer lists (q_idx None for reuse).
    pool = (nb, block): the hierarchical indexer -- the first full layer's
    scores give a candidate pool of nb blocks of `block` entries, and later
    reindex layers select inside it.
    swa_rings are updated in place.  Returns (outs, lses, idx_lists) per layer.
    """
    B = cache.batch
    cu = np.arange(B + 1, dtype=np.int32)
    outs, lses, idxs = [], [], []
    last_idx = None
    cand = None
    for li, mode in enumerate(modes):
        if mode == "full" and new_token is not None:
            kv_append(cache, new_token, cu, w_comp, new_idx_row)
        swa_append(swa_rings[li], swa_rows[li], cu, cache.n_tokens)
        if mode in ("full", "reindex"):
            hw = None if head_w is None else head_w[li]
            if mode == "reindex" and cand is not None:
                last_idx = indexer_topk_in_pool(cache, q_idx[li], cand, pool[1], k, hw)
            else:
                last_idx = indexer_topk(cache, q_idx[li], k, hw)
            if mode == "full" and pool is not None and cand is None:
                cand = indexer_pool(cache, q_idx[li], pool[1], pool[0], hw)
        elif last_idx is None:
            raise ValueError("reuse layer with no preceding full/reindex layer")
        o, l = sparse_attn(cache, q[li], last_idx, swa_rings[li], scale)
        outs.append(o)
        lses.append(l)
        idxs.append(last_idx)
    return outs, lses, idxs


# ---------------------------------------------------------------- CED and the 40-layer plan

def ced_project(h_bits, w_bits) -> np.ndarray:
    """The decoder's global KV rows from one hidden state [P2 四、"CED：上半段模型
    的 KV 由下半段代算"]: h bf16 bits [rows, d_model], w bf16 bits [n_out,
    d_model] (a row per output channel) -> fp32 [rows, n_out], each output the
    fp64 sum of its d_model products rounded once."""
    h = np.ascontiguousarray(h_bits, np.uint16)
    w = np.ascontiguousarray(w_bits, np.uint16)
    assert h.ndim == 2 and w.ndim == 2 and h.shape[1] == w.shape[1]
    out = np.empty((h.shape[0], w.shape[0]), np.float32)
    lib().orc_ced_project(_p(h, C.c_uint16), h.shape[0], h.shape[1], _p(w, C.c_uint16), w.shape[0],
                          _p(out, C.c_float))
    return out


def csa2_plan():
    """The pages' CSA2 layer plan [P2 四、"CSA2：三种模式，40 层只存 4 份"]: one
    (name, tokens per entry, layer modes) per stored cache, in layer order.
    Encoder: three groups of one Full and five Reuse layers, each group with
    its own 2->1 cache.  Decoder: one cache read by its five groups, (Full +
    3 Reuse) and then four times (Reindex + 3 Reuse); its entries are one per
    token, computed by the CED projection.  The encoder's two layers outside
    these groups have no mode in the pages and are not part of the plan."""
    enc = [(f"encoder{i}", 2, ["full"] + ["reuse"] * 5) for i in range(3)]
    dec = ("decoder", 1, ["full"] + ["reuse"] * 3 + (["reindex"] + ["reuse"] * 3) * 4)
    return enc + [dec]


def model_decode(groups, k, scale, pool=None):
    """One decode step of every CSA2 layer in plan order.  groups: one dict
    per cache with `cache`, `modes`, the per-layer lists `q`, `q_idx`,
    `rings`, `swa_rows`, the new indexer-key rows `idx_row`, and the new
    entries' source: `token` + `w_comp` (an encoder cache, 2->1 compressor)
    or `ced_h` + `ced_w` (the decoder cache: one entry per token from the CED
    projection).  pool = (nb, block) for groups with a Reindex layer.  Rings
    are updated in place.  Returns (outs, lses, idxs) per group."""
    res = []
    for g in groups:
        if g.get("ced_h") is not None:
            new, w = ced_project(g["ced_h"], g["ced_w"]), None
        else:
            new, w = g["token"], g["w_comp"]
        use_pool = pool if "reindex" in g["modes"] else None
        res.append(layer_group_decode(g["cache"], g["modes"], new, g["idx_row"], w, g["q"], g["q_idx"],
                                      g["rings"], g["swa_rows"], k, scale, pool=use_pool))
    return res
