"""Python binding of libcskv.so, the gfx950 CSA2 FP4 sparse-decode library.

Argument marshalling only: each function checks tensor placement, dtype and
shape, then calls the C entry point of the same name on the current HIP
stream.  Every step of the path runs in the library's HIP kernels; there is
no other code path.  If the library is not built, importing works but the
first call raises.

Tensors: device (cuda) tensors, contiguous.  bf16 data may be passed as
torch.bfloat16 or as int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _build

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EWORKSPACE = -3
EHIP = -4
STATUS_OVERFLOW = 1
STATUS_ODD_ENTRY_APPEND = 2
STATUS_BAD_STATE = 4
STATUS_BAD_PAGE = 8
MODE_FULL, MODE_REINDEX, MODE_REUSE = 0, 1, 2
IDX_BF16, IDX_FP4 = 0, 1
SWA_BF16, SWA_FP8 = 0, 1
KV_F32, KV_MX16 = 0, 1
MODES = {"full": MODE_FULL, "reindex": MODE_REINDEX, "reuse": MODE_REUSE}
KERNEL_APPEND, KERNEL_SWA_APPEND, KERNEL_INDEXER_SCAN, KERNEL_TOPK_SELECT, KERNEL_ATTENTION = 1, 2, 3, 4, 5
KERNEL_COMPRESS = 6
OP_INDEXER_TOPK, OP_SPARSE_ATTN, OP_LAYER_GROUP, OP_INDEXER_POOL, OP_INDEXER_IN_POOL = 1, 2, 3, 4, 5

EXPORTS = ("cskv_kv_append_fp4", "cskv_kv_append_fp4_mfma", "cskv_append_workspace_bytes", "cskv_swa_append", "cskv_swa_append_fp8",
           "cskv_indexer_topk",
           "cskv_indexer_topk_pool", "cskv_indexer_topk_in_pool", "cskv_sparse_attn_decode",
           "cskv_layer_group_decode", "cskv_layer_group_decode_pooled", "cskv_layer_group_decode_noalloc",
           "cskv_workspace_bytes",
           "cskv_workspace_bytes_pool", "cskv_entry_bytes", "cskv_cache_entry_bytes", "cskv_last_error",
           "cskv_ced_project", "cskv_model_decode", "cskv_model_workspace_bytes",
           "cskv_timer_enable", "cskv_timer_pause", "cskv_timer_read", "cskv_timer_disable_all")


class CskvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"cskv error {code}: {msg}")
        self.code = code


class CacheDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("capacity", C.c_int32), ("dim", C.c_int32),
                ("rope_dim", C.c_int32), ("k_group", C.c_int32), ("v_group", C.c_int32),
                ("idx_dim", C.c_int32),
                ("k_codes", C.c_void_p), ("k_scales", C.c_void_p), ("v_codes", C.c_void_p),
                ("v_scales", C.c_void_p), ("idx_keys", C.c_void_p), ("n_tokens", C.c_void_p),
                ("pending", C.c_void_p), ("status", C.c_void_p), ("idx_format", C.c_int32),
                ("idx_scales", C.c_void_p), ("swa_format", C.c_int32), ("k_format", C.c_int32),
                ("ratio", C.c_int32), ("page_size", C.c_int32), ("max_pages", C.c_int32),
                ("n_pages", C.c_int32), ("block_table", C.c_void_p)]


class LayerDesc(C.Structure):
    _fields_ = [("mode", C.c_int32), ("q", C.c_void_p), ("q_idx", C.c_void_p),
                ("head_w", C.c_void_p), ("swa", C.c_void_p), ("swa_row", C.c_void_p),
                ("idx", C.c_void_p), ("out", C.c_void_p), ("lse", C.c_void_p)]


class GroupDesc(C.Structure):
    _fields_ = [("cache", C.c_void_p), ("layers", C.c_void_p), ("n_layers", C.c_int32),
                ("new_tokens", C.c_void_p), ("w_comp", C.c_void_p), ("ced_h", C.c_void_p),
                ("ced_w", C.c_void_p), ("d_model", C.c_int32), ("new_idx_rows", C.c_void_p),
                ("pool_blocks", C.c_int32), ("pool_block", C.c_int32)]


_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(_build.LIB)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.cskv_kv_append_fp4.argtypes = [vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.cskv_kv_append_fp4_mfma.argtypes = [vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.cskv_append_workspace_bytes.argtypes = [i32, vp]
        L.cskv_append_workspace_bytes.restype = sz
        L.cskv_swa_append.argtypes = [vp, i32, i32, i32, vp, vp, i32, vp, vp]
        L.cskv_swa_append_fp8.argtypes = [vp, i32, i32, i32, vp, vp, i32, vp, vp]
        L.cskv_indexer_topk.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, sz, vp]
        L.cskv_sparse_attn_decode.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, C.c_float, vp, vp, vp, sz,
                                              vp]
        L.cskv_layer_group_decode.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, C.c_float,
                                              vp, sz, vp]
        L.cskv_layer_group_decode_pooled.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, C.c_float,
                                                     i32, i32, vp, sz, vp]
        L.cskv_layer_group_decode_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, C.c_float, vp]
        L.cskv_indexer_topk_pool.argtypes = [vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, sz, vp]
        L.cskv_indexer_topk_in_pool.argtypes = [vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, sz, vp]
        L.cskv_workspace_bytes.argtypes = [vp, i32, i32, i32, i32]
        L.cskv_workspace_bytes.restype = sz
        L.cskv_workspace_bytes_pool.argtypes = [vp, i32, i32, i32, i32, i32, i32]
        L.cskv_workspace_bytes_pool.restype = sz
        L.cskv_entry_bytes.argtypes = [i32] * 5
        L.cskv_entry_bytes.restype = sz
        L.cskv_cache_entry_bytes.argtypes = [vp]
        L.cskv_ced_project.argtypes = [vp, C.c_int64, i32, vp, i32, vp, vp]
        L.cskv_model_decode.argtypes = [vp, i32, i32, i32, i32, i32, C.c_float, vp, sz, vp]
        L.cskv_model_workspace_bytes.argtypes = [vp, i32, i32, i32, i32]
        L.cskv_model_workspace_bytes.restype = sz
        L.cskv_cache_entry_bytes.restype = sz
        L.cskv_last_error.restype = C.c_char_p
        L.cskv_timer_enable.argtypes = [i32, i32]
        L.cskv_timer_pause.argtypes = [i32, i32]
        L.cskv_timer_read.argtypes = [i32, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        for f in ("cskv_kv_append_fp4", "cskv_swa_append", "cskv_swa_append_fp8", "cskv_indexer_topk",
                  "cskv_indexer_topk_pool",
                  "cskv_indexer_topk_in_pool", "cskv_sparse_attn_decode", "cskv_layer_group_decode",
                  "cskv_layer_group_decode_pooled", "cskv_layer_group_decode_noalloc", "cskv_ced_project", "cskv_model_decode", "cskv_timer_enable", "cskv_timer_pause", "cskv_timer_read",
                  "cskv_timer_disable_all"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != OK:
        raise CskvError(rc, lib().cskv_last_error().decode())


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _keep_for(stream, *tensors) -> None:
    """Tensors the binding allocated for a call enqueued on `stream`: tell the
    caching allocator that stream uses them, so their memory is not handed
    out again before that stream's work is done (a no-op on the current
    stream)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _ptr(t: Optional[torch.Tensor], dtypes, name, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return C.c_void_p(t.data_ptr())


F32 = (torch.float32,)
I32 = (torch.int32,)
U8 = (torch.uint8,)
B16 = (torch.bfloat16, torch.int16, torch.uint16)


@dataclass
class Cache:
    """Device planes of one layer group's shared cache (torch-allocated, caller-owned)."""
    batch: int
    capacity: int
    k_group: int
    v_group: int
    idx_dim: int
    k_codes: torch.Tensor
    k_scales: torch.Tensor
    v_codes: Optional[torch.Tensor]
    v_scales: Optional[torch.Tensor]
    idx_keys: torch.Tensor
    n_tokens: torch.Tensor
    pending: torch.Tensor
    status: torch.Tensor
    dim: int = 576
    rope_dim: int = 64
    idx_format: int = 0                          # IDX_BF16, or IDX_FP4 (idx_keys u8 codes + idx_scales)
    idx_scales: Optional[torch.Tensor] = None
    swa_format: int = 0                          # window rings used with it: SWA_BF16, or SWA_FP8 (uint8 rings)
    k_format: int = 0                            # KV_F32, or KV_MX16 (k_group 16, uint8 scale planes)
    ratio: int = 2                               # tokens per entry: 2 (compressed pairs) or 1
    page_size: int = 0                           # paged planes: entries per page (0: [batch][capacity])
    n_pages: int = 0
    block_table: Optional[torch.Tensor] = None   # paged: int32 [batch][capacity // page_size]

    @classmethod
    def allocate_paged(cls, batch, capacity, page_size, n_pages, block_table, k_group=32, v_group=0,
                       idx_dim=128, dim=576, rope_dim=64, device="cuda", idx_format=0, swa_format=0,
                       k_format=0, ratio=2):
        """A cache whose planes are n_pages pages of page_size entries
        ([n_pages][page_size][row]); block_table (int32 [batch][capacity //
        page_size], caller-owned) names each sequence's page of every
        page-sized run of its entries."""
        c = cls.allocate(n_pages, page_size, k_group, v_group, idx_dim, dim, rope_dim, device, idx_format,
                         swa_format, k_format, ratio)
        c.batch, c.capacity = batch, capacity
        z = lambda *s, dt: torch.zeros(*s, dtype=dt, device=device)
        c.n_tokens, c.pending = z(batch, dt=torch.int32), z(batch, dim, dt=torch.float32)
        c.page_size, c.n_pages, c.block_table = page_size, n_pages, block_table
        return c

    @classmethod
    def allocate(cls, batch, capacity, k_group=32, v_group=0, idx_dim=128, dim=576, rope_dim=64,
                 device="cuda", idx_format=0, swa_format=0, k_format=0, ratio=2):
        dv = dim - rope_dim
        z = lambda *s, dt: torch.zeros(*s, dtype=dt, device=device)
        fp4 = idx_format == IDX_FP4
        st = torch.uint8 if k_format == KV_MX16 else torch.float32
        return cls(batch, capacity, k_group, v_group, idx_dim,
                   z(batch, capacity, dim // 2, dt=torch.uint8),
                   z(batch, capacity, dim // k_group, dt=st),
                   z(batch, capacity, dv // 2, dt=torch.uint8) if v_group else None,
                   z(batch, capacity, dv // v_group, dt=st) if v_group else None,
                   z(batch, capacity, idx_dim // 2, dt=torch.uint8) if fp4
                   else z(batch, capacity, idx_dim, dt=torch.int16),
                   z(batch, dt=torch.int32), z(batch, dim, dt=torch.float32),
                   z(4, dt=torch.int32), dim, rope_dim, idx_format,
                   z(batch, capacity, idx_dim // 16, dt=torch.uint8) if fp4 else None, swa_format, k_format,
                   ratio)

    def desc(self) -> CacheDesc:
        p = lambda t: None if t is None else t.data_ptr()
        return CacheDesc(self.batch, self.capacity, self.dim, self.rope_dim, self.k_group,
                         self.v_group, self.idx_dim, p(self.k_codes), p(self.k_scales),
                         p(self.v_codes), p(self.v_scales), p(self.idx_keys), p(self.n_tokens),
                         p(self.pending), p(self.status), self.idx_format, p(self.idx_scales),
                         self.swa_format, self.k_format, self.ratio, self.page_size,
                         self.capacity // self.page_size if self.page_size else 0, self.n_pages,
                         p(self.block_table))

    def entry_bytes(self) -> int:
        """Bytes per entry in this cache's formats."""
        d = self.desc()
        n = lib().cskv_cache_entry_bytes(C.byref(d))
        if n == 0:
            raise CskvError(EINVAL, lib().cskv_last_error().decode())
        return int(n)


def workspace_bytes(cache: Cache, k: int, op: int = OP_INDEXER_TOPK, n_heads: int = 0,
                    window: int = 0) -> int:
    d = cache.desc()
    n = lib().cskv_workspace_bytes(C.byref(d), op, n_heads, k, window)
    if n == 0:
        raise CskvError(EINVAL, lib().cskv_last_error().decode())
    return int(n)


def workspace(cache: Cache, k: int, op: int = OP_INDEXER_TOPK, n_heads: int = 0,
              window: int = 0, pool=None) -> torch.Tensor:
    """Device workspace for an operation; pool = (pool_blocks, pool_block) for the
    hierarchical indexer's operations."""
    if pool is None:
        n = workspace_bytes(cache, k, op, n_heads, window)
    else:
        d = cache.desc()
        n = lib().cskv_workspace_bytes_pool(C.byref(d), op, n_heads, k, window, pool[0], pool[1])
        if n == 0:
            raise CskvError(EINVAL, lib().cskv_last_error().decode())
    return torch.empty(int(n), dtype=torch.uint8, device=cache.k_codes.device)


def entry_bytes(dim, rope_dim, k_group, v_group, idx_dim) -> int:
    return int(lib().cskv_entry_bytes(dim, rope_dim, k_group, v_group, idx_dim))


def append_workspace(n_rows: int, w_comp: Optional[torch.Tensor], device="cuda") -> torch.Tensor:
    nbytes = lib().cskv_append_workspace_bytes(n_rows, None if w_comp is None else w_comp.data_ptr())
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def kv_append_fp4(cache: Cache, tokens: torch.Tensor, cu_new: Optional[torch.Tensor],
                  w_comp: Optional[torch.Tensor], idx_rows: torch.Tensor, ws: Optional[torch.Tensor] = None,
                  stream=None, mfma: bool = False) -> None:
    """cskv_kv_append_fp4, or with mfma=True cskv_kv_append_fp4_mfma (the
    matrix-core compressor for appends of 512 rows or more)."""
    n = tokens.shape[0]
    tmp = None
    if ws is None and w_comp is not None:
        ws = tmp = append_workspace(n, w_comp, tokens.device)
    d = cache.desc()
    fn = lib().cskv_kv_append_fp4_mfma if mfma else lib().cskv_kv_append_fp4
    _check(fn(
        C.byref(d), _ptr(tokens, F32, "tokens", (n, cache.dim)),
        _ptr(cu_new, I32, "cu_new", (cache.batch + 1,)), n,
        _ptr(w_comp, F32, "w_comp", (cache.dim, 2 * cache.dim)),
        _ptr(idx_rows, B16, "idx_rows", (n, cache.idx_dim)),
        _ptr(ws, U8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)))
    _keep_for(stream, tmp)


def swa_append(ring: torch.Tensor, rows: torch.Tensor, cu_new: Optional[torch.Tensor],
               end_pos: torch.Tensor, stream=None) -> None:
    """Window rows into a ring: bf16 rings (cskv_swa_append) or FP8 E4M3 rings
    given as uint8 tensors (cskv_swa_append_fp8)."""
    B, W, D = ring.shape
    n = rows.shape[0]
    fp8 = ring.dtype == torch.uint8
    fn = lib().cskv_swa_append_fp8 if fp8 else lib().cskv_swa_append
    _check(fn(_ptr(ring, U8 if fp8 else B16, "ring"), B, W, D, _ptr(rows, F32, "rows", (n, D)),
              _ptr(cu_new, I32, "cu_new", (B + 1,)), n,
              _ptr(end_pos, I32, "end_pos", (B,)), _stream(stream)))


def indexer_topk(cache: Cache, q_idx: torch.Tensor, k: int, head_w: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 stream=None, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k indices [B, k]; with `scores` (f32 [B, capacity]) the score of
    every live entry is written there too."""
    B, H, Di = q_idx.shape
    tmp = []
    if out is None:
        out = torch.empty(B, k, dtype=torch.int32, device=q_idx.device)
        tmp.append(out)
    if ws is None:
        ws = workspace(cache, k)
        tmp.append(ws)
    d = cache.desc()
    _check(lib().cskv_indexer_topk(
        C.byref(d), _ptr(q_idx, B16, "q_idx", (cache.batch, H, cache.idx_dim)), H,
        _ptr(head_w, F32, "head_w", (cache.batch, H)), k, _ptr(out, I32, "out", (cache.batch, k)),
        _ptr(scores, F32, "scores", (cache.batch, cache.capacity)),
        _ptr(ws, U8, "ws"), ws.numel(), _stream(stream)))
    _keep_for(stream, *tmp)
    return out


def indexer_topk_pool(cache: Cache, q_idx: torch.Tensor, k: int, pool_blocks: int, pool_block: int,
                      head_w: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      out_pool: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      stream=None):
    """indexer_topk plus the hierarchical indexer's candidate pool [B, pool_blocks]."""
    B, H, Di = q_idx.shape
    tmp = []
    if out is None:
        out = torch.empty(B, k, dtype=torch.int32, device=q_idx.device)
        tmp.append(out)
    if out_pool is None:
        out_pool = torch.empty(B, pool_blocks, dtype=torch.int32, device=q_idx.device)
        tmp.append(out_pool)
    if ws is None:
        ws = workspace(cache, k, OP_INDEXER_POOL, pool=(pool_blocks, pool_block))
        tmp.append(ws)
    d = cache.desc()
    _check(lib().cskv_indexer_topk_pool(
        C.byref(d), _ptr(q_idx, B16, "q_idx", (cache.batch, H, cache.idx_dim)), H,
        _ptr(head_w, F32, "head_w", (cache.batch, H)), k, _ptr(out, I32, "out", (cache.batch, k)),
        pool_blocks, pool_block, _ptr(out_pool, I32, "out_pool", (cache.batch, pool_blocks)),
        _ptr(ws, U8, "ws"), ws.numel(), _stream(stream)))
    _keep_for(stream, *tmp)
    return out, out_pool


def indexer_topk_in_pool(cache: Cache, q_idx: torch.Tensor, k: int, pool: torch.Tensor, pool_block: int,
                         head_w: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k of this query's indexer scores among the entries of the pooled blocks."""
    B, H, Di = q_idx.shape
    nb = pool.shape[1]
    tmp = []
    if out is None:
        out = torch.empty(B, k, dtype=torch.int32, device=q_idx.device)
        tmp.append(out)
    if ws is None:
        ws = workspace(cache, k, OP_INDEXER_IN_POOL, pool=(nb, pool_block))
        tmp.append(ws)
    d = cache.desc()
    _check(lib().cskv_indexer_topk_in_pool(
        C.byref(d), _ptr(q_idx, B16, "q_idx", (cache.batch, H, cache.idx_dim)), H,
        _ptr(head_w, F32, "head_w", (cache.batch, H)), k, _ptr(pool, I32, "pool", (cache.batch, nb)),
        nb, pool_block, _ptr(out, I32, "out", (cache.batch, k)), _ptr(ws, U8, "ws"), ws.numel(),
        _stream(stream)))
    _keep_for(stream, *tmp)
    return out


def sparse_attn_decode(cache: Cache, q: torch.Tensor, idx: torch.Tensor, swa: torch.Tensor,
                       softmax_scale: float, swa_len: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None):
    B, H, D = q.shape
    k = idx.shape[1]
    W = swa.shape[1]
    dv = cache.dim - cache.rope_dim
    tmp = []
    if out is None:
        out = torch.empty(B, H, dv, dtype=torch.float32, device=q.device)
        tmp.append(out)
    if lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
        tmp.append(lse)
    if ws is None:
        ws = workspace(cache, k, OP_SPARSE_ATTN, H, W)
        tmp.append(ws)
    d = cache.desc()
    _check(lib().cskv_sparse_attn_decode(
        C.byref(d), _ptr(q, F32, "q", (cache.batch, H, cache.dim)), H,
        _ptr(idx, I32, "idx", (cache.batch, k)), k, _ptr(swa, U8 if cache.swa_format == SWA_FP8 else B16, "swa", (cache.batch, W, cache.dim)), W,
        _ptr(swa_len, I32, "swa_len", (cache.batch,)), float(softmax_scale),
        _ptr(out, F32, "out", (cache.batch, H, dv)), _ptr(lse, F32, "lse", (cache.batch, H)),
        _ptr(ws, U8, "ws"), ws.numel(), _stream(stream)))
    _keep_for(stream, *tmp)
    return out, lse


@dataclass
class Layer:
    """One layer of a CSA2 group; tensors as in cskv.h's cskv_layer."""
    mode: str
    q: torch.Tensor
    swa: torch.Tensor
    out: torch.Tensor
    q_idx: Optional[torch.Tensor] = None
    head_w: Optional[torch.Tensor] = None
    swa_row: Optional[torch.Tensor] = None
    idx: Optional[torch.Tensor] = None
    lse: Optional[torch.Tensor] = None


def layer_group_decode(cache: Cache, layers: Sequence[Layer], new_tokens: Optional[torch.Tensor],
                       w_comp: Optional[torch.Tensor], new_idx_rows: Optional[torch.Tensor],
                       k: int, window: int, softmax_scale: float, ws: Optional[torch.Tensor] = None,
                       stream=None, pool=None) -> None:
    """One decode step of a layer group; pool = (pool_blocks, pool_block) turns on
    the hierarchical indexer (cskv_layer_group_decode_pooled)."""
    B = cache.batch
    n_heads = layers[0].q.shape[1]
    n_idx_heads = next((L.q_idx.shape[1] for L in layers if L.q_idx is not None), 1)
    tmp = None
    if ws is None:
        ws = tmp = workspace(cache, k, OP_LAYER_GROUP, n_heads, window, pool=pool)
    arr = (LayerDesc * len(layers))()
    for i, L in enumerate(layers):
        dv = cache.dim - cache.rope_dim
        arr[i] = LayerDesc(MODES[L.mode], _ptr(L.q, F32, "q", (B, n_heads, cache.dim)),
                           _ptr(L.q_idx, B16, "q_idx", (B, n_idx_heads, cache.idx_dim)),
                           _ptr(L.head_w, F32, "head_w", (B, n_idx_heads)),
                           _ptr(L.swa, U8 if cache.swa_format == SWA_FP8 else B16, "swa", (B, window, cache.dim)),
                           _ptr(L.swa_row, F32, "swa_row", (B, cache.dim)),
                           _ptr(L.idx, I32, "idx", (B, k)),
                           _ptr(L.out, F32, "out", (B, n_heads, dv)),
                           _ptr(L.lse, F32, "lse", (B, n_heads)))
    d = cache.desc()
    args = (C.byref(d), arr, len(layers), _ptr(new_tokens, F32, "new_tokens", (B, cache.dim)),
            _ptr(w_comp, F32, "w_comp", (cache.dim, 2 * cache.dim)),
            _ptr(new_idx_rows, B16, "new_idx_rows", (B, cache.idx_dim)), n_idx_heads, n_heads, k,
            window, float(softmax_scale))
    if pool is None:
        _check(lib().cskv_layer_group_decode(*args, _ptr(ws, U8, "ws"), ws.numel(), _stream(stream)))
    else:
        _check(lib().cskv_layer_group_decode_pooled(*args, pool[0], pool[1], _ptr(ws, U8, "ws"), ws.numel(),
                                                    _stream(stream)))
    _keep_for(stream, tmp)


def layer_group_decode_noalloc(cache: Cache, layers: Sequence[Layer], new_tokens: Optional[torch.Tensor],
                               w_comp: Optional[torch.Tensor], new_idx_rows: Optional[torch.Tensor],
                               k: int, window: int, softmax_scale: float, stream=None) -> None:
    """layer_group_decode without a workspace argument: the library's own
    scratch (cskv_layer_group_decode_noalloc; nothing is allocated)."""
    B = cache.batch
    n_heads = layers[0].q.shape[1]
    n_idx_heads = next((L.q_idx.shape[1] for L in layers if L.q_idx is not None), 1)
    arr = (LayerDesc * len(layers))()
    dv = cache.dim - cache.rope_dim
    for i, L in enumerate(layers):
        arr[i] = LayerDesc(MODES[L.mode], _ptr(L.q, F32, "q", (B, n_heads, cache.dim)),
                           _ptr(L.q_idx, B16, "q_idx", (B, n_idx_heads, cache.idx_dim)),
                           _ptr(L.head_w, F32, "head_w", (B, n_idx_heads)),
                           _ptr(L.swa, U8 if cache.swa_format == SWA_FP8 else B16, "swa", (B, window, cache.dim)),
                           _ptr(L.swa_row, F32, "swa_row", (B, cache.dim)),
                           _ptr(L.idx, I32, "idx", (B, k)),
                           _ptr(L.out, F32, "out", (B, n_heads, dv)),
                           _ptr(L.lse, F32, "lse", (B, n_heads)))
    d = cache.desc()
    _check(lib().cskv_layer_group_decode_noalloc(
        C.byref(d), arr, len(layers), _ptr(new_tokens, F32, "new_tokens", (B, cache.dim)),
        _ptr(w_comp, F32, "w_comp", (cache.dim, 2 * cache.dim)),
        _ptr(new_idx_rows, B16, "new_idx_rows", (B, cache.idx_dim)), n_idx_heads, n_heads, k, window,
        float(softmax_scale), _stream(stream)))


def ced_project(h: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """CED projection: out[r][n] = sum_k h[r][k] w[n][k]; h bf16 bits (int16)
    [rows, d_model], w bf16 bits (int16) [n_out, d_model] -> fp32 [rows, n_out]."""
    rows, dm = h.shape
    n_out = w.shape[0]
    tmp = None
    if out is None:
        out = tmp = torch.empty(rows, n_out, dtype=torch.float32, device=h.device)
    _check(lib().cskv_ced_project(_ptr(h, B16, "h", (rows, dm)), rows, dm, _ptr(w, B16, "w", (n_out, dm)),
                                  n_out, _ptr(out, F32, "out", (rows, n_out)), _stream(stream)))
    _keep_for(stream, tmp)
    return out


@dataclass
class Group:
    """One group of the layer plan (cskv_group): the layers sharing `cache`
    and the source of the step's new entries -- new_tokens (+ w_comp for
    the 2->1 compressor) or the CED projection of ced_h by ced_w."""
    cache: Cache
    layers: Sequence[Layer]
    new_idx_rows: Optional[torch.Tensor] = None
    new_tokens: Optional[torch.Tensor] = None
    w_comp: Optional[torch.Tensor] = None
    ced_h: Optional[torch.Tensor] = None
    ced_w: Optional[torch.Tensor] = None
    pool: Optional[tuple] = None


def _group_descs(groups: Sequence[Group], k: int, window: int):
    """ctypes descriptors of the groups (kept alive by the returned list)."""
    keep, descs = [], (GroupDesc * len(groups))()
    n_heads = groups[0].layers[0].q.shape[1]
    n_idx_heads = next((L.q_idx.shape[1] for g in groups for L in g.layers if L.q_idx is not None), 1)
    for gi, g in enumerate(groups):
        c, B = g.cache, g.cache.batch
        d = c.desc()
        arr = (LayerDesc * len(g.layers))()
        dv = c.dim - c.rope_dim
        for i, L in enumerate(g.layers):
            arr[i] = LayerDesc(MODES[L.mode], _ptr(L.q, F32, "q", (B, n_heads, c.dim)),
                               _ptr(L.q_idx, B16, "q_idx", (B, n_idx_heads, c.idx_dim)),
                               _ptr(L.head_w, F32, "head_w", (B, n_idx_heads)),
                               _ptr(L.swa, U8 if c.swa_format == SWA_FP8 else B16, "swa", (B, window, c.dim)),
                               _ptr(L.swa_row, F32, "swa_row", (B, c.dim)),
                               _ptr(L.idx, I32, "idx", (B, k)),
                               _ptr(L.out, F32, "out", (B, n_heads, dv)),
                               _ptr(L.lse, F32, "lse", (B, n_heads)))
        dm = 0 if g.ced_h is None else g.ced_h.shape[1]
        pb, pbk = g.pool if g.pool else (0, 0)
        descs[gi] = GroupDesc(C.addressof(d), C.addressof(arr), len(g.layers),
                              _ptr(g.new_tokens, F32, "new_tokens", (B, c.dim)),
                              _ptr(g.w_comp, F32, "w_comp", (c.dim, 2 * c.dim)),
                              _ptr(g.ced_h, B16, "ced_h", (B, dm)), _ptr(g.ced_w, B16, "ced_w", (c.dim, dm)), dm,
                              _ptr(g.new_idx_rows, B16, "new_idx_rows", (B, c.idx_dim)), pb, pbk)
        keep += [d, arr]
    return descs, keep, n_idx_heads, n_heads


def model_workspace(groups: Sequence[Group], k: int, window: int) -> torch.Tensor:
    descs, keep, _, n_heads = _group_descs(groups, k, window)
    n = lib().cskv_model_workspace_bytes(descs, len(groups), n_heads, k, window)
    if n == 0:
        raise CskvError(EINVAL, lib().cskv_last_error().decode())
    return torch.empty(int(n), dtype=torch.uint8, device=groups[0].cache.k_codes.device)


def model_decode(groups: Sequence[Group], k: int, window: int, softmax_scale: float,
                 ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step of every group of the layer plan (cskv_model_decode)."""
    tmp = None
    if ws is None:
        ws = tmp = model_workspace(groups, k, window)
    descs, keep, n_idx_heads, n_heads = _group_descs(groups, k, window)
    _check(lib().cskv_model_decode(descs, len(groups), n_idx_heads, n_heads, k, window, float(softmax_scale),
                                   _ptr(ws, U8, "ws"), ws.numel(), _stream(stream)))
    _keep_for(stream, tmp)


# ---------------------------------------------------------------- timers

def timer_enable(kind: int, max_launches: int) -> None:
    _check(lib().cskv_timer_enable(kind, max_launches))


def timer_pause(kind: int, paused: bool) -> None:
    _check(lib().cskv_timer_pause(kind, int(bool(paused))))


def timer_read(kind: int):
    ms = C.c_double()
    n = C.c_int32()
    _check(lib().cskv_timer_read(kind, C.byref(ms), C.byref(n)))
    return ms.value, n.value


def timer_disable_all() -> None:
    _check(lib().cskv_timer_disable_all())
