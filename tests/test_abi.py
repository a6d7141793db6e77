"""The C ABI without a GPU: the library loads, exports every function that
include/cskv.h declares, and its host-only parts (byte helpers, argument
checks that reject a call before anything is enqueued) behave as declared.
No call here reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

import compressed_sparse_kv_append_amd as ck
from compressed_sparse_kv_append_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cskv.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cskv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_build.LIB):
        pytest.fail(f"{_build.LIB} not built: run __graft_entry__.build() first")
    return ck.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10, names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"declared in cskv.h but not exported: {missing}"
    assert set(ck.EXPORTS) <= set(names), set(ck.EXPORTS) - set(names)


def test_entry_bytes(L):
    # 576 dims: 288 code bytes + 4 B per group scale + 2 B per indexer-key dim
    assert ck.entry_bytes(576, 64, 32, 0, 128) == 288 + 72 + 256
    assert ck.entry_bytes(576, 64, 64, 0, 128) == 288 + 36 + 256
    # split value plane: 512 dims at group 128 adds 256 + 16
    assert ck.entry_bytes(576, 64, 32, 128, 128) == 288 + 72 + 256 + 256 + 16
    assert ck.entry_bytes(576, 64, 100, 0, 128) == 0   # group must divide dim


def _desc(**over):
    d = dict(batch=2, capacity=64, dim=576, rope_dim=64, k_group=32, v_group=0, idx_dim=64,
             k_codes=0x10000, k_scales=0x20000, v_codes=None, v_scales=None, idx_keys=0x30000,
             n_tokens=0x40000, pending=0x50000, status=0x60000, idx_format=0, idx_scales=None, swa_format=0,
             k_format=0, ratio=2, page_size=0, max_pages=0, n_pages=0, block_table=None)
    d.update(over)
    return ck.CacheDesc(*[d[f] for f, _ in ck.CacheDesc._fields_])


def _err(L):
    return L.cskv_last_error().decode()


def test_cache_entry_bytes_in_each_format(L):
    n = lambda **o: L.cskv_cache_entry_bytes(C.byref(_desc(**o)))
    # fp32 scales, bf16 indexer keys: the shape-only helper's figure
    assert n(k_group=64, idx_dim=128) == ck.entry_bytes(576, 64, 64, 0, 128) == 288 + 36 + 256
    assert n(k_group=32, v_group=128, v_codes=0x70000, v_scales=0x80000, idx_dim=64) == \
        ck.entry_bytes(576, 64, 32, 128, 64)
    # the pages' formats with split planes: the value row (512 latent dims,
    # E2M1 + one byte per 16) is their 288 B main entry and the FP4 indexer
    # key their 72 B; the key plane adds the 576-dim row with its RoPE dims
    pages = dict(k_format=1, k_group=16, v_group=16, v_codes=0x70000, v_scales=0x80000, idx_dim=128,
                 idx_format=1, idx_scales=0x90000)
    key_row = 576 // 2 + 576 // 16
    assert n(**pages) == key_row + 288 + 72
    assert n(**pages) - key_row == 360
    # shared planes: the key row carries the values
    assert n(**dict(pages, v_group=0, v_codes=None, v_scales=None)) == 324 + 72
    assert n(k_format=1, k_group=32) == 0 and "k_group" in _err(L)


@pytest.mark.parametrize("over,code,text", [
    (dict(dim=512), ck.EUNSUPPORTED, "dim"),
    (dict(k_group=128), ck.EUNSUPPORTED, "k_group"),
    (dict(v_group=48), ck.EUNSUPPORTED, "v_group"),
    (dict(idx_dim=96), ck.EUNSUPPORTED, "idx_dim"),
    (dict(batch=0), ck.EINVAL, "batch"),
    (dict(capacity=0), ck.EINVAL, "capacity"),
    (dict(k_codes=None), ck.EINVAL, "NULL"),
    (dict(k_scales=0x20004), ck.EINVAL, "aligned"),
    (dict(v_group=128), ck.EINVAL, "value plane"),
    (dict(idx_format=2), ck.EUNSUPPORTED, "idx_format"),
    (dict(idx_format=1), ck.EINVAL, "idx_scales"),
    (dict(idx_scales=0x68000), ck.EINVAL, "idx_scales"),
    (dict(idx_format=1, idx_scales=0x68004), ck.EINVAL, "aligned"),
    (dict(swa_format=2), ck.EUNSUPPORTED, "swa_format"),
    (dict(k_format=2), ck.EUNSUPPORTED, "k_format"),
    (dict(k_format=1), ck.EUNSUPPORTED, "k_group"),
    (dict(k_group=16), ck.EUNSUPPORTED, "k_group"),
    (dict(k_format=1, k_group=16, v_group=32), ck.EUNSUPPORTED, "v_group"),
    (dict(ratio=0), ck.EUNSUPPORTED, "ratio"),
    (dict(ratio=3), ck.EUNSUPPORTED, "ratio"),
])
def test_cache_descriptor_rejected_before_launch(L, over, code, text):
    d = _desc(**over)
    rc = L.cskv_kv_append_fp4(C.byref(d), C.c_void_p(0x70000), None, 2, None,
                              C.c_void_p(0x80000), None, 0, None)
    assert rc == code and text in _err(L), (rc, _err(L))
    assert L.cskv_workspace_bytes(C.byref(d), ck.OP_INDEXER_TOPK, 0, 512, 0) == 0


def test_ced_and_model_arguments_rejected_before_launch(L):
    vp = C.c_void_p
    h, w, out = vp(0x100000), vp(0x200000), vp(0x300000)
    # d_model a multiple of 128, n_out a multiple of 16, aligned pointers
    assert L.cskv_ced_project(h, 32, 4000, w, 576, out, None) == ck.EUNSUPPORTED and "d_model" in _err(L)
    assert L.cskv_ced_project(h, 32, 4096, w, 570, out, None) == ck.EUNSUPPORTED and "n_out" in _err(L)
    assert L.cskv_ced_project(vp(0x100008), 32, 4096, w, 576, out, None) == ck.EINVAL
    assert L.cskv_ced_project(None, 32, 4096, w, 576, out, None) == ck.EINVAL
    assert L.cskv_ced_project(h, -1, 4096, w, 576, out, None) == ck.EINVAL
    # the 2->1 compressor on a one-entry-per-token cache
    d1 = _desc(ratio=1)
    need = L.cskv_append_workspace_bytes(2, vp(0x110000))
    assert L.cskv_kv_append_fp4(C.byref(d1), vp(0x70000), None, 2, vp(0x110000), vp(0x80000), vp(0xB0000),
                                need, None) == ck.EUNSUPPORTED and "ratio" in _err(L)
    # model decode: group checks come before any launch
    d = _desc()
    lay = ck.LayerDesc(ck.MODE_FULL, 0xC0000, 0xA0000, None, 0xE0000, None, 0x90000, 0xF0000, None)
    g = ck.GroupDesc(C.addressof(d), C.addressof(lay), 1, 0x70000, None, 0x100000, 0x200000, 4096, 0x80000, 0, 0)
    arr = (ck.GroupDesc * 1)(g)
    assert L.cskv_model_decode(arr, 1, 4, 16, 512, 128, C.c_float(0.04), vp(0xB0000), 1 << 30,
                               None) == ck.EINVAL and "exclusive" in _err(L)
    assert L.cskv_model_decode(arr, 0, 4, 16, 512, 128, C.c_float(0.04), vp(0xB0000), 1 << 30, None) == ck.EINVAL
    arr[0].new_tokens = None
    arr[0].d_model = 1000
    assert L.cskv_model_decode(arr, 1, 4, 16, 512, 128, C.c_float(0.04), vp(0xB0000), 1 << 30,
                               None) == ck.EUNSUPPORTED and "d_model" in _err(L)
    assert L.cskv_model_workspace_bytes(arr, 1, 16, 512, 128) == 0
    arr[0].d_model = 4096
    ws = L.cskv_model_workspace_bytes(arr, 1, 16, 512, 128)
    group = L.cskv_workspace_bytes(C.byref(d), ck.OP_LAYER_GROUP, 16, 512, 128)
    assert ws == group + 2 * 576 * 4            # the projected rows (4608 B, 256-aligned) + the group's
    assert L.cskv_model_decode(arr, 1, 4, 16, 512, 128, C.c_float(0.04), vp(0xB0000), ws - 1,
                               None) == ck.EWORKSPACE


def test_call_arguments_rejected_before_launch(L):
    d = _desc()
    vp = C.c_void_p
    # cu_new NULL needs one row per sequence
    assert L.cskv_kv_append_fp4(C.byref(d), vp(0x70000), None, 3, None, vp(0x80000), None, 0, None) == ck.EINVAL
    # a compressor append needs its workspace
    need = L.cskv_append_workspace_bytes(2, vp(0x110000))
    # compressor rows (fp32), then one 16-byte plan record per row and a count,
    # each region rounded to 256 bytes
    assert need == 4608 + 256 + 256 and L.cskv_append_workspace_bytes(2, None) == 256
    assert L.cskv_kv_append_fp4(C.byref(d), vp(0x70000), None, 2, vp(0x110000), vp(0x80000), vp(0xB0000),
                                need - 1, None) == ck.EWORKSPACE
    assert L.cskv_kv_append_fp4_mfma(C.byref(d), vp(0x70000), None, 2, vp(0x110000), vp(0x80000),
                                     vp(0xB0000), need - 1, None) == ck.EWORKSPACE
    # 512 rows and more: the same regions, then W split into bf16 high and
    # low parts for the matrix-core compressor (576 x 1152 x 2 x 2 bytes)
    assert L.cskv_append_workspace_bytes(512, vp(0x110000)) == 512 * 2304 + 512 * 16 + 256 + 576 * 1152 * 4
    # top-k: k out of range, too many heads, workspace too small
    ws = L.cskv_workspace_bytes(C.byref(d), ck.OP_INDEXER_TOPK, 0, 512, 0)
    assert ws > 0
    out = vp(0x90000)
    assert L.cskv_indexer_topk(C.byref(d), vp(0xA0000), 4, None, 0, out, None, vp(0xB0000), ws, None) == ck.EUNSUPPORTED
    assert L.cskv_indexer_topk(C.byref(d), vp(0xA0000), 65, None, 512, out, None, vp(0xB0000), ws, None) == ck.EUNSUPPORTED
    assert L.cskv_indexer_topk(C.byref(d), vp(0xA0000), 4, None, 512, out, None, vp(0xB0000), ws - 1, None) == ck.EWORKSPACE
    assert L.cskv_indexer_topk(C.byref(d), vp(0xA0000), 4, None, 512, out, None, None, ws, None) == ck.EWORKSPACE
    # attention: heads not a multiple of 16, missing window, workspace too small
    # (k = 2048 with a 1024-row window is split over several blocks, whose
    # partial softmaxes need workspace)
    aws = L.cskv_workspace_bytes(C.byref(d), ck.OP_SPARSE_ATTN, 16, 2048, 1024)
    assert aws > 256
    assert L.cskv_sparse_attn_decode(C.byref(d), vp(0xC0000), 24, vp(0xD0000), 512, vp(0xE0000), 128,
                                     None, C.c_float(0.04), vp(0xF0000), None, vp(0xB0000), aws,
                                     None) == ck.EUNSUPPORTED
    assert L.cskv_sparse_attn_decode(C.byref(d), vp(0xC0000), 16, vp(0xD0000), 512, None, 128,
                                     None, C.c_float(0.04), vp(0xF0000), None, vp(0xB0000), aws,
                                     None) == ck.EINVAL
    assert L.cskv_sparse_attn_decode(C.byref(d), vp(0xC0000), 16, vp(0xD0000), 2048, vp(0xE0000), 1024,
                                     None, C.c_float(0.04), vp(0xF0000), None, vp(0xB0000), aws - 1,
                                     None) == ck.EWORKSPACE
    assert L.cskv_workspace_bytes(C.byref(d), 9, 16, 512, 128) == 0
    # attention addresses a sequence's rows with 32-bit offsets: capacity <= 2^23
    big = _desc(capacity=(1 << 23) + 1)
    bws = L.cskv_workspace_bytes(C.byref(big), ck.OP_SPARSE_ATTN, 16, 512, 128)
    assert L.cskv_sparse_attn_decode(C.byref(big), vp(0xC0000), 16, vp(0xD0000), 512, vp(0xE0000), 128,
                                     None, C.c_float(0.04), vp(0xF0000), None, vp(0xB0000), bws,
                                     None) == ck.EUNSUPPORTED and "capacity" in _err(L)
    # window append: dim not a multiple of 4 (bf16) or of 16 (FP8)
    assert L.cskv_swa_append(vp(0x100000), 2, 128, 578, vp(0x70000), None, 2, vp(0x40000), None) == ck.EUNSUPPORTED
    assert L.cskv_swa_append_fp8(vp(0x100000), 2, 128, 580, vp(0x70000), None, 2, vp(0x40000), None) == ck.EUNSUPPORTED


def test_layer_group_checks_every_layer_first(L):
    d = _desc()
    vp = C.c_void_p
    ws = L.cskv_workspace_bytes(C.byref(d), ck.OP_LAYER_GROUP, 16, 512, 128)
    # a REUSE layer with no FULL/REINDEX before it is rejected before anything runs
    layers = (ck.LayerDesc * 2)()
    layers[0] = ck.LayerDesc(ck.MODE_REUSE, 0xC0000, None, None, 0x100000, None, None, 0xF0000, None)
    layers[1] = ck.LayerDesc(ck.MODE_FULL, 0xC0000, 0xA0000, None, 0x100000, None, 0x90000, 0xF0000, None)
    rc = L.cskv_layer_group_decode(C.byref(d), layers, 2, None, None, None, 4, 16, 512, 128,
                                   C.c_float(0.04), vp(0xB0000), ws, None)
    assert rc == ck.EINVAL and "REUSE" in _err(L)
    layers[0].mode = 7
    rc = L.cskv_layer_group_decode(C.byref(d), layers, 2, None, None, None, 4, 16, 512, 128,
                                   C.c_float(0.04), vp(0xB0000), ws, None)
    assert rc == ck.EINVAL and "mode" in _err(L)


def test_pool_arguments_rejected_before_launch(L):
    d = _desc()
    vp = C.c_void_p
    ws = L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_INDEXER_POOL, 0, 512, 0, 2048, 8)
    assert ws > L.cskv_workspace_bytes(C.byref(d), ck.OP_INDEXER_TOPK, 0, 512, 0)
    assert L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_INDEXER_IN_POOL, 0, 512, 0, 2048, 8) >= 2 * 2048 * 8 * 8
    # block size, pool size, pool too small for k
    for nb, blk, text in ((2048, 3, "pool_block"), (0, 8, "pool_blocks"), (4096, 8, "pool_blocks"),
                          (64, 8, "too small")):
        assert L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_INDEXER_POOL, 0, 512, 0, nb, blk) == 0
        assert text in _err(L)
        rc = L.cskv_indexer_topk_pool(C.byref(d), vp(0xA0000), 4, None, 512, vp(0x90000), nb, blk,
                                      vp(0x98000), vp(0xB0000), ws, None)
        assert rc == ck.EUNSUPPORTED and text in _err(L), (rc, _err(L))
    # missing pool output, workspace too small
    assert L.cskv_indexer_topk_pool(C.byref(d), vp(0xA0000), 4, None, 512, vp(0x90000), 2048, 8, None,
                                    vp(0xB0000), ws, None) == ck.EINVAL
    assert L.cskv_indexer_topk_pool(C.byref(d), vp(0xA0000), 4, None, 512, vp(0x90000), 2048, 8,
                                    vp(0x98000), vp(0xB0000), ws - 1, None) == ck.EWORKSPACE
    wi = L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_INDEXER_IN_POOL, 0, 512, 0, 2048, 8)
    assert L.cskv_indexer_topk_in_pool(C.byref(d), vp(0xA0000), 4, None, 512, None, 2048, 8, vp(0x90000),
                                       vp(0xB0000), wi, None) == ck.EINVAL
    assert L.cskv_indexer_topk_in_pool(C.byref(d), vp(0xA0000), 4, None, 512, vp(0x98000), 2048, 8,
                                       vp(0x90000), vp(0xB0000), wi - 1, None) == ck.EWORKSPACE
    # the pooled layer group needs more workspace than the plain one
    g0 = L.cskv_workspace_bytes(C.byref(d), ck.OP_LAYER_GROUP, 16, 512, 128)
    g1 = L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_LAYER_GROUP, 16, 512, 128, 2048, 8)
    assert g1 > g0 and L.cskv_workspace_bytes_pool(C.byref(d), ck.OP_LAYER_GROUP, 16, 512, 128, 0, 0) == g0



def test_noalloc_step_beyond_its_scratch_is_refused(L):
    # 32 sequences x 600K entries: the score keys alone (4 B per cache row)
    # pass the built-in 64 MiB scratch; refused before any device call
    d = _desc(batch=32, capacity=600000, k_group=64, idx_dim=128)
    need = L.cskv_workspace_bytes(C.byref(d), ck.OP_LAYER_GROUP, 64, 512, 128)
    assert need > (64 << 20)
    rc = L.cskv_layer_group_decode_noalloc(C.byref(d), None, 1, None, None, None, 64, 64, 512, 128,
                                           C.c_float(0.04), None)
    assert rc == ck.EWORKSPACE and "scratch" in _err(L), (rc, _err(L))
    # a step within the scratch passes this check; its arguments are checked
    # before the scratch is looked up (no layer array: EINVAL, no device call)
    small = _desc(batch=2, capacity=5000, k_group=64, idx_dim=128)
    rc = L.cskv_layer_group_decode_noalloc(C.byref(small), None, 1, None, None, None, 64, 64, 512, 128,
                                           C.c_float(0.04), None)
    assert rc == ck.EINVAL and "layers" in _err(L), (rc, _err(L))


def test_paged_cache_descriptor_rejected_before_launch(L):
    """A paged cache: a power-of-two page of at least 64 entries, capacity =
    max_pages x page_size, a block table, and planes under 2 GiB."""
    vp = C.c_void_p
    ok = dict(capacity=256, page_size=64, max_pages=4, n_pages=8, block_table=0x70000)
    tok, idx = vp(0x80000), vp(0x90000)
    def append(**over):
        d = _desc(**{**ok, **over})
        return L.cskv_kv_append_fp4(C.byref(d), tok, None, 2, None, idx, None, 0, None)
    assert append(page_size=48, max_pages=5, capacity=240) == ck.EUNSUPPORTED    # not a power of two
    assert append(page_size=32, max_pages=8) == ck.EUNSUPPORTED                  # below 64
    assert append(max_pages=3) == ck.EINVAL                                      # capacity != pages x size
    assert append(block_table=None) == ck.EINVAL
    assert append(n_pages=0) == ck.EINVAL
    assert append(page_size=1 << 20, max_pages=1, capacity=1 << 20, n_pages=8) == ck.EUNSUPPORTED   # > 2 GiB
    assert append(page_size=-64) == ck.EINVAL
