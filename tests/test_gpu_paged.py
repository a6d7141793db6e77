"""Paged cache planes: a block table per sequence maps each page-sized run of
its entries to a page of shared planes [P2 三、"突破六：系统层，不改模型改部署"
(KV allocated in fixed-size pages, PagedAttention-style)].

A paged cache holds the same entries as a dense one, only in other rows, so
every result must be the dense cache's bit for bit: the appends (entries
mode, decode pairs through the compressor, a planned chunk of 512+ rows),
the indexer top-k (full and pooled scans), attention and the layer-group
step, in every storage format.  The block tables are seeded shuffles with
pages to spare and pages of different sequences interleaved.  The dense
path is checked against the oracle by the other parity tests.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import dev, host  # noqa: E402

PLANES = ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "idx_scales")


@pytest.fixture(scope="module")
def ck():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_kv_append_amd as ck
    ck.lib()
    return ck


def _twins(ck, batch, cap, page, kg, vg, idx_dim, seed, idx_format=0, k_format=0, spare=5):
    """A dense cache and a paged cache of the same shape; the paged one's
    table is a seeded shuffle of batch * cap / page pages among n_pages."""
    dense = ck.Cache.allocate(batch, cap, kg, vg, idx_dim, idx_format=idx_format, k_format=k_format)
    max_pages = cap // page
    n_pages = batch * max_pages + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pages)[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    paged = ck.Cache.allocate_paged(batch, cap, page, n_pages, dev(table), kg, vg, idx_dim,
                                    idx_format=idx_format, k_format=k_format)
    return dense, paged, table


def _assert_same(dense, paged, table, page):
    torch.cuda.synchronize()
    nt = host(dense.n_tokens)
    assert np.array_equal(nt, host(paged.n_tokens))
    assert int(host(dense.status)[0]) == int(host(paged.status)[0])
    for b in range(dense.batch):
        if nt[b] % 2 == 1:
            assert np.array_equal(host(dense.pending[b]), host(paged.pending[b]))
    for name in PLANES:
        gd, gp = getattr(dense, name), getattr(paged, name)
        if gd is None:
            continue
        hd, hp = host(gd), host(gp)
        hp = hp.reshape(-1, *hd.shape[2:])
        for b in range(dense.batch):
            e = int(min(nt[b] // dense.ratio, dense.capacity))
            rows = (table[b][np.arange(e) // page].astype(np.int64) * page + np.arange(e) % page)
            if not np.array_equal(hd[b, :e].view(np.uint8), hp[rows].view(np.uint8)):
                raise AssertionError(f"{name} differs for sequence {b}")


def _load(ck, caches, w, lens):
    """Entries-mode append of seeded rows (one call for the batch) to every cache."""
    rows = np.concatenate([synth.cache_entries(w, b, n) for b, n in enumerate(lens)])
    keys = np.concatenate([synth.cache_idx_keys(w, b)[:n] for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for c in caches:
        ck.kv_append_fp4(c, dev(rows), dev(cu), None, dev(keys))


def _chunk(ck, caches, w, lens, salt, mfma=False):
    toks = np.concatenate([synth.prefill_tokens(w, b + salt, n) for b, n in enumerate(lens)])
    irows = np.concatenate([synth.prefill_idx_rows(w, b + salt, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for c in caches:
        ck.kv_append_fp4(c, dev(toks), dev(cu), dev(synth.w_comp(w)), dev(irows), mfma=mfma)


def _step(ck, c, w, step, pool=None):
    st = synth.step_inputs(w, step)
    rings = [dev(r) for r in st.swa_ring]
    B, k = w.batch, w.topk
    layers = []
    for li, mode in enumerate(w.layers):
        layers.append(ck.Layer(mode=mode, q=dev(st.q[li]), swa=rings[li],
                               out=torch.empty(B, w.q_heads, 512, device="cuda"),
                               lse=torch.empty(B, w.q_heads, device="cuda"),
                               q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                               swa_row=dev(st.swa_row[li]),
                               idx=torch.empty(B, k, dtype=torch.int32, device="cuda")
                               if mode != "reuse" else None))
    ck.layer_group_decode(c, layers, dev(st.token), dev(synth.w_comp(w)), dev(st.idx_row), k, w.window,
                          1 / math.sqrt(576), pool=pool)
    torch.cuda.synchronize()
    outs = [host(r) for r in rings]
    for L in layers:
        outs += [host(L.out), host(L.lse)] + ([host(L.idx)] if L.idx is not None else [])
    return outs


def _same_outputs(a, b):
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"output {i} differs between dense and paged"


@pytest.mark.parametrize("page", [64, 256])
@pytest.mark.parametrize("kg,vg,idx_format,k_format", [(32, 128, 0, 0), (64, 0, 1, 0), (16, 16, 1, 1)])
def test_paged_layer_group_matches_dense(ck, page, kg, vg, idx_format, k_format):
    """Ragged sequences (an empty one, some shorter than k, one spanning
    many pages), a prefill chunk through the planned compressor, then three
    Full + Reindex + Reuse steps: planes, counts, pending tokens, indices,
    outputs and LSE identical to the dense cache."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=5, entries=3000)
    lens = [3000, 0, 130, 700, 2049]
    cap = 4096
    dense, paged, table = _twins(ck, w.batch, cap, page, kg, vg, w.idx_dim, seed=page + kg,
                                 idx_format=idx_format, k_format=k_format)
    _load(ck, (dense, paged), w, lens)
    _assert_same(dense, paged, table, page)
    _chunk(ck, (dense, paged), w, [3, 600, 1, 0, 9], salt=7)       # 613 rows: the planned path
    _assert_same(dense, paged, table, page)
    for step in range(3):
        _same_outputs(_step(ck, dense, w, step), _step(ck, paged, w, step))
        _assert_same(dense, paged, table, page)


def test_paged_pooled_indexer_and_mfma_chunk(ck):
    """The hierarchical indexer's pooled scan reads entries through the
    table too; the matrix-core compressor writes through it."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=4, entries=5000)
    lens = [5000, 4100, 900, 4500]
    page = 128
    dense, paged, table = _twins(ck, w.batch, 6144, page, 64, 0, w.idx_dim, seed=3)
    _load(ck, (dense, paged), w, lens)
    _chunk(ck, (dense, paged), w, [700, 1, 2, 0], salt=5, mfma=True)
    _assert_same(dense, paged, table, page)
    for step in range(2):
        _same_outputs(_step(ck, dense, w, step, pool=(256, 8)), _step(ck, paged, w, step, pool=(256, 8)))
        _assert_same(dense, paged, table, page)


def test_paged_append_through_a_bad_page_flags_and_writes_nothing(ck):
    """An entry whose page the table does not map (-1, or past n_pages)
    raises CSKV_STATUS_BAD_PAGE; no plane row changes for it."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=2, entries=100)
    page, cap = 64, 256
    max_pages = cap // page
    n_pages = 2 * max_pages
    table = np.arange(n_pages, dtype=np.int32).reshape(2, max_pages)
    table[0, 1] = -1                  # entries 64 .. 127 of sequence 0
    table[1, 1] = n_pages + 3         # entries 64 .. 127 of sequence 1
    paged = ck.Cache.allocate_paged(2, cap, page, n_pages, dev(table), 32, 0, w.idx_dim)
    before = host(paged.k_codes).copy()
    _load(ck, (paged,), w, [100, 100])
    torch.cuda.synchronize()
    assert int(host(paged.status)[0]) & ck.STATUS_BAD_PAGE
    after = host(paged.k_codes)
    # rows of the mapped pages were written, no other row changed
    written = set()
    for b in range(2):
        for e in range(100):
            pg = table[b, e // page]
            if 0 <= pg < n_pages:
                written.add(int(pg) * page + e % page)
    changed = set(np.nonzero((before.reshape(-1, 288) != after.reshape(-1, 288)).any(axis=1))[0].tolist())
    assert changed <= written, sorted(changed - written)[:8]
