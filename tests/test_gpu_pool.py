"""GPU parity of the hierarchical sparse indexer [P2 "层级稀疏索引器：后面的
层只在候选池里找"]: the candidate pool built from a full layer's scan, the
top-k inside the pool, and the layer group with the pool turned on, each
bit for bit against the oracle (integer-valued indexer inputs, exact scores).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import TOL, assert_cache_equal, attn_rel_err, dev, host, load_entries, pair  # noqa: E402


@pytest.fixture(scope="module")
def ck():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_kv_append_amd as ck
    ck.lib()
    return ck


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


def _bf16_int(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _cache(ck, orc, lens, idx_dim, seed, key_fn=None, cap=None):
    g = np.random.default_rng(seed)
    B = len(lens)
    cap = cap or max(max(lens), 1) + 3
    gc, hc = pair(B, cap, 64, 0, idx_dim)
    keys = [key_fn(g, n) if key_fn else synth.int_bf16(g, (n, idx_dim)) for n in lens]
    load_entries(gc, hc, [np.zeros((n, 576), np.float32) for n in lens], keys)
    return g, gc, hc


def _pool_case(ck, orc, lens, idx_dim, heads, k, nb, block, seed, key_fn=None, head_w=None):
    g, gc, hc = _cache(ck, orc, lens, idx_dim, seed, key_fn)
    B = len(lens)
    q = synth.int_bf16(g, (B, heads, idx_dim))
    q2 = synth.int_bf16(g, (B, heads, idx_dim))
    hw = None if head_w is None else dev(head_w)
    idx, pool = ck.indexer_topk_pool(gc, dev(q), k, nb, block, head_w=hw)
    want_pool = orc.indexer_pool(hc, q, block, nb, head_w)
    want_idx = orc.indexer_topk(hc, q, k, head_w)
    got_pool, got_idx = host(pool), host(idx)
    for b in range(B):
        assert np.array_equal(got_pool[b], want_pool[b]), (b, lens[b], np.flatnonzero(got_pool[b] != want_pool[b])[:8])
        assert np.array_equal(got_idx[b], want_idx[b]), (b, lens[b])
    # a second query inside the device pool (equal to the oracle's)
    sel = host(ck.indexer_topk_in_pool(gc, dev(q2), k, pool, block, head_w=hw))
    want = orc.indexer_topk_in_pool(hc, q2, want_pool, block, k, head_w)
    for b in range(B):
        assert np.array_equal(sel[b], want[b]), (b, lens[b], np.flatnonzero(sel[b] != want[b])[:8])
    return got_pool, sel


def test_pool_and_topk_in_pool_ragged(ck, orc):
    # empty, below k, whole-pool (<= nb blocks), short last block, several
    # block-select slices (> 4096 blocks)
    lens = [0, 5, 300, 700, 1203, 5001, 40003]
    _pool_case(ck, orc, lens, 64, 4, 64, nb=96, block=8, seed=60)


def test_pool_many_sequences(ck, orc):
    """130 sequences: both the top-k and the pool's block select take the
    4-wave slice blocks of large batches; ragged lengths up to several block
    slices (> 4096 blocks of 8), with ties."""
    g = np.random.default_rng(68)
    lens = [int(x) for x in g.integers(0, 40000, size=130)]
    lens[:5] = [0, 5, 700, 36000, 39000]
    few = lambda g, n: synth.int_bf16(g, (n, 64), -2, 2)
    _pool_case(ck, orc, lens, 64, 4, 64, nb=96, block=8, seed=69, key_fn=few)


def test_pool_full_shape_blocks_of_8(ck, orc):
    # the pages' shape: 2048 blocks of 8 (16,384 positions), top-512, 64 x 128
    _pool_case(ck, orc, [70001, 20000, 16384, 16385], 128, 64, 512, nb=2048, block=8, seed=61)


@pytest.mark.parametrize("block", [2, 4, 16])
def test_pool_other_block_sizes(ck, orc, block):
    _pool_case(ck, orc, [3001, 999, 4100], 64, 4, 100, nb=(100 + block) // block + 20, block=block,
               seed=62 + block)


def test_pool_ties_take_lower_blocks(ck, orc):
    zero = lambda g, n: np.zeros((n, 64), np.uint16)
    pool, sel = _pool_case(ck, orc, [9000, 2000], 64, 4, 64, nb=40, block=8, seed=66, key_fn=zero)
    assert np.array_equal(pool[0], np.arange(40)) and np.array_equal(sel[0], np.arange(64))

    def few(g, n):           # keys in {0, 1} on one coordinate: two block scores
        k = np.zeros((n, 64), np.float32)
        k[:, 5] = g.integers(0, 2, n) * (g.random(n) < 0.02)
        return _bf16_int(k)
    _pool_case(ck, orc, [12000, 800], 64, 4, 128, nb=64, block=8, seed=67, key_fn=few,
               head_w=np.ones((2, 4), np.float32))


def test_layer_group_pooled_matches_oracle(ck, orc):
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=4, entries=3000)
    pool = (80, 8)
    gc, hc = pair(w.batch, 3100, w.k_group, w.v_group, w.idx_dim)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(w.batch)],
                 [synth.cache_idx_keys(w, b) for b in range(w.batch)])
    st = synth.step_inputs(w, 0)
    W = synth.w_comp(w)
    B = w.batch
    grings = [dev(r) for r in st.swa_ring]
    layers = []
    for li, mode in enumerate(w.layers):
        layers.append(ck.Layer(mode=mode, q=dev(st.q[li]), swa=grings[li],
                               out=torch.empty(B, w.q_heads, 512, device="cuda"),
                               lse=torch.empty(B, w.q_heads, device="cuda"),
                               q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                               swa_row=dev(st.swa_row[li]),
                               idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda")
                               if mode != "reuse" else None))
    scale = 1 / math.sqrt(576)
    ck.layer_group_decode(gc, layers, dev(st.token), dev(W), dev(st.idx_row), w.topk, w.window, scale, pool=pool)
    hrings = [r.copy() for r in st.swa_ring]
    outs, lses, idxs = orc.layer_group_decode(hc, w.layers, st.token, st.idx_row, W, st.q, st.q_idx, hrings,
                                              st.swa_row, w.topk, scale, pool=pool)
    plain = orc.layer_group_decode(*_fresh(w, orc), w.topk, scale)[2]
    torch.cuda.synchronize()
    assert_cache_equal(gc, hc)
    assert "reindex" in w.layers
    for li, L in enumerate(layers):
        assert np.array_equal(host(grings[li]), hrings[li])
        if L.idx is not None:
            assert np.array_equal(host(L.idx), idxs[li]), f"layer {li} indices differ"
        assert attn_rel_err(host(L.out), outs[li]).max() <= TOL
    # the pool changed the reindex layer's selection (so the test sees it)
    ri = w.layers.index("reindex")
    assert not np.array_equal(idxs[ri], plain[ri])


def _fresh(w, orc):
    """The same step's oracle inputs on a fresh cache, without the pool."""
    hc = orc.Cache.empty(w.batch, 3100, 576, 64, w.k_group, w.v_group, w.idx_dim)
    ents = [synth.cache_entries(w, b) for b in range(w.batch)]
    keys = [synth.cache_idx_keys(w, b) for b in range(w.batch)]
    cu = np.concatenate([[0], np.cumsum([len(e) for e in ents])]).astype(np.int32)
    orc.kv_append(hc, np.concatenate(ents).astype(np.float32), cu, None, np.concatenate(keys))
    st = synth.step_inputs(w, 0)
    return (hc, w.layers, st.token, st.idx_row, synth.w_comp(w), st.q, st.q_idx,
            [r.copy() for r in st.swa_ring], st.swa_row)
