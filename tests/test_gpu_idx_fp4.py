"""GPU parity of the FP4 indexer-key format [P2 四、"890 字节是怎么算出来的"
(a 128-dim indexer key in FP4 takes 72 B); P2 四、"P4 main KV" (E2M1, one
8-bit scale per 16 channels)]: the append's codes and E8M0 scales, the FP4
scan's top-k, the candidate pool and the layer group, each bit for bit
against the oracle (integer-valued indexer inputs: every score is exact).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import TOL, assert_cache_equal, attn_rel_err, dev, host, load_entries, pair  # noqa: E402

FP4 = 1


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


def _cache(lens, idx_dim, seed, key_fn=None, cap=None):
    g = np.random.default_rng(seed)
    cap = cap or max(max(lens), 1) + 3
    gc, hc = pair(len(lens), cap, 64, 0, idx_dim, idx_format=FP4)
    keys = [key_fn(g, n) if key_fn else synth.int_bf16(g, (n, idx_dim)) for n in lens]
    load_entries(gc, hc, [np.zeros((n, 576), np.float32) for n in lens], keys)
    return g, gc, hc


def test_append_writes_fp4_keys(ck, orc):
    # entries mode, then the compressor with pending tokens, ragged
    g, gc, hc = _cache([0, 17, 300, 1], 128, seed=70)
    assert_cache_equal(gc, hc)
    # values spanning many binades and zero groups
    def wide(g, n):
        x = g.standard_normal((n, 64)) * 2.0 ** g.integers(-20, 20, (n, 1))
        x[:, 16:32] = 0
        return _bf16_int(x.astype(np.float32))
    g, gc, hc = _cache([40, 3], 64, seed=71, key_fn=wide)
    assert_cache_equal(gc, hc)
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    toks = g.standard_normal((7, 576)).astype(np.float32)
    irows = synth.int_bf16(g, (7, 64))
    cu = np.array([0, 4, 7], np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows))
    orc.kv_append(hc, toks, cu, W, irows)
    assert_cache_equal(gc, hc)


def _topk_case(ck, orc, lens, idx_dim, heads, k, seed, key_fn=None, head_w=None):
    g, gc, hc = _cache(lens, idx_dim, seed, key_fn)
    q = synth.int_bf16(g, (len(lens), heads, idx_dim))
    hw = None if head_w is None else dev(head_w)
    got = host(ck.indexer_topk(gc, dev(q), k, head_w=hw))
    want = orc.indexer_topk(hc, q, k, head_w)
    for b in range(len(lens)):
        assert np.array_equal(got[b], want[b]), (b, lens[b], np.flatnonzero(got[b] != want[b])[:8])
    return gc, hc, q


@pytest.mark.parametrize("idx_dim,heads", [(128, 64), (64, 4), (128, 17)])
def test_fp4_topk_exact_ragged(ck, orc, idx_dim, heads):
    lens = [0, 1, 511, 513, 777, 4096 + 37, 20000, 40003]
    _topk_case(ck, orc, lens, idx_dim, heads, 512, seed=72 + idx_dim + heads)


def test_fp4_topk_ties_and_weights(ck, orc):
    zero = lambda g, n: np.zeros((n, 128), np.uint16)
    _topk_case(ck, orc, [9000, 600], 128, 64, 512, seed=75, key_fn=zero)
    hw = synth.head_weights_int(6, 3, 64)
    _topk_case(ck, orc, [3000, 64, 9000], 128, 64, 512, seed=76, head_w=hw)


def test_fp4_pool_and_topk_in_pool(ck, orc):
    g, gc, hc = _cache([70001, 20000, 5, 16385], 128, seed=77)
    q = synth.int_bf16(g, (4, 64, 128))
    q2 = synth.int_bf16(g, (4, 64, 128))
    idx, pool = ck.indexer_topk_pool(gc, dev(q), 512, 2048, 8)
    assert np.array_equal(host(pool), orc.indexer_pool(hc, q, 8, 2048))
    assert np.array_equal(host(idx), orc.indexer_topk(hc, q, 512))
    sel = ck.indexer_topk_in_pool(gc, dev(q2), 512, pool, 8)
    assert np.array_equal(host(sel), orc.indexer_topk_in_pool(hc, q2, host(pool), 8, 512))


def test_fp4_layer_group_matches_oracle(ck, orc):
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=3, entries=2500)
    gc, hc = pair(w.batch, 2600, w.k_group, w.v_group, w.idx_dim, idx_format=FP4)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(w.batch)],
                 [synth.cache_idx_keys(w, b) for b in range(w.batch)])
    st = synth.step_inputs(w, 0)
    W = synth.w_comp(w)
    B = w.batch
    grings = [dev(r) for r in st.swa_ring]
    layers = [ck.Layer(mode=m, q=dev(st.q[li]), swa=grings[li],
                       out=torch.empty(B, w.q_heads, 512, device="cuda"),
                       lse=torch.empty(B, w.q_heads, device="cuda"),
                       q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                       swa_row=dev(st.swa_row[li]),
                       idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda") if m != "reuse" else None)
              for li, m in enumerate(w.layers)]
    scale = 1 / math.sqrt(576)
    pool = (80, 8)
    ck.layer_group_decode(gc, layers, dev(st.token), dev(W), dev(st.idx_row), w.topk, w.window, scale, pool=pool)
    hrings = [r.copy() for r in st.swa_ring]
    outs, lses, idxs = orc.layer_group_decode(hc, w.layers, st.token, st.idx_row, W, st.q, st.q_idx, hrings,
                                              st.swa_row, w.topk, scale, pool=pool)
    torch.cuda.synchronize()
    assert_cache_equal(gc, hc)
    for li, L in enumerate(layers):
        if L.idx is not None:
            assert np.array_equal(host(L.idx), idxs[li]), f"layer {li} indices differ"
        assert attn_rel_err(host(L.out), outs[li]).max() <= TOL
