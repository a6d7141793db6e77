"""GPU parity of the CED projection, of one-entry-per-token caches and of one
decode step of the pages' whole CSA2 layer plan (three encoder caches of
Full + 5 Reuse, the decoder cache read by Full + 3 Reuse and four Reindex +
3 Reuse groups) against the oracle."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import (TOL, assert_cache_equal, attn_rel_err, dev, host, load_entries,  # noqa: E402
                             lse_tol)


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


def _bits(x):
    a = np.ascontiguousarray(x, np.float32)
    b = (a.view(np.uint32) >> 16).astype(np.uint16)
    return b


def _int_bf16(g, shape, lo, hi, scale=1.0):
    """bf16 bits of integers in [lo, hi] times a power of two (exact)."""
    return _bits(g.integers(lo, hi + 1, shape).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("rows,d_model", [(1, 4096), (32, 4096), (100, 256), (130, 1024)])
def test_ced_project_exact_on_integer_inputs(ck, orc, rows, d_model):
    # small integers times 2^-10: every partial sum is representable, so the
    # MFMA result is exact in any order and equals the oracle bit for bit
    g = np.random.default_rng(600 + rows)
    h = _int_bf16(g, (rows, d_model), -8, 8)
    w = _int_bf16(g, (576, d_model), -4, 4, 2.0 ** -10)
    got = host(ck.ced_project(dev(h), dev(w)))
    assert np.array_equal(got, orc.ced_project(h, w))


def test_ced_project_general_inputs_within_bound(ck, orc):
    g = np.random.default_rng(610)
    rows, dm = 70, 1024
    h = _bits(g.standard_normal((rows, dm)))
    w = _bits(g.standard_normal((576, dm)) * 0.02)
    got = host(ck.ced_project(dev(h), dev(w))).astype(np.float64)
    ref = orc.ced_project(h, w).astype(np.float64)
    hv = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wv = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # fp32 sums of exact products: (d_model + 4) roundings of at most 2^-24
    # times the sum of magnitudes, plus the oracle's own final rounding
    bound = (dm + 4) * 2.0 ** -24 * (np.abs(hv) @ np.abs(wv).T) + 2.0 ** -24 * np.abs(ref)
    assert (np.abs(got - ref) <= bound).all()


def test_ratio_one_cache_append_and_attention(ck, orc):
    g = np.random.default_rng(620)
    lens = [300, 1, 0, 77]
    B = len(lens)
    gc = ck.Cache.allocate(B, 400, 32, 0, 64, ratio=1)
    hc = orc.Cache.empty(B, 400, 576, 64, 32, 0, 64, ratio=1)
    load_entries(gc, hc, [synth.normal(g, (n, 576)) for n in lens], [synth.int_bf16(g, (n, 64)) for n in lens])
    assert_cache_equal(gc, hc)
    # an odd number of entries is fine at ratio 1: one more each
    load_entries(gc, hc, [synth.normal(g, (1, 576)) for _ in lens], [synth.int_bf16(g, (1, 64)) for _ in lens])
    assert_cache_equal(gc, hc)
    assert host(gc.n_tokens).tolist() == [n + 1 for n in lens]
    # top-k and attention over the ratio-1 entries; window length = token count
    qi = synth.int_bf16(g, (B, 4, 64))
    idx = host(ck.indexer_topk(gc, dev(qi), 64))
    assert np.array_equal(idx, orc.indexer_topk(hc, qi, 64))
    q = synth.normal(g, (B, 16, 576))
    ring = synth.normal_bf16_trunc(g, (B, 128, 576))
    scale = 1 / math.sqrt(576)
    out, lse = ck.sparse_attn_decode(gc, dev(q), dev(idx), dev(ring), scale)
    ref, rlse = orc.sparse_attn(hc, q, idx, ring, scale)
    assert attn_rel_err(host(out), ref).max() <= TOL
    sl = np.minimum(hc.n_tokens, 128).astype(np.int32)
    assert (np.abs(host(lse) - rlse) <= lse_tol(hc, q, idx, ring, sl, scale)).all()


def _plan_case(ck, orc, g, B, enc_entries, dec_entries, heads, iheads, dm, pool):
    """Device and host caches and step inputs for every group of the plan."""
    plan = synth.CSA2_PLAN
    dev_groups, host_groups = [], []
    W = (g.standard_normal((576, 1152)) * 0.02).astype(np.float32)
    for name, ratio, modes in plan:
        n = dec_entries if ratio == 1 else enc_entries
        gc = ck.Cache.allocate(B, n + 8, 64, 0, 64, ratio=ratio)
        hc = orc.Cache.empty(B, n + 8, 576, 64, 64, 0, 64, ratio=ratio)
        load_entries(gc, hc, [synth.student_t3(g, (n, 576)) for _ in range(B)],
                     [synth.int_bf16(g, (n, 64)) for _ in range(B)])
        L = len(modes)
        q = [synth.normal(g, (B, heads, 576)) for _ in range(L)]
        qi = [None if m == "reuse" else synth.int_bf16(g, (B, iheads, 64)) for m in modes]
        rings = [synth.normal_bf16_trunc(g, (B, 128, 576)) for _ in range(L)]
        rows = [synth.normal(g, (B, 576)) for _ in range(L)]
        irow = synth.int_bf16(g, (B, 64))
        hg = dict(cache=hc, modes=modes, q=q, q_idx=qi, rings=[r.copy() for r in rings], swa_rows=rows,
                  idx_row=irow)
        layers = [ck.Layer(mode=m, q=dev(q[i]), swa=dev(rings[i]), swa_row=dev(rows[i]),
                           q_idx=None if qi[i] is None else dev(qi[i]),
                           out=torch.empty(B, heads, 512, device="cuda"), lse=torch.empty(B, heads, device="cuda"),
                           idx=torch.empty(B, 512, dtype=torch.int32, device="cuda") if m != "reuse" else None)
                  for i, m in enumerate(modes)]
        dgrp = ck.Group(cache=gc, layers=layers, new_idx_rows=dev(irow),
                        pool=pool if "reindex" in modes else None)
        if ratio == 1:
            h = _int_bf16(g, (B, dm), -8, 8)
            wc = _int_bf16(g, (576, dm), -4, 4, 2.0 ** -10)
            hg.update(ced_h=h, ced_w=wc)
            dgrp.ced_h, dgrp.ced_w = dev(h), dev(wc)
        else:
            tok = synth.normal(g, (B, 576))
            hg.update(token=tok, w_comp=W)
            dgrp.new_tokens, dgrp.w_comp = dev(tok), dev(W)
        dev_groups.append(dgrp)
        host_groups.append(hg)
    return dev_groups, host_groups


@pytest.mark.parametrize("pool", [None, (128, 8)])
def test_model_decode_whole_plan(ck, orc, pool):
    g = np.random.default_rng(630 + (pool is not None))
    B, heads = 2, 16
    dev_groups, host_groups = _plan_case(ck, orc, g, B, enc_entries=1500, dec_entries=3001, heads=heads,
                                         iheads=4, dm=512, pool=pool)
    scale = 1 / math.sqrt(576)
    ck.model_decode(dev_groups, 512, 128, scale)
    res = orc.model_decode(host_groups, 512, scale, pool=pool)
    torch.cuda.synchronize()
    for gi, (dg, hg, (outs, lses, idxs)) in enumerate(zip(dev_groups, host_groups, res)):
        assert_cache_equal(dg.cache, hg["cache"])
        for li, L in enumerate(dg.layers):
            assert np.array_equal(host(L.swa), hg["rings"][li]), f"group {gi} layer {li}: window ring"
            if L.idx is not None:
                assert np.array_equal(host(L.idx), idxs[li]), f"group {gi} layer {li}: indices"
            err = attn_rel_err(host(L.out), outs[li])
            assert err.max() <= TOL, f"group {gi} layer {li}: max rel err {err.max():.3e}"
            sl = np.minimum(hg["cache"].n_tokens, 128).astype(np.int32)
            tol = lse_tol(hg["cache"], hg["q"][li], idxs[li], hg["rings"][li], sl, scale)
            assert (np.abs(host(L.lse) - lses[li]) <= tol).all(), f"group {gi} layer {li}: lse"
    # the decoder cache took one entry per token, the encoders one per pair
    assert host(dev_groups[3].cache.n_tokens).tolist() == [3002] * B
    assert host(dev_groups[0].cache.n_tokens).tolist() == [3001] * B
