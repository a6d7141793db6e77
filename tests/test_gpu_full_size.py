"""Parity at the full sizes of the four large workloads, through the entry
point and launch configuration the bench times (one cskv_layer_group_decode
step over the whole batch).

The oracle recomputes sampled sequences one by one: their cache rows, step
inputs and expected results come from the seeded generators in synth/.  The
other sequences of the batch hold filler of the same value law drawn on the
GPU with a seeded torch generator; they go through the same launches and are
checked by properties that hold at any size (selected indices ascending,
distinct and in range; outputs and log-sum-exps finite).  Sequences are
independent, so the filler cannot change a sampled sequence's results.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import TOL, attn_rel_err, dev, host  # noqa: E402


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


def _filler_rows(w, b, n):
    """fp32 [n, dim] on the GPU with the workload's value law (not the oracle's data)."""
    g = torch.Generator(device="cuda").manual_seed(1_000_003 * (w.seed + 1) + b)
    z = torch.randn(n, w.dim, generator=g, device="cuda")
    if w.entry_law == "t3":
        chi = torch.randn(n, w.dim, 3, generator=g, device="cuda").square().sum(-1)
        z = z / torch.sqrt(chi / 3)
    elif w.entry_law == "outliers":
        z = torch.where(torch.rand(n, w.dim, generator=g, device="cuda") < 0.01, z * 20, z)
    return z.contiguous()


def _filler_keys(w, b, n):
    g = torch.Generator(device="cuda").manual_seed(2_000_003 * (w.seed + 1) + b)
    v = torch.randint(-8, 9, (n, w.idx_dim), generator=g, device="cuda").to(torch.bfloat16)
    return v.view(torch.int16).contiguous()


def _build(ck, orc, w, cap, sampled):
    """Device cache of the whole batch (entries mode, one sequence per call)
    and a one-sequence host mirror for every sampled sequence."""
    gc = ck.Cache.allocate(w.batch, cap, w.k_group, w.v_group, w.idx_dim)
    E = synth.entry_counts(w)
    mirrors = {}
    for b in range(w.batch):
        n = int(E[b])
        if n == 0:
            continue
        if b in sampled:
            rows_h, keys_h = synth.cache_entries(w, b), synth.cache_idx_keys(w, b)
            rows, keys = dev(rows_h), dev(keys_h)
            hc = orc.Cache.empty(1, cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim)
            orc.kv_append(hc, rows_h, np.array([0, n], np.int32), None, keys_h)
            mirrors[b] = hc
        else:
            rows, keys = _filler_rows(w, b, n), _filler_keys(w, b, n)
        cu = np.zeros(w.batch + 1, np.int32)
        cu[b + 1:] = n
        ck.kv_append_fp4(gc, rows, dev(cu), None, keys)
    for b in sampled:
        if b not in mirrors:
            mirrors[b] = orc.Cache.empty(1, cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim)
    torch.cuda.synchronize()
    return gc, mirrors


def _step(ck, orc, w, gc, mirrors, st, W_h, pool=None):
    """One layer-group step on the device, then the oracle per sampled sequence
    (pool: the hierarchical indexer's (pool_blocks, pool_block))."""
    B = w.batch
    scale = 1 / math.sqrt(w.dim)
    layers = []
    for li, mode in enumerate(w.layers):
        layers.append(ck.Layer(mode=mode, q=dev(st.q[li]), swa=dev(st.swa_ring[li]),
                               q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                               swa_row=dev(st.swa_row[li]),
                               out=torch.empty(B, w.q_heads, w.vdim, device="cuda"),
                               lse=torch.empty(B, w.q_heads, device="cuda"),
                               idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda")
                               if mode != "reuse" else None))
    ws = ck.workspace(gc, w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window, pool=pool)
    ck.layer_group_decode(gc, layers, dev(st.token), dev(W_h), dev(st.idx_row), w.topk, w.window,
                          scale, ws=ws, pool=pool)
    torch.cuda.synchronize()
    assert int(host(gc.status)[0]) == 0

    # properties of every sequence
    E = np.clip(host(gc.n_tokens).astype(np.int64) // 2, 0, gc.capacity)
    for li, L in enumerate(layers):
        assert np.isfinite(host(L.out)).all(), f"layer {li}: non-finite output"
        lse = host(L.lse)
        assert np.isfinite(lse[E > 0]).all(), f"layer {li}: non-finite lse"
        if L.idx is not None:
            ix = host(L.idx)
            for b in range(B):
                m = min(int(E[b]), w.topk)
                row = ix[b]
                assert np.all(row[m:] == -1) and np.all(row[:m] >= 0) and np.all(row[:m] < E[b])
                assert np.all(np.diff(row[:m]) > 0), f"layer {li} seq {b}: indices not ascending"

    # the oracle on each sampled sequence
    for b, hc in mirrors.items():
        sl = slice(b, b + 1)
        rings = [r[sl].copy() for r in st.swa_ring]
        outs, lses, idxs = orc.layer_group_decode(
            hc, w.layers, st.token[sl], st.idx_row[sl], W_h, [q[sl] for q in st.q],
            [None if qi is None else qi[sl] for qi in st.q_idx], rings,
            [r[sl] for r in st.swa_row], w.topk, scale, pool=pool)
        e = int(hc.entries()[0])
        assert int(host(gc.n_tokens)[b]) == int(hc.n_tokens[0])
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "idx_scales"):
            gt = getattr(gc, name)
            if gt is None:
                continue
            assert np.array_equal(host(gt[b, :e]).view(np.uint8), getattr(hc, name)[0, :e].view(np.uint8)), \
                f"seq {b}: {name} differs"
        for li, L in enumerate(layers):
            assert np.array_equal(host(L.swa[sl]).view(np.uint16), rings[li]), f"seq {b} layer {li}: window"
            if L.idx is not None:
                assert np.array_equal(host(L.idx[sl]), idxs[li]), f"seq {b} layer {li}: indices differ"
            err = attn_rel_err(host(L.out[sl]), outs[li])
            assert err.max() <= TOL, f"seq {b} layer {li}: max rel err {err.max():.3e}"
            assert np.abs(host(L.lse[sl]) - lses[li]).max() < 1e-4
    return layers


def test_full_decode_64k_b32(ck, orc):
    """32 sequences x 32,768 entries (64K tokens), group 64, Student-t(3)."""
    w = synth.WORKLOADS["decode_64k_b32"]
    gc, mirrors = _build(ck, orc, w, w.entries + 8, sampled={0, 17, 31})
    _step(ck, orc, w, gc, mirrors, synth.step_inputs(w, 0), synth.w_comp(w))


def test_full_decode_1m_b1(ck, orc):
    """One sequence of 500,000 entries (1M tokens), group 32: the scan and the
    top-k at full length, every output against the oracle."""
    w = synth.WORKLOADS["decode_1m_b1"]
    gc, mirrors = _build(ck, orc, w, w.entries + 8, sampled={0})
    _step(ck, orc, w, gc, mirrors, synth.step_inputs(w, 0), synth.w_comp(w))


def test_full_group_128k_b64(ck, orc):
    """Full + Reindex + 3 Reuse on a shared cache, 64 sequences x 65,536 entries."""
    w = synth.WORKLOADS["group_128k_b64"]
    gc, mirrors = _build(ck, orc, w, w.entries + 8, sampled={0, 41, 63})
    _step(ck, orc, w, gc, mirrors, synth.step_inputs(w, 0), synth.w_comp(w))


def test_full_group_128k_b64_pooled(ck, orc):
    """The same layer group with the hierarchical indexer at the pages' size:
    the full layer's pool of 2048 blocks of 8 entries, the reindex layer
    selecting inside it."""
    w = synth.WORKLOADS["group_128k_b64"]
    gc, mirrors = _build(ck, orc, w, w.entries + 8, sampled={5, 62})
    st = synth.step_inputs(w, 0)
    layers = _step(ck, orc, w, gc, mirrors, st, synth.w_comp(w), pool=(2048, 8))
    # every sequence: the reindex layer's entries lie in the full layer's pool,
    # rebuilt here from the same cache state and the full layer's query
    fi, ri = w.layers.index("full"), w.layers.index("reindex")
    idx, pool = ck.indexer_topk_pool(gc, dev(st.q_idx[fi]), w.topk, 2048, 8)
    torch.cuda.synchronize()
    assert torch.equal(idx, layers[fi].idx)
    pool, sel = host(pool), host(layers[ri].idx)
    for b in range(w.batch):
        s = sel[b][sel[b] >= 0]
        assert len(s) == w.topk and set((s // 8).tolist()) <= set(pool[b].tolist()), f"seq {b}"


def test_full_mixed_ragged_b256(ck, orc):
    """256 ragged sequences (2K-32K tokens) with split K (g32) / V (g128) planes:
    a 16,384-token prefill chunk through the compressor on sequence 0 and one
    token on every other sequence in one append, then one decode step."""
    w = synth.WORKLOADS["mixed_ragged_b256"]
    E = synth.entry_counts(w)
    cap = int(E.max()) + w.chunk_tokens // 2 + 8
    sampled = {0, 100, 255}
    gc, mirrors = _build(ck, orc, w, cap, sampled)
    W_h = synth.w_comp(w)
    lens = [w.chunk_tokens] + [1] * (w.batch - 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    toks = torch.empty(int(cu[-1]), w.dim, device="cuda")
    irows = torch.empty(int(cu[-1]), w.idx_dim, dtype=torch.int16, device="cuda")
    host_rows = {}
    for b in range(w.batch):
        n = lens[b]
        if b in sampled:
            t_h, i_h = synth.prefill_tokens(w, b, n), synth.prefill_idx_rows(w, b, n)
            toks[cu[b]:cu[b + 1]] = dev(t_h)
            irows[cu[b]:cu[b + 1]] = dev(i_h)
            host_rows[b] = (t_h, i_h)
        else:
            toks[cu[b]:cu[b + 1]] = _filler_rows(w, 10_000 + b, n)
            irows[cu[b]:cu[b + 1]] = _filler_keys(w, 10_000 + b, n)
    W = dev(W_h)
    ck.kv_append_fp4(gc, toks, dev(cu), W, irows, ws=ck.append_workspace(int(cu[-1]), W))
    for b, (t_h, i_h) in host_rows.items():
        orc.kv_append(mirrors[b], t_h, np.array([0, len(t_h)], np.int32), W_h, i_h)
    torch.cuda.synchronize()
    _step(ck, orc, w, gc, mirrors, synth.step_inputs(w, 0), W_h)


def test_full_model_plan_64k_b32(ck, orc):
    """The pages' whole layer plan at the size bench.py times for it: 32
    sequences x 64K tokens, three encoder caches of 32,768 entries (2->1,
    Full + 5 Reuse each) and the decoder cache of 65,536 one-per-token
    entries fed by the CED projection (Full + 3 Reuse, then four Reindex +
    3 Reuse), one cskv_model_decode step.  Sequence 5 is drawn on the host
    in every cache and checked against the oracle (cache rows, windows,
    indices, outputs); the others are GPU filler checked by invariants."""
    B, T, kg, Di, Hi, Hq, K, W, dm = 32, 65536, 64, 128, 64, 64, 512, 128, 512
    sb = 5
    plan = orc.csa2_plan()
    g = np.random.default_rng(640)
    scale = 1 / math.sqrt(576)
    Wc = (g.standard_normal((576, 1152)) * 0.02).astype(np.float32)
    dev_groups, host_groups = [], []
    for gi, (name, ratio, modes) in enumerate(plan):
        E = T // ratio
        gc = ck.Cache.allocate(B, E + 8, kg, 0, Di, ratio=ratio)
        hc = orc.Cache.empty(1, E + 8, 576, 64, kg, 0, Di, ratio=ratio)
        for b in range(B):
            cu = np.zeros(B + 1, np.int32)
            cu[b + 1:] = E
            if b == sb:
                rows_h, keys_h = synth.student_t3(g, (E, 576)), synth.int_bf16(g, (E, Di))
                orc.kv_append(hc, rows_h, np.array([0, E], np.int32), None, keys_h)
                rows, keys = dev(rows_h), dev(keys_h)
            else:
                fw = synth.scaled(synth.WORKLOADS["decode_64k_b32"], seed=50 + gi)
                rows, keys = _filler_rows(fw, b, E), _filler_keys(fw, b, E)
            ck.kv_append_fp4(gc, rows, dev(cu), None, keys)
        L = len(modes)
        q = [synth.normal(g, (B, Hq, 576)) for _ in range(L)]
        qi = [None if m == "reuse" else synth.int_bf16(g, (B, Hi, Di)) for m in modes]
        rings = [synth.normal_bf16_trunc(g, (B, W, 576)) for _ in range(L)]
        srows = [synth.normal(g, (B, 576)) for _ in range(L)]
        irow = synth.int_bf16(g, (B, Di))
        layers = [ck.Layer(mode=m, q=dev(q[i]), swa=dev(rings[i]), swa_row=dev(srows[i]),
                           q_idx=None if qi[i] is None else dev(qi[i]),
                           out=torch.empty(B, Hq, 512, device="cuda"), lse=torch.empty(B, Hq, device="cuda"),
                           idx=torch.empty(B, K, dtype=torch.int32, device="cuda") if m != "reuse" else None)
                  for i, m in enumerate(modes)]
        dgrp = ck.Group(cache=gc, layers=layers, new_idx_rows=dev(irow))
        sl = slice(sb, sb + 1)
        hg = dict(cache=hc, modes=modes, q=[x[sl] for x in q], q_idx=[None if x is None else x[sl] for x in qi],
                  rings=[r[sl].copy() for r in rings], swa_rows=[r[sl] for r in srows], idx_row=irow[sl])
        if ratio == 1:
            h = synth.int_bf16(g, (B, dm))
            wc = synth.int_bf16(g, (576, dm))
            dgrp.ced_h, dgrp.ced_w = dev(h), dev(wc)
            hg.update(ced_h=h[sl], ced_w=wc)
        else:
            tok = synth.normal(g, (B, 576))
            dgrp.new_tokens, dgrp.w_comp = dev(tok), dev(Wc)
            hg.update(token=tok[sl], w_comp=Wc)
        dev_groups.append(dgrp)
        host_groups.append(hg)
    ck.model_decode(dev_groups, K, W, scale)
    res = orc.model_decode(host_groups, K, scale)
    torch.cuda.synchronize()
    for gi, (dg, hg, (outs, lses, idxs)) in enumerate(zip(dev_groups, host_groups, res)):
        gc, hc = dg.cache, hg["cache"]
        assert int(host(gc.status)[0]) == 0
        nt = host(gc.n_tokens)
        assert int(nt[sb]) == int(hc.n_tokens[0])
        e = int(hc.entries()[0])
        for name in ("k_codes", "k_scales", "idx_keys"):
            assert np.array_equal(host(getattr(gc, name)[sb, :e]).view(np.uint8),
                                  getattr(hc, name)[0, :e].view(np.uint8)), f"group {gi}: {name} differs"
        E = np.clip(nt.astype(np.int64) // gc.ratio, 0, gc.capacity)
        for li, L in enumerate(dg.layers):
            assert np.isfinite(host(L.out)).all() and np.isfinite(host(L.lse)).all(), f"group {gi} layer {li}"
            assert np.array_equal(host(L.swa[sb:sb + 1]).view(np.uint16), hg["rings"][li]), \
                f"group {gi} layer {li}: window"
            if L.idx is not None:
                ix = host(L.idx)
                for b in range(B):
                    m = min(int(E[b]), K)
                    assert np.all(ix[b, m:] == -1) and np.all(np.diff(ix[b, :m]) > 0) and ix[b, m - 1] < E[b]
                assert np.array_equal(ix[sb:sb + 1], idxs[li]), f"group {gi} layer {li}: indices differ"
            err = attn_rel_err(host(L.out[sb:sb + 1]), outs[li])
            assert err.max() <= TOL, f"group {gi} layer {li}: max rel err {err.max():.3e}"
            assert np.abs(host(L.lse[sb:sb + 1]) - lses[li]).max() < 1e-4, f"group {gi} layer {li}: lse"
