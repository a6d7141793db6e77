"""Parity at the full sizes of the four large workloads, through the entry
point and launch configuration the bench times (one cskv_layer_group_decode
step over the whole batch).

Every sequence is checked against the oracle.  Sequences with a complete
host mirror are compared in everything the step produces: cache rows,
window rings, top-k indices, attention outputs and log-sum-exps.  Their
inputs come from the seeded generators in synth/, or are drawn on the GPU
with a seeded torch generator and copied to the host before anything of the
library touches them (the 64K x 32 batch: its 32 sequences of 32,768 entries
would take minutes to draw on the host).  The other sequences of the large
batches hold GPU-drawn cache entries and host-drawn indexer keys; an
index-only mirror holds their keys (the oracle's append copies bf16 key rows
verbatim, and zero entries quantise to zero codes and +0 scales, which is
what the mirror's untouched planes hold), so their top-k indices are compared
on every sequence.  The step's own inputs (new tokens, queries, windows) are
host-drawn for every sequence.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import TOL, attn_rel_err, dev, host, lse_tol  # noqa: E402


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
    """fp32 [n, dim] on the GPU with the workload's value law (a seeded torch generator)."""
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


class Mirrors:
    """Host mirrors of a device batch: `full` (sorted sequence ids) in one
    complete oracle cache, every other sequence in an index-only cache."""

    def __init__(self, orc, w, cap, full, batch):
        self.full = sorted(full)
        self.rest = [b for b in range(batch) if b not in set(full)]
        self.hf = orc.Cache.empty(len(self.full), cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim)
        self.hi = orc.Cache.empty(len(self.rest), cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim) \
            if self.rest else None
        self.pos_f = {b: i for i, b in enumerate(self.full)}
        self.pos_i = {b: i for i, b in enumerate(self.rest)}


def _build(ck, orc, w, cap, full, host_rows="synth"):
    """Device cache of the whole batch (entries mode, one sequence per call)
    and its mirrors.  Sequences in `full` take synth rows and keys
    (host_rows="synth") or GPU filler copied to the host ("filler"); the
    others take GPU filler entries and synth keys."""
    gc = ck.Cache.allocate(w.batch, cap, w.k_group, w.v_group, w.idx_dim)
    E = synth.entry_counts(w)
    m = Mirrors(orc, w, cap, full, w.batch)
    full_rows, full_keys = {}, {}
    for b in range(w.batch):
        n = int(E[b])
        if b in m.pos_f and host_rows == "synth":
            rows_h, keys_h = synth.cache_entries(w, b), synth.cache_idx_keys(w, b)
            rows, keys = dev(rows_h), dev(keys_h)
        elif b in m.pos_f:
            rows, keys = _filler_rows(w, b, n), _filler_keys(w, b, n)
            rows_h, keys_h = host(rows), host(keys)
        else:
            rows, keys_h = _filler_rows(w, b, n), synth.cache_idx_keys(w, b)
            keys = dev(keys_h)
        if b in m.pos_f:
            full_rows[b], full_keys[b] = rows_h, keys_h
        else:
            m.hi.idx_keys[m.pos_i[b], :n] = keys_h
            m.hi.n_tokens[m.pos_i[b]] = 2 * n
        if n:
            cu = np.zeros(w.batch + 1, np.int32)
            cu[b + 1:] = n
            ck.kv_append_fp4(gc, rows, dev(cu), None, keys)
    if m.full:
        lens = [len(full_keys[b]) for b in m.full]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        orc.kv_append(m.hf, np.concatenate([full_rows[b] for b in m.full]), cu, None,
                      np.concatenate([full_keys[b] for b in m.full]))
    torch.cuda.synchronize()
    return gc, m


def _sub(x, seqs):
    return None if x is None else np.ascontiguousarray(x[seqs])


def _step(ck, orc, w, gc, m, st, W_h, pool=None):
    """One layer-group step on the device, then the oracle on both mirrors
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
    nt = host(gc.n_tokens)

    for seqs, hc, whole in ((m.full, m.hf, True), (m.rest, m.hi, False)):
        if not seqs:
            continue
        rings = [_sub(r, seqs).copy() for r in st.swa_ring]
        outs, lses, idxs = orc.layer_group_decode(
            hc, w.layers, _sub(st.token, seqs), _sub(st.idx_row, seqs), W_h, [_sub(q, seqs) for q in st.q],
            [_sub(qi, seqs) for qi in st.q_idx], rings, [_sub(r, seqs) for r in st.swa_row], w.topk, scale,
            pool=pool)
        assert np.array_equal(nt[seqs], hc.n_tokens)
        for li, L in enumerate(layers):
            if L.idx is not None:
                got = host(L.idx)[seqs]
                bad = [seqs[i] for i in range(len(seqs)) if not np.array_equal(got[i], idxs[li][i])]
                assert not bad, f"layer {li}: indices differ for sequences {bad[:8]}"
        if not whole:
            continue
        for i, b in enumerate(seqs):
            e = int(hc.entries()[i])
            for name in ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "idx_scales"):
                gt = getattr(gc, name)
                if gt is None:
                    continue
                assert np.array_equal(host(gt[b, :e]).view(np.uint8), getattr(hc, name)[i, :e].view(np.uint8)), \
                    f"seq {b}: {name} differs"
        for li, L in enumerate(layers):
            assert np.array_equal(host(L.swa)[seqs].view(np.uint16), rings[li]), f"layer {li}: window"
            err = attn_rel_err(host(L.out)[seqs], outs[li])
            assert err.max() <= TOL, f"layer {li}: max rel err {err.max():.3e} (seq {seqs[int(err.max(1).argmax())]})"
            idx_l = idxs[li]
            tol = lse_tol(hc, _sub(st.q[li], seqs), idx_l, rings[li], hc.n_tokens, scale)
            d = np.abs(host(L.lse)[seqs] - lses[li])
            assert (d <= tol).all(), f"layer {li}: lse error {d.max():.3e} over its bound"
    # every output finite
    for li, L in enumerate(layers):
        assert np.isfinite(host(L.out)).all(), f"layer {li}: non-finite output"
    return layers


def test_full_decode_64k_b32(ck, orc):
    """32 sequences x 32,768 entries (64K tokens), group 64, Student-t(3):
    every sequence in full, and the indexer's fp32 scores of every entry of
    every sequence (out_scores) against the oracle's exact scores."""
    w = synth.WORKLOADS["decode_64k_b32"]
    gc, m = _build(ck, orc, w, w.entries + 8, full=set(range(w.batch)), host_rows="filler")
    st = synth.step_inputs(w, 0)
    _step(ck, orc, w, gc, m, st, synth.w_comp(w))
    # scores of the cache as the step left it, for the full layer's query
    scores = torch.full((w.batch, gc.capacity), float("nan"), device="cuda")
    ck.indexer_topk(gc, dev(st.q_idx[0]), w.topk, scores=scores)
    torch.cuda.synchronize()
    sc = host(scores)
    E = m.hf.entries()
    for b in range(w.batch):
        want = orc.indexer_scores(m.hf.idx_keys[b, :E[b]], st.q_idx[0][b])
        assert np.array_equal(sc[b, :E[b]].astype(np.float64), want), f"seq {b}: scores differ"
        assert np.isnan(sc[b, E[b]:]).all(), f"seq {b}: rows past the entries were written"


def test_full_decode_64k_b32_fp4_key_scores(ck, orc):
    """The pages' FP4 indexer keys at 32 x 32,768: the appended codes and
    E8M0 scales of every entry bit for bit against the oracle's quantisation
    of the same key rows, and the scan's fp32 score of every entry
    (out_scores) exactly against the oracle's scores over the keys it
    quantised and dequantised itself (integer-valued inputs: exact sums).
    The main entries are zero rows; the scores do not read them."""
    w = synth.WORKLOADS["decode_64k_b32"]
    n = w.entries
    gc = ck.Cache.allocate(w.batch, n + 8, w.k_group, w.v_group, w.idx_dim, idx_format=1)
    zeros = torch.zeros(n, w.dim, device="cuda")
    keys_h = []
    for b in range(w.batch):
        kb = _filler_keys(w, b, n)
        keys_h.append(host(kb))
        cu = np.zeros(w.batch + 1, np.int32)
        cu[b + 1:] = n
        ck.kv_append_fp4(gc, zeros, dev(cu), None, kb)
    st = synth.step_inputs(w, 0)
    scores = torch.full((w.batch, gc.capacity), float("nan"), device="cuda")
    ck.indexer_topk(gc, dev(st.q_idx[0]), w.topk, scores=scores)
    torch.cuda.synchronize()
    sc, codes_g, scales_g = host(scores), host(gc.idx_keys), host(gc.idx_scales)
    for b in range(w.batch):
        codes, scl = orc.quantize_mx16(keys_h[b].reshape(-1))
        assert np.array_equal(codes_g[b, :n].reshape(-1), codes), f"seq {b}: FP4 key codes differ"
        assert np.array_equal(scales_g[b, :n].reshape(-1), scl), f"seq {b}: E8M0 key scales differ"
        deq = orc.dequantize_mx16(codes, scl, n * w.idx_dim)
        kbits = (deq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).reshape(n, w.idx_dim)
        want = orc.indexer_scores(kbits, st.q_idx[0][b])
        assert np.array_equal(sc[b, :n].astype(np.float64), want), f"seq {b}: scores differ"
        assert np.isnan(sc[b, n:]).all(), f"seq {b}: rows past the entries were written"


def test_full_decode_1m_b1(ck, orc):
    """One sequence of 500,000 entries (1M tokens), group 32: the scan and the
    top-k at full length, every output against the oracle."""
    w = synth.WORKLOADS["decode_1m_b1"]
    gc, m = _build(ck, orc, w, w.entries + 8, full={0})
    _step(ck, orc, w, gc, m, synth.step_inputs(w, 0), synth.w_comp(w))


def test_full_group_128k_b64(ck, orc):
    """Full + Reindex + 3 Reuse on a shared cache, 64 sequences x 65,536
    entries: indices of both index-producing layers on every sequence,
    everything on a seeded sample."""
    w = synth.WORKLOADS["group_128k_b64"]
    gc, m = _build(ck, orc, w, w.entries + 8, full={0, 41, 63})
    _step(ck, orc, w, gc, m, synth.step_inputs(w, 0), synth.w_comp(w))


def test_full_group_128k_b64_pooled(ck, orc):
    """The same layer group with the hierarchical indexer at the pages' size:
    the full layer's pool of 2048 blocks of 8 entries, the reindex layer
    selecting inside it; indices on every sequence."""
    w = synth.WORKLOADS["group_128k_b64"]
    gc, m = _build(ck, orc, w, w.entries + 8, full={5, 62})
    st = synth.step_inputs(w, 0)
    layers = _step(ck, orc, w, gc, m, st, synth.w_comp(w), pool=(2048, 8))
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
    token on every other sequence in one append, then one decode step;
    indices on every sequence, everything on a seeded sample."""
    w = synth.WORKLOADS["mixed_ragged_b256"]
    E = synth.entry_counts(w)
    cap = int(E.max()) + w.chunk_tokens // 2 + 8
    full = {0, 100, 255}
    gc, m = _build(ck, orc, w, cap, full)
    W_h = synth.w_comp(w)
    lens = [w.chunk_tokens] + [1] * (w.batch - 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    toks = torch.empty(int(cu[-1]), w.dim, device="cuda")
    irows = torch.empty(int(cu[-1]), w.idx_dim, dtype=torch.int16, device="cuda")
    host_rows = {}
    for b in range(w.batch):
        n = lens[b]
        if b in full:
            t_h, i_h = synth.prefill_tokens(w, b, n), synth.prefill_idx_rows(w, b, n)
            toks[cu[b]:cu[b + 1]] = dev(t_h)
            irows[cu[b]:cu[b + 1]] = dev(i_h)
            host_rows[b] = (t_h, i_h)
        else:
            toks[cu[b]:cu[b + 1]] = _filler_rows(w, 10_000 + b, n)
            irows[cu[b]:cu[b + 1]] = _filler_keys(w, 10_000 + b, n)
    W = dev(W_h)
    ck.kv_append_fp4(gc, toks, dev(cu), W, irows, ws=ck.append_workspace(int(cu[-1]), W))
    fl = [lens[b] for b in m.full]
    orc.kv_append(m.hf, np.concatenate([host_rows[b][0] for b in m.full]),
                  np.concatenate([[0], np.cumsum(fl)]).astype(np.int32), W_h,
                  np.concatenate([host_rows[b][1] for b in m.full]))
    # the index-only mirror: one token each (its values reach no indexer key:
    # it waits as the pending half of the next pair)
    nr = len(m.rest)
    orc.kv_append(m.hi, np.zeros((nr, w.dim), np.float32), np.arange(nr + 1, dtype=np.int32), W_h,
                  np.zeros((nr, w.idx_dim), np.uint16))
    torch.cuda.synchronize()
    _step(ck, orc, w, gc, m, synth.step_inputs(w, 0), W_h)


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
    plan = synth.CSA2_PLAN
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
