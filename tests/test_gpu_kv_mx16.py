"""GPU parity of the main-entry scale form with one E8M0 byte per 16 channels
[P2 四、"P4 main KV" (E2M1 codes, an 8-bit scale per 16 channels)]: the key
and value planes written bit for bit by both append modes, every code at
every scale read back exactly by the attention, and attention and the layer
group over such caches against the oracle."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import (TOL, assert_cache_equal, attn_rel_err, dev, host, load_entries,  # noqa: E402
                             lse_tol, pair)

MX16 = 1


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


def _hard_rows(g, n):
    """Rows that stress the 16-channel quantiser: heavy tails, zero and
    negative-zero groups, group maxima at and next to powers of two, values
    on and next to the E2M1 midpoints, scales at both ends of the E8M0 range."""
    rows = synth.student_t3(g, (n, 576))
    rows[0, :16] = 0.0                              # an all-zero group
    rows[0, 16:32] = -0.0
    rows[1, :16] = np.float32(4.0)                  # amax exactly 2^2
    rows[1, 16:32] = np.nextafter(np.float32(4.0), np.float32(0))
    rows[1, 32:48] = np.float32(2.0 ** -126)        # the smallest normal
    rows[1, 48:64] = np.float32(1e-40)              # subnormals: scale clamps at 2^-127
    rows[1, 64:80] = np.float32(3e38)               # near the largest float
    rows[1, 80:96] = -np.float32(7.9) * np.float32(2.0 ** 100)   # saturates to -6 x scale
    s = np.float32(0.5)                             # amax 3 -> scale 2^(1-2)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for i, m in enumerate(mids):
        x = np.float32(m * s)
        rows[2, 96 + 2 * i] = np.nextafter(x, np.float32(0))
        rows[2, 97 + 2 * i] = x
    rows[2, 110], rows[2, 111] = np.float32(3.0), np.float32(-1.5)
    rows[3] *= np.float32(1e30)
    return rows.astype(np.float32)


@pytest.mark.parametrize("v_group", [0, 16])
def test_append_mx16_entries_bitexact(ck, orc, v_group):
    g = np.random.default_rng(300 + v_group)
    gc, hc = pair(3, 700, 16, v_group, 64, k_format=MX16)
    lens = [5, 0, 650]
    rows = [_hard_rows(g, n) if n else np.zeros((0, 576), np.float32) for n in lens]
    keys = [synth.int_bf16(g, (n, 64)) for n in lens]
    load_entries(gc, hc, rows, keys)
    assert_cache_equal(gc, hc)
    rows2 = [synth.normal(g, (n, 576)) for n in (3, 2, 1)]
    keys2 = [synth.int_bf16(g, (n, 64)) for n in (3, 2, 1)]
    load_entries(gc, hc, rows2, keys2)
    assert_cache_equal(gc, hc)


@pytest.mark.parametrize("v_group", [0, 16])
def test_append_mx16_compressor_bitexact(ck, orc, v_group):
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    gc, hc = pair(3, 64, 16, v_group, 64, k_format=MX16)
    g = np.random.default_rng(310 + v_group)
    Wd = dev(W)
    for lens in [(7, 4, 1), (1, 0, 2), (3, 5, 1), (0, 1, 0), (40, 2, 3)]:
        toks = synth.normal(g, (sum(lens), 576))
        toks[::3] *= np.float32(20.0)
        irows = synth.int_bf16(g, (sum(lens), 64))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ck.kv_append_fp4(gc, dev(toks), dev(cu), Wd, dev(irows))
        orc.kv_append(hc, toks, cu, W, irows)
        assert_cache_equal(gc, hc)


@pytest.mark.parametrize("v_group", [0, 16])
def test_every_mx16_code_reads_back_exactly(ck, orc, v_group):
    # one cached entry per sequence, a zero query and no window: the softmax
    # puts weight 1 on that entry, so the output is its value row, bit for bit
    g = np.random.default_rng(320 + v_group)
    B, H = 2, 16
    gc, hc = pair(B, 8, 16, v_group, 64, k_format=MX16)
    kc = g.integers(0, 256, (B, 288), dtype=np.uint8)
    kc[0, :256] = np.arange(256)                    # every pair of codes
    ks = g.integers(100, 151, (B, 36), dtype=np.uint8)
    gc.k_codes[:, 0] = torch.from_numpy(kc).cuda()
    gc.k_scales[:, 0] = torch.from_numpy(ks).cuda()
    if v_group:
        vc = g.integers(0, 256, (B, 256), dtype=np.uint8)
        vs = g.integers(100, 151, (B, 32), dtype=np.uint8)
        gc.v_codes[:, 0] = torch.from_numpy(vc).cuda()
        gc.v_scales[:, 0] = torch.from_numpy(vs).cuda()
    gc.n_tokens.fill_(2)
    q = torch.zeros(B, H, 576, device="cuda")
    idx = torch.full((B, 16), -1, dtype=torch.int32, device="cuda")
    idx[:, 0] = 0
    ring = torch.zeros(B, 4, 576, dtype=torch.int16, device="cuda")
    out, lse = ck.sparse_attn_decode(gc, q, idx, ring, 0.04, swa_len=torch.zeros(B, dtype=torch.int32, device="cuda"))
    got = host(out)
    for b in range(B):
        want = (orc.dequantize_mx16(vc[b], vs[b], 512) if v_group
                else orc.dequantize_mx16(kc[b], ks[b], 576)[:512]).astype(np.float32)
        for h in range(H):
            assert np.array_equal(got[b, h], want), np.flatnonzero(got[b, h] != want)[:8]
    assert np.all(host(lse) == 0.0)


def _attn_case(ck, orc, v_group, lens, heads, k, nswa, seed, law="normal", fp8=False, window=128):
    g = np.random.default_rng(seed)
    B = len(lens)
    gc, hc = pair(B, max(lens) + 5, 16, v_group, 64, swa_format=int(fp8), k_format=MX16)
    ents = [synth.student_t3(g, (n, 576)) if law == "t3" else synth.normal(g, (n, 576)) for n in lens]
    load_entries(gc, hc, ents, [np.zeros((n, 64), np.uint16) for n in lens])
    q = synth.normal(g, (B, heads, 576))
    idx = np.full((B, k), -1, np.int32)
    for b, n in enumerate(lens):
        sel = np.sort(g.choice(n, size=min(k, n), replace=False)) if n else np.zeros(0, np.int64)
        idx[b, :len(sel)] = sel
    if fp8:
        ring = np.zeros((B, window, 576), np.uint8)
        rows = g.standard_normal((B * window, 576)).astype(np.float32) * 2
        orc.swa_append(ring, rows, (np.arange(B + 1) * window).astype(np.int32), np.full(B, window, np.int32))
        gring = torch.from_numpy(ring).cuda()
    else:
        ring = synth.normal_bf16_trunc(g, (B, window, 576))
        gring = dev(ring)
    sl = np.array(nswa, np.int32)
    scale = 1 / math.sqrt(576)
    out, lse = ck.sparse_attn_decode(gc, dev(q), dev(idx), gring, scale, swa_len=dev(sl))
    ref, rlse = orc.sparse_attn(hc, q, idx, ring, scale, swa_len=sl)
    out, lse = host(out), host(lse)
    err = attn_rel_err(out, ref)
    assert err.max() <= TOL, f"max rel err {err.max():.3e}"
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    tol = lse_tol(hc, q, idx, ring, sl, scale)
    d = np.abs(np.where(fin, lse, 0) - np.where(fin, rlse, 0))
    assert (d <= tol).all(), f"lse error {d.max():.3e} over its bound"
    print(f"max rel err {err.max():.2e}, lse max err / bound {(d / tol).max():.3f}")


@pytest.mark.parametrize("v_group,law,fp8", [(0, "t3", False), (16, "normal", False),
                                              (16, "t3", True), (0, "normal", True)])
def test_attention_mx16(ck, orc, v_group, law, fp8):
    _attn_case(ck, orc, v_group, lens=[700, 40, 513, 0], heads=32, k=512, nswa=[128, 5, 0, 77],
               seed=330 + v_group + int(fp8), law=law, fp8=fp8)


@pytest.mark.parametrize("v_group", [0, 16])
def test_attention_mx16_edge_cases(ck, orc, v_group):
    # no keys at all, only window keys, a single key, k not a multiple of 32
    _attn_case(ck, orc, v_group, lens=[0, 0, 1, 100], heads=16, k=37, nswa=[0, 3, 0, 128], seed=340 + v_group)


@pytest.mark.parametrize("batch,v_group", [(32, 0), (64, 16)])
def test_attention_mx16_mixed_splits(ck, orc, batch, v_group):
    g = np.random.default_rng(350 + batch)
    lens = [int(n) for n in g.integers(0, 900, batch)]
    lens[0], lens[1], lens[2] = 0, 511, 512
    nswa = [int(n) for n in g.integers(0, 129, batch)]
    nswa[0], nswa[3] = 0, 128
    _attn_case(ck, orc, v_group, lens=lens, heads=64, k=512, nswa=nswa, seed=360 + batch, law="t3")


@pytest.mark.parametrize("v_group,fp8", [(0, False), (16, True)])
def test_layer_group_mx16(ck, orc, v_group, fp8):
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=3, entries=2000, k_group=16, v_group=v_group)
    B = w.batch
    gc, hc = pair(B, 2100, 16, v_group, w.idx_dim, swa_format=int(fp8), k_format=MX16)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(B)],
                 [synth.cache_idx_keys(w, b) for b in range(B)])
    st = synth.step_inputs(w, 0)
    if fp8:
        rings = []
        for r in st.swa_ring:
            vals = (r.astype(np.uint32) << 16).view(np.float32)
            rings.append(np.vectorize(orc.e4m3_encode, otypes=[np.uint8])(vals))
        grings = [torch.from_numpy(r.copy()).cuda() for r in rings]
    else:
        rings = st.swa_ring
        grings = [dev(r) for r in rings]
    layers = [ck.Layer(mode=m, q=dev(st.q[li]), swa=grings[li],
                       out=torch.empty(B, w.q_heads, 512, device="cuda"),
                       lse=torch.empty(B, w.q_heads, device="cuda"),
                       q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                       swa_row=dev(st.swa_row[li]),
                       idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda") if m != "reuse" else None)
              for li, m in enumerate(w.layers)]
    W = synth.w_comp(w)
    scale = 1 / math.sqrt(576)
    ck.layer_group_decode(gc, layers, dev(st.token), dev(W), dev(st.idx_row), w.topk, w.window, scale)
    hrings = [r.copy() for r in rings]
    outs, lses, idxs = orc.layer_group_decode(hc, w.layers, st.token, st.idx_row, W, st.q, st.q_idx, hrings,
                                              st.swa_row, w.topk, scale)
    torch.cuda.synchronize()
    assert_cache_equal(gc, hc)
    for li, L in enumerate(layers):
        got = host(grings[li])
        assert np.array_equal(got.view(np.uint8), hrings[li].view(np.uint8)), f"layer {li} window ring differs"
        if L.idx is not None:
            assert np.array_equal(host(L.idx), idxs[li])
        assert attn_rel_err(host(L.out), outs[li]).max() <= TOL


def test_live_cache_rows_in_the_pages_formats(ck, orc):
    # a device cache in the pages' formats, filled by the append: the value
    # row (512 latent dims) is 288 B, the FP4 indexer key 72 B, and the
    # library's per-entry figure is the sum of every plane's row
    gc, hc = pair(2, 40, 16, 16, 128, idx_format=1, k_format=MX16)
    g = np.random.default_rng(370)
    load_entries(gc, hc, [synth.normal(g, (n, 576)) for n in (30, 7)], [synth.int_bf16(g, (n, 128)) for n in (30, 7)])
    assert_cache_equal(gc, hc)
    row = lambda t: t[0, 0].numel() * t.element_size()
    assert row(gc.v_codes) + row(gc.v_scales) == 288
    assert row(gc.idx_keys) + row(gc.idx_scales) == 72
    planes = (gc.k_codes, gc.k_scales, gc.v_codes, gc.v_scales, gc.idx_keys, gc.idx_scales)
    assert gc.entry_bytes() == sum(row(t) for t in planes) == 324 + 288 + 72
