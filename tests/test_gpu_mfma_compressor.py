"""The matrix-core compressor of large appends (cskv_kv_append_fp4_mfma).

Its entries are a product with bf16 high/low splits and fp32 accumulation in
an unspecified order, so they are held to a bound instead of bit equality:
per output, |e - sum_j W_rj u_j| <= 2.53e-4 * sum_j |W_rj u_j| (the header's
derivation: 3.02 * 2^-16 for the dropped split parts, 3455 * 2^-24 for an
fp32 sum of 3456 terms in any order).  The oracle's fp32 entry is itself
within 24 * 2^-24 of that sum (its fixed order), so the test allows
2.53e-4 + 1.5e-6 of sum_j |W_rj u_j| between the two, computed in fp64 for
every element.  The quantiser after it must be exact: the codes and scales
are the oracle's quantisation of the kernel's own entry rows, which the call
leaves in its workspace.  Pending tokens, token counts, indexer keys and the
status follow the exact path bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import assert_cache_equal, dev, host, load_entries, pair  # noqa: E402

BOUND = 2.53e-4 + 1.5e-6


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


def _completed(n_tokens, lens, pending, toks):
    """(input row, sequence, entry, x_even, x_odd) of every row that completes
    an entry, from the token counts before the append (host side)."""
    out = []
    row = 0
    for b, m in enumerate(lens):
        p = int(n_tokens[b])
        for q in range(m):
            pos = p + q
            if pos % 2 == 1:
                xe = toks[row + q - 1] if q > 0 else pending[b]
                out.append((row + q, b, pos // 2, xe, toks[row + q]))
        row += m
    return out


def _check_mfma_append(ck, orc, w, lens, k_group, v_group, seed_salt=0, sample=None, cached=True):
    """cached: the sequences first hold their seeded workload entries; else
    the cache starts empty."""
    E = synth.entry_counts(w) if cached else np.zeros(w.batch, np.int64)
    cap = int(E.max()) + max(lens) // 2 + 8
    gc, hc = pair(w.batch, cap, k_group, v_group, w.idx_dim)
    if cached:
        load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(w.batch)],
                     [synth.cache_idx_keys(w, b) for b in range(w.batch)])
    W = synth.w_comp(w)
    # a first append leaves odd token counts (pending tokens) on some sequences
    first = [1 if b % 2 else 0 for b in range(w.batch)]
    t1 = np.concatenate([synth.prefill_tokens(w, b + 50, n) for b, n in enumerate(first)])
    r1 = np.concatenate([synth.prefill_idx_rows(w, b + 50, n) for b, n in enumerate(first)])
    cu1 = np.concatenate([[0], np.cumsum(first)]).astype(np.int32)
    ck.kv_append_fp4(gc, dev(t1), dev(cu1), dev(W), dev(r1))
    orc.kv_append(hc, t1, cu1, W, r1)
    assert_cache_equal(gc, hc)
    nt0, pend0 = hc.n_tokens.copy(), hc.pending.copy()

    toks = np.concatenate([synth.prefill_tokens(w, b + seed_salt, n) for b, n in enumerate(lens)])
    irows = np.concatenate([synth.prefill_idx_rows(w, b + seed_salt, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = len(toks)
    assert n >= 512, "the matrix-core path serves appends of 512 rows or more"
    ws = ck.append_workspace(n, dev(W), "cuda")
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows), ws=ws, mfma=True)
    orc.kv_append(hc, toks, cu, W, irows)        # the exact path: counts, pending, keys, status
    torch.cuda.synchronize()
    ent = host(ws).view(np.float32)[: n * w.dim].reshape(n, w.dim)

    # counts, pending tokens, status and indexer keys as on the exact path
    assert np.array_equal(host(gc.n_tokens), hc.n_tokens)
    assert int(host(gc.status)[0]) == int(hc.status[0])
    for b in range(w.batch):
        if hc.n_tokens[b] % 2 == 1:
            assert np.array_equal(host(gc.pending[b]), hc.pending[b]), f"pending differs, seq {b}"
    assert np.array_equal(host(gc.idx_keys).view(np.uint16), hc.idx_keys.view(np.uint16))

    done = _completed(nt0, lens, pend0, toks)
    if sample is not None:
        done = done[::max(1, len(done) // sample)]
    kc, ks = host(gc.k_codes), host(gc.k_scales)
    vc = host(gc.v_codes) if gc.v_codes is not None else None
    vs = host(gc.v_scales) if gc.v_scales is not None else None
    Wd = W.astype(np.float64)
    worst = 0.0
    for r, b, e, xe, xo in done:
        u = np.concatenate([xe, xo]).astype(np.float64)
        ref = orc.compress_pair(W, xe, xo).astype(np.float64)
        mag = np.abs(Wd) @ np.abs(u)
        got = ent[r].astype(np.float64)
        err = np.abs(got - ref)
        ok = err <= BOUND * mag
        assert ok.all(), f"row {r}: |e - oracle| {err[~ok].max():.3e} over the bound"
        worst = max(worst, float((err / np.where(mag > 0, mag, 1)).max()))
        # the quantiser applied to the kernel's own entry, exactly
        codes, scales = orc.quantize_row(ent[r], k_group)
        assert np.array_equal(kc[b, e], codes) and np.array_equal(ks[b, e].view(np.uint32), scales.view(np.uint32)), \
            f"row {r}: key-plane codes or scales differ from the quantisation of its entry"
        if vc is not None:
            codes, scales = orc.quantize_row(ent[r][:512], v_group)
            assert np.array_equal(vc[b, e], codes) and np.array_equal(vs[b, e].view(np.uint32),
                                                                       scales.view(np.uint32))
    return worst, len(done)


@pytest.mark.parametrize("k_group,v_group", [(32, 0), (64, 0), (32, 128)])
def test_mfma_compressor_within_bound(ck, orc, k_group, v_group):
    """A ragged append of 1,205 rows over 6 sequences (one 1,001-token chunk,
    odd starts from pending tokens, an empty sequence): every entry element
    within the bound, codes exact for the kernel's entries."""
    w = synth.scaled(synth.WORKLOADS["mixed_ragged_b256"], batch=6, ragged_tokens=(200, 1200), chunk_tokens=1001)
    worst, cnt = _check_mfma_append(ck, orc, w, [1001, 3, 0, 200, 1, 0], k_group, v_group)
    print(f"{cnt} entries, worst |e - oracle| / sum|W u| = {worst:.2e}")


def test_mfma_compressor_small_appends_are_exact(ck, orc):
    """Below 512 rows the entry point takes the exact path: bit for bit."""
    w = synth.scaled(synth.WORKLOADS["mixed_ragged_b256"], batch=4, ragged_tokens=(100, 400), chunk_tokens=1)
    W = synth.w_comp(w)
    E = synth.entry_counts(w)
    gc, hc = pair(4, int(E.max()) + 200, 32, 0, w.idx_dim)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(4)],
                 [synth.cache_idx_keys(w, b) for b in range(4)])
    lens = [300, 7, 0, 2]
    toks = np.concatenate([synth.prefill_tokens(w, b, n) for b, n in enumerate(lens)])
    irows = np.concatenate([synth.prefill_idx_rows(w, b, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows), mfma=True)
    orc.kv_append(hc, toks, cu, W, irows)
    assert_cache_equal(gc, hc)


def test_mfma_compressor_full_chunk(ck, orc):
    """The ragged workload's 16,384-token chunk on sequence 0 plus one token
    on 255 others (about 8,320 entries through the matrix cores) onto an
    empty cache with pending tokens on every other sequence; 64 sampled
    entries checked against the oracle."""
    w = synth.WORKLOADS["mixed_ragged_b256"]
    lens = [w.chunk_tokens] + [1] * (w.batch - 1)
    worst, cnt = _check_mfma_append(ck, orc, w, lens, w.k_group, w.v_group, sample=64, cached=False)
    print(f"{cnt} sampled entries, worst |e - oracle| / sum|W u| = {worst:.2e}")
