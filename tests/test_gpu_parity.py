"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Codes, scales, indexer keys, pending tokens, counters and top-k indices must
match bit for bit; attention outputs within 2e-3 of the fp64 oracle (max
abs error over max abs reference value per sequence and head).
"""
import dataclasses
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import (TOL, assert_cache_equal, attn_rel_err, dev, host, load_entries, lse_tol,  # noqa: E402
                             pair)


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


# ---------------------------------------------------------------- append

def _hard_rows(g, n):
    """Rows that stress the quantiser: heavy tails, zero groups, values on and
    next to the rounding midpoints, tiny and negative-zero channels."""
    rows = synth.student_t3(g, (n, 576))
    rows[0, :32] = 0.0                       # an all-zero group
    rows[1, :] = -0.0
    rows[2, 32:64] = np.float32(1e-38)       # subnormal-adjacent scales
    rows[2, 40] = np.float32(-1e-39)
    a = np.float32(3.0)
    s = a / np.float32(6.0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for i, m in enumerate(mids):
        x = np.float32(m * s)
        rows[3, 64 + 3 * i: 64 + 3 * i + 3] = [np.nextafter(x, np.float32(0)), x, np.nextafter(x, np.float32(9))]
    rows[3, 64:96][np.arange(32) >= 21] = 0
    rows[3, 95] = a
    rows[4] *= np.float32(1e30)              # huge values
    return rows.astype(np.float32)


@pytest.mark.parametrize("k_group,v_group", [(32, 0), (64, 0), (32, 128), (64, 32)])
def test_append_entries_mode_bitexact(ck, orc, k_group, v_group):
    g = np.random.default_rng(100 + k_group + v_group)
    gc, hc = pair(3, 700, k_group, v_group, 64)
    lens = [5, 0, 650]
    rows = [_hard_rows(g, n) if n else np.zeros((0, 576), np.float32) for n in lens]
    keys = [synth.int_bf16(g, (n, 64)) for n in lens]
    load_entries(gc, hc, rows, keys)
    assert_cache_equal(gc, hc)
    # a second call appends after the first
    rows2 = [synth.normal(g, (n, 576)) for n in (3, 2, 1)]
    keys2 = [synth.int_bf16(g, (n, 64)) for n in (3, 2, 1)]
    load_entries(gc, hc, rows2, keys2)
    assert_cache_equal(gc, hc)


def test_append_compressor_pairs_pending_bitexact(ck, orc):
    w = synth.WORKLOADS["tiny_t4096"]
    W = synth.w_comp(w)
    gc, hc = pair(3, 64, 32, 0, 64)
    g = np.random.default_rng(7)
    Wd = dev(W)
    for call, lens in enumerate([(7, 4, 1), (1, 0, 2), (3, 5, 1), (0, 1, 0), (40, 2, 3)]):
        toks = synth.normal(g, (sum(lens), 576))
        toks[::3] *= np.float32(20.0)
        irows = synth.int_bf16(g, (sum(lens), 64))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ck.kv_append_fp4(gc, dev(toks), dev(cu), Wd, dev(irows))
        orc.kv_append(hc, toks, cu, W, irows)
        assert_cache_equal(gc, hc)


@pytest.mark.parametrize("k_group,v_group,idx_dim,fmt", [(32, 128, 128, "f32"), (64, 0, 64, "f32"),
                                                        (16, 16, 128, "mx16"), (32, 0, 128, "idx_fp4")])
def test_append_compressor_large_calls_bitexact(ck, orc, k_group, v_group, idx_dim, fmt):
    """Appends of 512 rows or more take the planned, tiled compressor: more
    than 1024 sequences (the plan covers them in rounds), empty sequences,
    sequences that start on a pending token, long runs of both parities, and
    one sequence whose rows would pass capacity (left untouched, flagged).
    Everything must equal the oracle bit for bit, over three calls."""
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    Wd = dev(W)
    B, cap = 1100, 400
    # the pages' 16-channel E8M0 entries and FP4 indexer keys take the
    # planned path's block quantiser, fp32 scales with bf16 keys its wave one
    gc, hc = pair(B, cap, k_group, v_group, idx_dim, idx_format=1 if fmt == "idx_fp4" else 0,
                  k_format=1 if fmt == "mx16" else 0)
    g = np.random.default_rng(31 + k_group)
    for call in range(3):
        lens = g.integers(0, 3, size=B)
        lens[g.integers(0, B, size=6)] = g.integers(100, 301, size=6)
        lens[7] = 0
        if call == 2:
            lens[1099] = 2 * cap + 2      # past capacity whatever the parity: rejected
        if call == 1:
            lens[:] = np.minimum(lens, 1)
            lens[:600] = 1                # a few hundred single rows; >= 512 rows in all
        toks = synth.normal(g, (int(lens.sum()), 576))
        toks[::5] *= np.float32(30.0)
        irows = synth.int_bf16(g, (int(lens.sum()), idx_dim))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        assert cu[-1] >= 512
        ck.kv_append_fp4(gc, dev(toks), dev(cu), Wd, dev(irows))
        orc.kv_append(hc, toks, cu, W, irows)
        assert_cache_equal(gc, hc)
    assert int(host(gc.status)[0]) == ck.STATUS_OVERFLOW


@pytest.mark.parametrize("rows", [511, 512, 4097])
def test_append_compressor_paths_agree(ck, orc, rows):
    """One long sequence just below, at and above the row count where the
    planned path starts, onto an odd token count (a pending partner)."""
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    gc, hc = pair(2, 2200, 32, 0, 64)
    g = np.random.default_rng(rows)
    first = synth.normal(g, (1, 576))
    ir0 = synth.int_bf16(g, (1, 64))
    cu0 = np.array([0, 1, 1], np.int32)
    ck.kv_append_fp4(gc, dev(first), dev(cu0), dev(W), dev(ir0))
    orc.kv_append(hc, first, cu0, W, ir0)
    toks = synth.normal(g, (rows, 576))
    irows = synth.int_bf16(g, (rows, 64))
    cu = np.array([0, rows, rows], np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows))
    orc.kv_append(hc, toks, cu, W, irows)
    assert_cache_equal(gc, hc)


def test_append_compressor_max_batch(ck, orc):
    """The largest batch (65,535 sequences), two rows each through the
    compressor in one call: the plan covers the sequences in 64 rounds and
    the tiled kernel 1,024 row tiles.  Every sequence ends with one entry;
    whole planes are compared with the oracle bit for bit."""
    B = 65535
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    gc, hc = pair(B, 2, 32, 0, 64)
    g = np.random.default_rng(55)
    toks = synth.normal(g, (2 * B, 576))
    irows = synth.int_bf16(g, (2 * B, 64))
    cu = (2 * np.arange(B + 1)).astype(np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows))
    orc.kv_append(hc, toks, cu, W, irows)
    torch.cuda.synchronize()
    assert int(host(gc.status)[0]) == 0 == int(hc.status[0])
    assert np.array_equal(host(gc.n_tokens), hc.n_tokens)
    for name in ("k_codes", "k_scales", "idx_keys"):
        got = host(getattr(gc, name)[:, :1]).view(np.uint8)
        want = getattr(hc, name)[:, :1].view(np.uint8)
        assert np.array_equal(got, want), f"{name} differs"


def test_append_one_row_per_sequence_and_overflow(ck, orc):
    w = synth.WORKLOADS["tiny_t4096"]
    W = synth.w_comp(w)
    gc, hc = pair(2, 2, 64, 0, 128)
    g = np.random.default_rng(8)
    for step in range(6):           # the 5th and 6th tokens would need entry 2 of 2
        tok = synth.normal(g, (2, 576))
        ir = synth.int_bf16(g, (2, 128))
        ck.kv_append_fp4(gc, dev(tok), None, dev(W), dev(ir))
        orc.kv_append(hc, tok, np.arange(3, dtype=np.int32), W, ir)
        assert_cache_equal(gc, hc)
    # tokens 1-4 fill both entries, token 5 waits as pending, token 6 would need entry 2
    assert int(host(gc.status)[0]) == ck.STATUS_OVERFLOW
    assert list(host(gc.n_tokens)) == [5, 5]


def test_append_entries_onto_pending_is_rejected(ck, orc):
    gc, hc = pair(2, 8, 32, 0, 64)
    g = np.random.default_rng(9)
    W = synth.w_comp(synth.WORKLOADS["tiny_t4096"])
    tok = synth.normal(g, (1, 576))
    irow = synth.int_bf16(g, (1, 64))
    cu = np.array([0, 1, 1], np.int32)
    ck.kv_append_fp4(gc, dev(tok), dev(cu), dev(W), dev(irow))
    orc.kv_append(hc, tok, cu, W, irow)
    rows = synth.normal(g, (2, 576))
    keys = synth.int_bf16(g, (2, 64))
    load_entries(gc, hc, [rows[:1], rows[1:]], [keys[:1], keys[1:]])
    torch.cuda.synchronize()
    assert int(host(gc.status)[0]) == ck.STATUS_ODD_ENTRY_APPEND
    assert list(host(gc.n_tokens)) == [1, 2]


def test_swa_append_ring(ck, orc):
    g = np.random.default_rng(10)
    B, W = 3, 8
    ring = synth.normal_bf16_trunc(g, (B, W, 576))
    lens = [11, 1, 0]
    rows = synth.normal(g, (sum(lens), 576))
    rows[0, :4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.3895314e38]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    end = np.array([20, 3, 5], np.int32)
    gr = dev(ring)
    ck.swa_append(gr, dev(rows), dev(cu), dev(end))
    hr = ring.copy()
    orc.swa_append(hr, rows, cu, end)
    torch.cuda.synchronize()
    assert np.array_equal(host(gr), hr)


# ---------------------------------------------------------------- indexer + top-k

def _indexer_case(ck, orc, lens, idx_dim, heads, k, seed, key_fn=None, q_fn=None, head_w=None, cap=None):
    g = np.random.default_rng(seed)
    B = len(lens)
    cap = cap or max(max(lens), 1) + 3
    gc, hc = pair(B, cap, 64, 0, idx_dim)
    ents = [np.zeros((n, 576), np.float32) for n in lens]
    keys = [key_fn(g, n) if key_fn else synth.int_bf16(g, (n, idx_dim)) for n in lens]
    load_entries(gc, hc, ents, keys)
    q = q_fn(g) if q_fn else synth.int_bf16(g, (B, heads, idx_dim))
    got = host(ck.indexer_topk(gc, dev(q), k, head_w=None if head_w is None else dev(head_w)))
    want = orc.indexer_topk(hc, q, k, head_w)
    for b in range(B):
        assert np.array_equal(got[b], want[b]), (b, lens[b], np.flatnonzero(got[b] != want[b])[:8])
    return got


@pytest.mark.parametrize("idx_dim,heads", [(64, 4), (128, 64), (128, 17), (64, 64)])
def test_indexer_topk_exact_ragged(ck, orc, idx_dim, heads):
    lens = [0, 1, 511, 512, 513, 777, 4096 + 37, 20000]
    _indexer_case(ck, orc, lens, idx_dim, heads, 512, seed=idx_dim + heads)


def test_indexer_topk_long_sequences_merge_slices(ck, orc):
    """Sequences longer than one slice (4096 keys) go through the per-slice
    candidate lists and the merge, while short ones in the same batch are
    selected from their keys directly."""
    lens = [36864, 36865, 80000, 700, 0]
    _indexer_case(ck, orc, lens, 128, 64, 512, seed=40)
    _indexer_case(ck, orc, [50000, 36900], 64, 4, 2048, seed=41)
    zero = lambda g, n: np.zeros((n, 64), np.uint16)
    got = _indexer_case(ck, orc, [90000, 40000], 64, 4, 512, seed=42, key_fn=zero)
    assert np.array_equal(got[0], np.arange(512)) and np.array_equal(got[1], np.arange(512))


@pytest.mark.parametrize("distinct", [False, True])
@pytest.mark.parametrize("lens", [[210000, 9000, 180000, 80000, 0, 300], [210000, 9000, 300]])
def test_indexer_topk_two_level_merge(ck, orc, distinct, lens):
    """Caches past the bound select's 524,288 entries select by slices and
    merge; 25 or more slices merge the slices' lists in groups of 8 first.
    Six sequences (4096-key slices): 52 slices in use (a last group of 4),
    44, 20 (groups of 8, 8 and 4), 3 (one group: its list is the answer) and
    short ones.  Three sequences (8192-key slices on 1024-thread blocks): 26
    slices in use (a last group of 2), 2 and a short one.  Many tied scores
    or few."""
    if distinct:
        key_fn = None
    else:
        key_fn = lambda g, n: synth.int_bf16(g, (n, 64), -1, 1)
    _indexer_case(ck, orc, lens, 64, 4, 512, seed=77 + distinct + len(lens), key_fn=key_fn, cap=530000)


def test_indexer_topk_grouped_bound_select(ck, orc):
    """Capacities from 131,073 to 524,288 entries: the bound comes from the
    maxima of groups of 1, 2 or 4 consecutive 16-entry tiles, the smallest
    group that fits the sequence's entries in one block, and the final
    select gathers up to 128 slices' candidate lists, slices with more than
    32 candidates in a second read.  Long sequences of each group size beside
    short and empty ones; many tied scores with k = 2048."""
    _indexer_case(ck, orc, [200000, 1000, 0, 5000], 64, 16, 512, seed=47, cap=250000)
    ties = lambda g, n: synth.int_bf16(g, (n, 64), -1, 1)
    _indexer_case(ck, orc, [300000, 130000, 600, 200000], 64, 16, 2048, seed=48, key_fn=ties, cap=400000)
    _indexer_case(ck, orc, [524288, 4097], 64, 4, 512, seed=49, cap=524288)


def test_indexer_topk_many_sequences(ck, orc):
    """Batches of 128 sequences or more select their slices with 4-wave
    blocks: ragged lengths from empty to several slices, with ties."""
    g = np.random.default_rng(91)
    lens = [int(x) for x in g.integers(0, 14000, size=130)]
    lens[:4] = [0, 1, 512, 4096 + 1]
    key_fn = lambda g, n: synth.int_bf16(g, (n, 64), -2, 2)
    _indexer_case(ck, orc, lens, 64, 4, 512, seed=92, key_fn=key_fn)


def test_indexer_topk_merge_candidate_counts(ck, orc):
    """Capacities past the bound select's range: slices hold 4096 entries;
    the merge reads k candidates per full slice and min(k, entries) of the
    last one.  Lengths put the last slice at 1,
    k, k + 1 and 4096 entries and the candidate count on both sides of 5120,
    where the merge changes from 10 to 36 candidates per thread."""
    s = 4096
    lens = [8 * s + 1, 8 * s + 512, 8 * s + 513, 10 * s, 10 * s + 1, 10 * s + 511]
    _indexer_case(ck, orc, lens, 64, 4, 512, seed=43, cap=530000)
    _indexer_case(ck, orc, [s + 100, 2 * s + 2047, 2 * s + 2048, 2 * s + 2049], 64, 4, 2048, seed=44, cap=530000)


def test_indexer_topk_capacity_far_beyond_entries(ck, orc):
    """A cache allocated far beyond what it holds: the scan sizes each
    sequence's runs from its live entries, not from the capacity, so every
    block of a sequence shares its few thousand entries; the select paths
    for capacities inside and past the bound select's range both stay exact."""
    lens = [5000, 3000, 0, 4097, 700]
    _indexer_case(ck, orc, lens, 128, 64, 512, seed=45, cap=100000)
    _indexer_case(ck, orc, lens, 64, 4, 512, seed=46, cap=500000)


def test_indexer_topk_head_weights_and_small_k(ck, orc):
    hw = synth.head_weights_int(5, 3, 64)
    _indexer_case(ck, orc, [3000, 64, 9000], 128, 64, 512, seed=11, head_w=hw)
    _indexer_case(ck, orc, [3000, 64, 9000], 128, 64, 1, seed=12, head_w=hw)
    _indexer_case(ck, orc, [3000, 64, 9000], 128, 64, 2048, seed=13)


def test_indexer_topk_all_ties_take_lowest_indices(ck, orc):
    zero = lambda g, n: np.zeros((n, 128), np.uint16)
    got = _indexer_case(ck, orc, [10000, 600], 128, 64, 512, seed=14, key_fn=zero)
    assert np.array_equal(got[0], np.arange(512)) and np.array_equal(got[1], np.arange(512))


def test_indexer_topk_few_distinct_scores(ck, orc):
    # keys in {0, 1} on one coordinate -> scores take 2 values, thousands tied
    def keys(g, n):
        k = np.zeros((n, 64), np.float32)
        k[:, 3] = g.integers(0, 2, n)
        return _bf16_int(k)

    def q(g):
        x = np.zeros((2, 4, 64), np.float32)
        x[:, :, 3] = 1
        return _bf16_int(x)
    _indexer_case(ck, orc, [7000, 900], 64, 4, 512, seed=15, key_fn=keys, q_fn=q)


def test_indexer_topk_negative_scores_and_signed_zero(ck, orc):
    # negative head weights make every score <= 0, with many -0 and +0 values
    hw = -np.ones((2, 4), np.float32)
    hw[:, 0] = 0
    _indexer_case(ck, orc, [5000, 700], 64, 4, 512, seed=16, head_w=hw)


# ---------------------------------------------------------------- attention

def _attn_case(ck, orc, k_group, v_group, lens, heads, k, nswa, seed, window=128, law="normal"):
    g = np.random.default_rng(seed)
    B = len(lens)
    cap = max(lens) + 5
    gc, hc = pair(B, cap, k_group, v_group, 64)
    ents = [synth.student_t3(g, (n, 576)) if law == "t3" else synth.normal(g, (n, 576)) for n in lens]
    load_entries(gc, hc, ents, [np.zeros((n, 64), np.uint16) for n in lens])
    q = synth.normal(g, (B, heads, 576))
    idx = np.full((B, k), -1, np.int32)
    for b, n in enumerate(lens):
        sel = np.sort(g.choice(n, size=min(k, n), replace=False)) if n else np.zeros(0, np.int64)
        idx[b, :len(sel)] = sel
    ring = synth.normal_bf16_trunc(g, (B, window, 576))
    sl = np.array(nswa, np.int32)
    scale = 1 / math.sqrt(576)
    out, lse = ck.sparse_attn_decode(gc, dev(q), dev(idx), dev(ring), scale, swa_len=dev(sl))
    ref, rlse = orc.sparse_attn(hc, q, idx, ring, scale, swa_len=sl)
    out, lse = host(out), host(lse)
    err = attn_rel_err(out, ref)
    assert err.max() <= TOL, f"max rel err {err.max():.3e}"
    finite = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), finite)
    tol = lse_tol(hc, q, idx, ring, sl, scale)
    d = np.abs(np.where(finite, lse, 0) - np.where(finite, rlse, 0))
    assert (d <= tol).all(), f"lse error {d.max():.3e} over its bound at {np.unravel_index((d / tol).argmax(), d.shape)}"
    print(f"lse max err {d.max():.2e}, max err / bound {(d / tol).max():.3f}")
    return err


@pytest.mark.parametrize("k_group,v_group,law", [(32, 0, "normal"), (64, 0, "t3"), (32, 128, "normal"),
                                                  (64, 64, "t3"), (64, 32, "normal"), (64, 128, "t3")])
def test_attention_parity(ck, orc, k_group, v_group, law):
    err = _attn_case(ck, orc, k_group, v_group, lens=[700, 40, 513], heads=32, k=512,
                     nswa=[128, 5, 0], seed=20 + k_group + v_group, law=law)
    print(f"attention max rel err {err.max():.2e}")


def test_attention_edge_cases(ck, orc):
    # no keys at all, only window keys, a single key, k not a multiple of 32
    _attn_case(ck, orc, 32, 0, lens=[0, 0, 1, 100], heads=16, k=37, nswa=[0, 3, 0, 128], seed=30)


def test_attention_longest_selection_and_window(ck, orc):
    # k = 2048 selected entries and a 1024-row window with 64 heads: the most
    # chunks a sequence can have, spread over several splits per head group
    _attn_case(ck, orc, 64, 0, lens=[2600, 2100], heads=64, k=2048, nswa=[1024, 700], seed=33,
               window=1024)


@pytest.mark.parametrize("batch", [32, 64])
def test_attention_mixed_splits(ck, orc, batch):
    # 64 heads over 32 or 64 sequences: enough blocks that a split carries
    # entry chunks and window chunks together (two splits per head group at
    # 32 sequences, one at 64); ragged lengths, empty sequences, part windows
    g = np.random.default_rng(40 + batch)
    lens = [int(n) for n in g.integers(0, 900, batch)]
    lens[0], lens[1], lens[2] = 0, 511, 512
    nswa = [int(n) for n in g.integers(0, 129, batch)]
    nswa[0], nswa[3] = 0, 128
    _attn_case(ck, orc, 64, 0, lens=lens, heads=64, k=512, nswa=nswa, seed=50 + batch, law="t3")


def test_attention_result_independent_of_batch(ck, orc):
    # The same sequences attended in one batch of 64 (one mixed split per head
    # group) and in batches of 4 (kind-pure splits merged by log-sum-exp):
    # only rounding may differ -- the probabilities enter P.V as bf16 high +
    # low pairs (2^-17 relative) scaled to a running maximum that the two
    # layouts reach in different orders, so outputs agree to 2^-14 per row.
    g = np.random.default_rng(77)
    B = 64
    lens = [int(n) for n in g.integers(0, 900, B)]
    nswa = np.array([int(n) for n in g.integers(0, 129, B)], np.int32)
    cap = max(lens) + 5
    gc, hc = pair(B, cap, 64, 0, 64)
    ents = [synth.student_t3(g, (n, 576)) for n in lens]
    load_entries(gc, hc, ents, [np.zeros((n, 64), np.uint16) for n in lens])
    q = synth.normal(g, (B, 64, 576))
    idx = np.full((B, 512), -1, np.int32)
    for b, n in enumerate(lens):
        sel = np.sort(g.choice(n, size=min(512, n), replace=False))
        idx[b, :len(sel)] = sel
    ring = synth.normal_bf16_trunc(g, (B, 128, 576))
    out, lse = ck.sparse_attn_decode(gc, dev(q), dev(idx), dev(ring), 0.04, swa_len=dev(nswa))
    out, lse = host(out), host(lse)
    for b0 in range(0, B, 4):
        sl = slice(b0, b0 + 4)
        sub = dataclasses.replace(gc, batch=4, k_codes=gc.k_codes[sl], k_scales=gc.k_scales[sl],
                                  idx_keys=gc.idx_keys[sl], n_tokens=gc.n_tokens[sl], pending=gc.pending[sl])
        o2, l2 = ck.sparse_attn_decode(sub, dev(q[sl]), dev(idx[sl]), dev(ring[sl]), 0.04, swa_len=dev(nswa[sl]))
        o2, l2 = host(o2), host(l2)
        assert attn_rel_err(out[sl], o2.astype(np.float64)).max() <= 2.0 ** -14
        fin = np.isfinite(l2)
        assert np.array_equal(np.isfinite(lse[sl]), fin)
        assert np.abs(lse[sl][fin] - l2[fin]).max(initial=0) <= 2e-5


def test_attention_invalid_indices_are_skipped(ck, orc):
    g = np.random.default_rng(31)
    gc, hc = pair(1, 50, 64, 0, 64)
    load_entries(gc, hc, [synth.normal(g, (40, 576))], [np.zeros((40, 64), np.uint16)])
    q = synth.normal(g, (1, 16, 576))
    idx = np.array([[5, -1, 39, 40, 1 << 30, -7, 0, 12]], np.int32)
    ring = synth.normal_bf16_trunc(g, (1, 4, 576))
    sl = np.array([2], np.int32)
    out, lse = ck.sparse_attn_decode(gc, dev(q), dev(idx), dev(ring), 0.05, swa_len=dev(sl))
    ref, rlse = orc.sparse_attn(hc, q, idx, ring, 0.05, swa_len=sl)
    assert attn_rel_err(host(out), ref).max() <= TOL


# ---------------------------------------------------------------- whole step

def _layers(ck, w, st, gdev_rings, B, k):
    layers = []
    for li, mode in enumerate(w.layers):
        layers.append(ck.Layer(mode=mode, q=dev(st.q[li]), swa=gdev_rings[li],
                               out=torch.empty(B, w.q_heads, 512, device="cuda"),
                               lse=torch.empty(B, w.q_heads, device="cuda"),
                               q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                               swa_row=dev(st.swa_row[li]),
                               idx=torch.empty(B, k, dtype=torch.int32, device="cuda")
                               if mode != "reuse" else None))
    return layers


def _run_group(ck, orc, w, gc, hc, step=0):
    st = synth.step_inputs(w, step)
    W = synth.w_comp(w)
    B = w.batch
    grings = [dev(r) for r in st.swa_ring]
    layers = _layers(ck, w, st, grings, B, w.topk)
    ck.layer_group_decode(gc, layers, dev(st.token), dev(W), dev(st.idx_row), w.topk, w.window,
                          1 / math.sqrt(576))
    hrings = [r.copy() for r in st.swa_ring]
    outs, lses, idxs = orc.layer_group_decode(hc, w.layers, st.token, st.idx_row, W, st.q, st.q_idx,
                                              hrings, st.swa_row, w.topk, 1 / math.sqrt(576))
    torch.cuda.synchronize()
    assert_cache_equal(gc, hc)
    errs = []
    for li, L in enumerate(layers):
        assert np.array_equal(host(grings[li]), hrings[li]), f"layer {li} window ring differs"
        if L.idx is not None:
            assert np.array_equal(host(L.idx), idxs[li]), f"layer {li} indices differ"
        e = attn_rel_err(host(L.out), outs[li])
        assert e.max() <= TOL, f"layer {li} max rel err {e.max():.3e}"
        assert np.abs(host(L.lse) - lses[li]).max() < 1e-4
        errs.append(float(e.max()))
    return errs


def test_tiny_t4096_full_step(ck, orc):
    """The tiny workload in full: 4095 tokens through the compressor, then one
    decode step (the 4096th token completes entry 2047)."""
    w = synth.WORKLOADS["tiny_t4096"]
    W = synth.w_comp(w)
    gc, hc = pair(1, 2048 + 8, w.k_group, w.v_group, w.idx_dim)
    toks = synth.prefill_tokens(w, 0, w.prefill_tokens)
    irows = synth.prefill_idx_rows(w, 0, w.prefill_tokens)
    cu = np.array([0, len(toks)], np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows))
    orc.kv_append(hc, toks, cu, W, irows)
    assert_cache_equal(gc, hc)
    errs = _run_group(ck, orc, w, gc, hc)
    assert int(host(gc.n_tokens)[0]) == 4096
    print("tiny_t4096 max rel err", errs)


def test_layer_group_modes_small(ck, orc):
    """Full + Reindex + 3 Reuse on a shared cache, batch 4 (the layer-group
    workload at a size the oracle finishes quickly), two consecutive steps."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=4, entries=3000)
    gc, hc = pair(4, 3010, w.k_group, w.v_group, w.idx_dim)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(4)],
                 [synth.cache_idx_keys(w, b) for b in range(4)])
    _run_group(ck, orc, w, gc, hc, step=0)
    _run_group(ck, orc, w, gc, hc, step=1)
    assert list(host(gc.n_tokens)) == [6002] * 4


def test_mixed_ragged_split_planes_small(ck, orc):
    """Ragged batch with split K (g32) / V (g128) planes, a prefill chunk through
    the compressor on sequence 0 and one token on the others, then one step."""
    w = synth.scaled(synth.WORKLOADS["mixed_ragged_b256"], batch=6, ragged_tokens=(200, 3000),
                     chunk_tokens=1001)
    E = synth.entry_counts(w)
    cap = int(E.max()) + w.chunk_tokens // 2 + 8
    gc, hc = pair(6, cap, w.k_group, w.v_group, w.idx_dim)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(6)],
                 [synth.cache_idx_keys(w, b) for b in range(6)])
    W = synth.w_comp(w)
    lens = [w.chunk_tokens] + [1] * 5
    toks = np.concatenate([synth.prefill_tokens(w, b, n) for b, n in enumerate(lens)])
    irows = np.concatenate([synth.prefill_idx_rows(w, b, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ck.kv_append_fp4(gc, dev(toks), dev(cu), dev(W), dev(irows))
    orc.kv_append(hc, toks, cu, W, irows)
    assert_cache_equal(gc, hc)
    _run_group(ck, orc, w, gc, hc, step=0)
