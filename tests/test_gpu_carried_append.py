"""A layer-group decode step whose append rides on its first top-k.

For caches the bound select serves (4,097 to 524,288 entries, at most 64
sequences) cskv_layer_group_decode splits the compressor append of the step
[P2 三、"突破四" (2 tokens -> 1 entry)]: a head kernel writes the indexer key
of each completed entry, the pending tokens, the token counts and the window
row before the scan; the slice launch of the top-k compresses the entry and
its final launch quantises it into the cache, before attention reads it.

The results must be those of the same step made of separate calls (the
append, the window append, the indexer top-k, attention), bit for bit, in
every storage format, dense and paged, and those of the oracle.  Sequences
are ragged: an empty one, one at capacity (its completing token overflows and
is flagged), odd and even token counts over consecutive steps.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import dev, host, load_entries, pair  # noqa: E402
from tests.test_gpu_paged import PLANES, _twins  # noqa: E402
from tests.test_gpu_parity import _run_group  # noqa: E402

SCALE = 1 / math.sqrt(576)


@pytest.fixture(scope="module")
def ck():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_kv_append_amd as ck
    ck.lib()
    return ck


def test_carried_group_steps_match_the_oracle(ck, orc):
    """Full + Reindex + 3 Reuse over 5 ragged sequences of an 8,192-entry
    cache, three consecutive steps (a token that starts a pair, one that
    completes it, one that starts the next)."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=5, entries=8192)
    cap = 8192
    lens = [6000, 0, 4097, 700, cap]
    gc, hc = pair(5, cap, w.k_group, w.v_group, w.idx_dim)
    load_entries(gc, hc, [synth.cache_entries(w, b, n) for b, n in enumerate(lens)],
                 [synth.cache_idx_keys(w, b, n) for b, n in enumerate(lens)])
    for step in range(3):
        _run_group(ck, orc, w, gc, hc, step=step)
    nt = host(gc.n_tokens)
    assert list(nt[:4]) == [2 * n + 3 for n in lens[:4]]
    assert nt[4] == 2 * cap + 1                    # the completing token overflowed
    assert int(host(gc.status)[0]) & ck.STATUS_OVERFLOW


def _ring(c, w, st):
    if c.swa_format == 1:
        return torch.zeros(c.batch, w.window, 576, dtype=torch.uint8, device="cuda")
    return dev(st.swa_ring[0])


def _by_group(ck, c, w, st, ring, W):
    B, k = c.batch, w.topk
    L = ck.Layer(mode="full", q=dev(st.q[0]), swa=ring, out=torch.empty(B, w.q_heads, 512, device="cuda"),
                 lse=torch.empty(B, w.q_heads, device="cuda"), q_idx=dev(st.q_idx[0]),
                 swa_row=dev(st.swa_row[0]), idx=torch.empty(B, k, dtype=torch.int32, device="cuda"))
    ck.layer_group_decode(c, [L], dev(st.token), W, dev(st.idx_row), k, w.window, SCALE)
    return L.idx, L.out, L.lse


def _by_parts(ck, c, w, st, ring, W):
    ck.kv_append_fp4(c, dev(st.token), None, W, dev(st.idx_row))
    ck.swa_append(ring, dev(st.swa_row[0]), None, c.n_tokens)
    idx = ck.indexer_topk(c, dev(st.q_idx[0]), w.topk)
    out, lse = ck.sparse_attn_decode(c, dev(st.q[0]), idx, ring, SCALE)
    return idx, out, lse


def _same_planes(a, b, table=None, page=0):
    """Planes, counts, pending tokens and status of cache b equal those of
    dense cache a (b paged through `table` when given)."""
    torch.cuda.synchronize()
    nt = host(a.n_tokens)
    assert np.array_equal(nt, host(b.n_tokens))
    assert int(host(a.status)[0]) == int(host(b.status)[0])
    for s in range(a.batch):
        if nt[s] % 2 == 1:
            assert np.array_equal(host(a.pending[s]), host(b.pending[s])), f"pending of sequence {s}"
    for name in PLANES:
        ga, gb = getattr(a, name), getattr(b, name)
        if ga is None:
            continue
        ha, hb = host(ga), host(gb)
        for s in range(a.batch):
            e = int(min(nt[s] // a.ratio, a.capacity))
            if table is None:
                rows_b = hb[s, :e]
            else:
                flat = hb.reshape(-1, *ha.shape[2:])
                rows_b = flat[table[s][np.arange(e) // page].astype(np.int64) * page + np.arange(e) % page]
            assert np.array_equal(ha[s, :e].view(np.uint8), rows_b.view(np.uint8)), f"{name} of sequence {s}"


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kg,vg,idx_format,k_format,swa_format",
                         [(64, 0, 0, 0, 0), (32, 128, 1, 0, 1), (16, 16, 1, 1, 0)])
def test_carried_step_equals_separate_calls(ck, paged, kg, vg, idx_format, k_format, swa_format):
    """The group step (append carried by the top-k) against the append, the
    window append, the top-k and attention called one after the other on a
    twin cache: identical planes, counts, pending tokens, status, window
    rings, indices, outputs and LSE over three steps."""
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=6, entries=6144, layers=("full",))
    cap, page = 6144, 128
    lens = [5000, 0, 4097, 1, 6144, 2222]
    W = dev(synth.w_comp(w))
    ref = ck.Cache.allocate(w.batch, cap, kg, vg, w.idx_dim, idx_format=idx_format, swa_format=swa_format,
                            k_format=k_format)
    table = None
    if paged:
        _, got, table = _twins(ck, w.batch, cap, page, kg, vg, w.idx_dim, seed=kg + vg, idx_format=idx_format,
                               k_format=k_format)
        got.swa_format = swa_format
    else:
        got = ck.Cache.allocate(w.batch, cap, kg, vg, w.idx_dim, idx_format=idx_format, swa_format=swa_format,
                                k_format=k_format)
    rows = np.concatenate([synth.cache_entries(w, b, n) for b, n in enumerate(lens)])
    keys = np.concatenate([synth.cache_idx_keys(w, b, n) for b, n in enumerate(lens)])
    cu = dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    for c in (ref, got):
        ck.kv_append_fp4(c, dev(rows), cu, None, dev(keys))
    for step in range(3):
        st = synth.step_inputs(w, step)
        ring_ref, ring_got = _ring(ref, w, st), _ring(got, w, st)
        i_ref, o_ref, l_ref = _by_parts(ck, ref, w, st, ring_ref, W)
        i_got, o_got, l_got = _by_group(ck, got, w, st, ring_got, W)
        _same_planes(ref, got, table, page)
        assert np.array_equal(host(ring_ref), host(ring_got)), f"window ring, step {step}"
        assert np.array_equal(host(i_ref), host(i_got)), f"indices, step {step}"
        assert np.array_equal(host(o_ref).view(np.uint32), host(o_got).view(np.uint32)), f"outputs, step {step}"
        assert np.array_equal(host(l_ref).view(np.uint32), host(l_got).view(np.uint32)), f"lse, step {step}"
    assert int(host(got.status)[0]) & ck.STATUS_OVERFLOW


@pytest.mark.parametrize("batch,cap,lens_fn", [
    # capacity past 262,144: groups of 4 tiles in the slice launch, the 128-slice final launch
    (3, 300000, lambda g, B: [20000, 0, 4097]),
    # the largest batch that carries its append, and the first that does not
    (64, 5000, lambda g, B: [int(x) for x in g.integers(0, 5000, size=B)]),
    (65, 5000, lambda g, B: [int(x) for x in g.integers(0, 5000, size=B)]),
])
def test_carried_step_limits_equal_separate_calls(ck, batch, cap, lens_fn):
    """Steps at the carried path's limits against separate calls, bit for bit
    over two steps (one holding a pending token, one completing entries)."""
    g = np.random.default_rng(batch)
    lens = lens_fn(g, batch)
    lens[0] = min(max(lens[0], 4097), cap)         # one sequence past one slice
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=batch, entries=max(lens), layers=("full",))
    W = dev(synth.w_comp(w))
    ref, got = (ck.Cache.allocate(batch, cap, 64, 0, w.idx_dim) for _ in range(2))
    rows = np.concatenate([synth.cache_entries(w, b, n) for b, n in enumerate(lens)])
    keys = np.concatenate([synth.cache_idx_keys(w, b, n) for b, n in enumerate(lens)])
    cu = dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    for c in (ref, got):
        ck.kv_append_fp4(c, dev(rows), cu, None, dev(keys))
    for step in range(2):
        st = synth.step_inputs(w, step)
        ring_ref, ring_got = _ring(ref, w, st), _ring(got, w, st)
        i_ref, o_ref, l_ref = _by_parts(ck, ref, w, st, ring_ref, W)
        i_got, o_got, l_got = _by_group(ck, got, w, st, ring_got, W)
        _same_planes(ref, got)
        assert np.array_equal(host(ring_ref), host(ring_got)), f"window ring, step {step}"
        assert np.array_equal(host(i_ref), host(i_got)), f"indices, step {step}"
        assert np.array_equal(host(o_ref).view(np.uint32), host(o_got).view(np.uint32)), f"outputs, step {step}"
        assert np.array_equal(host(l_ref).view(np.uint32), host(l_got).view(np.uint32)), f"lse, step {step}"
