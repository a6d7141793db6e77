"""Checkpoint and resume of a cache through host memory.

A device cache's whole state -- the code and scale planes, the indexer keys,
the token counts, the pending odd tokens and the status word -- is copied to
the host (a checkpoint) and into a freshly allocated cache on the device (a
resume).  Both caches then take the same appends and decode step: every plane
and every output must be identical bit for bit, and the original must still
match the oracle.  The pages keep the compressed cache as the state of a
sequence (P1 "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
§3.1; P2 "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B
压缩到 890 B的？" 三、"突破六：系统层，不改模型改部署", where KV moves between
memory tiers), so nothing outside these fields may carry state between calls.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import assert_cache_equal, dev, host, load_entries, pair  # noqa: E402

STATE = ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "idx_scales", "n_tokens", "pending", "status")


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


def _checkpoint(c):
    torch.cuda.synchronize()
    return {n: getattr(c, n).cpu().clone() for n in STATE if getattr(c, n) is not None}


def _resume(ck, c, snap):
    r = ck.Cache.allocate(c.batch, c.capacity, c.k_group, c.v_group, c.idx_dim, idx_format=c.idx_format,
                          swa_format=c.swa_format, k_format=c.k_format)
    for n, t in snap.items():
        getattr(r, n).copy_(t.cuda())
    torch.cuda.synchronize()
    return r


def _chunk(w, lens, salt):
    """Host rows of an append of lens[b] tokens to sequence b (seeded by b + salt)."""
    toks = np.concatenate([synth.prefill_tokens(w, b + salt, n) for b, n in enumerate(lens)])
    irows = np.concatenate([synth.prefill_idx_rows(w, b + salt, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return toks, cu, irows


def _append(ck, c, w, chunk):
    toks, cu, irows = chunk
    ck.kv_append_fp4(c, dev(toks), dev(cu), dev(synth.w_comp(w)), dev(irows))


def _step(ck, c, w, step):
    """One layer-group decode step; returns every output on the host."""
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
                          1 / math.sqrt(576))
    torch.cuda.synchronize()
    outs = [host(r) for r in rings]
    for L in layers:
        outs += [host(L.out), host(L.lse)] + ([host(L.idx)] if L.idx is not None else [])
    return outs


def _assert_same_state(a, b):
    torch.cuda.synchronize()
    for n in STATE:
        ta, tb = getattr(a, n), getattr(b, n)
        if ta is None:
            assert tb is None
            continue
        assert torch.equal(ta.view(torch.uint8) if ta.dtype.is_floating_point else ta,
                           tb.view(torch.uint8) if tb.dtype.is_floating_point else tb), f"{n} differs"


@pytest.mark.parametrize("v_group,idx_format,k_format", [(128, 0, 0), (0, 1, 1)])
def test_cache_resume_from_host_snapshot(ck, orc, v_group, idx_format, k_format):
    """Split planes (key g32 / value g128) with bf16 indexer keys, and the
    pages' storage (E8M0 per 16 channels, FP4 indexer keys); odd token counts
    leave pending tokens in the checkpoint."""
    w = synth.scaled(synth.WORKLOADS["mixed_ragged_b256"], batch=5, ragged_tokens=(300, 1500),
                     chunk_tokens=301, v_group=v_group)
    kg = 16 if k_format else w.k_group
    vg = 0 if k_format else w.v_group
    E = synth.entry_counts(w)
    cap = int(E.max()) + 400
    gc, hc = pair(w.batch, cap, kg, vg, w.idx_dim, idx_format=idx_format, k_format=k_format)
    load_entries(gc, hc, [synth.cache_entries(w, b) for b in range(w.batch)],
                 [synth.cache_idx_keys(w, b) for b in range(w.batch)])
    first = _chunk(w, [301, 2, 7, 0, 1], salt=0)
    _append(ck, gc, w, first)
    orc.kv_append(hc, *first[:2], synth.w_comp(w), first[2])
    assert_cache_equal(gc, hc)
    nt = host(gc.n_tokens)
    assert (nt % 2 == 1).any(), "the checkpoint should hold pending tokens"

    snap = _checkpoint(gc)
    rc = _resume(ck, gc, snap)
    _assert_same_state(gc, rc)

    # the same appends and decode step on both
    second = _chunk(w, [1, 4, 1, 9, 2], salt=11)
    for c in (gc, rc):
        _append(ck, c, w, second)
    orc.kv_append(hc, *second[:2], synth.w_comp(w), second[2])
    _assert_same_state(gc, rc)
    assert_cache_equal(gc, hc)
    og, orr = _step(ck, gc, w, 0), _step(ck, rc, w, 0)
    for i, (a, b) in enumerate(zip(og, orr)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"output {i} differs after resume"
    _assert_same_state(gc, rc)
