"""Calls enqueued on a stream other than the current one.

The binding allocates temporaries (workspaces, outputs the caller did not
pass) with torch on the current stream and launches on the given stream; it
records them on that stream, so the caching allocator does not hand their
memory to the current stream's next allocations while the kernels still use
it.  Right after each call the test fills fresh allocations of the same
sizes on the current stream; the results must equal the same calls made on
the current stream.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from tests._gpu_util import dev, host  # noqa: E402


@pytest.fixture(scope="module")
def ck():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_kv_append_amd as ck
    ck.lib()
    return ck


def _cache(ck, w, lens, cap):
    c = ck.Cache.allocate(w.batch, cap, w.k_group, w.v_group, w.idx_dim)
    rows = np.concatenate([synth.cache_entries(w, b, n) for b, n in enumerate(lens)])
    keys = np.concatenate([synth.cache_idx_keys(w, b, n) for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ck.kv_append_fp4(c, dev(rows), dev(cu), None, dev(keys))
    return c


def _scribble(nbytes):
    # allocations the size of the call's temporaries, filled on the current stream
    return [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(4)]


def test_side_stream_calls_equal_current_stream_calls(ck):
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=4, entries=6000, layers=("full",))
    lens, cap = [6000, 4500, 300, 5000], 6144
    st = synth.step_inputs(w, 1)
    W = dev(synth.w_comp(w))
    side = torch.cuda.Stream()                      # default priority
    results = []
    for stream in (None, side):
        c = _cache(ck, w, lens, cap)
        torch.cuda.synchronize()
        idx = ck.indexer_topk(c, dev(st.q_idx[0]), w.topk, stream=stream)
        keep = _scribble(ck.workspace_bytes(c, w.topk))
        ring = dev(st.swa_ring[0])
        L = ck.Layer(mode="full", q=dev(st.q[0]), swa=ring,
                     out=torch.empty(w.batch, w.q_heads, 512, device="cuda"),
                     lse=torch.empty(w.batch, w.q_heads, device="cuda"), q_idx=dev(st.q_idx[0]),
                     swa_row=dev(st.swa_row[0]), idx=torch.empty(w.batch, w.topk, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        ck.layer_group_decode(c, [L], dev(st.token), W, dev(st.idx_row), w.topk, w.window, 1 / math.sqrt(576),
                              stream=stream)
        keep += _scribble(ck.workspace_bytes(c, w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window))
        torch.cuda.synchronize()
        del keep
        results.append([host(idx), host(L.idx), host(L.out), host(L.lse), host(ring), host(c.k_codes),
                        host(c.n_tokens)])
    for i, (a, b) in enumerate(zip(*results)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"result {i} differs on the side stream"
