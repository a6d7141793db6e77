"""A whole decode step captured once in a HIP graph and replayed step after
step: every replay leaves the cache, the selected indices, the outputs and the
log-sum-exps bit-identical to the same call made eagerly on a twin cache.
The replays are separated by eager work and synchronisations."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import compressed_sparse_kv_append_amd as ck
import synth
from _gpu_util import dev, host, load_entries, pair

pytestmark = pytest.mark.gpu

PLANES = ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "n_tokens", "pending", "status")


def _twin(gc):
    """A second device cache holding a copy of every plane of gc."""
    fields = {}
    for f in dataclasses.fields(gc):
        v = getattr(gc, f.name)
        fields[f.name] = v.clone() if isinstance(v, torch.Tensor) else v
    return ck.Cache(**fields)


def _io(w, st, B):
    layers = []
    for li, mode in enumerate(w.layers):
        layers.append(ck.Layer(mode=mode, q=dev(st.q[li]), swa=dev(st.swa_ring[li]),
                               q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                               swa_row=dev(st.swa_row[li]),
                               out=torch.zeros(B, w.q_heads, 512, device="cuda"),
                               lse=torch.zeros(B, w.q_heads, device="cuda"),
                               idx=torch.zeros(B, w.topk, dtype=torch.int32, device="cuda")
                               if mode != "reuse" else None))
    return layers


def test_layer_group_graph_replay_matches_eager():
    w = synth.scaled(synth.WORKLOADS["group_128k_b64"], batch=3, entries=2500)
    B = w.batch
    ge, he = pair(B, 2600, w.k_group, w.v_group, w.idx_dim)
    load_entries(ge, he, [synth.cache_entries(w, b) for b in range(B)],
                 [synth.cache_idx_keys(w, b) for b in range(B)])
    gg = _twin(ge)
    st = synth.step_inputs(w, 0)
    tok, irow, W = dev(st.token), dev(st.idx_row), dev(synth.w_comp(w))
    le, lg = _io(w, st, B), _io(w, st, B)
    scale = 1 / math.sqrt(576)
    wse = ck.workspace(ge, w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window)
    wsg = ck.workspace(gg, w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ck.layer_group_decode(gg, lg, tok, W, irow, w.topk, w.window, scale, ws=wsg)
    torch.cuda.synchronize()
    # capture records the step without running it
    assert np.array_equal(host(gg.n_tokens), host(ge.n_tokens))

    for rep in range(4):
        ck.layer_group_decode(ge, le, tok, W, irow, w.topk, w.window, scale, ws=wse)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in PLANES:
            a, b = getattr(ge, name), getattr(gg, name)
            if a is None:
                continue
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), \
                f"replay {rep}: cache plane {name} differs"
        for li, (x, y) in enumerate(zip(le, lg)):
            if x.idx is not None:
                assert torch.equal(x.idx, y.idx), f"replay {rep}: layer {li} indices differ"
            assert torch.equal(x.out.view(torch.int32), y.out.view(torch.int32)), \
                f"replay {rep}: layer {li} outputs differ"
            assert torch.equal(x.lse.view(torch.int32), y.lse.view(torch.int32)), \
                f"replay {rep}: layer {li} lse differs"
    assert int(host(ge.n_tokens)[0]) == 2 * 2500 + 4
