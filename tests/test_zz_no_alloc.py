"""The allocation-free layer-group step (cskv_layer_group_decode_noalloc,
called through the C ABI) against cskv_layer_group_decode with a caller
workspace: two twin caches stepped by the two entry points must agree bit
for bit (cache planes, window rings, indices, outputs, log-sum-exps), on two
calls in a row, the second with a smaller batch and cache.  Both run the
same kernels on the same inputs, so they are compared exactly."""
import ctypes as C
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


def _twin(ck, B, E, cap, seed):
    g = np.random.default_rng(seed)
    caches = [ck.Cache.allocate(B, cap, 64, 0, 128) for _ in range(2)]
    rows = synth.student_t3(g, (B * E, 576))
    keys = synth.int_bf16(g, (B * E, 128))
    cu = dev((np.arange(B + 1) * E).astype(np.int32))
    for c in caches:
        ck.kv_append_fp4(c, dev(rows), cu, None, dev(keys))
    return caches, g


def _layers(ck, B, g, modes, heads=64, k=512, window=128):
    q = [synth.normal(g, (B, heads, 576)) for _ in modes]
    qi = [None if m == "reuse" else synth.int_bf16(g, (B, 64, 128)) for m in modes]
    rings = [synth.normal_bf16_trunc(g, (B, window, 576)) for _ in modes]
    rows = [synth.normal(g, (B, 576)) for _ in modes]

    def make():
        return [ck.Layer(mode=m, q=dev(q[i]), swa=dev(rings[i]), swa_row=dev(rows[i]),
                         q_idx=None if qi[i] is None else dev(qi[i]),
                         out=torch.full((B, heads, 512), float("nan"), device="cuda"),
                         lse=torch.full((B, heads), float("nan"), device="cuda"),
                         idx=torch.full((B, k), -7, dtype=torch.int32, device="cuda") if m != "reuse" else None)
                for i, m in enumerate(modes)]
    return make(), make()


def _step_both(ck, B, E, seed, modes):
    caches, g = _twin(ck, B, E, E + 16, seed)
    la, lb = _layers(ck, B, g, modes)
    tok, irow = dev(synth.normal(g, (B, 576))), dev(synth.int_bf16(g, (B, 128)))
    W = dev((g.standard_normal((576, 1152)) * 0.02).astype(np.float32))
    scale = 1 / math.sqrt(576)
    ck.layer_group_decode(caches[0], la, tok, W, irow, 512, 128, scale)
    # the allocation-free entry point, called through the C ABI
    arr = (ck.LayerDesc * len(lb))()
    for i, L in enumerate(lb):
        arr[i] = ck.LayerDesc(ck.MODES[L.mode], L.q.data_ptr(), None if L.q_idx is None else L.q_idx.data_ptr(),
                              None, L.swa.data_ptr(), L.swa_row.data_ptr(),
                              None if L.idx is None else L.idx.data_ptr(), L.out.data_ptr(), L.lse.data_ptr())
    d = caches[1].desc()
    rc = ck.lib().cskv_layer_group_decode_noalloc(C.byref(d), arr, len(lb), tok.data_ptr(), W.data_ptr(),
                                                  irow.data_ptr(), 64, 64, 512, 128, C.c_float(scale),
                                                  C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == ck.OK, ck.lib().cskv_last_error().decode()
    torch.cuda.synchronize()
    a, b = caches
    for name in ("k_codes", "k_scales", "idx_keys", "n_tokens", "pending", "status"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    for i, (x, y) in enumerate(zip(la, lb)):
        assert torch.equal(x.swa, y.swa), f"layer {i}: window"
        assert torch.equal(x.out.view(torch.int32), y.out.view(torch.int32)), f"layer {i}: out"
        assert torch.equal(x.lse.view(torch.int32), y.lse.view(torch.int32)), f"layer {i}: lse"
        if x.idx is not None:
            assert torch.equal(x.idx, y.idx), f"layer {i}: indices"
            assert int((x.idx >= 0).sum()) == B * 512
        assert torch.isfinite(y.out).all()


def test_noalloc_step_matches_caller_workspace(ck):
    _step_both(ck, 4, 6000, 1, ("full", "reindex", "reuse"))
    _step_both(ck, 2, 1500, 2, ("full", "reuse"))
