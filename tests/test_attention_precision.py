"""Why attention multiplies in split bf16 (hi + lo) on the matrix cores.

The MFMA takes bf16 operands.  The E2M1 codes of an entry and the window's
bf16 rows are exact in bf16; the query and the probabilities times the value
group's scale are not, so the kernel feeds each as a hi + lo pair of bf16.
This CPU test replays that arithmetic in fp64 on the decode workloads'
seeded inputs (512 entries quantised by the oracle, the 128-row window, 64
query heads) and shows that rounding either operand to one bf16 breaks the
per-row tolerance of 2e-3 [P2 三、"突破四：滑动窗口和稀疏注意力"], while the
pair stays at rounding level.  It checks a design choice, not the kernel:
the kernel's parity tests hold it to the same tolerance.
"""
import math

import numpy as np
import pytest

import synth

TOL = 2e-3


def _bf16(x):
    """Round to the nearest bf16, ties to even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _row_errors(orc, w, k=512, pool=4096, seed=0):
    """Max per-row error of the four roundings for sequence 0 of workload w."""
    g = np.random.default_rng(seed)
    sel = np.sort(g.choice(pool, size=k, replace=False))
    raw = synth.cache_entries(w, 0, pool)[sel]
    kg, dim, dv = w.k_group, w.dim, w.vdim
    quant = [orc.quantize_row(r, kg) for r in raw]
    K = np.stack([orc.dequantize_row(p, s, dim, kg) for p, s in quant])
    sc = np.stack([s for _, s in quant]).astype(np.float64)           # [k, dim / kg]
    codes = np.nan_to_num(K / np.repeat(sc, kg, axis=1))                # E2M1 values, exact in bf16
    st = synth.step_inputs(w, 0, seqs=[0])
    win = (st.swa_ring[0][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = st.q[0][0].astype(np.float64)
    scale = 1 / math.sqrt(dim)
    keys = np.concatenate([K, win])
    ref_l = q @ keys.T * scale
    ref_p = np.exp(ref_l - ref_l.max(1, keepdims=True))
    ref = ref_p @ keys[:, :dv] / ref_p.sum(1, keepdims=True)
    out = {}
    for q_lo in (True, False):
        for p_lo in (True, False):
            qq = q if q_lo else _bf16(q)
            ge = np.einsum("hgd,kgd->hkg", qq.reshape(len(qq), -1, kg), codes.reshape(k, -1, kg))
            lg = np.concatenate([(ge * sc[None]).sum(2), qq @ win.T], 1) * scale
            p = np.exp(lg - lg.max(1, keepdims=True))
            o = np.zeros((len(q), dv))
            for gi in range(dv // kg):
                ps = p[:, :k] * sc[None, :, gi]
                s = slice(gi * kg, (gi + 1) * kg)
                o[:, s] = (ps if p_lo else _bf16(ps)) @ codes[:, s]
            pw = p[:, k:]
            o += (pw if p_lo else _bf16(pw)) @ win[:, :dv]
            o /= p.sum(1, keepdims=True)
            out[(q_lo, p_lo)] = float((np.abs(o - ref).max(1) / np.abs(ref).max(1)).max())
    return out


@pytest.mark.parametrize("name", ["decode_64k_b32", "group_128k_b64"])
def test_attention_needs_both_lo_halves(orc, name):
    e = _row_errors(orc, synth.WORKLOADS[name])
    assert e[(True, True)] < 1e-9
    assert e[(False, True)] > TOL, "q rounded to one bf16 fits the tolerance"
    assert e[(True, False)] > TOL, "P times the value scale rounded to one bf16 fits the tolerance"
