"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
mirror a device cache on the host, and the attention tolerance check."""
from __future__ import annotations

import numpy as np
import torch

import compressed_sparse_kv_append_amd as ck
import oracle as orc

TOL = 2e-3   # max_i |o_i - r_i| / max_i |r_i| per (sequence, head) row


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def pair(batch, capacity, k_group, v_group, idx_dim, idx_format=0, swa_format=0, k_format=0):
    """An empty device cache and its empty host mirror with the same shape."""
    g = ck.Cache.allocate(batch, capacity, k_group, v_group, idx_dim, idx_format=idx_format,
                          swa_format=swa_format, k_format=k_format)
    h = orc.Cache.empty(batch, capacity, 576, 64, k_group, v_group, idx_dim, idx_format=idx_format,
                        swa_format=swa_format, k_format=k_format)
    return g, h


def assert_cache_equal(g: ck.Cache, h: orc.Cache, seqs=None, check_pending=True):
    torch.cuda.synchronize()
    seqs = list(range(h.batch)) if seqs is None else list(seqs)
    nt = host(g.n_tokens)
    assert np.array_equal(nt[seqs], h.n_tokens[seqs]), (nt[seqs], h.n_tokens[seqs])
    for b in seqs:
        e = int(min(h.n_tokens[b] // h.ratio, h.capacity))
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "idx_keys", "idx_scales"):
            gt = getattr(g, name)
            if gt is None:
                continue
            ga = host(gt[b, :e])
            ha = getattr(h, name)[b, :e]
            if not np.array_equal(ga.view(np.uint8), ha.view(np.uint8)):
                bad = np.argwhere(ga.view(np.uint8).reshape(e, -1) != ha.view(np.uint8).reshape(e, -1))
                raise AssertionError(f"{name} differs for sequence {b}: first at {bad[:5].tolist()}")
        if check_pending and h.ratio == 2 and h.n_tokens[b] % 2 == 1:
            assert np.array_equal(host(g.pending[b]), h.pending[b]), f"pending differs, seq {b}"
    assert int(host(g.status)[0]) == int(h.status[0])


def attn_rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max abs error over max abs reference value."""
    num = np.abs(out.astype(np.float64) - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def load_entries(g: ck.Cache, h: orc.Cache, entries_per_seq, idx_keys_per_seq):
    """Entries-mode append of per-sequence rows on both sides."""
    lens = [len(e) for e in entries_per_seq]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = np.concatenate(entries_per_seq).astype(np.float32)
    keys = np.concatenate(idx_keys_per_seq).astype(np.uint16)
    ck.kv_append_fp4(g, dev(rows), dev(cu), None, dev(keys))
    orc.kv_append(h, rows, cu, None, keys)


def lse_tol(h: orc.Cache, q: np.ndarray, idx: np.ndarray, ring: np.ndarray, swa_len: np.ndarray,
            scale: float) -> np.ndarray:
    """Per (sequence, head) bound on |lse - lse_ref| from the arithmetic of the
    logits: q enters the bf16 products as a high + low bf16 pair (relative
    error <= 2^-17 per element) and the 576-term sums accumulate in fp32
    (<= 576 * 2^-24 relative to the sum of |terms|), the keys being exact
    (E2M1 codes times fp32 group scales, bf16 window rows).  A softmax-
    weighted mean of logit errors is at most the largest, so
      |d lse| <= 2^-14 * scale * max_j sum_d |q_d| |k_jd| + 1e-5
    (2^-14 > 2^-17 + 576 * 2^-24; 1e-5 covers the fp32 log-sum-exp itself)."""
    B, H, D = q.shape
    tol = np.full((B, H), 1e-5)
    for b in range(B):
        E = int(min(h.n_tokens[b] // h.ratio, h.capacity))
        keys = []
        for e in idx[b]:
            if 0 <= e < E and h.k_format == 1:
                keys.append(orc.dequantize_mx16(h.k_codes[b, e], h.k_scales[b, e], D))
            elif 0 <= e < E:
                keys.append(orc.dequantize_row(h.k_codes[b, e], h.k_scales[b, e], D, h.k_group))
        nw = int(min(swa_len[b], ring.shape[1]))
        if nw and ring.dtype == np.uint8:          # FP8 E4M3 rows
            keys.append(np.vectorize(orc.e4m3_value)(ring[b, :nw]).astype(np.float64))
        elif nw:
            keys.append((ring[b, :nw].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        if not keys:
            continue
        K = np.abs(np.vstack(keys))
        tol[b] += 2.0 ** -14 * scale * (np.abs(q[b].astype(np.float64)) @ K.T).max(axis=1)
    return tol
