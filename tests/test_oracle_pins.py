"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests uses the HIP library.  Each pin is chosen so that a
plausible mistake in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding or tie rule) fails at least one of them.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_numbers.json"), encoding="utf-8"))
GIB = 1 << 30


# ---------------------------------------------------------------- byte accounting

def test_first_generation_bytes_per_token(orc):
    g = GOLD["first_gen_bytes_per_token"]
    b = orc.kv_bytes(g["layers"], 1, g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert b == 389120
    assert abs(b - g["approx_bytes"]) / g["approx_bytes"] < g["rel_tol"]


def test_first_generation_context_sizes(orc):
    g = GOLD["first_gen_context_sizes"]
    per_tok = orc.kv_bytes(95, 1, 8, 128, 2)
    # the pages' "GB" here are binary GiB: 47.5 -> "48", 380.0 -> "380"
    assert per_tok * g["tokens_128k"] / GIB == pytest.approx(47.5)
    assert round(per_tok * g["tokens_128k"] / GIB) == g["printed_128k_gb"]
    assert per_tok * g["tokens_1m"] / GIB == pytest.approx(g["printed_1m_gb"])
    assert orc.kv_bytes(95, g["tokens_1m"], 8, 128, 2) == per_tok * g["tokens_1m"]


def test_fp16_64k_estimate(orc):
    g = GOLD["fp16_64k_estimate"]
    b = orc.kv_bytes(g["layers"], g["tokens"], g["heads"], g["head_dim"], g["elem_bytes"])
    assert b == 128849018880
    assert b / 1e11 == pytest.approx(g["printed_bytes_approx"] / 1e11, abs=0.005)
    assert b / GIB == g["printed_gb"]
    assert b / 4 / GIB == g["printed_quarter_gb"]
    half = orc.kv_bytes(g["layers"], g["tokens"] // 2, g["heads"], g["head_dim"], g["elem_bytes"])
    assert half / 4 / GIB == g["printed_32k_quarter_gb"]


def test_fp4_is_4x_fp16_before_scales(orc):
    g = GOLD["fp4_vs_fp16_ratio_before_scales"]
    d = 576
    fp16 = d * g["fp16_bits"] / 8
    fp4_no_scale = orc.fp4_row_bytes(d, d, 0.0)
    assert fp16 / fp4_no_scale == g["printed_ratio"]
    # with fp32 group scales the ratio is 16 / (4 + 32/g)
    for grp, ratio in ((32, 3.2), (64, 16 / 4.5)):
        assert fp16 / orc.fp4_row_bytes(d, grp, 4.0) == pytest.approx(ratio)


def test_mla_entry_dims():
    g = GOLD["mla_numbers_per_layer_token"]
    assert g["latent"] + g["rope"] == g["printed_total"] == 576


def test_fp4_entry_and_indexer_key_bytes(orc):
    m, i = GOLD["fp4_main_entry"], GOLD["fp4_indexer_key"]
    assert orc.fp4_row_bytes(m["dims"], m["scale_group"], m["scale_bytes"]) == m["printed_bytes"]
    assert orc.fp4_row_bytes(i["dims"], i["scale_group"], i["scale_bytes"]) == i["printed_bytes"]


def test_global_kv_per_token_900(orc):
    g = GOLD["global_kv_per_token"]
    ratios = [g["encoder_ratio"]] * g["encoder_copies"] + [g["decoder_ratio"]] * g["decoder_copies"]
    enc = orc.global_kv_per_token(ratios[:3], 288, 72)
    dec = orc.global_kv_per_token(ratios[3:], 288, 72)
    assert enc == g["printed_encoder_bytes"]
    assert dec == g["printed_decoder_bytes"]
    tot = orc.global_kv_per_token(ratios, 288, 72)
    assert tot == g["printed_estimate"]
    assert abs(tot - g["printed_reported"]) / g["printed_reported"] < 0.02
    first_gen = orc.kv_bytes(95, 1, 8, 128, 2)
    assert round(first_gen / g["printed_reported"]) == GOLD["reduction_factor"]["printed"]


def test_csa2_schedule_counts():
    g = GOLD["csa2_full_layers"]
    sched = g["encoder_group"] * g["encoder_groups"] + g["decoder_first"] + \
        g["decoder_rest"] * g["decoder_rest_groups"]
    assert sched.count("full") == g["printed_full"]
    # the pages' own group sizes add up to 38 of the 40 layers they state
    assert len(sched) == 38


# ---------------------------------------------------------------- E2M1 / bf16

def test_e2m1_value_set(orc):
    vals = [orc.e2m1_value(c) for c in range(16)]
    assert sorted(set(abs(v) for v in vals)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert vals[:8] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert vals[8:] == [-v for v in vals[:8]]
    assert math.copysign(1, vals[8]) == -1          # code 8 is -0


def test_e2m1_encode_round_trip_and_ties(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_value(c)) == c
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert orc.e2m1_encode(v) == c and orc.e2m1_encode(-v) == c | 8
    assert orc.e2m1_encode(1e30) == 7 and orc.e2m1_encode(-7.0) == 15
    assert orc.e2m1_encode(-1e-30) == 8 and orc.e2m1_encode(0.0) == 0


def test_e2m1_monotone(orc):
    xs = np.linspace(-8, 8, 4001)
    vals = [orc.e2m1_value(orc.e2m1_encode(float(x))) for x in xs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))


def test_bf16_matches_torch_on_samples(orc):
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(2000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 2000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([orc.bf16_from_f32(float(v)) for v in x], np.uint16)
    assert np.array_equal(ref, got)


@pytest.fixture(scope="module")
def exhaustive_bin(tmp_path_factory):
    out = tmp_path_factory.mktemp("native") / "exhaustive"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-o", str(out),
                    os.path.join(HERE, "native", "exhaustive.c"), "-ldl", "-lm"], check=True)
    return str(out)


def test_encoders_exhaustive_all_fp32(orc, exhaustive_bin):
    """Every finite fp32 pattern: E2M1 encode vs the threshold table and bf16
    rounding vs the integer formulation."""
    import oracle.build as ob
    r = subprocess.run([exhaustive_bin, ob.LIB, "0", str(1 << 32)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "e2m1_mismatch=0 bf16_mismatch=0" in r.stdout
    # the stored checksums the device encoders are checked against come
    # from this same oracle run
    with open(os.path.join(HERE, "golden", "encoder_checksums.json")) as f:
        g = json.load(f)
    assert f"e2m1_sum={g['e2m1_sum']} bf16_sum={g['bf16_sum']}" in r.stdout
    assert f"tested={g['tested']} " in r.stdout


def test_oracle_under_host_sanitizers(tmp_path):
    """The oracle's C built with AddressSanitizer and UndefinedBehaviorSanitizer
    (every report fatal), driven through every entry point on small caches
    whose planes are allocated at exactly their layout's size, in every
    storage format and over the edge cases it handles (empty, full and
    overflowing sequences, pending tokens, k past the entry count, -1 and
    out-of-range indices, empty windows, padded pools)."""
    import oracle.build as ob
    exe = tmp_path / "sanitize_oracle"
    flags = [f for f in ob.CFLAGS if f not in ("-O2", "-fPIC", "-shared", "-fopenmp")]
    subprocess.run(["gcc", *flags, "-O1", "-g", "-fno-omit-frame-pointer", "-Wno-unknown-pragmas",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", ob.SRC,
                    os.path.join(HERE, "native", "sanitize_oracle.c"), "-lm", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.rstrip().endswith("ok") and "runtime error" not in r.stderr, r.stderr[-4000:]


# ---------------------------------------------------------------- quantiser

def _codes(packed):
    return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(*packed.shape[:-1], -1)


@pytest.mark.parametrize("group", [32, 64])
def test_quantize_error_bound_and_full_scale_code(orc, group):
    g = np.random.default_rng(group)
    for law in ("normal", "t3"):
        x = g.standard_normal(576).astype(np.float32) if law == "normal" else \
            (g.standard_t(3, 576)).astype(np.float32)
        packed, scales = orc.quantize_row(x, group)
        deq = orc.dequantize_row(packed, scales, 576, group)
        s = np.repeat(scales.astype(np.float64), group)
        err = np.abs(x.astype(np.float64) - deq)
        assert np.all(err <= s * (1 + 2 ** -20))
        small = np.abs(x.astype(np.float64)) <= 2 * s
        assert np.all(err[small] <= s[small] * (0.25 + 2 ** -21))
        codes = _codes(packed).reshape(-1, group)
        assert np.all((codes & 7).max(axis=1) == 7)
        # the scale is absmax / 6 in fp32
        a = np.abs(x).reshape(-1, group).max(axis=1)
        assert np.array_equal(scales, (a / np.float32(6.0)).astype(np.float32))


def test_quantize_zero_group_and_signs(orc):
    x = np.zeros(64, np.float32)
    x[32:] = np.float32(1.0)
    x[33] = np.float32(-1e-3)      # rounds to zero magnitude but keeps its sign
    x[34] = np.float32(-0.0)
    packed, scales = orc.quantize_row(x, 32)
    codes = _codes(packed)
    assert scales[0] == 0 and not np.signbit(scales[0]) and np.all(codes[:32] == 0)
    assert scales[1] == np.float32(1.0) / np.float32(6.0)
    assert codes[33] == 8 and codes[34] == 8 and codes[32] == 7


def test_quantize_pack_order_low_nibble_first(orc):
    x = np.zeros(32, np.float32)
    x[0], x[1] = 6.0, -3.0          # codes 7 and 13
    packed, _ = orc.quantize_row(x, 32)
    assert packed[0] == 7 | (13 << 4)


def test_quantize_uses_true_division(orc):
    """x/s is an IEEE division, not a multiplication by a reciprocal: find an
    input where the two differ in the chosen code and check the division wins."""
    g = np.random.default_rng(3)
    found = 0
    for _ in range(20000):
        a = np.float32(g.uniform(0.5, 4.0))
        s = a / np.float32(6.0)
        mid = np.float32(g.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
        x = np.float32(mid * s)
        for cand in (x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(10))):
            q_div = np.float32(cand / s)
            q_rcp = np.float32(cand * (np.float32(1.0) / s))
            if q_div != q_rcp:
                row = np.zeros(32, np.float32)
                row[0], row[1] = a, cand
                packed, scales = orc.quantize_row(row, 32)
                assert scales[0] == s
                assert _codes(packed)[1] == orc.e2m1_encode(float(q_div))
                found += 1
    assert found > 0


# ---------------------------------------------------------------- compressor

def test_compress_selects_rows():
    import oracle as orc
    D = 576
    g = np.random.default_rng(1)
    xe, xo = g.standard_normal(D).astype(np.float32), g.standard_normal(D).astype(np.float32)
    W = np.zeros((D, 2 * D), np.float32)
    W[np.arange(D), np.arange(D)] = 1
    assert np.array_equal(orc.compress_pair(W, xe, xo), xe)
    W[:] = 0
    W[np.arange(D), D + np.arange(D)] = 1
    assert np.array_equal(orc.compress_pair(W, xe, xo), xo)
    W[:] = 0
    W[3, 7], W[3, D + 7] = 2.0, -1.0
    e = orc.compress_pair(W, xe, xo)
    assert e[3] == np.float32(np.float32(2 * xe[7]) - xo[7]) and np.all(np.delete(e, 3) == 0)


def test_compress_fma_order_within_a_block():
    """Inside a block of 2D/64 terms the fold runs upward: 1e8 + 1 rounds to
    1e8 in fp32, so (1e8 + 1) - 1e8 = 0, while any regrouping that adds 1
    last gives 1."""
    import oracle as orc
    D = 576                                   # blocks of 18 terms
    W = np.zeros((D, 2 * D), np.float32)
    W[0, :3] = 1.0
    xe = np.zeros(D, np.float32)
    xe[:3] = [1e8, 1.0, -1e8]
    assert orc.compress_pair(W, xe, np.zeros(D, np.float32))[0] == 0.0
    # a single rounding per term: after acc = -1, fma(1/3f, 3, acc) keeps the
    # product's low bits (a separate multiply would round 3 * (1/3f) to 1 first)
    W[:] = 0
    W[2, 0], W[2, 1] = -1.0, np.float32(1.0 / 3.0)
    xe3 = np.zeros(D, np.float32)
    xe3[:2] = [1.0, 3.0]
    exact = np.float64(np.float32(1.0 / 3.0)) * 3.0 - 1.0
    assert orc.compress_pair(W, xe3, np.zeros(D, np.float32))[2] == np.float32(exact)


def test_compress_blocks_of_18_and_pairwise_tree():
    """Block sums [1e8, 0, 4, 4]: the tree adds (4 + 4) before meeting 1e8 and
    gets 1e8 + 8 exactly; a fold over j (or blocks joined left to right)
    rounds 1e8 + 4 back to 1e8 twice.  Terms at j = 17 and j = 18 fall in
    different blocks: with blocks of 16, 4 + 4 would meet first."""
    import oracle as orc
    D = 576
    z = np.zeros(D, np.float32)
    W = np.zeros((D, 2 * D), np.float32)
    u = np.zeros(D, np.float32)
    W[5, [0, 36, 54]] = 1.0                   # blocks 0, 2, 3
    u[[0, 36, 54]] = [1e8, 4.0, 4.0]
    assert orc.compress_pair(W, u, z)[5] == np.float32(100000008.0)
    W[:] = 0
    u[:] = 0
    W[6, [0, 17, 18]] = 1.0                   # block 0 holds j = 0..17, block 1 starts at 18
    u[[0, 17, 18]] = [1e8, 4.0, 4.0]
    assert orc.compress_pair(W, u, z)[6] == np.float32(1e8)
    # the second half of u (x_odd) is blocks 32..63: x_odd[0] meets x_even's
    # block sums only at the last level of the tree
    W[:] = 0
    W[7, [0, D]] = 1.0
    assert orc.compress_pair(W, np.full(D, 1e8, np.float32) * (np.arange(D) == 0),
                             np.full(D, -1e8, np.float32) * (np.arange(D) == 0))[7] == 0.0


def test_compress_within_forward_error_bound():
    import oracle as orc
    D = 576
    g = np.random.default_rng(2)
    W = (g.standard_normal((D, 2 * D)) * 0.02).astype(np.float32)
    xe, xo = g.standard_normal(D).astype(np.float32), g.standard_normal(D).astype(np.float32)
    e = orc.compress_pair(W, xe, xo).astype(np.float64)
    u = np.concatenate([xe, xo]).astype(np.float64)
    ref = W.astype(np.float64) @ u
    # every term passes through at most 18 fused multiply-adds of its block
    # and 6 additions of the tree
    n, uu = 2 * D // 64 + 6, 2.0 ** -24
    gamma = n * uu / (1 - n * uu)
    bound = gamma * (np.abs(W.astype(np.float64)) @ np.abs(u))
    assert np.all(np.abs(e - ref) <= bound)


# ---------------------------------------------------------------- append state machine

def _small_cache(orc, B=3, cap=40, k_group=32, v_group=0, idx_dim=64):
    return orc.Cache.empty(B, cap, 576, 64, k_group, v_group, idx_dim)


def test_append_pairs_and_pending(orc):
    D = 576
    g = np.random.default_rng(4)
    W = (g.standard_normal((D, 2 * D)) * 0.02).astype(np.float32)
    lens = [7, 4, 1]
    toks = [g.standard_normal((n, D)).astype(np.float32) for n in lens]
    irow = [g.integers(-8, 9, (n, 64)).astype(np.float32).view(np.uint32) >> 16 for n in lens]
    irow = [r.astype(np.uint16) for r in irow]
    # one call with all rows
    c1 = _small_cache(orc)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    orc.kv_append(c1, np.concatenate(toks), cu, W, np.concatenate(irow))
    # token by token
    c2 = _small_cache(orc)
    for t in range(max(lens)):
        rows, irs, cu2 = [], [], [0]
        for b in range(3):
            if t < lens[b]:
                rows.append(toks[b][t]); irs.append(irow[b][t])
            cu2.append(len(rows))
        orc.kv_append(c2, np.array(rows), np.array(cu2, np.int32), W, np.array(irs))
    for f in ("k_codes", "k_scales", "idx_keys", "n_tokens"):
        assert np.array_equal(getattr(c1, f), getattr(c2, f)), f
    assert np.array_equal(c1.pending[[0, 2]], c2.pending[[0, 2]])
    assert list(c1.n_tokens) == lens and list(c1.entries()) == [3, 2, 0]
    assert np.array_equal(c1.pending[0], toks[0][6]) and np.array_equal(c1.pending[2], toks[2][0])
    # entry i of sequence 0 is the compressed pair (2i, 2i+1) with the key row of token 2i+1
    e = orc.compress_pair(W, toks[0][2], toks[0][3])
    pk, sc = orc.quantize_row(e, 32)
    assert np.array_equal(c1.k_codes[0, 1], pk) and np.array_equal(c1.k_scales[0, 1], sc)
    assert np.array_equal(c1.idx_keys[0, 1], irow[0][3])
    assert c1.status[0] == 0


def test_append_entries_mode_and_split_planes(orc):
    g = np.random.default_rng(5)
    c = _small_cache(orc, B=2, cap=8, k_group=32, v_group=128)
    rows = g.standard_normal((5, 576)).astype(np.float32)
    irs = np.zeros((5, 64), np.uint16)
    orc.kv_append(c, rows, np.array([0, 3, 5], np.int32), None, irs)
    assert list(c.n_tokens) == [6, 4]
    pk, sc = orc.quantize_row(rows[4], 32)
    assert np.array_equal(c.k_codes[1, 1], pk) and np.array_equal(c.k_scales[1, 1], sc)
    pv, sv = orc.quantize_row(rows[4][:512], 128)
    assert np.array_equal(c.v_codes[1, 1], pv) and np.array_equal(c.v_scales[1, 1], sv)
    assert sv.shape == (4,)


def test_append_overflow_and_odd_are_rejected(orc):
    c = _small_cache(orc, B=2, cap=2)
    rows = np.ones((4, 576), np.float32)
    irs = np.zeros((4, 64), np.uint16)
    orc.kv_append(c, rows, np.array([0, 3, 4], np.int32), None, irs)
    assert list(c.n_tokens) == [0, 2] and c.status[0] == orc.STATUS_OVERFLOW
    c.status[0] = 0
    c.n_tokens[1] = 3
    orc.kv_append(c, rows[:1], np.array([0, 0, 1], np.int32), None, irs[:1])
    assert c.status[0] == orc.STATUS_ODD_ENTRY_APPEND and c.n_tokens[1] == 3


def test_swa_ring_positions(orc):
    g = np.random.default_rng(6)
    B, W, D = 2, 4, 576
    ring = np.zeros((B, W, D), np.uint16)
    rows = g.standard_normal((7, D)).astype(np.float32)
    cu = np.array([0, 6, 7], np.int32)
    end = np.array([10, 2], np.int32)
    orc.swa_append(ring, rows, cu, end)
    # sequence 0: rows are positions 4..9, the last 4 (6..9) land in slots 2,3,0,1
    for q, pos in ((2, 6), (3, 7), (4, 8), (5, 9)):
        want = np.array([orc.bf16_from_f32(float(v)) for v in rows[q]], np.uint16)
        assert np.array_equal(ring[0, pos % W], want)
    assert np.array_equal(ring[1, 1], np.array([orc.bf16_from_f32(float(v)) for v in rows[6]],
                                               np.uint16))
    assert np.all(ring[1, [0, 2, 3]] == 0)


# ---------------------------------------------------------------- indexer + top-k

def _bf16_int(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_indexer_special_cases(orc):
    g = np.random.default_rng(8)
    K = g.integers(-8, 9, (50, 64))
    q = g.integers(-8, 9, (4, 64))
    # zero keys score zero
    assert np.all(orc.indexer_scores(_bf16_int(np.zeros((3, 64))), _bf16_int(q)) == 0)
    # a unit query picks one coordinate and ReLU drops negatives
    e = np.zeros((1, 64)); e[0, 5] = 1
    s = orc.indexer_scores(_bf16_int(K), _bf16_int(e))
    assert np.array_equal(s, np.maximum(K[:, 5], 0))
    # the ReLU acts per head before the head sum: +e5 and -e5 give |K5|, not 0
    s2 = orc.indexer_scores(_bf16_int(K), _bf16_int(np.stack([e[0], -e[0]])))
    assert np.array_equal(s2, np.abs(K[:, 5]))
    # q equal to a key row scores its squared norm (single head)
    s3 = orc.indexer_scores(_bf16_int(K), _bf16_int(K[7:8]))
    assert s3[7] == float((K[7] ** 2).sum())
    # head weights scale heads linearly; zero weights silence a head
    w = np.array([0, 2, 0, 0], np.float32)
    s4 = orc.indexer_scores(_bf16_int(K), _bf16_int(q), w)
    assert np.array_equal(s4, 2 * np.maximum(K @ q[1], 0))
    # a transposed key layout would mix entries: entry j only depends on row j
    K2 = K.copy(); K2[10] = 0
    s5 = orc.indexer_scores(_bf16_int(K2), _bf16_int(q))
    s6 = orc.indexer_scores(_bf16_int(K), _bf16_int(q))
    assert s5[10] == 0 and np.array_equal(np.delete(s5, 10), np.delete(s6, 10))


def _valid_topk(s, k, out):
    E = len(s)
    n = min(k, E)
    sel = out[:n]
    assert np.all(out[n:] == -1) and np.all(np.diff(sel) > 0)
    S = set(sel.tolist())
    for i in S:
        for j in range(E):
            if j not in S:
                assert s[i] > s[j] or (s[i] == s[j] and i < j)


def test_topk_characterisation_with_ties(orc):
    g = np.random.default_rng(9)
    for trial in range(300):
        E = int(g.integers(0, 14))
        k = int(g.integers(1, 10))
        s = g.integers(0, 3, E).astype(np.float64) if trial % 2 else g.standard_normal(E)
        out = orc.topk(s, k)
        _valid_topk(s, k, out)


def test_topk_all_equal_takes_lowest_indices(orc):
    out = orc.topk(np.zeros(1000), 512)
    assert np.array_equal(out, np.arange(512))
    out = orc.topk(np.zeros(300), 512)
    assert np.array_equal(out[:300], np.arange(300)) and np.all(out[300:] == -1)


def test_topk_exhaustive_tiny(orc):
    """All score vectors over {0,1,2}^6 and every k: the output is the unique
    set allowed by the (score desc, index asc) order."""
    import itertools
    for s in itertools.product([0.0, 1.0, 2.0], repeat=6):
        s = np.array(s)
        for k in range(1, 8):
            _valid_topk(s, k, orc.topk(s, k))


# ---------------------------------------------------------------- FP8 window rows

def _e4m3_by_fields(v):
    s, e, m = v >> 7, (v >> 3) & 15, v & 7
    mag = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_values_and_round_trip(orc):
    vals = []
    for v in range(256):
        if v & 0x7F == 0x7F:
            assert math.isnan(orc.e4m3_value(v))
            continue
        x = orc.e4m3_value(v)
        assert x == _e4m3_by_fields(v)
        assert orc.e4m3_encode(x) == v                 # every finite value encodes to itself
        vals.append(x)
    assert max(vals) == 448.0 and min(v for v in vals if v > 0) == 2.0 ** -9
    assert len(set(vals)) == 253                         # +0 and -0 compare equal


def test_e4m3_rounding_ties_and_saturation(orc):
    pos = sorted({orc.e4m3_value(v) for v in range(0x7F)})
    for a, b in zip(pos, pos[1:]):
        mid = (a + b) / 2
        ca, cb = orc.e4m3_encode(a), orc.e4m3_encode(b)
        assert orc.e4m3_encode(mid) == (ca if ca % 2 == 0 else cb)      # ties to the even mantissa
        assert orc.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0))) == ca
        assert orc.e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == cb
    assert orc.e4m3_encode(448.0) == 0x7E and orc.e4m3_encode(1e30) == 0x7E
    assert orc.e4m3_encode(-500.0) == 0xFE and orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(2.0 ** -11) == 0x00 and orc.e4m3_encode(-(2.0 ** -10) * 1.01) == 0x81


def test_attention_with_fp8_window_is_the_decoded_rows(orc):
    g = np.random.default_rng(40)
    n = 20
    c8 = orc.Cache.empty(1, n, 576, 64, 32, 0, 64, swa_format=1)
    c16 = orc.Cache.empty(1, n, 576, 64, 32, 0, 64)
    ents = g.standard_normal((n, 576)).astype(np.float32)
    for c in (c8, c16):
        orc.kv_append(c, ents, np.array([0, n], np.int32), None, np.zeros((n, 64), np.uint16))
    rows = g.standard_normal((6, 576)).astype(np.float32)
    ring8 = np.zeros((1, 8, 576), np.uint8)
    orc.swa_append(ring8, rows, np.array([0, 6], np.int32), np.array([6], np.int32))
    assert ring8[0, 3, 7] == orc.e4m3_encode(rows[3, 7]) and not ring8[0, 6:].any()
    # the same rows as bf16 (exact: E4M3 values have 4 significant bits)
    dec = np.vectorize(orc.e4m3_value)(ring8).astype(np.float32)
    ring16 = _bf16_int(dec)
    q = g.standard_normal((1, 16, 576)).astype(np.float32)
    idx = np.array([[0, 5, 19, -1]], np.int32)
    o8, l8 = orc.sparse_attn(c8, q, idx, ring8, 0.04, swa_len=np.array([6], np.int32))
    o16, l16 = orc.sparse_attn(c16, q, idx, ring16, 0.04, swa_len=np.array([6], np.int32))
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)


# ---------------------------------------------------------------- FP4 indexer key

def test_e8m0_values(orc):
    assert orc.e8m0_value(127) == 1.0 and orc.e8m0_value(128) == 2.0 and orc.e8m0_value(125) == 0.25
    assert orc.e8m0_value(0) == 2.0 ** -127 and orc.e8m0_value(254) == 2.0 ** 127


def _mx_group(orc, vals):
    x = _bf16_int(np.asarray(vals, np.float32))
    codes, scales = orc.quantize_mx16(x)
    return codes, scales, orc.dequantize_mx16(codes, scales, len(vals))


def test_mx16_scale_rule_at_binade_edges(orc):
    # largest magnitude a: scale 2^(floor(log2 a) - 2)
    for a, e in ((1.0, -2), (1.99, -2), (2.0, -1), (6.0, 0), (7.0, 0), (8.0, 1), (0.375, -4), (1000.0, 7)):
        a = float(np.float32(a))
        vals = [0.0] * 15 + [a]
        codes, scales, deq = _mx_group(orc, vals)
        assert scales[0] == e + 127, (a, scales[0])
    # 7 / 1 is past 6: it saturates to 6 (the MX rule clamps)
    assert _mx_group(orc, [0.0] * 15 + [7.0])[2][15] == 6.0
    # an all-zero group: byte 0, zero codes
    codes, scales, deq = _mx_group(orc, [0.0] * 16)
    assert scales[0] == 0 and not codes.any() and not deq.any()


def test_mx16_integers_and_round_trip(orc):
    # a group holding -8..8 has scale 2: x / 2 in steps of 0.5, nearest E2M1
    # value with ties to the even code, worked out by hand
    ints = np.arange(-8, 8).astype(np.float32)               # -8..7: one group, largest magnitude 8
    codes, scales, deq = _mx_group(orc, ints)
    want = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 5: 4, 6: 6, 7: 8, 8: 8}
    assert scales[0] == 128
    assert [deq[i] for i in range(16)] == [float(np.sign(v)) * want[abs(int(v))] for v in ints]
    # values already on the grid of their group survive exactly
    g = np.random.default_rng(30)
    for _ in range(200):
        e = int(g.integers(-6, 6))
        grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        v = g.choice(grid, 16) * g.choice([-1, 1], 16) * 2.0 ** e
        v[0] = 6 * 2.0 ** e                                  # pins the group's scale
        assert np.array_equal(_mx_group(orc, v)[2], v)
    # 128 dims take 64 code bytes + 8 scale bytes = 72 B, the pages' figure
    codes, scales = orc.quantize_mx16(_bf16_int(np.ones(128, np.float32)))
    assert codes.nbytes + scales.nbytes == 72 == orc.fp4_row_bytes(128, 16, 1)


def test_mx16_main_entry_form(orc):
    g = np.random.default_rng(32)
    # on bf16-representable inputs the fp32 form and the bf16 form agree
    for _ in range(50):
        x = _bf16_int(g.standard_normal(576).astype(np.float32) * 2.0 ** g.integers(-8, 8))
        xf = (x.astype(np.uint32) << 16).view(np.float32)
        c1, s1 = orc.quantize_mx16(x)
        c2, s2 = orc.quantize_mx16_f32(xf)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # fp32 inputs at a binade edge: 7.999 has floor(log2) 2 -> scale 1 -> saturates to 6
    codes, scales = orc.quantize_mx16_f32(np.array([7.999] + [0.0] * 15, np.float32))
    assert scales[0] == 127 and orc.dequantize_mx16(codes, scales, 16)[0] == 6.0
    # on-grid groups survive exactly
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = g.choice(grid, 576) * g.choice([-1, 1], 576)
    v[::16] = 6.0
    v = v * 2.0 ** np.repeat(g.integers(-5, 5, 36), 16)
    codes, scales = orc.quantize_mx16_f32(v.astype(np.float32))
    assert np.array_equal(orc.dequantize_mx16(codes, scales, 576), v)


def test_attention_over_mx16_entries_is_attention_over_their_values(orc):
    # rows on the E2M1 x 2^e grid of every 16-channel group dequantise exactly
    # under both scale forms, so attention agrees bit for bit
    g = np.random.default_rng(33)
    n = 30
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    ents = g.choice(grid, (n, 576)) * g.choice([-1, 1], (n, 576))
    ents[:, ::16] = 6.0
    ents = (ents * 2.0 ** np.repeat(g.integers(-3, 3, (n, 36)), 16, axis=1)).astype(np.float32)
    cm = orc.Cache.empty(1, n, 576, 64, 16, 16, 64, k_format=1)
    cf = orc.Cache.empty(1, n, 576, 64, 16, 16, 64)
    for c in (cm, cf):
        orc.kv_append(c, ents, np.array([0, n], np.int32), None, np.zeros((n, 64), np.uint16))
    assert cm.k_scales.dtype == np.uint8 and cm.k_scales.shape == (1, n, 36) and cm.v_scales.shape == (1, n, 32)
    q = g.standard_normal((1, 16, 576)).astype(np.float32)
    idx = np.array([[0, 3, 29, 17, -1]], np.int32)
    ring = _bf16_int(g.standard_normal((1, 4, 576)).astype(np.float32))
    om, lm = orc.sparse_attn(cm, q, idx, ring, 0.04, swa_len=np.array([2], np.int32))
    of, lf = orc.sparse_attn(cf, q, idx, ring, 0.04, swa_len=np.array([2], np.int32))
    assert np.array_equal(om, of) and np.array_equal(lm, lf)


def test_fp4_cache_scores_use_the_dequantised_keys(orc):
    g = np.random.default_rng(31)
    n, Di = 300, 64
    keys = _bf16_int(g.integers(-8, 9, (n, Di)))
    c = orc.Cache.empty(1, n, 576, 64, 32, 0, Di, idx_format=1)
    orc.kv_append(c, np.zeros((n, 576), np.float32), np.array([0, n], np.int32), None, keys)
    for j in (0, 7, 299):
        codes, scales = orc.quantize_mx16(keys[j])
        assert np.array_equal(c.idx_keys[0, j], codes) and np.array_equal(c.idx_scales[0, j], scales)
    # the dequantised keys are bf16-exact: scoring them as a bf16 plane gives the same ranking
    deq = np.stack([orc.dequantize_mx16(c.idx_keys[0, j], c.idx_scales[0, j], Di) for j in range(n)])
    q = _bf16_int(g.integers(-8, 9, (1, 4, Di)))
    b16 = _bf16_int(deq.astype(np.float32))
    assert np.array_equal(orc.indexer_topk(c, q, 50)[0], orc.topk(orc.indexer_scores(b16, q[0]), 50))
    assert not np.array_equal(orc.indexer_topk(c, q, 50)[0], orc.topk(orc.indexer_scores(keys, q[0]), 50))


# ---------------------------------------------------------------- candidate pool

def _pool_by_subsets(s, block, nb):
    """The pool found by trying every set of blocks: the unique set of
    min(nb, blocks) blocks in which every member beats every non-member
    on (block maximum, then lower block index)."""
    import itertools
    E = len(s)
    nblk = -(-E // block)
    bm = [max(s[i * block:(i + 1) * block]) for i in range(nblk)]
    m = min(nb, nblk)
    found = []
    for S in itertools.combinations(range(nblk), m):
        inside = set(S)
        if all(bm[i] > bm[j] or (bm[i] == bm[j] and i < j)
               for i in inside for j in range(nblk) if j not in inside):
            found.append(list(S))
    assert len(found) == 1
    return found[0] + [-1] * (nb - m)


def test_pool_blocks_brute_force_tiny(orc):
    g = np.random.default_rng(21)
    for trial in range(400):
        E = int(g.integers(0, 13))
        block = int(g.integers(1, 4))
        nb = int(g.integers(1, 6))
        s = g.integers(0, 3, E).astype(np.float64) if trial % 2 else g.standard_normal(E)
        assert list(orc.pool_blocks(s, block, nb)) == _pool_by_subsets(list(s), block, nb)


def test_pool_blocks_hand_built(orc):
    # blocks of 8 over 27 entries: maxima 5 (block 0), 9 (block 1), 5 (block 2),
    # 7 (block 3, the short one: entries 24..26)
    s = np.zeros(27)
    s[3], s[12], s[20], s[26] = 5, 9, 5, 7
    assert list(orc.pool_blocks(s, 8, 2)) == [1, 3]
    assert list(orc.pool_blocks(s, 8, 3)) == [0, 1, 3]        # tie 5 = 5: block 0 before block 2
    assert list(orc.pool_blocks(s, 8, 6)) == [0, 1, 2, 3, -1, -1]
    assert list(orc.pool_blocks(np.zeros(0), 8, 2)) == [-1, -1]
    # within the pool, selection follows the entry scores, not the block maxima
    pool = np.array([1, 3], np.int32)
    assert list(orc.topk_in_pool(s, pool, 8, 3)) == [8, 12, 26]   # 9, 7, then the lowest 0 (entry 8)
    assert list(orc.topk_in_pool(s, pool, 8, 12)) == list(range(8, 16)) + [24, 25, 26, -1]


def test_topk_in_pool_brute_force_tiny(orc):
    g = np.random.default_rng(22)
    for trial in range(300):
        E = int(g.integers(0, 14))
        block = int(g.integers(1, 4))
        nb = int(g.integers(1, 5))
        k = int(g.integers(1, 8))
        s = g.integers(0, 3, E).astype(np.float64) if trial % 2 else g.standard_normal(E)
        pool = orc.pool_blocks(s, block, nb)
        q = g.integers(0, 3, E).astype(np.float64)        # a second query's scores
        out = orc.topk_in_pool(q, pool, block, k)
        ent = [j for b in pool if b >= 0 for j in range(b * block, min((b + 1) * block, E))]
        n = min(k, len(ent))
        sel = list(out[:n])
        assert all(x == -1 for x in out[n:]) and sel == sorted(sel) and set(sel) <= set(ent)
        for i in sel:
            for j in ent:
                if j not in sel:
                    assert q[i] > q[j] or (q[i] == q[j] and i < j)


def test_topk_in_pool_closed_forms(orc):
    g = np.random.default_rng(23)
    # every block pooled: the pool changes nothing
    s = g.integers(0, 4, 500).astype(np.float64)
    pool = orc.pool_blocks(s, 8, 2048)
    assert list(pool[:63]) == list(range(63)) and np.all(pool[63:] == -1)
    assert np.array_equal(orc.topk_in_pool(s, pool, 8, 64), orc.topk(s, 64))
    # the pool's own scores, all distinct, k <= nb: the k best entries lie in
    # the k best blocks, so the pooled top-k is the top-k
    for E, nb, k in ((4000, 64, 64), (4003, 100, 37), (20000, 2048, 512)):
        s = g.permutation(E).astype(np.float64)
        pool = orc.pool_blocks(s, 8, nb)
        assert np.array_equal(orc.topk_in_pool(s, pool, 8, k), orc.topk(s, k))


def test_pool_on_a_cache_matches_the_score_form(orc):
    cache = _small_cache(orc, B=2, cap=300)
    g = np.random.default_rng(24)
    for b, n in enumerate((300, 131)):
        keys = _bf16_int(g.integers(-8, 9, (n, 64)))
        orc.kv_append(cache, np.zeros((n, 576), np.float32), np.array([0] * (b + 1) + [n] * (2 - b), np.int32),
                      None, keys)
    q = _bf16_int(g.integers(-8, 9, (2, 4, 64)))
    q2 = _bf16_int(g.integers(-8, 9, (2, 4, 64)))
    pool = orc.indexer_pool(cache, q, 8, 16)
    out = orc.indexer_topk_in_pool(cache, q2, pool, 8, 50)
    for b, n in enumerate((300, 131)):
        keys = cache.idx_keys[b, :n]
        assert np.array_equal(pool[b], orc.pool_blocks(orc.indexer_scores(keys, q[b]), 8, 16))
        assert np.array_equal(out[b], orc.topk_in_pool(orc.indexer_scores(keys, q2[b]), pool[b], 8, 50))


# ---------------------------------------------------------------- attention

def _attn_cache(orc, entries, group=32):
    """Cache holding the given fp32 entries for one sequence."""
    n = entries.shape[0]
    c = orc.Cache.empty(1, n, 576, 64, group, 0, 64)
    orc.kv_append(c, entries, np.array([0, n], np.int32), None, np.zeros((n, 64), np.uint16))
    return c


def test_attention_equal_logits_gives_mean(orc):
    g = np.random.default_rng(10)
    c = _attn_cache(orc, g.standard_normal((6, 576)).astype(np.float32))
    idx = np.array([[0, 2, 5, -1]], np.int32)
    swa = _bf16_int(g.integers(-3, 4, (1, 4, 576)))
    out, lse = orc.sparse_attn(c, np.zeros((1, 2, 576), np.float32), idx, swa, 1 / 24,
                               swa_len=np.array([2], np.int32))
    vals = [orc.dequantize_row(c.k_codes[0, j], c.k_scales[0, j], 576, 32)[:512] for j in (0, 2, 5)]
    vals += [(swa[0, s, :512].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
             for s in range(2)]
    assert np.allclose(out[0, 0], np.mean(vals, axis=0), rtol=0, atol=1e-14)
    assert lse[0, 1] == pytest.approx(math.log(5), abs=1e-14)


def test_attention_single_key_and_dominant_key(orc):
    g = np.random.default_rng(11)
    ent = g.standard_normal((3, 576)).astype(np.float32)
    c = _attn_cache(orc, ent)
    deq = [orc.dequantize_row(c.k_codes[0, j], c.k_scales[0, j], 576, 32) for j in range(3)]
    swa = np.zeros((1, 1, 576), np.uint16)
    q = g.standard_normal((1, 1, 576)).astype(np.float32)
    out, lse = orc.sparse_attn(c, q, np.array([[1]], np.int32), swa, 0.5,
                               swa_len=np.array([0], np.int32))
    assert np.array_equal(out[0, 0], deq[1][:512])
    assert lse[0, 0] == pytest.approx(0.5 * float(q[0, 0].astype(np.float64) @ deq[1]), rel=1e-13)
    # make key 2 dominate by > 60 in logit: the others weigh <= 2 e^-60
    qd = (deq[2] / np.dot(deq[2], deq[2]) * 200.0).astype(np.float32)[None, None]
    out, _ = orc.sparse_attn(c, qd, np.array([[0, 1, 2]], np.int32), swa, 1.0,
                             swa_len=np.array([0], np.int32))
    l = [float(qd[0, 0].astype(np.float64) @ d) for d in deq]
    assert l[2] - max(l[0], l[1]) > 60
    assert np.allclose(out[0, 0], deq[2][:512], rtol=0, atol=1e-24)


def test_attention_lse_merge_and_permutation(orc):
    g = np.random.default_rng(12)
    c = _attn_cache(orc, g.standard_normal((20, 576)).astype(np.float32))
    q = g.standard_normal((1, 3, 576)).astype(np.float32)
    swa = _bf16_int(g.integers(-4, 5, (1, 8, 576)))
    idx = np.array([[1, 4, 7, 11, 19]], np.int32)
    joint, lj = orc.sparse_attn(c, q, idx, swa, 1 / 24, swa_len=np.array([8], np.int32))
    sp, ls = orc.sparse_attn(c, q, idx, swa, 1 / 24, swa_len=np.array([0], np.int32))
    sw, lw = orc.sparse_attn(c, q, np.full((1, 5), -1, np.int32), swa, 1 / 24,
                             swa_len=np.array([8], np.int32))
    m = np.maximum(ls, lw)
    wa, wb = np.exp(ls - m), np.exp(lw - m)
    merged = (sp * wa[..., None] + sw * wb[..., None]) / (wa + wb)[..., None]
    assert np.allclose(joint, merged, rtol=1e-12, atol=1e-14)
    assert np.allclose(lj, m + np.log(wa + wb), rtol=1e-13)
    perm, lp = orc.sparse_attn(c, q, idx[:, ::-1].copy(), swa, 1 / 24, swa_len=np.array([8], np.int32))
    assert np.allclose(perm, joint, rtol=1e-13, atol=1e-15) and np.allclose(lp, lj, rtol=1e-14)


def test_attention_out_of_range_indices_skipped_and_empty(orc):
    g = np.random.default_rng(13)
    c = _attn_cache(orc, g.standard_normal((4, 576)).astype(np.float32))
    q = g.standard_normal((1, 2, 576)).astype(np.float32)
    swa = np.zeros((1, 2, 576), np.uint16)
    a, la = orc.sparse_attn(c, q, np.array([[0, 9, -5, 2]], np.int32), swa, 0.1,
                            swa_len=np.array([0], np.int32))
    b, lb = orc.sparse_attn(c, q, np.array([[0, 2]], np.int32), swa, 0.1,
                            swa_len=np.array([0], np.int32))
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    e, le = orc.sparse_attn(c, q, np.array([[-1]], np.int32), swa, 0.1,
                            swa_len=np.array([0], np.int32))
    assert np.all(e == 0) and np.all(np.isneginf(le))


# ---------------------------------------------------------------- modes

def test_modes_reindex_and_reuse_reproduce_full(orc):
    import synth
    w = synth.scaled(synth.WORKLOADS["tiny_t4096"], batch=2, entries=300, prefill_tokens=None,
                     entry_law="normal", layers=("full", "reindex", "reuse"))
    cache = orc.Cache.empty(2, 310, 576, 64, 32, 0, 64)
    ents = np.concatenate([synth.cache_entries(w, b) for b in range(2)])
    keys = np.concatenate([synth.cache_idx_keys(w, b) for b in range(2)])
    orc.kv_append(cache, ents, np.array([0, 300, 600], np.int32), None, keys)
    st = synth.step_inputs(w)
    Wc = synth.w_comp(w)
    # give the reindex layer the full layer's indexer query, the reuse layer its q and window
    q_idx = [st.q_idx[0], st.q_idx[0], None]
    q = [st.q[0], st.q[1], st.q[0]]
    rings = [st.swa_ring[0].copy(), st.swa_ring[1].copy(), st.swa_ring[0].copy()]
    rows = [st.swa_row[0], st.swa_row[1], st.swa_row[0]]
    outs, lses, idxs = orc.layer_group_decode(cache, w.layers, st.token, st.idx_row, Wc, q, q_idx,
                                              rings, rows, 64, 1 / 24)
    assert np.array_equal(idxs[0], idxs[1]) and np.array_equal(idxs[2], idxs[1])
    assert np.array_equal(outs[2], outs[0]) and np.array_equal(lses[2], lses[0])
    assert not np.array_equal(outs[1], outs[0])
    assert list(cache.n_tokens) == [601, 601]


def test_modes_with_candidate_pool(orc):
    """The layer group with the hierarchical indexer: a pool holding every
    block changes nothing; a small pool confines the reindex layer's
    selection to the full layer's pool blocks."""
    import synth
    w = synth.scaled(synth.WORKLOADS["tiny_t4096"], batch=2, entries=300, prefill_tokens=None,
                     entry_law="normal", layers=("full", "reindex", "reuse"))
    ents = np.concatenate([synth.cache_entries(w, b) for b in range(2)])
    keys = np.concatenate([synth.cache_idx_keys(w, b) for b in range(2)])
    st = synth.step_inputs(w)
    Wc = synth.w_comp(w)
    res = {}
    for name, pool in (("none", None), ("all", (2048, 8)), ("small", (6, 8))):
        cache = orc.Cache.empty(2, 310, 576, 64, 32, 0, 64)
        orc.kv_append(cache, ents, np.array([0, 300, 600], np.int32), None, keys)
        rings = [r.copy() for r in st.swa_ring]
        res[name] = orc.layer_group_decode(cache, w.layers, st.token, st.idx_row, Wc, st.q, st.q_idx,
                                           rings, st.swa_row, 40, 1 / 24, pool=pool)
        if name == "small":
            cand = orc.indexer_pool(cache, st.q_idx[0], 8, 6)
    for a, b in zip(res["none"][2], res["all"][2]):
        assert np.array_equal(a, b)
    assert np.array_equal(res["small"][2][0], res["none"][2][0])          # full layer: unchanged
    assert not np.array_equal(res["small"][2][1], res["none"][2][1])
    for b in range(2):
        allowed = {8 * int(p) + r for p in cand[b] if p >= 0 for r in range(8)}
        sel = res["small"][2][1][b]
        assert set(sel[sel >= 0].tolist()) <= allowed and np.sum(sel >= 0) == 40



# ---------------------------------------------------------------- CED projection and the layer plan

def _bf16_bits(x):
    """bf16 bits of values that bf16 holds exactly (small integers, powers of two)."""
    a = np.asarray(x, np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), a), "not exact in bf16"
    return bits


def test_ced_project_identity_and_one_hot(orc):
    g = np.random.default_rng(500)
    h = g.integers(-8, 9, (5, 600)).astype(np.float32)
    eye = np.zeros((576, 600), np.float32)
    eye[np.arange(576), np.arange(576)] = 1
    assert np.array_equal(orc.ced_project(_bf16_bits(h), _bf16_bits(eye)), h[:, :576])
    # a one-hot hidden state picks one input column of w: out[n] = w[n][j]
    # (a transposed operand would pick row j instead)
    w = g.integers(-4, 5, (576, 600)).astype(np.float32)
    for j in (0, 17, 599):
        e = np.zeros((1, 600), np.float32)
        e[0, j] = 1
        assert np.array_equal(orc.ced_project(_bf16_bits(e), _bf16_bits(w))[0], w[:, j])


def test_ced_project_rank_one_and_linearity(orc):
    g = np.random.default_rng(501)
    dm = 256
    a = g.integers(-3, 4, 576).astype(np.float32)
    b = g.integers(-3, 4, dm).astype(np.float32)
    h = g.integers(-8, 9, (4, dm)).astype(np.float32)
    w = np.outer(a, b)                                 # w[n][k] = a[n] b[k]
    got = orc.ced_project(_bf16_bits(h), _bf16_bits(w))
    hb = [sum(int(x) * int(y) for x, y in zip(row, b)) for row in h]
    assert np.array_equal(got, np.array([[float(s * int(an)) for an in a] for s in hb], np.float32))
    h2 = g.integers(-8, 9, (4, dm)).astype(np.float32)
    w2 = g.integers(-4, 5, (576, dm)).astype(np.float32)
    lhs = orc.ced_project(_bf16_bits(h + h2), _bf16_bits(w2))
    rhs = orc.ced_project(_bf16_bits(h), _bf16_bits(w2)) + orc.ced_project(_bf16_bits(h2), _bf16_bits(w2))
    assert np.array_equal(lhs, rhs)


def test_ced_project_brute_force_and_rounding(orc):
    g = np.random.default_rng(502)
    # tiny integer case against exact integer arithmetic
    h = g.integers(-8, 9, (3, 40))
    w = g.integers(-4, 5, (7, 40))
    want = np.array([[sum(int(h[r, k]) * int(w[n, k]) for k in range(40)) for n in range(7)] for r in range(3)])
    assert np.array_equal(orc.ced_project(_bf16_bits(h), _bf16_bits(w)), want.astype(np.float32))
    # general bf16 inputs: within one fp32 rounding of the exact sum (math.fsum)
    hb = (g.standard_normal((2, 300)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = (g.standard_normal((5, 300)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    hv = (hb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wv = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = orc.ced_project(hb, wb)
    for r in range(2):
        for n in range(5):
            terms = hv[r] * wv[n]
            exact = math.fsum(terms)
            bound = abs(exact) * 2.0 ** -24 + 300 * 2.0 ** -53 * np.abs(terms).sum()
            assert abs(float(got[r, n]) - exact) <= bound


def test_csa2_plan_matches_the_pages(orc):
    g = GOLD["csa2_full_layers"]
    plan = orc.csa2_plan()
    enc, dec = plan[:3], plan[3]
    assert len(plan) == 4                                       # 4 stored copies
    assert all(m == g["encoder_group"] for _, _, m in enc)
    assert dec[2] == g["decoder_first"] + g["decoder_rest"] * g["decoder_rest_groups"]
    modes = [m for _, _, ms in plan for m in ms]
    assert modes.count("full") == g["printed_full"] and len(modes) == 38
    kv = GOLD["global_kv_per_token"]
    assert [r for _, r, _ in plan] == [kv["encoder_ratio"]] * kv["encoder_copies"] + \
        [kv["decoder_ratio"]] * kv["decoder_copies"]


def test_synth_plan_is_the_oracle_plan(orc):
    # the GPU workloads take the layer plan from synth; it must be the plan
    # the oracle follows and the page's counts
    import synth
    g = GOLD["csa2_full_layers"]
    assert [(n, r, list(m)) for n, r, m in synth.CSA2_PLAN] == [(n, r, list(m)) for n, r, m in orc.csa2_plan()]
    modes = [m for _, _, ms in synth.CSA2_PLAN for m in ms]
    assert modes.count("full") == g["printed_full"] and len(synth.CSA2_PLAN) == 4


def test_plan_caches_in_the_pages_formats_hold_900_bytes_per_token(orc):
    # live caches of the plan in the pages' formats (E2M1 + one E8M0 byte per
    # 16 channels, split value plane; FP4 indexer keys): per token, each
    # cache's value row (the 512 latent dims) and indexer key over its ratio
    kv = GOLD["global_kv_per_token"]
    total = 0.0
    for _, ratio, _ in orc.csa2_plan():
        c = orc.Cache.empty(1, 4, k_group=16, v_group=16, idx_dim=128, idx_format=1, k_format=1, ratio=ratio)
        row = c.v_codes[0, 0].nbytes + c.v_scales[0, 0].nbytes + c.idx_keys[0, 0].nbytes + c.idx_scales[0, 0].nbytes
        assert row == 360
        total += row / ratio
    assert total == kv["printed_estimate"]
    assert abs(total - kv["printed_reported"]) / kv["printed_reported"] < 0.02


def test_ratio_one_cache_stores_one_entry_per_token(orc):
    # the same entries appended to a ratio-1 and a ratio-2 cache: identical
    # planes, n_tokens m vs 2m; attention with the window length given is equal
    g = np.random.default_rng(503)
    rows = g.standard_normal((30, 576)).astype(np.float32)
    keys = g.integers(-8, 9, (30, 64)).astype(np.float32)
    keys = (keys.view(np.uint32) >> 16).astype(np.uint16)
    c1 = orc.Cache.empty(1, 40, k_group=32, idx_dim=64, ratio=1)
    c2 = orc.Cache.empty(1, 40, k_group=32, idx_dim=64, ratio=2)
    cu = np.array([0, 30], np.int32)
    orc.kv_append(c1, rows, cu, None, keys)
    orc.kv_append(c2, rows, cu, None, keys)
    assert c1.n_tokens[0] == 30 and c2.n_tokens[0] == 60
    assert np.array_equal(c1.entries(), c2.entries())
    for name in ("k_codes", "k_scales", "idx_keys"):
        assert np.array_equal(getattr(c1, name), getattr(c2, name))
    # a ratio-1 cache takes entries at any token count; the compressor is refused
    orc.kv_append(c1, rows[:1], np.array([0, 1], np.int32), None, keys[:1])
    assert c1.n_tokens[0] == 31 and c1.status[0] == 0
    with pytest.raises(ValueError):
        orc.kv_append(c1, rows[:2], np.array([0, 2], np.int32), np.zeros((576, 1152), np.float32), keys[:2])
    q = g.standard_normal((1, 8, 576)).astype(np.float32)
    idx = np.array([[0, 5, 29, -1]], np.int32)
    ring = (g.standard_normal((1, 16, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sl = np.array([9], np.int32)
    c1.n_tokens[0] = 30
    o1, l1 = orc.sparse_attn(c1, q, idx, ring, 0.05, swa_len=sl)
    o2, l2 = orc.sparse_attn(c2, q, idx, ring, 0.05, swa_len=sl)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # without swa_len the window length is the token count: 16 here (ring full)
    o3, _ = orc.sparse_attn(c1, q, idx, ring, 0.05)
    o4, _ = orc.sparse_attn(c1, q, idx, ring, 0.05, swa_len=np.array([16], np.int32))
    assert np.array_equal(o3, o4)


def test_model_decode_is_the_plan_of_layer_groups(orc):
    # a tiny two-cache plan: an encoder group and the decoder group; each
    # group's results are those of its own layer group, the decoder's new
    # entry being the CED projection of the hidden state
    g = np.random.default_rng(504)
    B, dm = 2, 64
    enc = orc.Cache.empty(B, 64, k_group=32, idx_dim=64)
    dec = orc.Cache.empty(B, 64, k_group=32, idx_dim=64, ratio=1)
    for c in (enc, dec):
        orc.kv_append(c, g.standard_normal((B * 20, 576)).astype(np.float32), np.array([0, 20, 40], np.int32),
                      None, (g.integers(-8, 9, (B * 20, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    plan = [("encoder0", 2, ["full", "reuse"]), ("decoder", 1, ["full", "reuse", "reindex", "reuse"])]
    W = (g.standard_normal((576, 1152)) * 0.02).astype(np.float32)
    hid = _bf16_bits(g.integers(-8, 9, (B, dm)).astype(np.float32))
    wced = _bf16_bits(g.integers(-4, 5, (576, dm)).astype(np.float32) * np.float32(2.0 ** -6))
    groups, twins = [], []
    for (name, ratio, modes), c in zip(plan, (enc, dec)):
        n = len(modes)
        grp = dict(cache=c, modes=modes, idx_row=(g.integers(-8, 9, (B, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16),
                   q=[g.standard_normal((B, 8, 576)).astype(np.float32) for _ in range(n)],
                   q_idx=[None if m == "reuse" else (g.integers(-8, 9, (B, 2, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for m in modes],
                   rings=[np.zeros((B, 8, 576), np.uint16) for _ in range(n)],
                   swa_rows=[g.standard_normal((B, 576)).astype(np.float32) for _ in range(n)])
        if ratio == 1:
            grp.update(ced_h=hid, ced_w=wced)
        else:
            grp.update(token=g.standard_normal((B, 576)).astype(np.float32), w_comp=W)
        groups.append(grp)
        twin = dict(grp, cache=orc.Cache(**{k: (v.copy() if isinstance(v, np.ndarray) else v)
                                            for k, v in c.__dict__.items()}),
                    rings=[r.copy() for r in grp["rings"]])
        twins.append(twin)
    res = orc.model_decode(groups, 16, 0.05, pool=(4, 2))
    # the encoder group by itself
    t = twins[0]
    o, l, i = orc.layer_group_decode(t["cache"], t["modes"], t["token"], t["idx_row"], t["w_comp"], t["q"],
                                     t["q_idx"], t["rings"], t["swa_rows"], 16, 0.05)
    assert all(np.array_equal(a, b) for a, b in zip(o, res[0][0]))
    # the decoder group: entries-mode append of the projected rows, pooled reindex
    t = twins[1]
    rows = orc.ced_project(hid, wced)
    o, l, i = orc.layer_group_decode(t["cache"], t["modes"], rows, t["idx_row"], None, t["q"], t["q_idx"],
                                     t["rings"], t["swa_rows"], 16, 0.05, pool=(4, 2))
    assert all(np.array_equal(a, b) for a, b in zip(o, res[1][0]))
    assert all(np.array_equal(a, b) for a, b in zip(i, res[1][2]))
    assert dec.n_tokens.tolist() == [21, 21] and enc.n_tokens.tolist() == [41, 41]
    assert np.array_equal(dec.k_codes, t["cache"].k_codes)
