"""Pins of the oracle against things other than itself: format specs, library
routines, closed forms, brute force and the constants the pages print.

CPU only.  A plausible slip in the oracle (a dropped term, a wrong sign, an
off-by-one in visibility, a transposed operand) fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codec
from oracle import csa as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs
def _all_e4m3_values():
    c = np.arange(256, dtype=np.uint8)
    return c, codec.e4m3_decode(c)


def test_e4m3_decode_matches_torch_float8():
    c, v = _all_e4m3_values()
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(v) & np.isnan(ref)
    assert np.all(both_nan | (v == ref))
    assert np.array_equal(np.signbit(v[~both_nan]), np.signbit(ref[~both_nan]))


def test_e4m3_anchor_values_of_the_spec():
    _, v = _all_e4m3_values()
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert v[0x38] == 1.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:0x7F]) > 0)          # positive codes are monotone


def _brute_nearest(x, table):
    """Nearest finite table value, ties to the even code (code & 1 == 0)."""
    out = []
    for xv in x:
        a = abs(xv)
        best = None
        for code, tv in table:
            d = abs(a - tv)
            key = (d, code & 1)
            if best is None or key < best[0]:
                best = (key, code)
        out.append(best[1] | (0x80 if math.copysign(1.0, xv) < 0 and len(table) > 16 else 0)
                   | (0x8 if math.copysign(1.0, xv) < 0 and len(table) <= 16 else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_is_nearest_even_by_brute_force():
    c, v = _all_e4m3_values()
    table = [(int(k), float(v[k])) for k in range(0x7F)]     # positive finite
    rng = np.random.default_rng(1)
    mids = (v[1:0x7E] + v[2:0x7F]) / 2.0                      # exact midpoints
    x = np.concatenate([rng.uniform(-500, 500, 300), rng.normal(0, 0.01, 300), mids, -mids,
                        v[:0x7F], [0.0, -0.0, 449.0, 1e6, -1e6]])
    got = codec.e4m3_encode(x)
    assert np.array_equal(got, _brute_nearest(x, table))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 1e-3, 20000)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3_encode(x.astype(np.float64)), ref)


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e30, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codec.bf16_encode(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codec.bf16_decode(ref), back)


def test_e2m1_table_and_brute_force():
    v = codec.e2m1_decode(np.arange(16))
    assert list(v[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]     # OCP MX v1.0 table
    assert list(v[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    table = [(k, float(v[k])) for k in range(8)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-8, 8, 500), mids, [-m for m in mids], [7.0, 100.0]])
    assert np.array_equal(codec.e2m1_encode(x), _brute_nearest(x, table))


def test_fp4_to_fp8_dequant_is_lossless():
    """The FP4 QAT section of the llm-tech overview: E2M1 -> E4M3 loses nothing
    (two more exponent bits).  Every E2M1 magnitude times 2^e, for the shifts
    that keep it inside the E4M3 range, is an E4M3 value."""
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    assert g["fp4_to_fp8_dequant_lossless"]["value"] is True
    e2 = codec.e2m1_decode(np.arange(16))
    for e in range(-8, 7):
        x = e2 * 2.0 ** e
        assert np.array_equal(codec.e4m3_decode(codec.e4m3_encode(x)), x)


def test_fp8_row_scale_is_smallest_power_of_two():
    rng = np.random.default_rng(5)
    amax = np.concatenate([rng.lognormal(0, 4, 2000), 448.0 * 2.0 ** np.arange(-10, 10),
                           np.nextafter(448.0 * 2.0 ** np.arange(-10, 10), np.inf)])
    s = codec.fp8_row_scale(amax)
    for a, sv in zip(amax, s):
        e = -200
        while a > 448.0 * 2.0 ** e:                       # brute-force search
            e += 1
        assert sv == 2.0 ** max(e, -126)
    assert codec.fp8_row_scale([0.0])[0] == 1.0


def test_mxfp4_scale_and_elements_brute_force():
    rng = np.random.default_rng(6)
    x = (rng.normal(0, 1, (64, 64)) * rng.lognormal(0, 3, (64, 1))).astype(np.float32)
    codes, e8 = codec.mxfp4_encode(x)
    e2 = codec.e2m1_decode(np.arange(8))
    for r in range(64):
        for b in range(2):
            blk = x[r, 32 * b: 32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            E = -300
            while 2.0 ** (E + 1 + 2) <= amax:            # largest E with 2^(E+2) <= amax
                E += 1
            assert int(e8[r, b]) - 127 == E
            for i in range(32):                         # nearest of the scaled table
                a = abs(blk[i]) / 2.0 ** E
                d = np.abs(e2 - a)
                cand = np.flatnonzero(d == d.min())
                want = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
                assert codes[r, 32 * b + i] & 7 == want
    deq = codec.mxfp4_decode(codes, e8)
    assert np.all(np.abs(deq) <= 6.0 * np.ldexp(1.0, np.repeat(e8.astype(int) - 127, 32, 1)))


def test_kv_row_layout_is_about_half_of_bf16():
    """llm-tech overview: RoPE dims BF16 + rest FP8 roughly halves the KV volume."""
    assert O.row_bytes("fp8", 512, 64) == 576
    assert 0.5 <= O.row_bytes("fp8", 512, 64) / (2 * 512) < 0.6
    rng = np.random.default_rng(7)
    v = rng.normal(0, 1, (32, 512))
    rows, s = O.pack_rows(v, "fp8", 64)
    back = O.unpack_rows(rows, s, "fp8", 512, 64)
    # RoPE dims are exactly BF16 of the values; bulk within half an E4M3 step
    assert np.array_equal(back[:, 448:], codec.bf16_decode(codec.bf16_encode(v[:, 448:])))
    assert np.all(np.abs(back[:, :448] - v[:, :448]) <= np.abs(v[:, :448]) / 16 + s[:, None] * 2.0 ** -10)


# -------------------------------------------------------------- compressor
def test_compress_m1_is_identity():
    x = synth.normal(0, 2, (37, 16))
    g = synth.normal(0, 6, (16,)) * 0.02
    assert np.array_equal(O.compress(x, g, np.array([0.3]), 1), x)


def test_compress_zero_weights_is_block_mean_and_tail_dropped():
    x = synth.normal(0, 2, (4 * 9 + 3, 8))
    c = O.compress(x, np.zeros(8), np.zeros(4), 4)
    assert c.shape == (9, 8)
    np.testing.assert_allclose(c, x[:36].reshape(9, 4, 8).mean(axis=1), rtol=1e-14, atol=1e-15)


def test_compress_constant_block_is_that_constant():
    x = np.repeat(synth.normal(0, 3, (5, 1, 8)), 4, axis=1).reshape(20, 8)
    c = O.compress(x, synth.normal(0, 6, (8,)), synth.normal(0, 7, (4,)), 4)
    np.testing.assert_allclose(c, x[::4], rtol=1e-14, atol=1e-15)


def test_compress_basis_vectors_give_softmax_weights():
    m, D = 4, 8
    g = np.array([0.5, -1.0, 2.0, 0.1, 0, 0, 0, 0])
    b = np.array([0.2, 0.3, -0.4, 1.0])
    x = np.eye(D)[:m]
    a = g[:m] + b
    want = [math.exp(ai) / sum(math.exp(aj) for aj in a) for ai in a]
    c = O.compress(x, g, b, m)[0]
    np.testing.assert_allclose(c[:m], want, rtol=1e-14)
    assert np.all(c[m:] == 0)


def test_compress_weights_depend_on_the_token_not_just_the_slot():
    """Not average pooling (kenelite analysis 5.2): permuting the tokens of a block
    with zero slot bias permutes nothing in the output, but changing one token's
    gate response changes the weights."""
    x = synth.normal(0, 11, (4, 6))
    g = synth.normal(0, 12, (6,))
    c1 = O.compress(x, g, np.zeros(4), 4)
    c2 = O.compress(x[[2, 0, 3, 1]], g, np.zeros(4), 4)
    np.testing.assert_allclose(c1, c2, rtol=1e-13)
    assert not np.allclose(c1, x.mean(axis=0, keepdims=True))


# ------------------------------------------------------------------ indexer
def test_indexer_basis_keys_closed_form():
    q = synth.normal(0, 20, (3, 5))
    w = synth.normal(0, 21, (3,))
    s = O.indexer_scores(q, w, np.eye(5))
    want = [sum(w[h] * max(0.0, q[h, j]) for h in range(3)) for j in range(5)]
    np.testing.assert_allclose(s, want, rtol=1e-15)


def test_indexer_brute_force_tiny():
    q = synth.normal(0, 22, (2, 4))
    w = synth.normal(0, 23, (2,))
    k = synth.normal(0, 24, (7, 4))
    s = O.indexer_scores(q, w, k)
    for j in range(7):
        acc = 0.0
        for h in range(2):
            d = 0.0
            for i in range(4):
                d += q[h, i] * k[j, i]
            acc += w[h] * (d if d > 0 else 0.0)
        assert abs(s[j] - acc) <= 1e-14 * (1 + abs(acc))


def test_indexer_relu_blocks_negative_heads():
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[-2.0, 3.0]])
    assert O.indexer_scores(q, np.array([5.0, 7.0]), k)[0] == 21.0


# --------------------------------------------------------------------- top-k
def test_topk_equals_full_sort_tiny_with_ties():
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(0, 40))
        k = int(rng.integers(1, 20))
        s = rng.integers(-3, 4, n).astype(np.float64) * 0.5      # many ties, exact zeros
        full = sorted(range(n), key=lambda j: (-s[j], j))
        want = sorted(full[:k]) + [-1] * (k - min(k, n))
        assert list(O.topk_select(s, k)) == want


def test_topk_k_at_least_n_takes_everything():
    s = synth.normal(0, 25, (9,))
    assert list(O.topk_select(s, 12)) == list(range(9)) + [-1] * 3


# ------------------------------------------------------------------ attention
def _sdpa(q, k, v, mask, tau):
    """torch CPU float64 scaled_dot_product_attention, q [T,H,D], k/v [S,D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1,H,T,D]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[1], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask)[None, None], scale=tau)
    return o[0].permute(1, 0, 2).numpy()


def _csa_pipeline(x, q, m, k, W, sink, tau, gate, bias):
    """Oracle CSA layer on float64 data: compress -> indexer -> top-k -> attention."""
    T = x.shape[0]
    ent = O.compress(x, gate, bias, m)
    N = ent.shape[0]
    qI = synth.normal(0, 30, (T, 2, x.shape[1]))
    w = synth.normal(0, 31, (T, 2))
    sel = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        nt = int(O.n_visible(t, m, N))
        sel[t] = O.topk_select(O.indexer_scores(qI[t], w[t], ent[:nt]), k)
    return O.csa_prefill(q, ent, sel, x, W, sink, tau)


def test_csa_m1_full_topk_no_window_no_sink_is_dense_causal_attention():
    T, H, D = 48, 3, 16
    x = synth.normal(0, 40, (T, D))
    q = synth.normal(0, 41, (T, H, D))
    tau = 1 / math.sqrt(D)
    o, _ = _csa_pipeline(x, q, 1, T, 0, None, tau, synth.normal(0, 42, (D,)), np.zeros(1))
    mask = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(o, _sdpa(q, x, x, mask, tau), rtol=1e-12, atol=1e-13)


def test_hca_m_prime_equal_T_is_single_entry_attention():
    T, H, D = 64, 2, 8
    x = synth.normal(0, 43, (T, D))
    q = synth.normal(0, 44, (T, H, D))
    ent = O.compress(x, synth.normal(0, 45, (D,)), synth.normal(0, 46, (T,)), T)
    o, lse = O.hca_prefill(q, ent, T, x, 0, None, 0.3)
    np.testing.assert_array_equal(o[:-1], 0.0)
    assert np.all(lse[:-1] == -np.inf)
    np.testing.assert_allclose(o[-1], np.repeat(ent, H, axis=0), rtol=1e-14)


def test_hca_m1_no_window_is_dense_causal_attention():
    T, H, D = 40, 2, 8
    x = synth.normal(0, 47, (T, D))
    q = synth.normal(0, 48, (T, H, D))
    ent = O.compress(x, np.zeros(D), np.zeros(1), 1)
    o, _ = O.hca_prefill(q, ent, 1, x, 0, None, 0.5)
    np.testing.assert_allclose(o, _sdpa(q, x, x, np.tril(np.ones((T, T), dtype=bool)), 0.5),
                               rtol=1e-12, atol=1e-13)


def test_no_visible_entries_is_sliding_window_attention():
    T, H, D, W = 30, 2, 8, 5
    x = synth.normal(0, 49, (T, D))
    q = synth.normal(0, 50, (T, H, D))
    ent = O.compress(x, np.zeros(D), np.zeros(64), 64)          # T < 64 -> no entries
    assert ent.shape[0] == 0
    o, _ = O.hca_prefill(q, ent, 64, x, W, None, 0.4)
    i, j = np.indices((T, T))
    band = (j <= i) & (j > i - W)
    np.testing.assert_allclose(o, _sdpa(q, x, x, band, 0.4), rtol=1e-12, atol=1e-13)


def test_window_and_entries_equal_brute_force_concatenated_softmax():
    T, H, D, W, m, k = 24, 2, 4, 6, 4, 3
    x = synth.normal(0, 51, (T, D))
    q = synth.normal(0, 52, (T, H, D))
    ent = O.compress(x, synth.normal(0, 53, (D,)), synth.normal(0, 54, (m,)), m)
    rng = np.random.default_rng(9)
    sel = np.full((T, k), -1)
    for t in range(T):
        nt = int(O.n_visible(t, m, ent.shape[0]))
        pick = np.sort(rng.permutation(nt)[:k])
        sel[t, :len(pick)] = pick
    sink = np.array([0.7, -0.2])
    o, _ = O.csa_prefill(q, ent, sel, x, W, sink, 0.5)
    for t in range(T):
        rows = [ent[j] for j in sel[t] if j >= 0] + [x[u] for u in range(max(0, t - W + 1), t + 1)]
        for h in range(H):
            logits = [0.5 * sum(q[t, h, d] * r[d] for d in range(D)) for r in rows]
            z = math.exp(sink[h]) + sum(math.exp(lv) for lv in logits)
            want = [sum(math.exp(lv) * r[d] for lv, r in zip(logits, rows)) / z for d in range(D)]
            np.testing.assert_allclose(o[t, h], want, rtol=1e-12, atol=1e-14)


def test_sink_closed_form():
    q = synth.normal(0, 55, (3, 8))
    E = synth.normal(0, 56, (10, 8))
    o0, lse0 = O.attend(q, E, None, 0.3)
    sig = np.array([-1.0, 0.0, 2.5])
    o1, lse1 = O.attend(q, E, sig, 0.3)
    z0 = np.exp(lse0)
    np.testing.assert_allclose(o1, o0 * (z0 / (z0 + np.exp(sig)))[:, None], rtol=1e-13)
    np.testing.assert_allclose(lse1, np.log(z0 + np.exp(sig)), rtol=1e-14)


def test_empty_set_and_sink_only():
    o, lse = O.attend(np.ones((2, 4)), np.zeros((0, 4)), None, 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    o, lse = O.attend(np.ones((2, 4)), np.zeros((0, 4)), np.array([0.5, -3.0]), 1.0)
    assert np.all(o == 0)
    np.testing.assert_allclose(lse, [0.5, -3.0])


def test_merge_of_disjoint_partials_equals_union_softmax():
    q = synth.normal(0, 57, (4, 8))
    A = synth.normal(0, 58, (7, 8))
    Wn = synth.normal(0, 59, (5, 8))
    sig = synth.normal(0, 60, (4,))
    op, lp = O.attend(q, A, None, 0.35)
    merged = O.swa_merge(q, Wn, op, lp, sig, 0.35)
    whole, _ = O.attend(q, np.concatenate([A, Wn]), sig, 0.35)
    np.testing.assert_allclose(merged, whole, rtol=1e-13, atol=1e-15)
    # merging with an empty partial (lse = -inf) is plain window attention + sink
    only_w, _ = O.attend(q, Wn, sig, 0.35)
    np.testing.assert_allclose(O.swa_merge(q, Wn, np.zeros((4, 8)), np.full(4, -np.inf), sig, 0.35),
                               only_w, rtol=1e-13)


def test_decode_equals_prefill_at_the_same_position():
    T, H, D, W, m = 37, 2, 8, 8, 4
    x = synth.normal(0, 61, (T, D))
    q = synth.normal(0, 62, (T, H, D))
    ent = O.compress(x, synth.normal(0, 63, (D,)), synth.normal(0, 64, (m,)), m)
    sig = np.array([0.1, -0.4])
    ring = np.zeros((W, D))
    for p in range(T):
        ring[p % W] = x[p]
    t = T - 1
    o_pre, _ = O.hca_prefill(q, ent, m, x, W, sig, 0.3)
    o_dec, _ = O.hca_decode(q[t], ent, m, ent.shape[0], ring, t, W, sig, 0.3)
    np.testing.assert_allclose(o_dec, o_pre[t], rtol=1e-14)
    sel = O.topk_select(synth.normal(0, 65, (ent.shape[0],)), 4)
    o_pre2, _ = O.csa_prefill(q, ent, np.tile(sel, (T, 1)), x, W, sig, 0.3)
    o_dec2, _ = O.csa_decode(q[t], ent, sel, ring, t, W, sig, 0.3)
    np.testing.assert_allclose(o_dec2, o_pre2[t], rtol=1e-14)


# ---------------------------------------------------------------- counting
def test_entry_counts_and_visibility_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    assert 10 ** 6 // g["hca_block_m_prime"]["value"] == g["hca_entries_at_1e6_tokens"]["value_approx"]
    cfg = synth.get_config
    assert cfg("csa_prefill_32k").m == g["csa_block_m"]["value"]
    assert cfg("hca_prefill_128k").m == g["hca_block_m_prime"]["value"]
    assert cfg("csa_prefill_32k").k == g["csa_topk_flash"]["value"]
    assert cfg("csa_decode_1m").k == g["csa_topk_pro"]["value"]
    assert all(c.W == g["sliding_window"]["value"] for c in synth.CONFIGS.values())
    assert cfg("csa_decode_1m").N == 262144 and cfg("hybrid_decode_1m").N_hca == 8192
    for T, m in [(2048, 4), (32768, 4), (131072, 128), (1000, 7)]:
        N = T // m
        nt = O.n_visible(np.arange(T), m, N)
        # sum_t min(N, floor((t+1)/m)) = m * N (N - 1) / 2 + N * (T - m N + 1)
        assert int(nt.sum()) == m * N * (N - 1) // 2 + N * (T - m * N + 1)
        assert nt[m - 2] == 0 and nt[m - 1] == 1 and nt[-1] == N


def test_generator_slices_are_consistent():
    full = synth.normal(3, 7, (101,))
    assert np.array_equal(synth.normal(3, 7, (40,), start=33), full[33:73])
    z = synth.normal(0, 1, (200000,))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


def test_decode_append_equals_prefill_compression_and_keeps_the_last_window():
    """Appending tokens one by one must leave the caches prefill builds: each
    closed block's entry equals the entry `compress` gives for the whole
    prefix (the block's tokens only), and the window slots hold the latest W
    positions, position p in slot p mod W."""
    rng = np.random.default_rng(21)
    T, D, m, W = 61, 16, 4, 8
    x = rng.standard_normal((T, D))
    g = rng.standard_normal(D) * 0.3
    b = rng.standard_normal(m) * 0.3
    p0, p1 = 6, 58                      # starts inside block 1, stops inside block 14
    entries, window = O.decode_append(x, g, b, m, W, p0, p1)
    full = O.compress(x[:p1], g, b, m)
    assert sorted(entries) == list(range(p0 // m, p1 // m))   # blocks closed by the steps: 1 .. 13
    for j, c in entries.items():
        np.testing.assert_allclose(c, full[j], rtol=1e-13, atol=1e-13)
    assert window == {p % W: p for p in range(p1 - W, p1)}
    # m' = 128 blocks: none closes before position 127; the window is the last W of the steps
    e2, w2 = O.decode_append(x, g, b, 128, W, 0, T)
    assert e2 == {} and sorted(w2.values()) == list(range(T - W, T))


# ------------------------------------------------------------ MXFP4 pins
def _mx_golden():
    return json.load(open(os.path.join(GOLDEN, "mxfp4_blocks.json")))


def test_mxfp4_decode_hand_worked_blocks():
    """OCP MX v1.0 decode of hand-worked blocks: an E8M0 byte e is exactly
    2^(e-127) and each element is its E2M1 table value times that scale
    (a bias of 128 or a wrong table entry fails here)."""
    for blk in _mx_golden()["decode_blocks"]:
        codes = np.array(blk["codes"], dtype=np.uint8)[None, :]
        got = codec.mxfp4_decode(codes, np.array([[blk["e8m0"]]], dtype=np.uint8))[0]
        if "values" in blk:
            want = np.array(blk["values"], dtype=np.float64)
        else:
            want = np.array([math.ldexp(v, blk["values_exp2"]) for v in blk["values_mant"]])
        assert np.array_equal(got, want), blk["note"]
        assert np.array_equal(np.signbit(got), np.signbit(want)), blk["note"]


def test_mxfp4_row_packing_puts_element_2i_in_the_low_nibble():
    """The stored MXFP4 row layout: byte i holds element 2i in its low nibble
    and element 2i+1 in its high nibble; one E8M0 byte per 32 elements (a
    nibble swap or a per-block scale mix-up fails here)."""
    row = _mx_golden()["packed_row"]
    v = np.array(row["values"], dtype=np.float64)[None, :]
    packed, e8 = O.pack_rows(v, "mxfp4")
    assert packed.tolist() == [row["bytes"]]
    assert e8.tolist() == [row["e8m0"]]
    back = O.unpack_rows(np.array([row["bytes"]], np.uint8), np.array([row["e8m0"]], np.uint8), "mxfp4", 64)
    assert np.array_equal(back, v)


def test_mxfp4_round_trip_is_the_nearest_scaled_e2m1_value():
    """decode(encode(x)) is, element by element, the nearest value of
    {+-2^E v : v an E2M1 magnitude} with E the block's shared exponent found
    by brute force (largest E with 2^(E+2) <= amax), ties to the even code,
    saturating at 6 * 2^E."""
    rng = np.random.default_rng(61)
    x = (rng.normal(0, 1, (24, 64)) * rng.lognormal(0, 2, (24, 1))).astype(np.float32).astype(np.float64)
    x[3, :32] = 0.0                                   # an all-zero block
    x[5, 7] = -0.0
    codes, e8 = codec.mxfp4_encode(x)
    got = codec.mxfp4_decode(codes, e8)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(x.shape[0]):
        for blk in range(2):
            seg = x[r, 32 * blk: 32 * blk + 32]
            amax = float(np.max(np.abs(seg)))
            if amax == 0.0:
                E = -127
            else:
                E = -300
                while 2.0 ** (E + 1 + 2) <= amax:
                    E += 1
            for i in range(32):
                a = abs(seg[i]) / 2.0 ** E
                best = min(range(8), key=lambda c: (abs(mags[c] - a), c & 1))
                want = math.copysign(mags[best] * 2.0 ** E, seg[i])
                assert got[r, 32 * blk + i] == want, (r, blk, i)


def test_kv_cache_is_about_two_percent_of_a_bf16_gqa8_cache():
    """kenelite analysis section 8: at long context the KV cache is about 2 % of
    a BF16 GQA-8, head-dim-128 cache.  Per token and per layer pair (CSA and
    HCA alternate: llm-tech overview) this layout stores a CSA entry (576-byte
    row + 4-byte scale) and an indexer key (64 FP8 + 4-byte scale) every m = 4
    tokens and an HCA entry every m' = 128 tokens; the sliding windows are a
    fixed 128 rows per layer and vanish per token at 1M."""
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    assert g["csa_hca_alternate"]["value"] is True
    base = g["kv_cache_vs_bf16_gqa8_hd128"]["baseline"]
    bf16_per_layer = 2 * base["kv_heads"] * base["head_dim"] * base["bytes_per_value"]    # K and V
    m, mh = g["csa_block_m"]["value"], g["hca_block_m_prime"]["value"]
    entry = O.row_bytes("fp8", 512, 64) + 4
    key = O.row_bytes("fp8", 64, 0) + 4
    T, W = 1 << 20, g["sliding_window"]["value"]
    csa = (T // m) * (entry + key) + W * entry
    hca = (T // mh) * entry + W * entry
    ratio = (csa + hca) / (2 * T * bf16_per_layer)
    assert abs(ratio - g["kv_cache_vs_bf16_gqa8_hd128"]["value_approx"]) < 0.005, ratio


# ------------------------------------------- RMSNorm and partial RoPE pins
def test_rms_norm_matches_torch_and_gives_unit_rms():
    """10100 analysis, section 3 item 1: RMSNorm of query / KV entries.
    Against torch's own rms_norm (float64) and the closed forms: with unit
    gain and eps = 0 every row has mean square 1; a constant row becomes
    sign * gain."""
    rng = np.random.default_rng(71)
    x = rng.normal(0, 3, (40, 64))
    gain = rng.normal(1, 0.1, 64)
    got = O.rms_norm(x, gain, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(gain), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)
    unit = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(unit * unit, axis=1), 1.0, rtol=1e-14)
    const = O.rms_norm(np.full((2, 64), -2.5), gain, 0.0)
    np.testing.assert_allclose(const, np.tile(-gain, (2, 1)), rtol=1e-14)


def _exact_theta(R):
    """Frequencies that are powers of two, so that every position * theta
    below is exact in binary32 and the angle algebra holds exactly."""
    return 2.0 ** -np.arange(R // 2, dtype=np.float64)


def test_rope_rotates_consecutive_pairs_of_the_trailing_dims_only():
    """Partial RoPE touches only the last R dims, pair by pair: a basis
    vector in the bulk is unchanged; one at dim D - R + 2i moves only within
    (D - R + 2i, D - R + 2i + 1), by the pair's angle; position 0 is the
    identity."""
    D, R = 16, 8
    theta = _exact_theta(R)
    for d in range(D):
        e = np.zeros((1, D)); e[0, d] = 1.0
        y = O.rope(e, [3], theta, R)[0]
        if d < D - R:
            assert np.array_equal(y, e[0])
            continue
        i = (d - (D - R)) // 2
        a = 3 * theta[i]
        pair = [D - R + 2 * i, D - R + 2 * i + 1]
        assert np.all(y[[k for k in range(D) if k not in pair]] == 0.0)
        if (d - (D - R)) % 2 == 0:
            np.testing.assert_allclose(y[pair], [math.cos(a), math.sin(a)], rtol=1e-15, atol=1e-16)
        else:
            np.testing.assert_allclose(y[pair], [-math.sin(a), math.cos(a)], rtol=1e-15, atol=1e-16)
    x = synth.normal(0, 72, (5, D))
    assert np.array_equal(O.rope(x, np.zeros(5), theta, R), x)


def test_rope_preserves_norms_and_scores_depend_on_relative_position_only():
    """Rotations preserve each pair's length, and the RoPE part of a score
    <R_p q, R_s k> equals <q, R_(s-p) k>: it depends on s - p only (exact
    here: the angles are exact binary32 products)."""
    D, R = 64, 16
    theta = _exact_theta(R)
    q = synth.normal(0, 73, (6, D))
    k = synth.normal(0, 74, (6, D))
    ps = np.array([0, 5, 17, 33, 100, 7])
    ss = np.array([3, 5, 40, 2, 100, 70])
    rq = O.rope(q, ps, theta, R)
    rk = O.rope(k, ss, theta, R)
    np.testing.assert_allclose(np.linalg.norm(rq[:, D - R:].reshape(6, -1, 2), axis=2),
                               np.linalg.norm(q[:, D - R:].reshape(6, -1, 2), axis=2), rtol=1e-14)
    lhs = np.sum(rq[:, D - R:] * rk[:, D - R:], axis=1)
    rel = O.rope(k, ss - ps, theta, R)
    rhs = np.sum(q[:, D - R:] * rel[:, D - R:], axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # composition: rotating by p then by s is rotating by p + s
    np.testing.assert_allclose(O.rope(O.rope(q, ps, theta, R), ss, theta, R), O.rope(q, ps + ss, theta, R),
                               rtol=1e-12, atol=1e-13)


def test_compressed_entry_takes_the_position_of_its_block_end():
    """A block of m equal tokens compresses to that token (softmax weights sum
    to 1), so after the post-processing its entry must equal the token
    post-processed at the block's last position (m-1, 2m-1, ...), the
    position at which the entry becomes visible to queries."""
    D, R, m = 32, 8, 4
    theta = _exact_theta(R)
    tok = synth.normal(0, 75, (5, 1, D))
    x = np.repeat(tok, m, axis=1).reshape(5 * m, D)
    gain = synth.normal(0, 76, (D,)) * 0.1 + 1.0
    c = O.compress(x, synth.normal(0, 77, (D,)), synth.normal(0, 78, (m,)), m)
    pos = O.entry_positions(5, m, pos0=8)
    assert list(pos) == [11, 15, 19, 23, 27]
    got = O.post_rows(c, pos, gain, 1e-6, theta, R)
    want = O.post_rows(tok[:, 0], pos, gain, 1e-6, theta, R)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # m = 1 gives every token its own position
    assert list(O.entry_positions(4, 1, pos0=3)) == [3, 4, 5, 6]


def test_restore_state_equals_the_uninterrupted_state():
    """Prefix reuse (kenelite analysis 16): restoring the entries of the
    complete blocks, recomputing the incomplete block and rebuilding the
    window from the last raw tokens gives the state that processing every
    position leaves: entries = compression of all complete blocks, the
    window = the last W positions, the tail = the incomplete block."""
    rng = np.random.default_rng(41)
    for m, W, P in [(4, 16, 103), (4, 16, 100), (128, 128, 700), (3, 8, 5), (4, 128, 64)]:
        D = 8
        x = rng.standard_normal((P + 40, D))
        g = rng.standard_normal(D) * 0.3
        b = rng.standard_normal(m) * 0.3
        p0 = (max(0, min(P - W, P)) // m) * m
        n_r = rng.integers(p0 // m, P // m + 1)              # restored blocks: at least those below p0
        restored = O.compress(x[: n_r * m], g, b, m)
        entries, window, tail = O.restore_state(restored, x[p0:P], g, b, m, W, p0)
        full = O.compress(x[:P], g, b, m)
        assert entries.shape == full.shape
        np.testing.assert_allclose(entries, full, rtol=0, atol=1e-12)
        e_dec, w_dec = O.decode_append(x, g, b, m, W, 0, P)
        assert window == {s: q for s, q in w_dec.items() if q >= P - W}
        assert sorted(window.values()) == list(range(max(0, P - W), P))
        assert tail == list(range((P // m) * m, P))
        if e_dec:
            np.testing.assert_allclose(entries[sorted(e_dec)], np.stack([e_dec[j] for j in sorted(e_dec)]), atol=1e-12)
