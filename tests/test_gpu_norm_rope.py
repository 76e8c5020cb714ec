"""GPU parity of the RMSNorm / partial-RoPE post-processing (csa_norm_rope)
that csa_compress_kv and csa_decode_append apply to stored rows and the
attention entry points apply to queries, against the oracle's post_rows.

Stored rows: every code must be the quantisation of a value within the
propagated float32 bound of the oracle's processed entry (compressor bound
carried through the norm and the rotation).  Queries: the oracle processes
the BF16 query values, rounds them back to BF16 and attends; the attention
tolerance is the one of the plain parity tests.
"""
import math

import numpy as np
import pytest

import synth
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _post(lib, D, rope_dims, gain=True, pos0=0, eps=1e-6, layer=0):
    """(library NormRope, float64 gain or None, float32 theta or None)."""
    g = None
    if gain:
        g = (1.0 + synth.tensor(0, "norm_gain", (D,), std=0.1, layer=layer)).astype(np.float32)
    th = Hx.rope_theta(rope_dims) if rope_dims else None
    nr = lib.NormRope(gain=None if g is None else Hx.to_dev(g), eps=eps, rope_dims=rope_dims,
                      theta=None if th is None else Hx.to_dev(th), pos0=pos0)
    return nr, (None if g is None else g.astype(np.float64)), th


def _check_post_rows(rows, sc, fmt, D, R, c, e, gain, eps, th, rope_dims, positions, max_frac=2e-3):
    cp = O.post_rows(c, positions, gain, eps, th, rope_dims)
    ep = Hx.post_error_bound(c, e, gain, eps, th, rope_dims)
    frac = Hx.check_compress(rows, sc, fmt, D, R, cp, ep)
    if fmt != "f32":
        assert frac <= max_frac, f"{frac:.2e} of codes differ from the oracle's packing"


# ================================================================ compress
POST_COMPRESS_CASES = [
    # name, tok fmt, store fmt, D, R (store), m, T, B, rope dims, gain, pos0
    ("csa_kv_bf16_fp8_D512_m4", "bf16", "fp8", 512, 64, 4, 1030, 2, 64, True, 0),
    ("hca_kv_bf16_fp8_D512_m128", "bf16", "fp8", 512, 64, 128, 128 * 9 + 5, 1, 64, True, 5000),
    ("f32_f32_D64_m4_cross_lane_pairs", "f32", "f32", 64, 0, 4, 2051, 2, 16, True, 3),
    ("f32_f32_D32_m7_rope_only", "f32", "f32", 32, 0, 7, 500, 1, 8, False, 0),
    ("idx_bf16_mxfp4_D64_m4_norm_only", "bf16", "mxfp4", 64, 0, 4, 2050, 1, 0, True, 0),
    ("f32_fp8_D64_R16_m4", "f32", "fp8", 64, 16, 4, 999, 2, 16, True, 1 << 20),
    # angles beyond 1.6e6 (the kernels' library-sincos fallback) next to smaller ones
    ("f32_f32_D64_m4_far_positions", "f32", "f32", 64, 0, 4, 999, 1, 16, True, 3_000_000),
    # m = 1: the packed quantise-only kernel (8 dims per lane)
    ("win_bf16_fp8_D512_m1", "bf16", "fp8", 512, 64, 1, 777, 1, 64, True, 100000),
    ("f32_fp8_D64_R16_m1", "f32", "fp8", 64, 16, 1, 777, 2, 16, True, 7),
    ("f32_f32_D32_m1", "f32", "f32", 32, 0, 1, 300, 1, 8, True, 0),
]


@pytest.mark.parametrize("name,tf,sf,D,R,m,T,B,rd,gain,pos0", POST_COMPRESS_CASES)
def test_compress_with_norm_rope(lib, name, tf, sf, D, R, m, T, B, rd, gain, pos0):
    x = synth.tensor(0, "kv", (B, T, D), rmsnorm=(tf == "bf16"), layer=9)
    g = synth.tensor(0, "gate", (D,), std=0.02, layer=9)
    b = synth.tensor(0, "bias", (m,), std=0.02, layer=9)
    if m == 1:
        g, b = np.zeros(D), np.ones(1)
    xd, xv = Hx.act(x, tf)
    N = T // m
    nr, gain64, th = _post(lib, D, rd, gain, pos0)
    out = lib.alloc_store(B, N + 2, D, sf, R, device=Hx.dev())
    lib.compress_kv(xd, m, Hx.to_dev(g.astype(np.float32)), Hx.to_dev(b.astype(np.float32)), out, out_row0=1,
                    post=nr)
    _sync()
    g32 = g.astype(np.float32).astype(np.float64)
    b32 = b.astype(np.float32).astype(np.float64)
    pos = O.entry_positions(N, m, pos0)
    for bi in range(B):
        rows = out.rows[bi, 1: 1 + N].cpu().numpy()
        sc = None if out.scales is None else out.scales[bi, 1: 1 + N].cpu().numpy()
        c = O.compress(xv[bi], g32, b32, m)
        e = None if m == 1 else Hx.compress_error_bound(xv[bi], g32, b32, m)
        _check_post_rows(rows, sc, sf, D, R, c, e, gain64, nr.eps, th, rd, pos)


def test_compress_post_none_and_zero_post_are_identical(lib):
    """A post-processing block with no gain and rope_dims = 0 stores the same
    bytes as no block at all."""
    import torch
    D, R, m, T = 512, 64, 4, 520
    x = synth.tensor(0, "kv", (1, T, D), rmsnorm=True, layer=10)
    xd, _ = Hx.act(x, "bf16")
    g = Hx.to_dev(synth.tensor(0, "gate", (D,), std=0.02).astype(np.float32))
    b = Hx.to_dev(synth.tensor(0, "bias", (m,), std=0.02).astype(np.float32))
    a = lib.alloc_store(1, T // m, D, "fp8", R, device=Hx.dev())
    c = lib.alloc_store(1, T // m, D, "fp8", R, device=Hx.dev())
    lib.compress_kv(xd, m, g, b, a)
    lib.compress_kv(xd, m, g, b, c, post=lib.NormRope())
    _sync()
    assert torch.equal(a.rows, c.rows) and torch.equal(a.scales, c.scales)


APPEND_POST_CASES = [
    # name, tok fmt, store fmt, D, R, m, tail rows, window slots, steps, rope dims
    ("csa_kv_bf16_fp8_D512_m4_window", "bf16", "fp8", 512, 64, 4, 4, 128, 140, 64),
    ("hca_kv_bf16_fp8_D512_m128", "bf16", "fp8", 512, 64, 128, 128, 0, 140, 64),
    ("f32_f32_D64_m3_window16", "f32", "f32", 64, 0, 3, 6, 16, 60, 16),
]


@pytest.mark.parametrize("name,tf,sf,D,R,m,Rt,W,steps,rd", APPEND_POST_CASES)
def test_decode_append_with_norm_rope(lib, name, tf, sf, D, R, m, Rt, W, steps, rd):
    """Tokens appended one per step with post-processing leave the bytes that
    prefill compression with the same post-processing (pos0 = 0) stores for
    every closed block; window rows are the processed tokens at their own
    positions, within the bound of the oracle's."""
    import torch
    p0s = [0, 5, m + 2]
    B = len(p0s)
    Tmax = max(p0s) + steps
    x = synth.tensor(0, "kv", (B, Tmax, D), rmsnorm=(tf == "bf16"), layer=11)
    g = synth.tensor(0, "gate", (D,), std=0.02, layer=11)
    bb = synth.tensor(0, "bias", (m,), std=0.02, layer=11)
    xd, xv = Hx.act(x, tf)
    gd, bd = Hx.to_dev(g.astype(np.float32)), Hx.to_dev(bb.astype(np.float32))
    nr, gain64, th = _post(lib, D, rd, True, 0, layer=11)
    ncap = Tmax // m + 2
    out = lib.alloc_store(B, ncap, D, sf, R, device=Hx.dev())
    out.rows.fill_(0xAB)
    win = None
    if W:
        win = lib.alloc_store(B, W, D, sf, R, device=Hx.dev())
        win.rows.fill_(0xCD)
    tail = torch.zeros((B, Rt, D), dtype=xd.dtype, device=Hx.dev())
    for b, p0 in enumerate(p0s):
        for q in range((p0 // m) * m, p0):
            tail[b, q % Rt] = xd[b, q]
    pos = torch.empty(B, dtype=torch.int64, device=Hx.dev())
    tok = torch.zeros((B, D), dtype=xd.dtype, device=Hx.dev())
    for st in range(steps):
        ps = [p0 + st for p0 in p0s]
        pos.copy_(torch.tensor(ps, dtype=torch.int64))
        for b, p in enumerate(ps):
            tok[b] = xd[b, p]
        lib.decode_append(tok, pos, tail, m, gd, bd, out, win, W, post=nr)
    ref = lib.alloc_store(B, ncap, D, sf, R, device=Hx.dev())
    lib.compress_kv(xd, m, gd, bd, ref, post=nr)
    _sync()
    g32 = g.astype(np.float32).astype(np.float64)
    b32 = bb.astype(np.float32).astype(np.float64)
    for b, p0 in enumerate(p0s):
        j0, j1 = p0 // m, (p0 + steps) // m
        assert j1 > j0
        assert torch.equal(out.rows[b, j0:j1], ref.rows[b, j0:j1]), "entry bytes differ from csa_compress_kv"
        sc = None
        if out.scales is not None:
            assert torch.equal(out.scales[b, j0:j1], ref.scales[b, j0:j1])
            sc = out.scales[b, j0:j1].cpu().numpy()
        c = O.compress(xv[b][j0 * m: j1 * m], g32, b32, m)
        e = Hx.compress_error_bound(xv[b][j0 * m: j1 * m], g32, b32, m)
        _check_post_rows(out.rows[b, j0:j1].cpu().numpy(), sc, sf, D, R, c, e, gain64, nr.eps, th, rd,
                         O.entry_positions(j1 - j0, m, j0 * m))
        keep = np.ones(ncap, bool)
        keep[j0:j1] = False
        assert np.all(out.rows[b].cpu().numpy()[keep] == 0xAB)
        if W:
            ps = np.arange(max(p0, p0 + steps - W), p0 + steps)       # the last W positions written
            slots = ps % W
            got = win.rows[b].cpu().numpy()[slots]
            gsc = None if win.scales is None else win.scales[b].cpu().numpy()[slots]
            _check_post_rows(got, gsc, sf, D, R, xv[b][ps], None, gain64, nr.eps, th, rd, ps)


# =============================================================== attention
def _attn_inputs(B, Tq, H, D, R, fmt, qf, n_kv, n_win, layer):
    q = synth.tensor(0, "q", (B, Tq, H, D), rmsnorm=False, layer=layer) * 1.7
    ckv = synth.tensor(0, "kv", (B, n_kv, D), rmsnorm=True, layer=layer)
    win = synth.tensor(0, "kv", (B, n_win, D), rmsnorm=True, layer=layer + 7)
    sink = synth.tensor(0, "sink", (H,), layer=layer).astype(np.float32)
    qd, qv = Hx.act(q, qf)
    cst, cdeq = Hx.upload_store(ckv, fmt, R)
    wst, wdeq = Hx.upload_store(win, fmt, R)
    return qd, qv, cst, cdeq, wst, wdeq, sink


@pytest.mark.parametrize("fmt,qf,H,D,R,T,m,k,W,gain,rd", [
    ("fp8", "bf16", 64, 512, 64, 700, 4, 64, 128, True, 64),      # MFMA kernel
    ("fp8", "bf16", 64, 512, 64, 300, 4, 96, 40, False, 64),      # MFMA kernel, rotation only
    ("fp8", "bf16", 32, 512, 64, 300, 4, 64, 128, True, 0),       # MFMA kernel, norm only
    ("f32", "f32", 4, 64, 0, 1000, 4, 64, 128, True, 16),         # general kernel
    ("fp8", "f32", 4, 64, 16, 500, 4, 32, 128, True, 16)])
def test_csa_prefill_with_query_norm_rope(lib, fmt, qf, H, D, R, T, m, k, W, gain, rd):
    import torch
    N = T // m
    qd, qv, cst, cdeq, wst, wdeq, sink = _attn_inputs(1, T, H, D, R, fmt, qf, N, T, layer=12)
    nr, gain64, th = _post(lib, D, rd, gain, layer=12)
    sel = Hx.random_selection(T, m, N, k, seed=13)
    out = torch.empty(qd.shape, dtype=qd.dtype, device=Hx.dev())
    lse = torch.empty((1, T, H), dtype=torch.float32, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.sparse_attn_prefill(qd, cst, N, Hx.to_dev(sel[None]), k, wst, W, Hx.to_dev(sink), tau, out, lse, q_post=nr)
    _sync()
    qp = Hx.post_queries(qv[0], np.arange(T), gain64, nr.eps, th, rd, qf == "bf16")
    want, want_lse = O.csa_prefill(qp, cdeq[0], sel, wdeq[0], W, sink.astype(np.float64), tau)
    Hx.check_attn(out.float().cpu().numpy()[0], want, bf16=(qf == "bf16"))
    np.testing.assert_allclose(lse.cpu().numpy()[0], want_lse, rtol=2e-3 if qf == "bf16" else 1e-4, atol=2e-3)


def test_hca_prefill_with_query_norm_rope(lib):
    import torch
    H, D, R, T, m, W = 64, 512, 64, 1000, 128, 128
    N = T // m
    qd, qv, cst, cdeq, wst, wdeq, sink = _attn_inputs(1, T, H, D, R, "fp8", "bf16", N, T, layer=13)
    nr, gain64, th = _post(lib, D, 64, True, layer=13)
    out = torch.empty(qd.shape, dtype=qd.dtype, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.hca_attn(qd, cst, m, N, None, wst, W, Hx.to_dev(sink), tau, out, q_post=nr)
    _sync()
    qp = Hx.post_queries(qv[0], np.arange(T), gain64, nr.eps, th, 64, True)
    want, _ = O.hca_prefill(qp, cdeq[0], m, wdeq[0], W, sink.astype(np.float64), tau)
    Hx.check_attn(out.float().cpu().numpy()[0], want)


def _decode_inputs(B, H, D, R, N, W, k, m, layer):
    q = synth.tensor(0, "q", (B, H, D), rmsnorm=False, layer=layer) * 0.6
    ckv = synth.tensor(0, "kv", (B, N, D), rmsnorm=True, layer=layer)
    ring = synth.tensor(0, "kv", (B, W, D), rmsnorm=True, layer=layer + 7)
    sink = synth.tensor(0, "sink", (H,), layer=layer).astype(np.float32)
    qd, qv = Hx.act(q, "bf16")
    cst, cdeq = Hx.upload_store(ckv, "fp8", R)
    rst, rdeq = Hx.upload_store(ring, "fp8", R)
    pos = np.array([m * N + b for b in range(B)], np.int64)
    pos[-1] = 61
    rng = np.random.default_rng(layer)
    sel = np.full((B, k), -1, np.int32)
    for b in range(B):
        nt = int(O.n_visible(pos[b], m, N))
        pick = np.sort(rng.permutation(nt)[:k])
        sel[b, : len(pick)] = pick
    return qd, qv, cst, cdeq, rst, rdeq, sink, pos, sel


def test_csa_decode_with_query_norm_rope(lib):
    """Split decode (workspace), the allocation-free entry point and the
    two-part form (partial, then swa_merge with the same post-processing)
    all process the query at its position and agree with the oracle; the
    two single-call forms give the same bits."""
    import torch
    B, H, D, R, N, k, W, m = 4, 128, 512, 64, 4000, 1024, 128, 4
    qd, qv, cst, cdeq, rst, rdeq, sink, pos, sel = _decode_inputs(B, H, D, R, N, W, k, m, 14)
    nr, gain64, th = _post(lib, D, 64, True, layer=14)
    ws = torch.empty(max(lib.attn_workspace(B, 1, H, D, k + W), 16), dtype=torch.uint8, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    sd, pd, skd = Hx.to_dev(sel), Hx.to_dev(pos), Hx.to_dev(sink)
    out = torch.empty(qd.shape, dtype=torch.bfloat16, device=Hx.dev())
    lib.sparse_attn_decode(qd, cst, N, sd, k, rst, pd, W, skd, tau, out, ws=ws, q_post=nr)
    out2 = torch.empty_like(out)
    lib.sparse_attn_decode_noalloc(qd, cst, N, sd, k, rst, pd, W, skd, tau, out2, q_post=nr)
    part = torch.empty(qd.shape, dtype=torch.float32, device=Hx.dev())
    plse = torch.empty((B, H), dtype=torch.float32, device=Hx.dev())
    lib.sparse_attn_decode(qd, cst, N, sd, k, rst, pd, W, skd, tau, part, lse=plse, flags=lib.ATTN_PARTIAL, ws=ws,
                           q_post=nr)
    merged = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=Hx.dev())
    lib.swa_merge(qd[:, None], rst, pd[:, None], W, lib.WIN_RING, part, plse, skd, tau, merged, q_post=nr)
    _sync()
    assert torch.equal(out, out2)
    got, gotm = out.float().cpu().numpy(), merged[:, 0].float().cpu().numpy()
    qp = Hx.post_queries(qv, pos, gain64, nr.eps, th, 64, True)
    for b in range(B):
        want, _ = O.csa_decode(qp[b], cdeq[b], sel[b], rdeq[b], int(pos[b]), W, sink.astype(np.float64), tau)
        Hx.check_attn(got[b], want)
        Hx.check_attn(gotm[b], want)


def test_hca_decode_with_query_norm_rope(lib):
    import torch
    B, H, D, R, N, W, m = 3, 128, 512, 64, 300, 128, 128
    qd, qv, cst, cdeq, rst, rdeq, sink, pos, _ = _decode_inputs(B, H, D, R, N, W, 1, m, 15)
    nr, gain64, th = _post(lib, D, 64, True, layer=15)
    ws = torch.empty(max(lib.attn_workspace(B, 1, H, D, N + W), 16), dtype=torch.uint8, device=Hx.dev())
    out = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.hca_attn(qd[:, None], cst, m, N, Hx.to_dev(pos[:, None]), rst, W, Hx.to_dev(sink), tau, out,
                 flags=lib.WIN_RING, ws=ws, q_post=nr)
    _sync()
    got = out.float().cpu().numpy()[:, 0]
    qp = Hx.post_queries(qv, pos, gain64, nr.eps, th, 64, True)
    for b in range(B):
        want, _ = O.hca_decode(qp[b], cdeq[b], m, N, rdeq[b], int(pos[b]), W, sink.astype(np.float64), tau)
        Hx.check_attn(got[b], want)


# ======================================================== full-size shapes
def test_compress_full_128k_with_norm_rope_sampled(lib):
    """CSA (m=4) and HCA (m'=128) compression of 131072 bf16 tokens, D=512,
    with RMSNorm and 64 rotated dims; sampled entries against the oracle."""
    T, D, R = 131072, 512, 64
    x = synth.tensor(0, "kv", (1, T, D), rmsnorm=True)
    xd, xv = Hx.act(x, "bf16")
    for m, layer in [(4, 0), (128, 1)]:
        g = synth.tensor(0, "gate", (D,), std=0.02, layer=layer).astype(np.float32)
        b = synth.tensor(0, "bias", (m,), std=0.02, layer=layer).astype(np.float32)
        nr, gain64, th = _post(lib, D, R, True, layer=layer)
        N = T // m
        out = lib.alloc_store(1, N, D, "fp8", R, device=Hx.dev())
        lib.compress_kv(xd, m, Hx.to_dev(g), Hx.to_dev(b), out, post=nr)
        _sync()
        rows = np.unique(np.concatenate([[0, N - 1], np.linspace(0, N - 1, 64).astype(int)]))
        tok = np.concatenate([xv[0, j * m:(j + 1) * m] for j in rows])
        g64, b64 = g.astype(np.float64), b.astype(np.float64)
        c = O.compress(tok, g64, b64, m)
        e = Hx.compress_error_bound(tok, g64, b64, m)
        _check_post_rows(out.rows[0].cpu().numpy()[rows], out.scales[0].cpu().numpy()[rows], "fp8", D, R, c, e,
                         gain64, nr.eps, th, R, (rows + 1) * m - 1)


def test_csa_prefill_32k_with_query_norm_rope_sampled(lib):
    """CSA prefill at 32768 tokens (H=64, D=512, k=512, W=128) with the
    query post-processing, in the benchmark's launch configuration."""
    import torch
    from tests.test_gpu_fullsize import _attn_prefill_stores, _q_device, _sample_rows
    T, m, D, R, H, k, W = 32768, 4, 512, 64, 64, 512, 128
    rows = _sample_rows(T, m, seed=21)
    cst, cdeq, wst, wdeq, qrows = _attn_prefill_stores(T, m, D, R, rows, "csa", 0)
    N = T // m
    sel = Hx.random_selection(T, m, N, k, seed=22)
    sink = synth.tensor(0, "sink", (H,)).astype(np.float32)
    nr, gain64, th = _post(lib, D, R, True, layer=21)
    qrows = np.asarray(qrows) * 1.5
    qd = _q_device(T, H, D, rows, qrows)
    qp = Hx.post_queries(Hx.bf16_vals(qrows), rows, gain64, nr.eps, th, R, True)
    out = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.sparse_attn_prefill(qd, cst, N, Hx.to_dev(sel[None]), k, wst, W, Hx.to_dev(sink), tau, out, q_post=nr)
    _sync()
    got = out[0, torch.as_tensor(rows, device=Hx.dev())].float().cpu().numpy()
    want = np.stack([O.attend(qp[i], np.concatenate([cdeq[sel[t][sel[t] >= 0]], wdeq[O.window_positions(t, W)]]),
                              sink.astype(np.float64), tau)[0] for i, t in enumerate(rows)])
    Hx.check_attn(got, want)


def test_decode_1m_with_query_norm_rope_sampled(lib):
    """CSA decode at 2^20 tokens of context (B=32, 262,144 entries each,
    k=1024, H=128) with the query post-processing; sampled sequences."""
    import torch
    from tests.test_gpu_fullsize import _filler_store
    B, ctx, D, R, H, W, k, m = 32, 1 << 20, 512, 64, 128, 128, 1024, 4
    N = ctx // m
    sampled = [0, B - 1]
    ckv = lib.alloc_store(B, N, D, "fp8", R, device=Hx.dev())
    ring = lib.alloc_store(B, W, D, "fp8", R, device=Hx.dev())
    deq = {}
    for b in range(B):
        if b in sampled:
            cv = synth.tensor(0, "kv", (N, D), rmsnorm=True, layer=30, start=b * N * D)
            rv = synth.tensor(0, "kv", (W, D), rmsnorm=True, layer=37, start=b * W * D)
            deq[b] = {}
            for name, vals, st in [("ckv", cv, ckv), ("ring", rv, ring)]:
                rws, sc = O.pack_rows(vals, "fp8", R)
                st.rows[b] = Hx.to_dev(rws)
                st.scales[b] = Hx.to_dev(sc)
                deq[b][name] = O.unpack_rows(rws, sc, "fp8", D, R)
                del rws, sc
            del cv, rv
        else:
            _filler_store(lib, ckv, b, N, D, "fp8", R, 6000 + b)
            _filler_store(lib, ring, b, W, D, "fp8", R, 7000 + b)
    rng = np.random.default_rng(31)
    sel = np.full((B, k), -1, np.int32)
    for b in range(B):
        sel[b] = np.sort(rng.permutation(N)[:k])
    q = synth.tensor(0, "q", (B, H, D), rmsnorm=False, layer=30) * 0.8
    sink = synth.tensor(0, "sink", (H,), layer=30).astype(np.float32)
    pos = np.full(B, ctx, np.int64)
    nr, gain64, th = _post(lib, D, R, True, layer=30)
    aws = torch.empty(max(lib.attn_workspace(B, 1, H, D, k + W), 16), dtype=torch.uint8, device=Hx.dev())
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.sparse_attn_decode(Hx.bf16_dev(q), ckv, N, Hx.to_dev(sel), k, ring, Hx.to_dev(pos), W, Hx.to_dev(sink), tau,
                           out, ws=aws, q_post=nr)
    _sync()
    got = out.float().cpu().numpy()
    qp = Hx.post_queries(Hx.bf16_vals(q), pos, gain64, nr.eps, th, R, True)
    for b in sampled:
        want, _ = O.csa_decode(qp[b], deq[b]["ckv"], sel[b].astype(np.int64), deq[b]["ring"], ctx, W,
                               sink.astype(np.float64), tau)
        Hx.check_attn(got[b], want)
