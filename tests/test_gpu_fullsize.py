"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times, checked on sampled outputs the oracle computes one by one.

Each stage is isolated: the stores a stage reads are packed by the oracle's
codec from seeded inputs and uploaded, so both sides consume identical bytes.
Rows and sequences that are not sampled are filled with other data; only
sampled outputs are compared, and those depend on oracle-known inputs only.
"""
import math

import numpy as np
import pytest

import synth
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu

T128 = 131072


def _sync():
    import torch
    torch.cuda.synchronize()


def _sample_rows(T, m, extra=12, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, m - 2, m - 1, m, 127, 128, 129, 4095, T // 2, T - 2, T - 1]
    return sorted(set([r for r in fixed if 0 <= r < T] + list(rng.integers(0, T, extra))))


def test_compress_full_128k_sampled(lib):
    """CSA (m=4) and HCA (m'=128) compression of 131072 bf16 tokens, D=512."""
    D, R = 512, 64
    x = synth.tensor(0, "kv", (1, T128, D), rmsnorm=True)
    xd, xv = Hx.act(x, "bf16")
    for m, layer in [(4, 0), (128, 1)]:
        g = synth.tensor(0, "gate", (D,), std=0.02, layer=layer).astype(np.float32)
        b = synth.tensor(0, "bias", (m,), std=0.02, layer=layer).astype(np.float32)
        N = T128 // m
        out = lib.alloc_store(1, N, D, "fp8", R, device=Hx.dev())
        lib.compress_kv(xd, m, Hx.to_dev(g), Hx.to_dev(b), out)
        _sync()
        rows = np.unique(np.concatenate([[0, N - 1], np.linspace(0, N - 1, 64).astype(int)]))
        got_rows = out.rows[0].cpu().numpy()[rows]
        got_s = out.scales[0].cpu().numpy()[rows]
        tok = np.concatenate([xv[0, j * m:(j + 1) * m] for j in rows])
        c = O.compress(tok, g.astype(np.float64), b.astype(np.float64), m)
        eps = Hx.compress_error_bound(tok, g.astype(np.float64), b.astype(np.float64), m)
        frac = Hx.check_compress(got_rows, got_s, "fp8", D, R, c, eps)
        assert frac <= 2e-3


def _prefill_indexer_inputs(T, m, H_I, d_I, rows, layer=0):
    """Oracle-packed compressed indexer keys for all entries; queries and head
    weights from the generator on the sampled rows, zero elsewhere."""
    N = T // m
    xi = synth.tensor(0, "idx_k", (T, d_I), rmsnorm=True, layer=layer)
    gi = synth.tensor(0, "idx_gate", (d_I,), std=0.02, layer=layer)
    bi = synth.tensor(0, "idx_bias", (m,), std=0.02, layer=layer)
    keys_vals = O.compress(Hx.bf16_vals(xi), gi.astype(np.float32), bi.astype(np.float32), m)
    kst, kdeq = Hx.upload_store(keys_vals[None], "fp8")
    import torch
    import long_context_attention_15_amd as lib
    w = np.zeros((T, H_I), np.float32)
    qst = lib.alloc_store(1, T * H_I, d_I, "fp8", device=Hx.dev())
    qst.rows.zero_()
    qst.scales.fill_(1.0)
    qdeq = {}
    for t in rows:
        qv = synth.tensor(0, "idx_q", (H_I, d_I), rmsnorm=True, layer=layer, start=t * H_I * d_I)
        w[t] = synth.tensor(0, "head_w", (H_I,), std=0.02, layer=layer, start=t * H_I).astype(np.float32)
        rr, sc = O.pack_rows(qv, "fp8")
        qst.rows[0, t * H_I:(t + 1) * H_I] = Hx.to_dev(rr)
        qst.scales[0, t * H_I:(t + 1) * H_I] = Hx.to_dev(sc)
        qdeq[t] = O.unpack_rows(rr, sc, "fp8", d_I)
    return N, kst, kdeq[0], qst, qdeq, w


@pytest.mark.parametrize("T,k", [(32768, 512), (T128, 512)])
def test_csa_indexer_prefill_full_sampled(lib, T, k):
    import torch
    m, H_I, d_I = 4, 8, 64
    rows = _sample_rows(T, m)
    N, kst, kdeq, qst, qdeq, w = _prefill_indexer_inputs(T, m, H_I, d_I, rows)
    sel = torch.empty((1, T, k), dtype=torch.int32, device=Hx.dev())
    nws = lib.indexer_topk_workspace(1, T, N, k)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=Hx.dev())
    lib.indexer_topk(qst, Hx.to_dev(w[None]), kst, N, None, 1, T, H_I, m, k, sel, ws)
    _sync()
    got = sel[0].cpu().numpy()
    flips = 0
    for t in rows:
        nt = int(O.n_visible(t, m, N))
        s = O.indexer_scores(qdeq[t], w[t].astype(np.float64), kdeq[:nt])
        err = Hx.score_error_bound(qdeq[t], w[t].astype(np.float64), kdeq[:nt])
        flips += Hx.check_topk(got[t], s, k, err)
    assert flips <= 2


def _attn_prefill_stores(T, m, D, R, rows, kind, layer):
    """Oracle-packed compressed entries (from seeded tokens) and the raw window
    store; queries from the generator on the sampled rows, zero elsewhere."""
    x = synth.tensor(0, "kv", (T, D), rmsnorm=True, layer=layer)
    xv = Hx.bf16_vals(x)
    g = synth.tensor(0, "gate", (D,), std=0.02, layer=layer).astype(np.float32)
    b = synth.tensor(0, "bias", (m,), std=0.02, layer=layer).astype(np.float32)
    ent = O.compress(xv, g.astype(np.float64), b.astype(np.float64), m)
    cst, cdeq = Hx.upload_store(ent[None], "fp8", R)
    wst, wdeq = Hx.upload_store(xv[None], "fp8", R)
    H = 64
    qrows = np.stack([synth.tensor(0, "q", (H, D), rmsnorm=True, layer=layer, start=t * H * D) for t in rows])
    return cst, cdeq[0], wst, wdeq[0], qrows


def _q_device(T, H, D, rows, qrows):
    """bf16 queries on the device: generator rows at the sampled positions,
    zeros elsewhere (never compared)."""
    import torch
    qd = torch.zeros((1, T, H, D), dtype=torch.bfloat16, device=Hx.dev())
    qd[0, torch.as_tensor(rows, device=Hx.dev())] = Hx.bf16_dev(qrows)
    return qd


@pytest.mark.parametrize("T", [32768, T128])
def test_csa_sparse_attn_prefill_full_sampled(lib, T):
    import torch
    m, D, R, H, k, W = 4, 512, 64, 64, 512, 128
    rows = _sample_rows(T, m, seed=1)
    cst, cdeq, wst, wdeq, qrows = _attn_prefill_stores(T, m, D, R, rows, "csa", 0)
    N = T // m
    sel = Hx.random_selection(T, m, N, k, seed=7) if T <= 32768 else None
    if sel is None:                          # only sampled rows matter; others attend to the first k
        sel = np.full((T, k), -1, np.int32)
        base = np.arange(k, dtype=np.int32)
        for t0 in range(0, T, 8192):
            t = np.arange(t0, min(T, t0 + 8192))
            nt = np.minimum(N, (t + 1) // m)
            sel[t] = np.where(base[None, :] < nt[:, None], base[None, :], -1)
        rng = np.random.default_rng(8)
        for t in rows:
            nt = int(O.n_visible(t, m, N))
            pick = np.sort(rng.permutation(nt)[:k])
            sel[t] = -1
            sel[t, :len(pick)] = pick
    sink = synth.tensor(0, "sink", (H,)).astype(np.float32)
    qd = _q_device(T, H, D, rows, qrows)
    qv = Hx.bf16_vals(qrows)
    out = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.sparse_attn_prefill(qd, cst, N, Hx.to_dev(sel[None]), k, wst, W, Hx.to_dev(sink), tau, out)
    _sync()
    got = out[0, torch.as_tensor(rows, device=Hx.dev())].float().cpu().numpy()
    want = np.stack([O.attend(qv[i], np.concatenate([cdeq[sel[t][sel[t] >= 0]], wdeq[O.window_positions(t, W)]]),
                              sink.astype(np.float64), tau)[0] for i, t in enumerate(rows)])
    Hx.check_attn(got, want)


def test_hca_attn_prefill_full_sampled(lib):
    import torch
    T, m, D, R, H, W = T128, 128, 512, 64, 64, 128
    rows = _sample_rows(T, m, seed=2)
    cst, cdeq, wst, wdeq, qrows = _attn_prefill_stores(T, m, D, R, rows, "hca", 1)
    N = T // m
    sink = synth.tensor(0, "sink", (H,), layer=1).astype(np.float32)
    qd = _q_device(T, H, D, rows, qrows)
    qv = Hx.bf16_vals(qrows)
    out = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.hca_attn(qd, cst, m, N, None, wst, W, Hx.to_dev(sink), tau, out)
    _sync()
    got = out[0, torch.as_tensor(rows, device=Hx.dev())].float().cpu().numpy()
    want = O.hca_prefill(qv, cdeq, m, wdeq, W, sink.astype(np.float64), tau, positions=rows)[0]
    Hx.check_attn(got, want)


def _filler_store(lib, st, b, n, D, fmt, R, seed):
    """Fill sequence b of a store with GPU-generated rows (not an oracle input)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((1, n, D), generator=g, device="cuda")
    x = (x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    sub = lib.Store(st.rows[b:b + 1], None if st.scales is None else st.scales[b:b + 1], st.cap, D, R, st.fmt)
    lib.compress_kv(x, 1, torch.zeros(D, device="cuda"), torch.ones(1, device="cuda"), sub)


def _decode_setup(lib, B, N, D, R, W, H_I, d_I, ifmt, sampled, layer):
    """Stores for B sequences: oracle-packed for the sampled ones, GPU filler
    for the others."""
    ckv = lib.alloc_store(B, N, D, "fp8", R, device=Hx.dev())
    keys = lib.alloc_store(B, N, d_I, ifmt, device=Hx.dev())
    ring = lib.alloc_store(B, W, D, "fp8", R, device=Hx.dev())
    deq = {}
    for b in range(B):
        if b in sampled:
            cv = synth.tensor(0, "kv", (N, D), rmsnorm=True, layer=layer, start=b * N * D)
            kv = synth.tensor(0, "idx_k", (N, d_I), rmsnorm=True, layer=layer, start=b * N * d_I)
            rv = synth.tensor(0, "kv", (W, D), rmsnorm=True, layer=layer + 7, start=b * W * D)
            out = {}
            for name, vals, st, fmt, r in [("ckv", cv, ckv, "fp8", R), ("keys", kv, keys, ifmt, 0),
                                           ("ring", rv, ring, "fp8", R)]:
                rows, sc = O.pack_rows(vals, fmt, r)
                st.rows[b] = Hx.to_dev(rows)
                st.scales[b] = Hx.to_dev(sc)
                out[name] = O.unpack_rows(rows, sc, fmt, vals.shape[1], r)
                del rows, sc
            deq[b] = out
            del cv, kv, rv
        else:
            _filler_store(lib, ckv, b, N, D, "fp8", R, 1000 + b)
            _filler_store(lib, keys, b, N, d_I, ifmt, 0, 2000 + b)
            _filler_store(lib, ring, b, W, D, "fp8", R, 3000 + b)
    return ckv, keys, ring, deq


@pytest.mark.parametrize("hybrid", [False, True])
def test_decode_1m_full_sampled(lib, hybrid):
    """CSA decode at 2^20 tokens of context (262,144 entries per sequence):
    B=32 with an FP8 indexer, or the hybrid B=16 with an MXFP4 indexer plus an
    HCA layer over 8,192 entries."""
    import torch
    B = 16 if hybrid else 32
    ctx, D, R, H, W, k, H_I, d_I, m, mh = 1 << 20, 512, 64, 128, 128, 1024, 8, 64, 4, 128
    N, Nh = ctx // m, ctx // mh
    ifmt = "mxfp4" if hybrid else "fp8"
    sampled = [0, B - 1]
    layer = 2 if hybrid else 3
    ckv, keys, ring, deq = _decode_setup(lib, B, N, D, R, W, H_I, d_I, ifmt, sampled, layer)
    # queries: generator values for every sequence (small)
    qI = synth.tensor(0, "idx_q", (B, H_I, d_I), rmsnorm=True, layer=layer)
    qst, qdeq = Hx.upload_store(qI, ifmt)
    w = synth.tensor(0, "head_w", (B, 1, H_I), std=0.02, layer=layer).astype(np.float32)
    q = synth.tensor(0, "q", (B, H, D), rmsnorm=True, layer=layer)
    sink = synth.tensor(0, "sink", (H,), layer=layer).astype(np.float32)
    pos = np.full(B, ctx, np.int64)
    sel = torch.empty((B, 1, k), dtype=torch.int32, device=Hx.dev())
    iws = torch.empty(max(lib.indexer_topk_workspace(B, 1, N, k), 16), dtype=torch.uint8, device=Hx.dev())
    lib.indexer_topk(qst, Hx.to_dev(w), keys, N, Hx.to_dev(pos), B, 1, H_I, m, k, sel, iws)
    _sync()
    sel_g = sel[:, 0].cpu().numpy()
    flips = 0
    for b in sampled:
        s = O.indexer_scores(qdeq[b], w[b, 0].astype(np.float64), deq[b]["keys"])
        err = Hx.score_error_bound(qdeq[b], w[b, 0].astype(np.float64), deq[b]["keys"])
        flips += Hx.check_topk(sel_g[b], s, k, err)
    assert flips <= 2
    # attention over the GPU's selection (checked above), oracle-known stores
    qd = Hx.bf16_dev(q)
    qv = Hx.bf16_vals(q)
    aws = torch.empty(max(lib.attn_workspace(B, 1, H, D, k + W), 16), dtype=torch.uint8, device=Hx.dev())
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=Hx.dev())
    tau = 1.0 / math.sqrt(D)
    lib.sparse_attn_decode(qd, ckv, N, sel[:, 0], k, ring, Hx.to_dev(pos), W, Hx.to_dev(sink), tau, out, ws=aws)
    _sync()
    got = out.float().cpu().numpy()
    for b in sampled:
        want, _ = O.csa_decode(qv[b], deq[b]["ckv"], sel_g[b].astype(np.int64), deq[b]["ring"], ctx, W,
                               sink.astype(np.float64), tau)
        Hx.check_attn(got[b], want)
    del ckv, keys
    if hybrid:
        hkv = lib.alloc_store(B, Nh, D, "fp8", R, device=Hx.dev())
        hring = lib.alloc_store(B, W, D, "fp8", R, device=Hx.dev())
        hdeq = {}
        for b in range(B):
            if b in sampled:
                hv = synth.tensor(0, "kv", (Nh, D), rmsnorm=True, layer=layer + 100, start=b * Nh * D)
                rv = synth.tensor(0, "kv", (W, D), rmsnorm=True, layer=layer + 107, start=b * W * D)
                hdeq[b] = {}
                for name, vals, st in [("hkv", hv, hkv), ("ring", rv, hring)]:
                    rows, sc = O.pack_rows(vals, "fp8", R)
                    st.rows[b] = Hx.to_dev(rows)
                    st.scales[b] = Hx.to_dev(sc)
                    hdeq[b][name] = O.unpack_rows(rows, sc, "fp8", D, R)
            else:
                _filler_store(lib, hkv, b, Nh, D, "fp8", R, 4000 + b)
                _filler_store(lib, hring, b, W, D, "fp8", R, 5000 + b)
        qh = synth.tensor(0, "q", (B, 1, H, D), rmsnorm=True, layer=layer + 100)
        sinkh = synth.tensor(0, "sink", (H,), layer=layer + 100).astype(np.float32)
        hws = torch.empty(max(lib.attn_workspace(B, 1, H, D, Nh + W), 16), dtype=torch.uint8, device=Hx.dev())
        outh = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=Hx.dev())
        lib.hca_attn(Hx.bf16_dev(qh), hkv, mh, Nh, Hx.to_dev(pos[:, None]), hring, W, Hx.to_dev(sinkh), tau, outh,
                     flags=lib.WIN_RING, ws=hws)
        _sync()
        goth = outh[:, 0].float().cpu().numpy()
        qhv = Hx.bf16_vals(qh)
        for b in sampled:
            want, _ = O.hca_decode(qhv[b, 0], hdeq[b]["hkv"], mh, Nh, hdeq[b]["ring"], ctx, W,
                                   sinkh.astype(np.float64), tau)
            Hx.check_attn(goth[b], want)
