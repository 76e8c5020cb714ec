"""GPU: prefix reuse (kenelite analysis, section 十六).  A decode state whose
compressed CSA / HCA entries are restored from storage, with the incomplete
block's tail and the window recomputed from raw tokens by csa_decode_rebuild
(zero SWA caching: no window rows are stored), is byte for byte the state of
an uninterrupted decode, and decoding on from it gives the same bits and
agrees with the oracle."""
import math

import numpy as np
import pytest

import synth
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu

B, D, R, H, W, m, mh = 3, 512, 64, 64, 128, 4, 128
dI, HI, k = 64, 8, 64
P = np.array([1000, 1161, 517])            # prefix lengths (positions 0 .. P-1 processed)
STEPS = 3                                  # decode steps after the prefix


def _sync():
    import torch
    torch.cuda.synchronize()


class _Inputs:
    def __init__(self, lib):
        import torch
        Tmax = int(P.max()) + STEPS
        self.x = synth.tensor(0, "kv", (B, Tmax, D), rmsnorm=True, layer=60)
        self.xi = synth.tensor(0, "idx_k", (B, Tmax, dI), rmsnorm=True, layer=60)
        self.xh = synth.tensor(0, "kv", (B, Tmax, D), rmsnorm=True, layer=61)
        self.xd, self.xv = Hx.act(self.x, "bf16")
        self.xid, self.xiv = Hx.act(self.xi, "bf16")
        self.xhd, self.xhv = Hx.act(self.xh, "bf16")
        f32 = lambda a: Hx.to_dev(np.asarray(a, np.float32))
        self.g = synth.tensor(0, "gate", (D,), std=0.02, layer=60).astype(np.float32)
        self.b = synth.tensor(0, "bias", (m,), std=0.02, layer=60).astype(np.float32)
        self.gi = synth.tensor(0, "idx_gate", (dI,), std=0.02, layer=60).astype(np.float32)
        self.bi = synth.tensor(0, "idx_bias", (m,), std=0.02, layer=60).astype(np.float32)
        self.gh = synth.tensor(0, "gate", (D,), std=0.02, layer=61).astype(np.float32)
        self.bh = synth.tensor(0, "bias", (mh,), std=0.02, layer=61).astype(np.float32)
        self.gd, self.bd, self.gid, self.bid, self.ghd, self.bhd = map(f32, [self.g, self.b, self.gi, self.bi,
                                                                            self.gh, self.bh])
        self.gain = (1.0 + synth.tensor(0, "norm_gain", (D,), std=0.1, layer=60)).astype(np.float32)
        self.theta = Hx.rope_theta(R)
        self.nr = lib.NormRope(gain=f32(self.gain), eps=1e-6, rope_dims=R, theta=Hx.to_dev(self.theta))
        self.bidx = torch.arange(B, device=Hx.dev())


class _State:
    """Decode caches of the B sequences: CSA KV entries + window ring, CSA
    indexer keys, HCA KV entries + window ring, and the raw tail rings."""

    def __init__(self, lib, fill):
        import torch
        self.ckv = lib.alloc_store(B, int(P.max()) // m + 8, D, "fp8", R, device=Hx.dev())
        self.keys = lib.alloc_store(B, int(P.max()) // m + 8, dI, "fp8", device=Hx.dev())
        self.hkv = lib.alloc_store(B, int(P.max()) // mh + 2, D, "fp8", R, device=Hx.dev())
        self.ring = lib.alloc_store(B, W, D, "fp8", R, device=Hx.dev())
        self.ring_h = lib.alloc_store(B, W, D, "fp8", R, device=Hx.dev())
        for st in [self.ckv, self.keys, self.hkv, self.ring, self.ring_h]:
            st.rows.fill_(fill)
            st.scales.fill_(float(fill))
        self.t_kv = torch.zeros((B, m, D), dtype=torch.bfloat16, device=Hx.dev())
        self.t_i = torch.zeros((B, m, dI), dtype=torch.bfloat16, device=Hx.dev())
        self.t_h = torch.zeros((B, mh, D), dtype=torch.bfloat16, device=Hx.dev())

    def append(self, lib, inp, pos):
        """One decode append per cache at positions pos (device int64 [B], -1: nothing)."""
        import torch
        p = torch.clamp(pos, min=0)
        lib.decode_append(inp.xd[inp.bidx, p].contiguous(), pos, self.t_kv, m, inp.gd, inp.bd, self.ckv, self.ring, W,
                          post=inp.nr)
        lib.decode_append(inp.xid[inp.bidx, p].contiguous(), pos, self.t_i, m, inp.gid, inp.bid, self.keys)
        lib.decode_append(inp.xhd[inp.bidx, p].contiguous(), pos, self.t_h, mh, inp.ghd, inp.bhd, self.hkv,
                          self.ring_h, W, post=inp.nr)


def _uninterrupted(lib, inp):
    import torch
    st = _State(lib, 0xAB)
    pos_tab = torch.from_numpy(np.where(np.arange(P.max())[:, None] < P[None, :], np.arange(P.max())[:, None],
                                        -1).astype(np.int64)).to(Hx.dev())
    for s in range(int(P.max())):
        st.append(lib, inp, pos_tab[s])
    return st


def _rebuild_rows(xd, p0, nrows):
    """tok [B][n][dim] with rows p0[b] .. p0[b] + nrows[b] - 1 of each sequence (padded)."""
    import torch
    n = int(nrows.max())
    idx = torch.from_numpy((p0[:, None] + np.arange(n)[None, :]).astype(np.int64)).to(Hx.dev())
    idx = torch.clamp(idx, max=xd.shape[1] - 1)
    return xd[torch.arange(B, device=Hx.dev())[:, None], idx].contiguous()


def _restored(lib, inp, ref):
    """Entries of complete blocks copied through host memory (the CSA caches
    one block short, so a restored prefix also recomputes a closed block);
    window rings start as garbage, tails as zeros; then csa_decode_rebuild."""
    import torch
    st = _State(lib, 0xCD)
    for b in range(B):
        for src, dst, mm, short in [(ref.ckv, st.ckv, m, 1), (ref.keys, st.keys, m, 1), (ref.hkv, st.hkv, mh, 0)]:
            n_r = int(P[b]) // mm - short
            dst.rows[b, :n_r] = src.rows[b, :n_r].cpu().to(Hx.dev())
            dst.scales[b, :n_r] = src.scales[b, :n_r].cpu().to(Hx.dev())
    for xd, tail, mm, gd, bd, out, win, post in [
            (inp.xd, st.t_kv, m, inp.gd, inp.bd, st.ckv, st.ring, inp.nr),
            (inp.xid, st.t_i, m, inp.gid, inp.bid, st.keys, None, None),
            (inp.xhd, st.t_h, mh, inp.ghd, inp.bhd, st.hkv, st.ring_h, inp.nr)]:
        p0 = (np.maximum(0, P - W) // mm) * mm
        nrows = P - p0
        tok = _rebuild_rows(xd, p0, nrows)
        lib.decode_rebuild(tok, Hx.to_dev(p0.astype(np.int64)), tail, mm, gd, bd, out, win, W if win else 0,
                           post=post, n_valid=Hx.to_dev(nrows.astype(np.int32)))
    return st


def _decode_steps(lib, inp, st):
    """STEPS decode steps from position P: appends, indexer + top-k, CSA
    sparse attention and HCA attention; returns the per-step outputs."""
    import torch
    outs = []
    tau = 1.0 / math.sqrt(D)
    for s in range(STEPS):
        pos = Hx.to_dev((P + s).astype(np.int64))
        st.append(lib, inp, pos)
        qI = synth.tensor(0, "idx_q", (B, HI, dI), rmsnorm=True, layer=70 + s)
        qst, _ = Hx.upload_store(qI, "fp8")
        w = Hx.to_dev(synth.tensor(0, "head_w", (B, 1, HI), std=0.02, layer=70 + s).astype(np.float32))
        Ncap, Nhcap = st.ckv.cap, st.hkv.cap
        sel = torch.empty((B, 1, k), dtype=torch.int32, device=Hx.dev())
        iws = torch.empty(max(lib.indexer_topk_workspace(B, 1, Ncap, k), 16), dtype=torch.uint8, device=Hx.dev())
        lib.indexer_topk(qst, w, st.keys, Ncap, pos, B, 1, HI, m, k, sel, iws)
        q = synth.tensor(0, "q", (B, H, D), rmsnorm=True, layer=70 + s)
        qh = synth.tensor(0, "q", (B, 1, H, D), rmsnorm=True, layer=80 + s)
        sink = Hx.to_dev(synth.tensor(0, "sink", (H,), layer=70).astype(np.float32))
        ws = torch.empty(max(lib.attn_workspace(B, 1, H, D, max(k, Nhcap) + W), 16), dtype=torch.uint8,
                         device=Hx.dev())
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=Hx.dev())
        lib.sparse_attn_decode(Hx.bf16_dev(q), st.ckv, Ncap, sel[:, 0], k, st.ring, pos, W, sink, tau, out, ws=ws)
        out_h = torch.empty((B, 1, H, D), dtype=torch.bfloat16, device=Hx.dev())
        lib.hca_attn(Hx.bf16_dev(qh), st.hkv, mh, Nhcap, pos[:, None], st.ring_h, W, sink, tau, out_h,
                     flags=lib.WIN_RING, ws=ws)
        _sync()
        outs.append((sel.cpu().numpy(), out.cpu(), out_h.cpu(), Hx.bf16_vals(q), Hx.bf16_vals(qh)))
    return outs


def test_restore_then_decode_equals_uninterrupted_decode(lib):
    import torch
    inp = _Inputs(lib)
    ref = _uninterrupted(lib, inp)
    rst = _restored(lib, inp, ref)
    _sync()
    # the decode state: byte for byte
    for b in range(B):
        for name, mm in [("ckv", m), ("keys", m), ("hkv", mh)]:
            n = int(P[b]) // mm
            a, c = getattr(ref, name), getattr(rst, name)
            assert torch.equal(a.rows[b, :n], c.rows[b, :n]), f"{name} entries differ (sequence {b})"
            assert torch.equal(a.scales[b, :n], c.scales[b, :n]), f"{name} scales differ (sequence {b})"
    for name in ["ring", "ring_h"]:
        a, c = getattr(ref, name), getattr(rst, name)
        assert torch.equal(a.rows, c.rows) and torch.equal(a.scales, c.scales), f"{name} differs"
    for name in ["t_kv", "t_i", "t_h"]:
        assert torch.equal(getattr(ref, name), getattr(rst, name)), f"{name} differs"
    # the restored state against the oracle's
    g64, b64 = inp.g.astype(np.float64), inp.b.astype(np.float64)
    gh64, bh64 = inp.gh.astype(np.float64), inp.bh.astype(np.float64)
    gain64 = inp.gain.astype(np.float64)
    for b in range(B):
        Pb = int(P[b])
        for xv, gg, bb, mm, st, ring in [(inp.xv, g64, b64, m, rst.ckv, rst.ring),
                                         (inp.xhv, gh64, bh64, mh, rst.hkv, rst.ring_h)]:
            p0 = (max(0, Pb - W) // mm) * mm
            n_r = Pb // mm - (1 if mm == m else 0)
            restored = O.compress(xv[b, : n_r * mm], gg, bb, mm)
            ent, window, tail = O.restore_state(restored, xv[b, p0:Pb], gg, bb, mm, W, p0)
            n = Pb // mm
            e = Hx.compress_error_bound(xv[b, : n * mm], gg, bb, mm)
            cp = O.post_rows(ent, O.entry_positions(n, mm), gain64, 1e-6, inp.theta, R)
            ep = Hx.post_error_bound(ent, e, gain64, 1e-6, inp.theta, R)
            frac = Hx.check_compress(st.rows[b, :n].cpu().numpy(), st.scales[b, :n].cpu().numpy(), "fp8", D, R,
                                     cp, ep)
            assert frac <= 2e-3
            slots = sorted(window)
            qs = np.array([window[s_] for s_ in slots])
            wp = O.post_rows(xv[b, qs], qs, gain64, 1e-6, inp.theta, R)
            wb = Hx.post_error_bound(xv[b, qs], None, gain64, 1e-6, inp.theta, R)
            Hx.check_compress(ring.rows[b, slots].cpu().numpy(), ring.scales[b, slots].cpu().numpy(), "fp8", D, R,
                              wp, wb)
            tl = (rst.t_kv if mm == m else rst.t_h)[b].float().cpu().numpy()
            assert np.array_equal(tl[[q % mm for q in tail]], xv[b, tail]), "tail rows are not the raw tokens"
    # decoding on: identical bits, and the oracle's outputs
    outs_ref = _decode_steps(lib, inp, ref)
    outs_rst = _decode_steps(lib, inp, rst)
    for (sa, oa, oha, _, _), (sb, ob, ohb, _, _) in zip(outs_ref, outs_rst):
        assert np.array_equal(sa, sb), "selections differ"
        assert torch.equal(oa, ob) and torch.equal(oha, ohb), "attention outputs differ"
    sel, out, out_h, qv, qhv = outs_rst[-1]
    pos = P + STEPS - 1
    tau = 1.0 / math.sqrt(D)
    sink = synth.tensor(0, "sink", (H,), layer=70).astype(np.float32).astype(np.float64)
    for b in range(B):
        n_vis = int(O.n_visible(int(pos[b]), m, rst.ckv.cap))
        cdeq = O.unpack_rows(rst.ckv.rows[b, :n_vis].cpu().numpy(), rst.ckv.scales[b, :n_vis].cpu().numpy(), "fp8",
                             D, R)
        rdeq = O.unpack_rows(rst.ring.rows[b].cpu().numpy(), rst.ring.scales[b].cpu().numpy(), "fp8", D, R)
        want, _ = O.csa_decode(qv[b], cdeq, sel[b, 0].astype(np.int64), rdeq, int(pos[b]), W, sink, tau)
        Hx.check_attn(out[b].float().numpy(), want)
        nh = int(O.n_visible(int(pos[b]), mh, rst.hkv.cap))
        hdeq = O.unpack_rows(rst.hkv.rows[b, :nh].cpu().numpy(), rst.hkv.scales[b, :nh].cpu().numpy(), "fp8", D, R)
        rhdeq = O.unpack_rows(rst.ring_h.rows[b].cpu().numpy(), rst.ring_h.scales[b].cpu().numpy(), "fp8", D, R)
        want_h, _ = O.hca_decode(qhv[b, 0], hdeq, mh, nh, rhdeq, int(pos[b]), W, sink, tau)
        Hx.check_attn(out_h[b, 0].float().numpy(), want_h)


def test_rebuild_skips_sequences_that_do_not_start_a_block(lib):
    """p0 not a multiple of m, or negative: nothing is written for that
    sequence; n_valid = 0 likewise."""
    import torch
    inp = _Inputs(lib)
    st = _State(lib, 0x5A)
    before = [st.ckv.rows.clone(), st.ring.rows.clone(), st.t_kv.clone()]
    tok = inp.xd[:, :40].contiguous()
    p0 = Hx.to_dev(np.array([2, -4, 8], np.int64))
    nv = Hx.to_dev(np.array([40, 40, 0], np.int32))
    lib.decode_rebuild(tok, p0, st.t_kv, m, inp.gd, inp.bd, st.ckv, st.ring, W, post=inp.nr, n_valid=nv)
    _sync()
    assert torch.equal(before[0], st.ckv.rows) and torch.equal(before[1], st.ring.rows)
    assert torch.equal(before[2], st.t_kv)
