"""The allocation-free decode entry point (csa_sparse_attn_decode_noalloc):
its split partials live in the library's per-device scratch array instead of
a caller workspace.  Two calls in a row, the second with fewer sequences and
a shorter selection, each equal bit for bit to csa_sparse_attn_decode with a
workspace (same kernels, same split plan) and within the bf16 tolerance of
the oracle.  Run after every other GPU test, or alone in a fresh process."""
import math

import numpy as np
import pytest

import synth
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu


def _case(lib, B, H, N, k, W, m, layer, pos_shift):
    import torch
    q = synth.tensor(0, "q", (B, H, 512), rmsnorm=True, layer=layer)
    ckv = synth.tensor(0, "kv", (B, N, 512), rmsnorm=True, layer=layer)
    ring = synth.tensor(0, "kv", (B, W, 512), rmsnorm=True, layer=layer + 7)
    sink = synth.tensor(0, "sink", (H,), layer=layer).astype(np.float32)
    qd, qv = Hx.act(q, "bf16")
    cst, cdeq = Hx.upload_store(ckv, "fp8", 64)
    rst, rdeq = Hx.upload_store(ring, "fp8", 64)
    pos = np.array([m * N + pos_shift + b for b in range(B)], np.int64)
    pos[-1] = 45                                         # a short sequence: partial window, few entries
    rng = np.random.default_rng(layer)
    sel = np.full((B, k), -1, np.int32)
    for b in range(B):
        nt = int(O.n_visible(pos[b], m, N))
        pick = np.sort(rng.permutation(nt)[:k])
        sel[b, : len(pick)] = pick
    tau = 1.0 / math.sqrt(512)
    sd, pd, skd = Hx.to_dev(sel), Hx.to_dev(pos), Hx.to_dev(sink)
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device=Hx.dev())
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device=Hx.dev())
    lib.sparse_attn_decode_noalloc(qd, cst, N, sd, k, rst, pd, W, skd, tau, out, lse=lse)
    ws = torch.empty(max(lib.attn_workspace(B, 1, H, 512, k + W), 16), dtype=torch.uint8, device=Hx.dev())
    assert lib.attn_workspace(B, 1, H, 512, k + W) > 0           # this shape splits its lists
    ref = torch.empty_like(out)
    ref_lse = torch.empty_like(lse)
    lib.sparse_attn_decode(qd, cst, N, sd, k, rst, pd, W, skd, tau, ref, lse=ref_lse, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "no-allocation output differs from the workspace entry point"
    assert torch.equal(lse, ref_lse)
    got = out.float().cpu().numpy()
    for b in range(B):
        want, want_lse = O.csa_decode(qv[b], cdeq[b], sel[b], rdeq[b], int(pos[b]), W, sink.astype(np.float64), tau)
        Hx.check_attn(got[b], want)
        np.testing.assert_allclose(lse[b].cpu().numpy(), want_lse, rtol=1e-4, atol=1e-4)


def test_noalloc_decode_two_calls_second_smaller(lib):
    _case(lib, B=6, H=128, N=3000, k=1024, W=128, m=4, layer=11, pos_shift=0)
    _case(lib, B=3, H=128, N=1500, k=512, W=128, m=4, layer=12, pos_shift=2)
