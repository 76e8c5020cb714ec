"""GPU tests of the one-pass long-list indexer's threshold path and of the
path a workgroup takes when it stops waiting for its query's other chunks.

The one-pass path (a query's chunks scored in one launch, each chunk's
statistic published in the workspace) forms a threshold T from those
statistics when ceil(k / #full chunks) <= 128.  A workgroup that stops
waiting takes T = 0, keeping every key as a candidate; the final selection
is exact either way.  CSA_INDEXER_SPIN_LIMIT sets the wait budget from the
host (0: every workgroup stops at once; 1: a mix), so every kernel still
exits normally.  The diagnostic counters say which paths ran."""
import os

import numpy as np
import pytest

from oracle import codec
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu


class _SpinLimit:
    def __init__(self, n):
        self.n = n

    def __enter__(self):
        self.old = os.environ.get("CSA_INDEXER_SPIN_LIMIT")
        os.environ["CSA_INDEXER_SPIN_LIMIT"] = str(self.n)

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["CSA_INDEXER_SPIN_LIMIT"]
        else:
            os.environ["CSA_INDEXER_SPIN_LIMIT"] = self.old


def _run(lib, qst, w, kst, N, pos, B, H_I, m, k):
    import torch
    sel = torch.full((B, 1, k), -7, dtype=torch.int32, device=Hx.dev())
    ws = torch.empty(max(lib.indexer_topk_workspace(B, 1, N, k), 16), dtype=torch.uint8, device=Hx.dev())
    lib.indexer_topk(qst, w, kst, N, Hx.to_dev(np.asarray(pos, np.int64)), B, 1, H_I, m, k, sel, ws)
    torch.cuda.synchronize()
    return sel[:, 0].cpu().numpy()


def _tie_inputs(lib, B, N, H_I, d_I, seed):
    rng = np.random.default_rng(seed)
    keys = rng.integers(-2, 3, (B, N, d_I)).astype(np.float64)
    keys[:, :, 0] = 2.0                       # amax 2 in every row: scale 2^-7, codes exact
    q = rng.integers(-1, 2, (B, H_I, d_I)).astype(np.float64)
    q[:, :, 1] = 1.0
    kst, kdeq = Hx.upload_store(keys, "fp8")
    qst, qdeq = Hx.upload_store(q, "fp8")
    assert np.array_equal(kdeq, keys) and np.array_equal(qdeq, q)
    return kst, qst, keys, q


@pytest.mark.parametrize("spin", [None, 0, 1])
def test_one_pass_threshold_path_with_exact_ties(lib, spin):
    """262,144 entries, k = 1024: 32 full chunks, ceil(k / 32) = 32 <= 128, so
    the chunks publish statistics and compact against the threshold.
    Integer inputs with w = 1 make every score exact and tie massively
    (exact zeros included): the sets must equal the oracle's, smaller index
    first, whether the workgroups wait (default), all stop at once (0) or
    some stop (1)."""
    import torch
    B, N, H_I, d_I, m, k = 3, 262144, 8, 64, 4, 1024
    kst, qst, keys, q = _tie_inputs(lib, B, N, H_I, d_I, 31)
    w = torch.ones((B, 1, H_I), dtype=torch.float32, device=Hx.dev())
    pos = [m * N + 1, m * N - 5, m * 200000 + 2]    # the last query sees 200,000 entries (ragged last chunk)
    lib.diag_counters(reset=True)
    if spin is None:
        sel = _run(lib, qst, w, kst, N, pos, B, H_I, m, k)
    else:
        with _SpinLimit(spin):
            sel = _run(lib, qst, w, kst, N, pos, B, H_I, m, k)
    diag = lib.diag_counters(reset=True)
    for b in range(B):
        nt = int(O.n_visible(pos[b], m, N))
        want = O.topk_select(O.indexer_scores(q[b], np.ones(H_I), keys[b, :nt]), k)
        assert np.array_equal(sel[b], want), f"sequence {b}"
    if spin is None:
        assert diag[lib.DIAG_INDEXER_GIVEUPS] == 0, diag
    if spin == 0:
        # every nonempty chunk of every query stopped waiting, so every key is
        # a candidate and every final selection took the many-candidate path
        nchunks = sum((int(O.n_visible(p, m, N)) + 8191) // 8192 for p in pos)
        assert diag[lib.DIAG_INDEXER_GIVEUPS] == nchunks, diag
        assert diag[lib.DIAG_INDEXER_WIDE_SELECT] == B, diag


def test_give_up_path_on_random_fp8_keys_at_the_1m_decode_shape(lib):
    """B = 32 sequences of 262,144 random FP8 indexer keys, k = 1024 (the 1M
    decode shape): the selections of the normal run, of a run where every
    workgroup stops waiting at once and of a mixed run are identical, and two
    sequences agree with the oracle."""
    import torch
    B, N, H_I, d_I, m, k = 32, 262144, 8, 64, 4, 1024
    gen = torch.Generator(device=Hx.dev())
    gen.manual_seed(23)

    def codes(shape):
        c = torch.randint(0, 256, shape, generator=gen, device=Hx.dev(), dtype=torch.int32)
        c = torch.where((c & 0x7F) == 0x7F, c - 1, c)          # no NaN codes
        return c.to(torch.uint8)

    krows, qrows = codes((B, N, d_I)), codes((B, H_I, d_I))
    ksc = torch.full((B, N), 2.0 ** -4, dtype=torch.float32, device=Hx.dev())
    qsc = torch.full((B, H_I), 2.0 ** -3, dtype=torch.float32, device=Hx.dev())
    w = (torch.randn((B, 1, H_I), generator=gen, device=Hx.dev()) * 0.5).contiguous()
    kst = lib.Store(krows, ksc, N, d_I, 0, lib.FP8_E4M3)
    qst = lib.Store(qrows, qsc, H_I, d_I, 0, lib.FP8_E4M3)
    pos = [m * N + (b % 3) for b in range(B)]
    lib.diag_counters(reset=True)
    ref = _run(lib, qst, w, kst, N, pos, B, H_I, m, k)
    assert lib.diag_counters(reset=True)[lib.DIAG_INDEXER_GIVEUPS] == 0
    with _SpinLimit(0):
        all_gave_up = _run(lib, qst, w, kst, N, pos, B, H_I, m, k)
    diag = lib.diag_counters(reset=True)
    assert diag[lib.DIAG_INDEXER_GIVEUPS] == B * 32 and diag[lib.DIAG_INDEXER_WIDE_SELECT] == B, diag
    with _SpinLimit(1):
        mixed = _run(lib, qst, w, kst, N, pos, B, H_I, m, k)
    lib.diag_counters(reset=True)
    assert np.array_equal(all_gave_up, ref)
    assert np.array_equal(mixed, ref)
    flips = 0
    for b in (0, 17):
        nt = int(O.n_visible(pos[b], m, N))
        kv = codec.e4m3_decode(krows[b, :nt].cpu().numpy()) * 2.0 ** -4
        qv = codec.e4m3_decode(qrows[b].cpu().numpy()) * 2.0 ** -3
        wv = w[b, 0].cpu().numpy().astype(np.float64)
        s_ = O.indexer_scores(qv, wv, kv)
        flips += Hx.check_topk(ref[b], s_, k, Hx.score_error_bound(qv, wv, kv))
    assert flips <= 2
