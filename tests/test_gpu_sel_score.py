"""GPU tests of csa_indexer_topk's sel_score output on every selection path.

The output pairs each selected index with the float32 score the selection
compared (the order key read back), -inf in padded slots, so that the
(score, index) pairs of selections over separate entry ranges can be merged
into one top-k (kenelite analysis 5.3: per-query top-k over the indexer
scores).  Checked here, path by path: the selection is identical with and
without the output, every selected score is within the float32 error bound of
the oracle's score of that entry (exactly equal on integer inputs, where every
score is exact), and the padding is -inf.  Paths: the streaming prefill
kernel, one chunk per query, chunks + merge, the one-pass long-list kernel
(including queries that see fewer than k entries, which are scored only when
the output is asked for) and the three-kernel long-list path."""
import numpy as np
import pytest

import synth
from oracle import csa as O
from tests import helpers as Hx

pytestmark = pytest.mark.gpu


def _inputs(B, Tq, N, H_I, d_I, fmt, layer):
    keys = synth.tensor(0, "idx_k", (B, N, d_I), rmsnorm=True, layer=layer)
    q = synth.tensor(0, "idx_q", (B, Tq * H_I, d_I), rmsnorm=True, layer=layer)
    w = synth.tensor(0, "head_w", (B, Tq, H_I), std=0.02, layer=layer).astype(np.float32)
    kst, kdeq = Hx.upload_store(keys, fmt)
    qst, qdeq = Hx.upload_store(q, fmt)
    return kst, kdeq, qst, qdeq.reshape(B, Tq, H_I, d_I), w


def _select(lib, qst, w, kst, N, pos, B, Tq, H_I, m, k, scores):
    import torch
    sel = torch.full((B, Tq, k), -7, dtype=torch.int32, device=Hx.dev())
    sc = torch.full((B, Tq, k), 7.0, dtype=torch.float32, device=Hx.dev()) if scores else None
    nws = lib.indexer_topk_workspace(B, Tq, N, k)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=Hx.dev())
    qp = None if pos is None else Hx.to_dev(np.asarray(pos, np.int64))
    lib.indexer_topk(qst, Hx.to_dev(w), kst, N, qp, B, Tq, H_I, m, k, sel, ws, sel_score=sc)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), None if sc is None else sc.cpu().numpy()


def _check(lib, qst, w, kst, kdeq, qdeq, N, pos, B, Tq, H_I, m, k, rows=None, exact=False):
    sel0, _ = _select(lib, qst, w, kst, N, pos, B, Tq, H_I, m, k, False)
    sel1, sc = _select(lib, qst, w, kst, N, pos, B, Tq, H_I, m, k, True)
    assert np.array_equal(sel0, sel1), "asking for the scores changed the selection"
    rows = range(Tq) if rows is None else rows
    for b in range(B):
        for i in rows:
            t = i if pos is None else pos[b][i]
            nt = int(O.n_visible(t, m, N))
            got, gs = sel1[b, i], sc[b, i]
            valid = got >= 0
            assert np.all(np.isneginf(gs[~valid])), "padded slots must hold -inf"
            assert int(valid.sum()) == min(k, nt)
            idx = got[valid].astype(np.int64)
            ref = O.indexer_scores(qdeq[b, i], w[b, i].astype(np.float64), kdeq[b, idx])
            if exact:
                assert np.array_equal(gs[valid].astype(np.float64), ref), (b, i)
            else:
                err = Hx.score_error_bound(qdeq[b, i], w[b, i].astype(np.float64), kdeq[b, idx])
                assert np.all(np.abs(gs[valid] - ref) <= err + 1e-6 * np.abs(ref)), (b, i)
    return sel1, sc


def test_sel_score_streaming_prefill(lib):
    """FP8 keys of 64 dims, 4096 queries: the single-pass streaming kernel."""
    T, m, k, H_I, d_I = 4096, 4, 512, 8, 64
    N = T // m
    kst, kdeq, qst, qdeq, w = _inputs(1, T, N, H_I, d_I, "fp8", 5)
    rows = sorted(set(range(0, T, 53)) | {0, 2, 3, 4, k * m - 1, k * m, T - 1})
    _check(lib, qst, w, kst, kdeq, qdeq, N, None, 1, T, H_I, m, k, rows=rows)


def test_sel_score_one_chunk(lib):
    """float32 keys of 32 dims: one chunk per query, selected in place."""
    T, m, k, H_I, d_I = 2048, 4, 64, 2, 32
    N = T // m
    kst, kdeq, qst, qdeq, w = _inputs(1, T, N, H_I, d_I, "f32", 6)
    rows = sorted(set(range(0, T, 31)) | {0, 3, 4, 255, 256, T - 1})
    _check(lib, qst, w, kst, kdeq, qdeq, N, None, 1, T, H_I, m, k, rows=rows)


def test_sel_score_chunks_and_merge(lib):
    """MXFP4 keys, 300 queries over 40,000 entries: two chunks per query,
    their candidates merged."""
    B, Tq, N, m, k, H_I, d_I = 1, 300, 40000, 4, 128, 8, 64
    kst, kdeq, qst, qdeq, w = _inputs(B, Tq, N, H_I, d_I, "mxfp4", 7)
    pos = [[m * N - 1 - 97 * i for i in range(Tq)]]
    _check(lib, qst, w, kst, kdeq, qdeq, N, pos, B, Tq, H_I, m, k, rows=range(0, Tq, 23))


def test_sel_score_one_pass_long_lists(lib):
    """One query per sequence over 20,000 entries (the one-pass kernel), and
    sequences that see fewer than k entries on the same path."""
    B, N, m, k, H_I, d_I = 4, 20000, 4, 1024, 8, 64
    kst, kdeq, qst, qdeq, w = _inputs(B, 1, N, H_I, d_I, "fp8", 8)
    pos = [[m * N + 3], [m * N - 17], [m * 600 + 1], [3]]        # 20000, 19995, 600 and 1 visible entries
    _check(lib, qst, w, kst, kdeq, qdeq, N, pos, B, 1, H_I, m, k)


def test_sel_score_exact_on_integer_inputs(lib):
    """Integer keys and queries with unit head weights make every score an
    exact small integer (massive ties): the returned scores equal the
    oracle's exactly."""
    B, N, H_I, d_I, m, k = 2, 50000, 8, 64, 4, 1024
    rng = np.random.default_rng(41)
    keys = rng.integers(-2, 3, (B, N, d_I)).astype(np.float64)
    keys[:, :, 0] = 2.0                            # amax 2 per row: scale 2^-7, codes exact
    q = rng.integers(-1, 2, (B, H_I, d_I)).astype(np.float64)
    q[:, :, 1] = 1.0
    kst, kdeq = Hx.upload_store(keys, "fp8")
    qst, qdeq = Hx.upload_store(q, "fp8")
    assert np.array_equal(kdeq, keys) and np.array_equal(qdeq, q)
    w = np.ones((B, 1, H_I), np.float32)
    pos = [[m * N + 2], [m * 31000 + 1]]
    _check(lib, qst, w, kst, kdeq, qdeq.reshape(B, 1, H_I, d_I), N, pos, B, 1, H_I, m, k, exact=True)


def test_sel_score_three_kernel_long_lists(lib):
    """More than 128 chunks of 8192 entries per query (1,050,000 entries):
    score, compact and final select as three launches; the second sequence
    sees 700 entries."""
    B, N, m, k, H_I, d_I = 2, 1050000, 4, 1024, 8, 64
    kst, kdeq, qst, qdeq, w = _inputs(B, 1, N, H_I, d_I, "fp8", 9)
    pos = [[m * N - 2], [m * 700]]
    _check(lib, qst, w, kst, kdeq, qdeq, N, pos, B, 1, H_I, m, k)


def _merge_pairs(parts, k):
    """Host merge of (score, global index) lists: the k largest scores, ties
    to the smaller index, returned in ascending index order (the order of the
    entry point's output)."""
    sc = np.concatenate([p[0] for p in parts])
    ix = np.concatenate([p[1] for p in parts])
    keep = ix >= 0
    sc, ix = sc[keep], ix[keep]
    order = np.lexsort((ix, -sc.astype(np.float64)))[:k]
    return np.sort(ix[order])


@pytest.mark.parametrize("N,k,split", [(50000, 1024, 23456), (3000, 512, 1000)])
def test_range_selections_merge_to_the_whole_selection(lib, N, k, split):
    """The entry range [0, N) split in two, as two devices holding halves of
    one sequence's compressed keys would hold it: each range is selected on
    its own (positions shifted so that a range sees the query's visible
    entries inside it), and merging the two (score, index) lists gives the
    selection of one call over the whole range, exactly (integer inputs make
    every score exact, with many ties)."""
    B, H_I, d_I, m = 1, 8, 64, 4
    rng = np.random.default_rng(43 + N)
    keys = rng.integers(-2, 3, (B, N, d_I)).astype(np.float64)
    keys[:, :, 0] = 2.0
    q = rng.integers(-1, 2, (B, H_I, d_I)).astype(np.float64)
    q[:, :, 1] = 1.0
    w = np.ones((B, 1, H_I), np.float32)
    qst, _ = Hx.upload_store(q, "fp8")
    for t in (m * N + 1, m * (split + 700) + 2):              # sees all N; sees 700 entries of the second range
        whole, _ = Hx.upload_store(keys, "fp8")
        sel, _ = _select(lib, qst, w, whole, N, [[t]], B, 1, H_I, m, k, False)
        nt = int(O.n_visible(t, m, N))
        parts = []
        for r0, r1 in ((0, split), (split, N)):
            part, _ = Hx.upload_store(keys[:, r0:r1], "fp8")
            seen = max(0, min(nt, r1) - r0)
            tp = m * seen - 1                                    # a position that sees exactly `seen` entries
            s_r, sc_r = _select(lib, qst, w, part, r1 - r0, [[tp]], B, 1, H_I, m, k, True)
            idx = s_r[0, 0].astype(np.int64)
            parts.append((sc_r[0, 0], np.where(idx >= 0, idx + r0, -1)))
        merged = _merge_pairs(parts, k)
        want = sel[0, 0][sel[0, 0] >= 0]
        assert np.array_equal(merged, want), t
