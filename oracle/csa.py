"""Oracle of the CSA / HCA hot path (test infrastructure only).

Plain, slow, float64 CPU model of what the hybrid attention of DeepSeek-V4
computes, written from the pages:

* CSA (llm-tech overview, "Compressed Sparse Attention"; kenelite analysis
  section 5.1 pipeline, 5.2 learned 4x compression, 5.3 Lightning Indexer and
  top-k): compress each block of m = 4 tokens' KV into one entry, score the
  compressed entries with the indexer, keep the top-k, attend to those.
* HCA (llm-tech overview, "Heavily Compressed Attention"; kenelite analysis
  section 6): compress m' = 128 tokens per entry, attend densely.
* Both add a 128-token sliding window of raw tokens (llm-tech overview, HCA
  section; kenelite analysis section 7) and an attention-sink logit per head
  (llm-tech overview, "other architecture details").

Where the pages leave an operator open, the spec of this project fixes it:
the compressor is a softmax over the block of per-token logits <x, g> + b_i
weighting the tokens' K/V; the indexer score is sum_h w_h * ReLU(q_h . k); a
query at position t sees compressed entry j iff (j+1)*m - 1 <= t; K = V = the
stored entry (shared KV); the sink is a per-head logit that enters only the
softmax denominator.

Only ``tests/``, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the HIP library never does.
"""
from __future__ import annotations

import numpy as np

from . import codec

NEG_INF = float("-inf")


# ---------------------------------------------------------------- visibility
def n_visible(t, m: int, n_entries: int):
    """Entries a query at position t may see: blocks [j*m, j*m+m-1] with
    j*m + m - 1 <= t, i.e. min(N, floor((t+1)/m))."""
    t = np.asarray(t, dtype=np.int64)
    return np.minimum(n_entries, (t + 1) // m)


def window_positions(t: int, W: int) -> np.ndarray:
    """Raw-token positions of the sliding window of a query at t: the last W
    tokens up to and including t."""
    return np.arange(max(0, t - W + 1), t + 1, dtype=np.int64)


# ------------------------------------------------------------------ compress
def compress(x: np.ndarray, gate: np.ndarray, bias: np.ndarray, m: int) -> np.ndarray:
    """Learned block compression (kenelite analysis section 5.2: each token's
    contribution weight is learned, not average pooling; section 6: the same
    with m' = 128).

    x [T, D] token K/V; gate [D]; bias [m].  For block j (tokens jm .. jm+m-1,
    an incomplete tail block is dropped):
        a_i = <x_{jm+i}, gate> + bias_i,   alpha = softmax(a),
        c_j = sum_i alpha_i x_{jm+i}.
    Returns c [floor(T/m), D] in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    N = T // m
    blocks = x[: N * m].reshape(N, m, D)
    a = blocks @ np.asarray(gate, np.float64) + np.asarray(bias, np.float64)[None, :]
    a = a - a.max(axis=1, keepdims=True)
    alpha = np.exp(a)
    alpha = alpha / alpha.sum(axis=1, keepdims=True)
    return np.einsum("nm,nmd->nd", alpha, blocks)


def decode_append(x: np.ndarray, gate: np.ndarray, bias: np.ndarray, m: int, W: int, p0: int, p1: int):
    """Decode-time cache maintenance of one sequence (kenelite analysis 16,
    inference infrastructure: only whole compression blocks enter the
    compressed cache, an incomplete tail block stays raw; llm-tech overview,
    HCA section: the sliding window holds the latest raw tokens).

    x [T, D] the sequence's tokens.  Positions < p0 were handled before, so
    the raw tail holds the tokens of the current block up to p0; positions
    p0 .. p1-1 arrive one per step.  Each step puts its token in window slot
    p mod W and in the tail; when the tail holds m tokens the block is
    compressed (as in `compress`) into entry p // m = (p+1)/m - 1 and the
    tail restarts.  Returns (entries {j: c_j [D]} for the blocks closed by
    these steps, window {slot: position} of the slots they wrote).
    """
    x = np.asarray(x, dtype=np.float64)
    tail = [x[q] for q in range((p0 // m) * m, p0)]
    entries, window = {}, {}
    for p in range(p0, p1):
        tail.append(x[p])
        window[p % W] = p
        if len(tail) == m:
            entries[p // m] = compress(np.stack(tail), gate, bias, m)[0]
            tail = []
    return entries, window


def restore_state(restored: np.ndarray, x_recent: np.ndarray, gate: np.ndarray, bias: np.ndarray, m: int, W: int,
                  p0: int):
    """Decode state of one sequence at position P rebuilt for prefix reuse
    (kenelite analysis 16, inference infrastructure: compressed CSA / HCA
    entries are restored from storage, the incomplete compression block at
    the end is recomputed, and under zero SWA caching the recent window is
    rebuilt from recomputed raw tokens instead of being stored).

    restored [n_r, D]: entries of the first n_r complete blocks, as stored.
    x_recent [P - p0, D]: raw tokens of positions p0 .. P-1 (p0 a multiple
    of m, p0 <= n_r m).  Returns (entries [P // m, D]: the restored ones,
    then blocks p0/m .. compressed from x_recent (the restored value is kept
    for a block that is both); window {slot q mod W: position q} for the
    last min(W, P) positions; tail: positions of the incomplete block).
    """
    x_recent = np.asarray(x_recent, np.float64)
    P = p0 + x_recent.shape[0]
    n_r = np.asarray(restored).shape[0]
    entries = [np.asarray(restored[j], np.float64) for j in range(min(n_r, P // m))]
    for j in range(len(entries), P // m):
        entries.append(compress(x_recent[j * m - p0: (j + 1) * m - p0], gate, bias, m)[0])
    window = {q % W: q for q in range(max(0, P - W), P)}
    tail = list(range((P // m) * m, P))
    D = x_recent.shape[1]
    return (np.stack(entries) if entries else np.zeros((0, D))), window, tail


# ---------------------------------------------- RMSNorm and partial RoPE
def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """RMSNorm of every last-axis row (10100 analysis, section 3 item 1,
    auxiliary optimisations: queries and KV entries are RMS-normalised, which
    keeps the logits from blowing up): x / sqrt(mean(x^2) + eps) * gain."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, np.float64)


def rope_angles(positions, theta) -> np.ndarray:
    """Rotation angle of pair i at a position: the binary32 product of the
    position (as binary32) and theta_i (binary32), the precision in which the
    kernels form it; [n, R/2] float64."""
    pos32 = np.asarray(positions, np.float64).astype(np.float32)
    th32 = np.asarray(theta, np.float32)
    return (pos32[:, None] * th32[None, :]).astype(np.float64)


def rope(x: np.ndarray, positions, theta, rope_dims: int) -> np.ndarray:
    """Partial rotary position embedding (10100 analysis, section 3 item 1:
    partial RoPE keeps relative position information; llm-tech overview:
    the RoPE dims are the ones kept in BF16): the last rope_dims dims of each
    row, taken as consecutive pairs (x_a, x_b), are rotated by the row's
    angle for that pair: (x_a cos - x_b sin, x_a sin + x_b cos).  Rows
    [n, D], positions [n], theta [rope_dims / 2]."""
    x = np.array(x, np.float64, copy=True)
    if rope_dims == 0:
        return x
    D = x.shape[-1]
    ang = rope_angles(positions, theta)
    c, s = np.cos(ang), np.sin(ang)
    a = x[:, D - rope_dims::2].copy()
    b = x[:, D - rope_dims + 1::2].copy()
    x[:, D - rope_dims::2] = a * c - b * s
    x[:, D - rope_dims + 1::2] = a * s + b * c
    return x


def entry_positions(n: int, m: int, pos0: int = 0) -> np.ndarray:
    """Position given to compressed entry j when it is rotated: the position
    of the last token of its block, pos0 + (j + 1) m - 1 (a block's entry
    becomes visible at that position, so a query there and the entry get
    the same angle; m = 1 gives each token its own position)."""
    return pos0 + (np.arange(n, dtype=np.int64) + 1) * m - 1


def post_rows(rows: np.ndarray, positions, gain=None, eps: float = 1e-6, theta=None, rope_dims: int = 0):
    """RMSNorm (when gain is given), then partial RoPE (when theta is given)
    of stored rows or queries at their positions."""
    y = np.asarray(rows, np.float64)
    if gain is not None:
        y = rms_norm(y, gain, eps)
    if theta is not None and rope_dims:
        y = rope(y, positions, theta, rope_dims)
    return y


# ------------------------------------------------------------- storage rows
def row_bytes(fmt: str, D: int, R: int = 0) -> int:
    if fmt == "f32":
        return 4 * D
    if fmt == "fp8":
        return (D - R) + 2 * R
    if fmt == "mxfp4":
        return D // 2
    raise ValueError(fmt)


def pack_rows(values: np.ndarray, fmt: str, R: int = 0):
    """Quantize rows [n, D] into the stored layout.

    f32   : D little-endian float32; no scale.
    fp8   : dims [0, D-R) as E4M3FN of x/s with one power-of-two scale s per
            row (float32 array), dims [D-R, D) as BF16 (kenelite analysis 8.2:
            RoPE dims BF16, the rest FP8).
    mxfp4 : D/2 bytes, element 2i in the low nibble of byte i, plus one E8M0
            per 32 elements.
    Values are first rounded to float32, the working precision of the kernels.
    Returns (rows uint8 [n, row_bytes], scales or None).
    """
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    n, D = v.shape
    if fmt == "f32":
        return np.ascontiguousarray(v.astype(np.float32)).view(np.uint8).reshape(n, 4 * D), None
    if fmt == "fp8":
        bulk = v[:, : D - R]
        amax = np.max(np.abs(bulk), axis=1) if D - R > 0 else np.zeros(n)
        s = codec.fp8_row_scale(amax)
        codes = codec.e4m3_encode(bulk / s[:, None])
        rope = codec.bf16_encode(v[:, D - R:]).view(np.uint8).reshape(n, 2 * R)
        rows = np.concatenate([codes, rope], axis=1)
        return np.ascontiguousarray(rows), s.astype(np.float32)
    if fmt == "mxfp4":
        codes, e8 = codec.mxfp4_encode(v)
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return np.ascontiguousarray(packed), np.ascontiguousarray(e8)
    raise ValueError(fmt)


def unpack_rows(rows: np.ndarray, scales, fmt: str, D: int, R: int = 0) -> np.ndarray:
    """Inverse of pack_rows: stored rows -> float64 values (exact)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    if fmt == "f32":
        return rows.view(np.float32).reshape(n, D).astype(np.float64)
    if fmt == "fp8":
        bulk = codec.e4m3_decode(rows[:, : D - R]) * np.asarray(scales, np.float64)[:, None]
        rope = codec.bf16_decode(np.ascontiguousarray(rows[:, D - R:]).view(np.uint16).reshape(n, R))
        return np.concatenate([bulk, rope], axis=1)
    if fmt == "mxfp4":
        codes = np.empty((n, D), dtype=np.uint8)
        codes[:, 0::2] = rows & 15
        codes[:, 1::2] = rows >> 4
        return codec.mxfp4_decode(codes, scales)
    raise ValueError(fmt)


def quantize(values: np.ndarray, fmt: str, R: int = 0) -> np.ndarray:
    """Round-trip through storage: what a consumer of the stored rows sees."""
    rows, s = pack_rows(values, fmt, R)
    return unpack_rows(rows, s, fmt, np.asarray(values).shape[1], R)


# ------------------------------------------------------------------- indexer
def indexer_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Lightning Indexer score of every key for one query (llm-tech overview,
    CSA section; kenelite analysis 5.3): I_j = sum_h w_h * ReLU(<q_h, k_j>).

    q_idx [H_I, d_I], w [H_I], keys [n, d_I] -> [n] float64.
    """
    dots = np.asarray(keys, np.float64) @ np.asarray(q_idx, np.float64).T   # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) highest scores, ties going to the smaller index; returned
    in ascending index order and padded with -1 to length k
    (kenelite analysis 5.3: top-512 / top-1024 compressed entries)."""
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    j = np.arange(n)
    order = np.lexsort((j, -scores))          # primary: score desc, then index asc
    take = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[: take.shape[0]] = take
    return out


# ----------------------------------------------------------------- attention
def attend(q: np.ndarray, entries: np.ndarray, sink, tau: float):
    """Softmax attention of H heads over shared entries (K = V = entry), with
    an optional per-head sink logit in the denominator only.

    q [H, D], entries [n, D], sink [H] or None (= -inf).
    logits l_{h,e} = tau <q_h, e>;  M = max(sink_h, max_e l);
    Z = e^{sink_h - M} + sum_e e^{l - M};  o_h = sum_e e^{l - M} e / Z;
    lse_h = M + ln Z.  With no entries and sink = -inf: o = 0, lse = -inf.
    """
    q = np.asarray(q, np.float64)
    E = np.asarray(entries, np.float64)
    H, D = q.shape
    sig = np.full(H, NEG_INF) if sink is None else np.asarray(sink, np.float64)
    if E.shape[0] == 0:
        lmax = np.full(H, NEG_INF)
        l = np.zeros((H, 0))
    else:
        l = tau * (q @ E.T)
        lmax = l.max(axis=1)
    M = np.maximum(sig, lmax)
    o = np.zeros((H, D))
    lse = np.full(H, NEG_INF)
    ok = M > NEG_INF
    if np.any(ok):
        p = np.exp(l[ok] - M[ok, None])
        z = np.exp(sig[ok] - M[ok]) + p.sum(axis=1)
        o[ok] = (p @ E) / z[:, None]
        lse[ok] = M[ok] + np.log(z)
    return o, lse


def csa_prefill(q, ckv, sel, win, W: int, sink, tau: float):
    """CSA core attention for every query of a prefill (kenelite analysis 5.1
    "Top-k Compressed Blocks -> Core Attention", section 7 sliding window).

    q [T, H, D]; ckv [N, D] compressed entries; sel [T, k] (-1 padded);
    win [T, D] raw tokens as stored; query t attends to {ckv[j] : j in sel[t]}
    plus win[t-W+1 .. t] plus the sink.
    """
    T, H, D = q.shape
    o = np.zeros((T, H, D))
    lse = np.zeros((T, H))
    for t in range(T):
        idx = sel[t][sel[t] >= 0]
        ent = np.concatenate([ckv[idx], win[window_positions(t, W)]], axis=0)
        o[t], lse[t] = attend(q[t], ent, sink, tau)
    return o, lse


def hca_prefill(q, hkv, m: int, win, W: int, sink, tau: float, positions=None):
    """HCA dense attention (kenelite analysis section 6; page 5 "applies heavier
    compression with dense attention"): query t attends to every visible entry
    j < n_t plus the window and the sink.  ``positions`` (default 0..T-1)
    gives each query's position."""
    T, H, D = q.shape
    N = hkv.shape[0]
    pos = np.arange(T) if positions is None else np.asarray(positions)
    o = np.zeros((T, H, D))
    lse = np.zeros((T, H))
    for i in range(T):
        t = int(pos[i])
        nt = int(n_visible(t, m, N))
        ent = np.concatenate([hkv[:nt], win[window_positions(t, W)]], axis=0)
        o[i], lse[i] = attend(q[i], ent, sink, tau)
    return o, lse


def ring_window(ring: np.ndarray, pos: int, W: int) -> np.ndarray:
    """Window rows of a decode query at position ``pos`` from a ring of W slots
    in which position p lives in slot p mod W."""
    return ring[window_positions(pos, W) % W]


def csa_decode(q, ckv, sel, ring, pos: int, W: int, sink, tau: float):
    """One decode token of one sequence: q [H, D], sel [k], ring [W, D]."""
    idx = sel[sel >= 0]
    ent = np.concatenate([ckv[idx], ring_window(ring, pos, W)], axis=0)
    return attend(q, ent, sink, tau)


def hca_decode(q, hkv, m: int, n_entries: int, ring, pos: int, W: int, sink, tau: float):
    nt = int(n_visible(pos, m, n_entries))
    ent = np.concatenate([hkv[:nt], ring_window(ring, pos, W)], axis=0)
    return attend(q, ent, sink, tau)


def swa_merge(q, win_rows, part_o, part_lse, sink, tau: float):
    """Merge a partial attention result (o_p normalised over its own entries,
    lse_p = ln sum e^{l}) with window attention and the sink:
        o = (e^{lse_p} o_p + sum_w e^{l_w} v_w) / (e^{lse_p} + sum_w e^{l_w} + e^{sink}).
    q [H, D], win_rows [n_w, D], part_o [H, D], part_lse [H]."""
    q = np.asarray(q, np.float64)
    Wr = np.asarray(win_rows, np.float64)
    H, D = q.shape
    sig = np.full(H, NEG_INF) if sink is None else np.asarray(sink, np.float64)
    lw = tau * (q @ Wr.T) if Wr.shape[0] else np.zeros((H, 0))
    lwmax = lw.max(axis=1) if Wr.shape[0] else np.full(H, NEG_INF)
    lp = np.asarray(part_lse, np.float64)
    M = np.maximum(np.maximum(sig, lwmax), lp)
    o = np.zeros((H, D))
    for h in range(H):
        if M[h] == NEG_INF:
            continue
        pw = np.exp(lw[h] - M[h])
        ep = np.exp(lp[h] - M[h])
        z = ep + pw.sum() + np.exp(sig[h] - M[h])
        o[h] = (ep * np.asarray(part_o[h], np.float64) + pw @ Wr) / z
    return o
