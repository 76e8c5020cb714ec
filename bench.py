"""Benchmark of the CSA + HCA hybrid attention hot path on one MI355X.

Headline: 128K-token prefill throughput of one CSA layer (m=4, indexer 8x64
FP8, top-512, window 128, sink) plus one HCA layer (m'=128, window 128,
sink), 64 query heads, head dim 512 (448 FP8 + 64 BF16 RoPE dims).  A step is
the whole path for both layers: compress KV, store the window, compress the
indexer keys, quantise the indexer queries, indexer + top-k, CSA sparse
attention; HCA compress, window, dense attention.  value = 131072 / step time.
Decode at 1M context (CSA B=32 FP8 indexer; hybrid B=16 MXFP4 indexer + HCA)
is reported alongside as microseconds per token.

Inputs are seeded synthetic data (torch's generator on the GPU; RMS-normalised
N(0,1) activations, N(0, 0.02^2) weights, N(0,1) sinks) of the workloads'
shapes, resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA+HCA attn tokens/s (128K prefill) + µs/token decode at 1M ctx; % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
FP32_VALU_TFLOPS = 157.3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ inputs
class Gen:
    """Seeded device-side synthetic data."""

    def __init__(self, seed=0):
        import torch
        self.g = torch.Generator(device="cuda")
        self.g.manual_seed(seed)

    def normal(self, shape, std=1.0, rms=False, dtype=None):
        import torch
        x = torch.randn(shape, generator=self.g, device="cuda", dtype=torch.float32)
        if rms:
            x = x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + 1e-6)
        if std != 1.0:
            x = x * std
        return x if dtype is None else x.to(dtype)


def norm_rope(csa, gen, D, R, base=10000.0):
    """RMSNorm (gain 1 + N(0, 0.1^2), eps 1e-6) and RoPE of the R trailing
    dims (theta_i = base^(-2i/R)) as the library's post-processing block."""
    import torch
    theta = torch.pow(torch.tensor(base, dtype=torch.float64),
                      -2.0 * torch.arange(R // 2, dtype=torch.float64) / R).float().cuda()
    return csa.NormRope(gain=1.0 + gen.normal((D,), std=0.1), eps=1e-6, rope_dims=R, theta=theta)


def quantised_rows(csa, gen, B, n, D, fmt, R, chunk_rows=1 << 18, cap=None):
    """A store of n RMS-normalised N(0,1) rows per batch element (cap >= n
    rows allocated), quantised by the library's own m = 1 compressor (as a
    prefill would have stored them)."""
    import torch
    st = csa.alloc_store(B, cap or n, D, fmt, R)
    zero = torch.zeros(D, device="cuda")
    one = torch.ones(1, device="cuda")
    for b in range(B):
        for r0 in range(0, n, chunk_rows):
            r1 = min(n, r0 + chunk_rows)
            x = gen.normal((1, r1 - r0, D), rms=True, dtype=torch.bfloat16)
            sub = csa.Store(st.rows[b:b + 1], None if st.scales is None else st.scales[b:b + 1], n, D, R, st.fmt)
            csa.compress_kv(x, 1, zero, one, sub, out_row0=r0)
    return st


# ---------------------------------------------------------------- workloads
class Prefill128K:
    """CSA + HCA prefill layers at T = 131072."""

    def __init__(self, csa, T=131072, H=64, D=512, R=64, W=128, k=512, HI=8, dI=64, m=4, mh=128):
        import torch
        self.csa, self.T, self.H, self.D, self.R, self.W, self.k = csa, T, H, D, R, W, k
        self.HI, self.dI, self.m, self.mh = HI, dI, m, mh
        g = Gen(0)
        bf = torch.bfloat16
        self.kv = g.normal((1, T, D), rms=True, dtype=bf)
        self.kv_h = g.normal((1, T, D), rms=True, dtype=bf)
        self.xi = g.normal((1, T, dI), rms=True, dtype=bf)
        self.qi = g.normal((1, T * HI, dI), rms=True, dtype=bf)
        self.w = g.normal((1, T, HI), std=0.02)
        self.q = g.normal((1, T, H, D), rms=True, dtype=bf)
        self.q_h = g.normal((1, T, H, D), rms=True, dtype=bf)
        self.gate = g.normal((D,), std=0.02)
        self.bias = g.normal((m,), std=0.02)
        self.gate_i = g.normal((dI,), std=0.02)
        self.bias_i = g.normal((m,), std=0.02)
        self.gate_h = g.normal((D,), std=0.02)
        self.bias_h = g.normal((mh,), std=0.02)
        self.sink = g.normal((H,))
        self.sink_h = g.normal((H,))
        self.zero_i = torch.zeros(dI, device="cuda")
        self.one = torch.ones(1, device="cuda")
        self.N, self.Nh = T // m, T // mh
        self.ckv = csa.alloc_store(1, self.N, D, "fp8", R)
        self.win = csa.alloc_store(1, T, D, "fp8", R)
        self.keys = csa.alloc_store(1, self.N, dI, "fp8")
        self.qst = csa.alloc_store(1, T * HI, dI, "fp8")
        self.hkv = csa.alloc_store(1, self.Nh, D, "fp8", R)
        self.win_h = csa.alloc_store(1, T, D, "fp8", R)
        self.sel = torch.empty((1, T, k), dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.out_h = torch.empty_like(self.q_h)
        nws = csa.indexer_topk_workspace(1, T, self.N, k)
        self.ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        self.tau = 1.0 / math.sqrt(D)
        self.post = norm_rope(csa, g, D, R)

    def ops(self, post=None):
        """The step; with `post`, RMSNorm + partial RoPE fused into the
        compressors (stored entries and window rows) and the attention
        kernels (queries)."""
        c = self.csa
        return [
            ("csa_compress_kv(m=4)", lambda: c.compress_kv(self.kv, self.m, self.gate, self.bias, self.ckv,
                                                           post=post)),
            ("csa_compress_kv(window)", lambda: c.compress_kv(self.kv, 1, self.gate, self.one, self.win, post=post)),
            ("csa_compress_kv(idx keys)", lambda: c.compress_kv(self.xi, self.m, self.gate_i, self.bias_i, self.keys)),
            ("csa_compress_kv(idx q)", lambda: c.compress_kv(self.qi, 1, self.zero_i, self.one, self.qst)),
            ("csa_indexer_topk", lambda: c.indexer_topk(self.qst, self.w, self.keys, self.N, None, 1, self.T,
                                                        self.HI, self.m, self.k, self.sel, self.ws)),
            ("csa_sparse_attn_prefill", lambda: c.sparse_attn_prefill(self.q, self.ckv, self.N, self.sel, self.k,
                                                                      self.win, self.W, self.sink, self.tau,
                                                                      self.out, q_post=post)),
            ("hca_compress_kv(m=128)", lambda: c.compress_kv(self.kv_h, self.mh, self.gate_h, self.bias_h, self.hkv,
                                                             post=post)),
            ("hca_compress_kv(window)", lambda: c.compress_kv(self.kv_h, 1, self.gate_h, self.one, self.win_h,
                                                              post=post)),
            ("hca_attn", lambda: c.hca_attn(self.q_h, self.hkv, self.mh, self.Nh, None, self.win_h, self.W,
                                            self.sink_h, self.tau, self.out_h, q_post=post)),
        ]

    # algorithmic work per launch
    def pairs(self, m, N, sel_k=None):
        """sum over queries of (compressed entries attended + window entries)."""
        T, W = self.T, self.W
        # window: sum_t min(W, t+1)
        win = W * (W + 1) // 2 + (T - W) * W
        # compressed: sum_t min(N, floor((t+1)/m)) (capped by k for CSA)
        tot = 0
        for t0 in range(0, T, 4096):
            import numpy as np
            t = np.arange(t0, min(T, t0 + 4096))
            nt = np.minimum(N, (t + 1) // m)
            if sel_k is not None:
                nt = np.minimum(nt, sel_k)
            tot += int(nt.sum())
        return tot + win

    def algorithmic(self):
        H, D = self.H, self.D
        csa_pairs = self.pairs(self.m, self.N, self.k)
        hca_pairs = self.pairs(self.mh, self.Nh)
        fl = lambda p: 4.0 * H * D * p          # QK^T and PV, 2 flops per MAC
        # indexer: every (query, visible compressed entry) pair scores H_I dot
        # products of d_I dims (the head-weighted ReLU sum is VALU work)
        idx_pairs = self.pairs(self.m, self.N) - (self.W * (self.W + 1) // 2 + (self.T - self.W) * self.W)
        return {
            "csa_sparse_attn_prefill": {"flops": fl(csa_pairs), "pairs": csa_pairs},
            "hca_attn": {"flops": fl(hca_pairs), "pairs": hca_pairs},
            "csa_indexer_topk": {"flops": 2.0 * self.HI * self.dI * idx_pairs, "pairs": idx_pairs},
        }


class Decode1M:
    """CSA decode (B=32, FP8 indexer) or hybrid decode (B=16, MXFP4 indexer +
    HCA layer) with 2^20 tokens of context per sequence."""

    def __init__(self, csa, hybrid, ctx=1 << 20, H=128, D=512, R=64, W=128, k=1024, HI=8, dI=64, m=4, mh=128):
        import torch
        self.csa, self.hybrid = csa, hybrid
        self.B = 16 if hybrid else 32
        B = self.B
        self.H, self.D, self.W, self.k, self.HI, self.dI, self.m, self.mh = H, D, W, k, HI, dI, m, mh
        self.N, self.Nh = ctx // m, ctx // mh
        g = Gen(1 if hybrid else 2)
        bf = torch.bfloat16
        ifmt = "mxfp4" if hybrid else "fp8"
        # one spare entry each: the step that closes the next block writes it
        self.ckv = quantised_rows(csa, g, B, self.N, D, "fp8", R, cap=self.N + 1)
        self.keys = quantised_rows(csa, g, B, self.N, dI, ifmt, 0, cap=self.N + 1)
        self.ring = quantised_rows(csa, g, B, W, D, "fp8", R)
        self.qi = g.normal((B, HI, dI), rms=True, dtype=bf)
        self.qst = csa.alloc_store(B, HI, dI, ifmt)
        self.w = g.normal((B, 1, HI), std=0.02)
        self.q = g.normal((B, H, D), rms=True, dtype=bf)
        self.sink = g.normal((H,))
        self.pos = torch.full((B,), ctx, dtype=torch.int64, device="cuda")
        self.sel = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.zero_i = torch.zeros(dI, device="cuda")
        self.one = torch.ones(1, device="cuda")
        nws = csa.indexer_topk_workspace(B, 1, self.N, k)
        self.iws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        aws = max(csa.attn_workspace(B, 1, H, D, k + W), csa.attn_workspace(B, 1, H, D, self.Nh + W))
        self.aws = torch.empty(max(aws, 16), dtype=torch.uint8, device="cuda")
        self.tau = 1.0 / math.sqrt(D)
        if hybrid:
            self.hkv = quantised_rows(csa, g, B, self.Nh, D, "fp8", R, cap=self.Nh + 1)
            self.ring_h = quantised_rows(csa, g, B, W, D, "fp8", R)
            self.q_h = g.normal((B, 1, H, D), rms=True, dtype=bf)
            self.sink_h = g.normal((H,))
            self.out_h = torch.empty_like(self.q_h)
        self.flush = torch.empty(1 << 29, dtype=torch.uint8, device="cuda")   # 512 MiB > the 256 MB MALL
        # cache maintenance of the step: the new token's KV and indexer key,
        # raw tails of the current blocks, compressor weights
        self.kv_tok = g.normal((B, D), rms=True, dtype=bf)
        self.ik_tok = g.normal((B, dI), rms=True, dtype=bf)
        self.kv_tail = g.normal((B, m, D), rms=True, dtype=bf)
        self.ik_tail = g.normal((B, m, dI), rms=True, dtype=bf)
        self.g_kv, self.b_kv = g.normal((D,), std=0.02), g.normal((m,), std=0.02)
        self.g_ik, self.b_ik = g.normal((dI,), std=0.02), g.normal((m,), std=0.02)
        if hybrid:
            self.hkv_tok = g.normal((B, D), rms=True, dtype=bf)
            self.h_tail = g.normal((B, mh, D), rms=True, dtype=bf)
            self.g_h, self.b_h = g.normal((D,), std=0.02), g.normal((mh,), std=0.02)
        self.post = norm_rope(csa, g, D, R)
        # positions at which the step closes a block (CSA every m tokens, HCA every m')
        self.pos_close_m = torch.full((B,), ctx + m - 1, dtype=torch.int64, device="cuda")
        self.pos_close_mh = torch.full((B,), ctx + mh - 1, dtype=torch.int64, device="cuda")

    def append_ops(self, pos, pos_h, post=None):
        """Cache maintenance of the step's new token (window slot, tails, and
        the compressed entry when a block closes at that position); `post`
        adds RMSNorm + partial RoPE to the KV rows written."""
        c = self.csa
        o = [
            ("csa_decode_append(kv)", lambda: c.decode_append(self.kv_tok, pos, self.kv_tail, self.m, self.g_kv,
                                                              self.b_kv, self.ckv, self.ring, self.W, post=post)),
            ("csa_decode_append(idx keys)", lambda: c.decode_append(self.ik_tok, pos, self.ik_tail, self.m,
                                                                    self.g_ik, self.b_ik, self.keys)),
        ]
        if self.hybrid:
            o.append(("hca_decode_append(kv)", lambda: c.decode_append(self.hkv_tok, pos_h, self.h_tail, self.mh,
                                                                       self.g_h, self.b_h, self.hkv, self.ring_h,
                                                                       self.W, post=post)))
        return o

    def ops(self, post=None):
        """The decode step; `post` adds RMSNorm + partial RoPE of the queries
        to the attention kernels."""
        c = self.csa
        o = [
            ("csa_compress_kv(idx q)", lambda: c.compress_kv(self.qi, 1, self.zero_i, self.one, self.qst)),
            ("csa_indexer_topk", lambda: c.indexer_topk(self.qst, self.w, self.keys, self.N, self.pos, self.B, 1,
                                                        self.HI, self.m, self.k, self.sel, self.iws)),
            ("csa_sparse_attn_decode", lambda: c.sparse_attn_decode(self.q, self.ckv, self.N, self.sel, self.k,
                                                                    self.ring, self.pos, self.W, self.sink,
                                                                    self.tau, self.out, ws=self.aws, q_post=post)),
        ]
        if self.hybrid:
            o.append(("hca_attn(decode)", lambda: c.hca_attn(self.q_h, self.hkv, self.mh, self.Nh, self.pos[:, None],
                                                             self.ring_h, self.W, self.sink_h, self.tau, self.out_h,
                                                             flags=c.WIN_RING, ws=self.aws, q_post=post)))
        return o

    def unfused_window_ops(self):
        """The step's CSA attention as the pages' two-part form: attention over
        the selected entries only (CSA_ATTN_PARTIAL: float32 partial + LSE),
        then swa_merge adds the window and the sink (the step fuses both)."""
        import torch
        c = self.csa
        if not hasattr(self, "part_o"):
            self.part_o = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
            self.part_lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
            self.out_m = torch.empty_like(self.q)
        return [
            ("csa_sparse_attn_decode(partial)", lambda: c.sparse_attn_decode(
                self.q, self.ckv, self.N, self.sel, self.k, self.ring, self.pos, self.W, self.sink, self.tau,
                self.part_o, lse=self.part_lse, flags=c.ATTN_PARTIAL, ws=self.aws)),
            ("swa_merge", lambda: c.swa_merge(self.q[:, None], self.ring, self.pos[:, None], self.W, c.WIN_RING,
                                              self.part_o, self.part_lse, self.sink, self.tau, self.out_m[:, None])),
        ]

    def invariant_ops(self):
        """The step's attention with CSA_BATCH_INVARIANT (no split lists)."""
        c = self.csa
        f = c.BATCH_INVARIANT
        o = [("csa_sparse_attn_decode", lambda: c.sparse_attn_decode(self.q, self.ckv, self.N, self.sel, self.k,
                                                                     self.ring, self.pos, self.W, self.sink,
                                                                     self.tau, self.out, flags=f, ws=self.aws))]
        if self.hybrid:
            o.append(("hca_attn(decode)", lambda: c.hca_attn(self.q_h, self.hkv, self.mh, self.Nh, self.pos[:, None],
                                                             self.ring_h, self.W, self.sink_h, self.tau, self.out_h,
                                                             flags=c.WIN_RING | f, ws=self.aws)))
        return o

    def algorithmic_bytes(self):
        """HBM bytes the method must move per step (no implementation overheads)."""
        B, N, k, W, H, D = self.B, self.N, self.k, self.W, self.H, self.D
        key_b = (32 + 2) if self.hybrid else (64 + 4)
        row_b = 576 + 4
        per = {
            "csa_indexer_topk": B * (N * key_b + self.HI * (key_b) + 4 * self.HI + 4 * k),
            "csa_sparse_attn_decode": B * ((k + W) * row_b + 2 * H * D * 2 + 4 * k),
        }
        if self.hybrid:
            per["hca_attn(decode)"] = B * ((self.Nh + W) * row_b + 2 * H * D * 2)
        return per


# ------------------------------------------------------------------ timing
def time_ops(ops, steps, warmup, flush=None):
    """Run the op list `steps` times after `warmup` untimed passes.  Events
    bracket every op on the current stream (the one the library launches on).
    Returns (total ms per step by the outer events, {op: mean ms})."""
    import torch
    for _ in range(warmup):
        for _, f in ops:
            f()
    torch.cuda.synchronize()
    per = {n: 0.0 for n, _ in ops}
    total = 0.0
    for s in range(steps):
        if flush is not None:
            flush.fill_(s & 255)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i, (_, f) in enumerate(ops):
            f()
            evs[i + 1].record()
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(ops):
            per[n] += evs[i].elapsed_time(evs[i + 1])
        total += evs[0].elapsed_time(evs[-1])
        log(f"step {s + 1}/{steps}: {evs[0].elapsed_time(evs[-1]):.3f} ms")
    return total / steps, {n: v / steps for n, v in per.items()}


def time_graph(ops, steps, flush=None):
    """The op list captured once in a HIP graph (after two eager passes on a
    side stream) and replayed `steps` times; events bracket each replay on
    the current stream.  Returns ms per replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            for _, f in ops:
                f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, f in ops:
            f()
    g.replay()
    torch.cuda.synchronize()
    total = 0.0
    for s in range(steps):
        if flush is not None:
            flush.fill_(s & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    log(f"graph replays: {total / steps:.3f} ms per step")
    del g
    return total / steps


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(T=131072, n_sample=512, budget_s=15.0):
    """The oracle on the host cores: the 128K CSA+HCA prefill, compressing all
    tokens and running indexer/top-k/attention on a stride sample of query
    rows; tokens/s extrapolated to all 131072 rows."""
    import numpy as np
    import synth
    from oracle import csa as O
    try:
        from threadpoolctl import threadpool_info
        pool = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        pool = os.cpu_count() or 1
    allowed = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    H, D, R, W, k, HI, dI, m, mh = 64, 512, 64, 128, 512, 8, 64, 4, 128
    N, Nh = T // m, T // mh
    tau = 1.0 / math.sqrt(D)
    t0 = time.perf_counter()
    kv = synth.tensor(0, "kv", (T, D), rmsnorm=True)
    kvh = synth.tensor(0, "kv", (T, D), rmsnorm=True, layer=1)
    xi = synth.tensor(0, "idx_k", (T, dI), rmsnorm=True)
    t_gen = time.perf_counter() - t0
    cpu0, wall0 = time.process_time(), time.perf_counter()
    t0 = time.perf_counter()
    ckv = O.quantize(O.compress(kv, synth.tensor(0, "gate", (D,), std=0.02),
                                synth.tensor(0, "bias", (m,), std=0.02), m), "fp8", R)
    win = O.quantize(kv, "fp8", R)
    keys = O.quantize(O.compress(xi, synth.tensor(0, "idx_gate", (dI,), std=0.02),
                                 synth.tensor(0, "idx_bias", (m,), std=0.02), m), "fp8")
    hkv = O.quantize(O.compress(kvh, synth.tensor(0, "gate", (D,), std=0.02, layer=1),
                                synth.tensor(0, "bias", (mh,), std=0.02, layer=1), mh), "fp8", R)
    winh = O.quantize(kvh, "fp8", R)
    t_compress = time.perf_counter() - t0
    rows = np.unique(np.linspace(0, T - 1, n_sample).astype(np.int64))
    sink = synth.tensor(0, "sink", (H,))
    sinkh = synth.tensor(0, "sink", (H,), layer=1)
    t0 = time.perf_counter()
    done = 0
    for t in rows:
        t = int(t)
        qi = O.quantize(synth.tensor(0, "idx_q", (HI, dI), rmsnorm=True, start=t * HI * dI), "fp8")
        w = synth.tensor(0, "head_w", (HI,), std=0.02, start=t * HI).astype(np.float32)
        nt = int(O.n_visible(t, m, N))
        sel = O.topk_select(O.indexer_scores(qi, w, keys[:nt]), k)
        q = synth.tensor(0, "q", (H, D), rmsnorm=True, start=t * H * D)
        idx = sel[sel >= 0]
        O.attend(q, np.concatenate([ckv[idx], win[O.window_positions(t, W)]]), sink, tau)
        qh = synth.tensor(0, "q", (H, D), rmsnorm=True, layer=1, start=t * H * D)
        nth = int(O.n_visible(t, mh, Nh))
        O.attend(qh, np.concatenate([hkv[:nth], winh[O.window_positions(t, W)]]), sinkh, tau)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t_rows = time.perf_counter() - t0
    busy = (time.process_time() - cpu0) / (time.perf_counter() - wall0)   # threads kept busy on average
    total = t_compress + t_rows * T / done
    return {"value": T / total, "unit": "tokens/s", "cores": max(1, math.ceil(busy)), "kind": "oracle",
            "cpu_model": model, "threads_busy_avg": round(busy, 2), "blas_threads": int(pool),
            "cpus_allowed": allowed,
            "sample": f"{done} of {T} query rows (stride sample) of the 128K CSA+HCA prefill, all tokens "
                      f"compressed; per-row time extrapolated to {T} rows (compress {t_compress:.1f} s, "
                      f"rows {t_rows:.1f} s, input generation {t_gen:.1f} s excluded)"}


# ------------------------------------------------------------- HBM traffic
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "csa_hca_prefill_128k_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "long_context_attention_15_amd", "csrc", "attn_m32.hip")


def recorded_traffic(op):
    """HBM bytes per launch of `op` from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    record under profiles/ (scaled by a plain copy's counters), or None when
    there is none or the kernel source changed since the counters were taken
    (the record carries the SHA-256 of the source it measured)."""
    import hashlib
    try:
        text = open(TRAFFIC_RECORD).read()
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic-record:"):
            f = dict(kv.split("=", 1) for kv in line.split()[1:])
            if f.get("op") == op and f.get("sha256") == sha:
                return float(f["bytes"])
    return None


# -------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (the reference for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path runs and is timed on a single MI355X; "
              "runs over several GPUs are not supported (--gpus 1 only).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    import long_context_attention_15_amd as csa
    csa.load()
    log(f"lib {csa.version()} on {torch.cuda.get_device_name(0)}")

    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, RMS-normalised N(0,1))",
              "config": {"workload": "CSA+HCA prefill, one CSA layer (m=4, FP8 indexer 8x64, top-512) + one HCA "
                                     "layer (m'=128), T=131072, H=64, D=512 (448 FP8 + 64 BF16), window 128, sink",
                         "global_batch": 1, "seq_len": 131072}}
    kernels = {}
    if args.only in ("all", "prefill"):
        log("prefill 128K: building inputs")
        pf = Prefill128K(csa)
        torch.cuda.synchronize()
        ms, per = time_ops(pf.ops(), args.steps, args.warmup)
        result["value"] = pf.T / (ms * 1e-3)
        result["ms_per_step"] = ms
        kernels.update({f"prefill/{n}": v for n, v in per.items()})
        alg = pf.algorithmic()
        dom = max((n for n in alg if n != "csa_indexer_topk"), key=lambda n: per[n])
        ach = alg[dom]["flops"] / (per[dom] * 1e-3) / 1e12
        result["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": ach / MFMA_BF16_TFLOPS, "traffic": recorded_traffic(dom)}
        result["prefill_ops_tflops"] = {n: alg[n]["flops"] / (per[n] * 1e-3) / 1e12 for n in alg}
        # the indexer scores FP8 keys on bf16 MFMAs (exact conversion), so its
        # peak is the bf16 one; top-k selection rides along in the same kernel
        ia = alg["csa_indexer_topk"]["flops"] / (per["csa_indexer_topk"] * 1e-3) / 1e12
        result["indexer_roofline"] = {"kernel": "csa_indexer_topk", "bound": "mfma", "achieved": ia,
                                      "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ia / MFMA_BF16_TFLOPS,
                                      "flops": alg["csa_indexer_topk"]["flops"]}
        # RMSNorm + partial RoPE fused into the step (stored rows and queries)
        ms_p, per_p = time_ops(pf.ops(pf.post), args.steps, args.warmup)
        result["norm_rope_prefill"] = {"ms_per_step": ms_p, "added_ms": ms_p - ms,
                                       "added_ms_per_op": {n: per_p[n] - per[n] for n in per
                                                           if "idx" not in n and "indexer" not in n}}
        del pf
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        dec = {}
        for hybrid in (False, True):
            name = "hybrid_decode_1m" if hybrid else "csa_decode_1m"
            log(f"{name}: building caches")
            d = Decode1M(csa, hybrid)
            torch.cuda.synchronize()
            csa.diag_counters(reset=True)
            ms, per = time_ops(d.ops(), args.decode_steps, 2, flush=d.flush)
            ms_g = time_graph(d.ops(), args.decode_steps, flush=d.flush)
            ab = d.algorithmic_bytes()
            # the step as a serving loop runs it (one HIP graph per step) and,
            # for reference, launched op by op from Python
            dec[name] = {"batch": d.B, "us_per_step": ms_g * 1e3, "us_per_token": ms_g * 1e3 / d.B,
                         "us_per_step_eager": ms * 1e3, "us_per_token_eager": ms * 1e3 / d.B,
                         "hbm_gbs": {n: ab[n] / (per[n] * 1e-3) / 1e9 for n in ab},
                         "hbm_frac": {n: ab[n] / (per[n] * 1e-3) / 1e9 / HBM_PEAK_GBS for n in ab}}
            kernels.update({f"{name}/{n}": v for n, v in per.items()})
            # cache maintenance of the new token (outside the step, whose caches
            # are given): at the step's position, and at positions that close a
            # block (every m-th token for CSA, every m'-th for HCA), where the
            # compressed entry is written too
            _, per_app = time_ops(d.append_ops(d.pos, d.pos), args.decode_steps, 2, flush=d.flush)
            _, per_close = time_ops(d.append_ops(d.pos_close_m, d.pos_close_mh), args.decode_steps, 2, flush=d.flush)
            dec[name]["append_us"] = {n: v * 1e3 for n, v in per_app.items()}
            dec[name]["append_block_close_us"] = {n: v * 1e3 for n, v in per_close.items()}
            # RMSNorm + partial RoPE: queries in the step, KV rows in the appends
            ms_gp = time_graph(d.ops(d.post), args.decode_steps, flush=d.flush)
            _, per_appp = time_ops(d.append_ops(d.pos_close_m, d.pos_close_mh, d.post), args.decode_steps, 2,
                                   flush=d.flush)
            dec[name]["norm_rope"] = {"us_per_step": ms_gp * 1e3, "added_us": (ms_gp - ms_g) * 1e3,
                                      "append_block_close_added_us": {n: (per_appp[n] - per_close[n]) * 1e3
                                                                      for n in per_close}}
            # row a7 on its own: partial attention + swa_merge (window and sink)
            _, per_sw = time_ops(d.unfused_window_ops(), args.decode_steps, 2, flush=d.flush)
            dec[name]["unfused_window_us"] = {n: v * 1e3 for n, v in per_sw.items()}
            # the attention with batch-invariant results (no split lists)
            _, per_inv = time_ops(d.invariant_ops(), args.decode_steps, 2, flush=d.flush)
            dec[name]["batch_invariant_attn_us"] = {n: v * 1e3 for n, v in per_inv.items()}
            # indexer workgroups that stopped waiting for their query's threshold
            # (exact either way, only slower) and final selects past their LDS budget
            diag = csa.diag_counters(reset=True)
            dec[name]["indexer_giveups"] = int(diag[csa.DIAG_INDEXER_GIVEUPS])
            dec[name]["indexer_wide_selects"] = int(diag[csa.DIAG_INDEXER_WIDE_SELECT])
            if diag[csa.DIAG_INDEXER_GIVEUPS]:
                log(f"{name}: {diag[csa.DIAG_INDEXER_GIVEUPS]} indexer workgroups gave up waiting")
            del d
            torch.cuda.empty_cache()
        result["decode"] = dec
    result["kernels_ms"] = kernels
    if not args.no_cpu_baseline and args.only in ("all", "prefill"):
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
