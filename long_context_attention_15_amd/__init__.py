"""Python binding of libcsa.so, the gfx950 CSA/HCA hybrid attention library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors, passed as raw pointers)
and the current HIP stream.  The names mirror the C entry points declared in
``include/csa.h``.  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa.so")

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
ATTN_PARTIAL = 1
WIN_RING = 2
BATCH_INVARIANT = 4
FMT_NAMES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "mxfp4": MXFP4}


class CsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class _CStore(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("cap", ctypes.c_int64),
                ("dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("row_bytes", ctypes.c_int32)]


class _CNormRope(ctypes.Structure):
    _fields_ = [("norm_gain", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("rope_dims", ctypes.c_int32),
                ("rope_theta", ctypes.c_void_p), ("pos0", ctypes.c_int64)]


@dataclass
class NormRope:
    """csa_norm_rope: RMSNorm (gain: float32 [dim] device tensor, or None) then
    partial RoPE of the last rope_dims dims (theta: float32 [rope_dims/2]
    device tensor) of stored rows or queries; pos0 = position of token row 0
    for csa_compress_kv."""
    gain: object = None
    eps: float = 1e-6
    rope_dims: int = 0
    theta: object = None
    pos0: int = 0

    def c(self) -> "_CNormRope":
        return _CNormRope(_ptr(self.gain), self.eps, self.rope_dims, _ptr(self.theta), self.pos0)


def _post(p):
    return None if p is None else ctypes.byref(p.c())


_lib: Optional[ctypes.CDLL] = None

_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "csa_version": ([], ctypes.c_char_p),
    "csa_status_string": ([_I], ctypes.c_char_p),
    "csa_last_error": ([], ctypes.c_char_p),
    "csa_compress_kv": ([_P, _I, _I, _I64, _I64, _I, _P, _P, _CStore, _I64, _P, _P], _I),
    "csa_decode_append": ([_P, _I, _I, _P, _P, _I, _I, _P, _P, _CStore, _CStore, _I, _P, _P], _I),
    "csa_decode_rebuild": ([_P, _I, _I, _I, _I64, _P, _P, _P, _I, _I, _P, _P, _CStore, _CStore, _I, _P, _P], _I),
    "csa_indexer_topk_workspace": ([_I, _I, _I64, _I], _SZ),
    "csa_indexer_topk": ([_CStore, _P, _CStore, _I64, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "csa_attn_workspace": ([_I, _I, _I, _I, _I64], _SZ),
    "csa_sparse_attn_prefill": ([_P, _I, _I, _I, _I, _CStore, _I64, _P, _I, _CStore, _I, _P, _F, _P, _P, _I,
                                 _P, _P], _I),
    "csa_sparse_attn_decode": ([_P, _I, _I, _I, _CStore, _I64, _P, _I, _CStore, _P, _I, _P, _F, _P, _P, _I, _P,
                                _SZ, _P, _P], _I),
    "hca_attn": ([_P, _I, _I, _I, _I, _CStore, _I, _I64, _P, _CStore, _I, _P, _F, _P, _P, _I, _P, _SZ, _P, _P], _I),
    "swa_merge": ([_P, _I, _I, _I, _I, _CStore, _P, _I, _I, _P, _P, _P, _F, _P, _P, _P], _I),
    "csa_diag_counters": ([_P, _I, _I], _I),
    "csa_sparse_attn_decode_noalloc": ([_P, _I, _I, _I, _CStore, _I64, _P, _I, _CStore, _P, _I, _P, _F, _P, _P, _I,
                                        _P, _P], _I),
}
EXPORTS = tuple(_SIGS)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcsa.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} not found: build it with long_context_attention_15_amd/build.py")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def version() -> str:
    return load().csa_version().decode()


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        raise CsaError(status, f"{what}: {lib.csa_status_string(status).decode()}: "
                               f"{lib.csa_last_error().decode()}")


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _fmt_of(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def row_bytes(fmt: int, dim: int, rope: int = 0) -> int:
    return {F32: 4 * dim, FP8_E4M3: dim - rope + 2 * rope, MXFP4: dim // 2}[fmt]


@dataclass
class Store:
    """An entry store in device memory: rows [B][cap][row_bytes] uint8 plus
    scales (float32 [B][cap] for FP8, uint8 [B][cap][dim/32] for MXFP4)."""
    rows: object
    scales: object
    cap: int
    dim: int
    rope: int
    fmt: int

    @property
    def row_bytes(self) -> int:
        return row_bytes(self.fmt, self.dim, self.rope)

    @property
    def B(self) -> int:
        return int(self.rows.shape[0])

    def c(self) -> _CStore:
        return _CStore(_ptr(self.rows), _ptr(self.scales), self.cap, self.dim, self.rope, self.fmt,
                       self.row_bytes)


def alloc_store(B: int, cap: int, dim: int, fmt, rope: int = 0, device="cuda") -> Store:
    """Allocate an (uninitialised) store with torch."""
    import torch
    fmt = FMT_NAMES.get(fmt, fmt)
    rb = row_bytes(fmt, dim, rope)
    rows = torch.empty((B, cap, rb), dtype=torch.uint8, device=device)
    if fmt == FP8_E4M3:
        scales = torch.empty((B, cap), dtype=torch.float32, device=device)
    elif fmt == MXFP4:
        scales = torch.empty((B, cap, dim // 32), dtype=torch.uint8, device=device)
    else:
        scales = None
    return Store(rows, scales, cap, dim, rope, fmt)


DIAG_INDEXER_GIVEUPS, DIAG_INDEXER_WIDE_SELECT, DIAG_COUNT = 0, 1, 4


def diag_counters(reset: bool = False):
    """csa_diag_counters: the device's diagnostic event counters (synchronises the device)."""
    buf = (ctypes.c_uint64 * DIAG_COUNT)()
    _check(load().csa_diag_counters(ctypes.cast(buf, ctypes.c_void_p), DIAG_COUNT, int(reset)), "csa_diag_counters")
    return [int(v) for v in buf]


# ------------------------------------------------------------- entry points
def compress_kv(tok, m: int, gate, bias, out: Store, out_row0: int = 0, post: Optional[NormRope] = None,
                stream=None):
    """csa_compress_kv: tok [B][T][dim] float32 or bfloat16 (rows contiguous)."""
    B, T, D = tok.shape
    assert tok.stride(2) == 1 and tok.stride(1) == D, "token rows must be contiguous"
    _check(load().csa_compress_kv(_ptr(tok), _fmt_of(tok), B, T, tok.stride(0), m, _ptr(gate), _ptr(bias),
                                  out.c(), out_row0, _post(post), _stream(stream)), "csa_compress_kv")


def decode_append(tok, pos, tail, m: int, gate, bias, out: Store, win: Optional[Store] = None, W: int = 0,
                  post: Optional[NormRope] = None, stream=None):
    """csa_decode_append: tok [B][dim] float32 or bfloat16, pos [B] int64, tail [B][R][dim] (tok's dtype,
    R a multiple of m); window row pos mod W of `win` when given, entry (pos+1)/m - 1 of `out` when a
    block closes."""
    B, D = tok.shape
    assert tok.is_contiguous() and tail.is_contiguous() and tail.dtype == tok.dtype and tail.shape[0] == B
    assert tail.shape[2] == D and pos.dtype.itemsize == 8 and pos.numel() == B
    wc = win.c() if win is not None else _CStore(None, None, 0, 0, 0, 0, 0)
    _check(load().csa_decode_append(_ptr(tok), _fmt_of(tok), B, _ptr(pos), _ptr(tail), int(tail.shape[1]), m,
                                    _ptr(gate), _ptr(bias), out.c(), wc, W, _post(post), _stream(stream)),
           "csa_decode_append")


def decode_rebuild(tok, p0, tail, m: int, gate, bias, out: Store, win: Optional[Store] = None, W: int = 0,
                   post: Optional[NormRope] = None, n_valid=None, stream=None):
    """csa_decode_rebuild: tok [B][n][dim] float32 or bfloat16 (rows contiguous), p0 int64 [B] (positions of
    row 0, multiples of m), n_valid int32 [B] or None; leaves tail, window and entries as decode appends at
    p0 .. p0 + n_valid - 1 would."""
    B, n, D = tok.shape
    assert tok.stride(2) == 1 and tok.stride(1) == D, "token rows must be contiguous"
    assert tail.is_contiguous() and tail.dtype == tok.dtype and tail.shape[0] == B and tail.shape[2] == D
    assert p0.dtype.itemsize == 8 and p0.numel() == B
    wc = win.c() if win is not None else _CStore(None, None, 0, 0, 0, 0, 0)
    assert n_valid is None or (n_valid.dtype.itemsize == 4 and n_valid.numel() == B)
    _check(load().csa_decode_rebuild(_ptr(tok), _fmt_of(tok), B, n, tok.stride(0), _ptr(p0), _ptr(n_valid), _ptr(tail),
                                     int(tail.shape[1]), m, _ptr(gate), _ptr(bias), out.c(), wc, W, _post(post),
                                     _stream(stream)), "csa_decode_rebuild")


def indexer_topk_workspace(B: int, Tq: int, n_entries: int, k: int) -> int:
    return int(load().csa_indexer_topk_workspace(B, Tq, n_entries, k))


def indexer_topk(q_idx: Store, head_w, keys: Store, n_entries: int, q_pos, B: int, Tq: int, H_I: int, m: int,
                 k: int, sel, ws=None, stream=None, sel_score=None):
    """csa_indexer_topk: writes sel [B][Tq][k] int32 (and, if given,
    sel_score [B][Tq][k] float32)."""
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().csa_indexer_topk(q_idx.c(), _ptr(head_w), keys.c(), n_entries, _ptr(q_pos), B, Tq, H_I, m, k,
                                   _ptr(sel), _ptr(sel_score), _ptr(ws), wsb, _stream(stream)), "csa_indexer_topk")


def attn_workspace(B: int, Tq: int, H: int, dim: int, max_list: int) -> int:
    return int(load().csa_attn_workspace(B, Tq, H, dim, max_list))


def sparse_attn_prefill(q, ckv: Store, n_entries: int, sel, k: int, win: Store, W: int, sink, sm_scale: float,
                        out, lse=None, flags: int = 0, q_post: Optional[NormRope] = None, stream=None):
    """csa_sparse_attn_prefill: q [B][T][H][dim]."""
    B, T, H, D = q.shape
    _check(load().csa_sparse_attn_prefill(_ptr(q), _fmt_of(q), B, T, H, ckv.c(), n_entries, _ptr(sel), k, win.c(),
                                          W, _ptr(sink), sm_scale, _ptr(out), _ptr(lse), flags, _post(q_post),
                                          _stream(stream)),
           "csa_sparse_attn_prefill")


def sparse_attn_decode(q, ckv: Store, n_entries: int, sel, k: int, ring: Store, pos, W: int, sink,
                       sm_scale: float, out, lse=None, flags: int = 0, ws=None, q_post: Optional[NormRope] = None,
                       stream=None):
    """csa_sparse_attn_decode: q [B][H][dim], pos int64 [B]."""
    B, H, D = q.shape
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().csa_sparse_attn_decode(_ptr(q), _fmt_of(q), B, H, ckv.c(), n_entries, _ptr(sel), k, ring.c(),
                                         _ptr(pos), W, _ptr(sink), sm_scale, _ptr(out), _ptr(lse), flags, _ptr(ws),
                                         wsb, _post(q_post), _stream(stream)), "csa_sparse_attn_decode")


def sparse_attn_decode_noalloc(q, ckv: Store, n_entries: int, sel, k: int, ring: Store, pos, W: int, sink,
                               sm_scale: float, out, lse=None, flags: int = 0, q_post: Optional[NormRope] = None,
                               stream=None):
    """csa_sparse_attn_decode_noalloc: as sparse_attn_decode, split partials in the library's device scratch."""
    B, H, D = q.shape
    _check(load().csa_sparse_attn_decode_noalloc(_ptr(q), _fmt_of(q), B, H, ckv.c(), n_entries, _ptr(sel), k,
                                                 ring.c(), _ptr(pos), W, _ptr(sink), sm_scale, _ptr(out), _ptr(lse),
                                                 flags, _post(q_post), _stream(stream)),
           "csa_sparse_attn_decode_noalloc")


def hca_attn(q, hkv: Store, m_prime: int, n_entries: int, q_pos, win: Store, W: int, sink, sm_scale: float,
             out, lse=None, flags: int = 0, ws=None, q_post: Optional[NormRope] = None, stream=None):
    """hca_attn: q [B][Tq][H][dim]; q_pos int64 [B][Tq] or None (prefill)."""
    B, Tq, H, D = q.shape
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().hca_attn(_ptr(q), _fmt_of(q), B, Tq, H, hkv.c(), m_prime, n_entries, _ptr(q_pos), win.c(), W,
                           _ptr(sink), sm_scale, _ptr(out), _ptr(lse), flags, _ptr(ws), wsb, _post(q_post),
                           _stream(stream)),
           "hca_attn")


def swa_merge(q, win: Store, q_pos, W: int, flags: int, part_out, part_lse, sink, sm_scale: float, out,
              q_post: Optional[NormRope] = None, stream=None):
    """swa_merge: q [B][Tq][H][dim]; part_out float32 like q; part_lse [B][Tq][H]."""
    B, Tq, H, D = q.shape
    _check(load().swa_merge(_ptr(q), _fmt_of(q), B, Tq, H, win.c(), _ptr(q_pos), W, flags, _ptr(part_out),
                            _ptr(part_lse), _ptr(sink), sm_scale, _ptr(out), _post(q_post), _stream(stream)),
           "swa_merge")
