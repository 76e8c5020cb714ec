"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the attention method itself: it only draws
numbers and shapes them into the workloads described on the pages (the
DeepSeek-V4 spec table on the kenelite analysis page, and the CSA/HCA sections
of the llm-tech overview).  Random numbers are produced by a counter-based
generator so that any slice of any tensor can be regenerated on its own:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state advances by the golden-ratio increment and
  each output is the published 64-bit finaliser of the state.
* Box-Muller: two uniforms in (0, 1] x [0, 1) give two N(0, 1) values.

A tensor is identified by (seed, stream); element ``i`` of it is a pure
function of (seed, stream, i).
"""
from __future__ import annotations

import numpy as np

from .configs import CONFIGS, Config, get_config  # noqa: F401

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_STREAM_MUL = 0xD1B54A32D192ED03
_MASK64 = (1 << 64) - 1


def _fmix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _fmix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, stream: int) -> int:
    """Starting SplitMix64 state for tensor ``stream`` under ``seed``."""
    return _fmix64_int((seed * 0x9E3779B97F4A7C15) ^ ((stream * _STREAM_MUL) & _MASK64))


def uint64_stream(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 sequence of a stream."""
    base = np.uint64(stream_base(seed, stream))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = base + idx * _GOLDEN
        return _fmix64(state)


def normal(seed: int, stream: int, shape, start: int = 0) -> np.ndarray:
    """N(0, 1) float64 values; element ``start + i`` of the stream for flat index i.

    Elements 2p and 2p+1 of a stream come from the Box-Muller pair p, so a slice
    that starts at an odd element still reproduces the full-stream values.
    """
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    n = int(np.prod(shape)) if len(shape) else 1
    if n == 0:
        return np.zeros(shape, dtype=np.float64)
    p0 = start // 2
    p1 = (start + n + 1) // 2
    r = uint64_stream(seed, stream, 2 * p0, 2 * (p1 - p0))
    hi = (r >> np.uint64(11)).astype(np.float64)
    u1 = (hi[0::2] + 1.0) * (2.0 ** -53)           # (0, 1]
    u2 = hi[1::2] * (2.0 ** -53)                    # [0, 1)
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = rad * np.cos(2.0 * np.pi * u2)
    z[1::2] = rad * np.sin(2.0 * np.pi * u2)
    off = start - 2 * p0
    return z[off:off + n].reshape(shape)


def rms_normalize(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Scale every last-axis row to unit root-mean-square (unit gain).

    This shapes the value distribution of the inputs ("activations after
    RMSNorm"); it is input preparation upstream of every library call.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


# Stream ids of the named tensors of one attention layer; a second layer adds
# LAYER_STRIDE to each.
STREAMS = {
    "q": 1, "kv": 2, "idx_k": 3, "idx_q": 4, "head_w": 5,
    "gate": 6, "bias": 7, "idx_gate": 8, "idx_bias": 9, "sink": 10, "norm_gain": 11,
}
LAYER_STRIDE = 100


def sid(name: str, layer: int = 0) -> int:
    return STREAMS[name] + LAYER_STRIDE * layer


def tensor(seed: int, name: str, shape, *, layer: int = 0, std: float = 1.0,
           rmsnorm: bool = False, start: int = 0) -> np.ndarray:
    """A named input tensor as float64: N(0, std^2), optionally RMS-normalised rows."""
    x = normal(seed, sid(name, layer), shape, start=start)
    if rmsnorm:
        x = rms_normalize(x)
    return x * std if std != 1.0 else x
