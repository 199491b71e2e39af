"""Seeded synthetic inputs (weights and token ids) for the streamed training step.

This module holds none of the training step's arithmetic: it draws numbers.
It is the one module that both the CPU oracle's tests and the benchmark use,
so that both sides see the same inputs. The generator is a counter-based
SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) with Box-Muller normals; its
definition is written out in ``csrc/synth/synth.c``. Every element depends only
on (seed, stream, index), so tensors of any size are drawn in parallel and
slices of a tensor can be drawn independently.

Streams: weight tensor ``i`` of the canonical tensor order draws from stream
``i``; token ids draw from stream ``TOKEN_STREAM``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

TOKEN_STREAM = 1 << 40
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmtsynth.so")
_lib = None


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def lib():
    """Load ``libmtsynth.so`` (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        L.synth_normal_f32.restype = None
        L.synth_uniform_i32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        L.synth_uniform_i32.restype = None
        L.synth_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.c_int64, ctypes.c_void_p]
        L.synth_words.restype = None
        _lib = L
    return _lib


def normal(seed: int, stream: int, shape, std: float = 1.0, offset: int = 0,
           out: np.ndarray | None = None) -> np.ndarray:
    """float32 array of ``std * N(0, 1)`` draws for elements ``offset ..``."""
    n = int(np.prod(shape, dtype=np.int64))
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    lib().synth_normal_f32(seed, stream, offset, n, float(std),
                           out.ctypes.data_as(ctypes.c_void_p), _threads())
    return out


def uniform_int(seed: int, stream: int, shape, n_values: int, offset: int = 0) -> np.ndarray:
    """int32 array of uniform draws in ``[0, n_values)``."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(shape, dtype=np.int32)
    lib().synth_uniform_i32(seed, stream, offset, n, int(n_values),
                            out.ctypes.data_as(ctypes.c_void_p), _threads())
    return out


def words(seed: int, stream: int, offset: int, n: int) -> np.ndarray:
    """Raw 64-bit generator words (for checking the generator against its definition)."""
    out = np.empty(n, dtype=np.uint64)
    lib().synth_words(seed, stream, offset, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def token_batch(seed: int, batch: int, seq: int, vocab: int):
    """Next-token batch: draw ``[batch, seq + 1]`` uniform ids, return
    ``tokens = ids[:, :seq]`` and ``targets = ids[:, 1:]`` (both int32, C order)."""
    ids = uniform_int(seed + 1, TOKEN_STREAM, (batch, seq + 1), vocab)
    return np.ascontiguousarray(ids[:, :seq]), np.ascontiguousarray(ids[:, 1:])


def init_tensor(seed: int, tensor_id: int, shape, is_gain: bool, std: float = 0.02,
                out: np.ndarray | None = None) -> np.ndarray:
    """Initial value of one weight tensor: norm gains are 1.0, every other
    tensor is N(0, std^2) drawn from stream ``tensor_id``."""
    if is_gain:
        if out is None:
            return np.ones(shape, dtype=np.float32)
        out.fill(1.0)
        return out
    return normal(seed, tensor_id, shape, std, out=out)
