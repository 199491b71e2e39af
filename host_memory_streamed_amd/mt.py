"""ctypes binding of ``libmt.so`` (declared in ``include/mt.h`` and
``include/mt_ops.h``): argument marshalling only. Every step of the training
path runs inside the library; nothing here computes.

Raises ``RuntimeError`` at first use if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmt.so")

MT_OK, MT_EINVAL, MT_EHOSTOOM, MT_EDEVOOM, MT_EHIP, MT_ENONFINITE, MT_ETIMEOUT, MT_ENOGRADS, MT_ESTATE = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)
MT_FP32, MT_BF16 = 0, 1
MT_KEEP_GRADS, MT_KERNEL_TIMING, MT_TRACE, MT_OVERLAP_OPT, MT_PROGRESS, MT_CACHE_NO_REFRESH = 1, 2, 4, 8, 16, 32
MT_BF16_GRADS = 64
MT_GEMM_NT, MT_GEMM_NN, MT_GEMM_TN = 0, 1, 2
PHASES = {0: "load", 1: "fwd", 2: "head", 3: "bwd", 4: "grad", 5: "adamw", 6: "ckpt_out", 7: "ckpt_in",
          8: "refresh"}
UNIT_EMB, UNIT_HEAD = -1, -2


class MTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class ModelConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "max_batch",
        "max_seq", "compute_dtype", "n_layer_buffers", "host_threads")] + [
        ("flags", ctypes.c_uint32), ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float)] + [
        (n, ctypes.c_double) for n in ("lr", "beta1", "beta2", "adam_eps", "weight_decay")] + [
        ("chunk_rows", ctypes.c_int32), ("ckpt_host", ctypes.c_int32), ("grad_ring_slots", ctypes.c_int32),
        ("wait_timeout_ms", ctypes.c_int32), ("micro_batches", ctypes.c_int32)]


class DeviceEnv(ctypes.Structure):
    _fields_ = [("copy_in", ctypes.c_void_p), ("compute", ctypes.c_void_p), ("copy_out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


class StepStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in (
        "step_ms", "forward_ms", "h2d_bytes", "d2h_bytes", "h2d_busy_ms", "d2h_busy_ms", "compute_busy_ms",
        "adamw_ms", "adamw_bytes", "tail_ms", "model_flops", "hw_flops")] + [
        ("tokens", ctypes.c_int64), ("step", ctypes.c_int64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class SchedEntry(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int32), ("unit", ctypes.c_int32), ("buffer", ctypes.c_int32),
                ("stream", ctypes.c_int32), ("t0_ms", ctypes.c_double), ("t1_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I32, _I64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "mt_tensor_count": (_I32, [ctypes.POINTER(ModelConfig)]),
    "mt_host_bytes": (ctypes.c_int, [ctypes.POINTER(ModelConfig), ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                     ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "mt_tensor_info": (ctypes.c_int, [ctypes.POINTER(ModelConfig), _I32, ctypes.c_char_p, _I32,
                                      ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "mt_device_plan": (ctypes.c_int, [ctypes.POINTER(ModelConfig), ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "mt_create": (ctypes.c_int, [ctypes.POINTER(ModelConfig), _P, ctypes.POINTER(DeviceEnv), ctypes.POINTER(_P)]),
    "mt_set_param": (ctypes.c_int, [_P, _I32, _P]),
    "mt_train_step": (ctypes.c_int, [_P, _P, _P, _I32, _I32, ctypes.POINTER(_F)]),
    "mt_token_losses": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(_I64)]),
    "mt_params": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_I64)]),
    "mt_grads": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_I64)]),
    "mt_opt_state": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_I64)]),
    "mt_stats": (ctypes.c_int, [_P, ctypes.POINTER(StepStats)]),
    "mt_kernel_stats": (ctypes.c_int, [_P, ctypes.POINTER(KernelStat), _I32, ctypes.POINTER(_I32)]),
    "mt_schedule": (ctypes.c_int, [_P, ctypes.POINTER(SchedEntry), _I32, ctypes.POINTER(_I32)]),
    "mt_trace_dump": (ctypes.c_int, [_P, ctypes.c_char_p]),
    "mt_device_bytes": (ctypes.c_int, [_P, ctypes.POINTER(_I64)]),
    "mt_sync": (ctypes.c_int, [_P]),
    "mt_layout_info": (ctypes.c_int, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "mt_last_error": (ctypes.c_char_p, [_P]),
    "mt_destroy": (None, [_P]),
    "mt_op_gemm": (ctypes.c_int, [_I32, _I32, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P]),
    "mt_op_gemm_variant": (ctypes.c_int, [_I32, _I32, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64,
                                          _I32, _P]),
    "mt_op_gemm_ws_bytes": (_I64, []),
    "mt_op_gemm_ws": (ctypes.c_int, [_I32, _I32, _P, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _I64,
                                     _P]),
    "mt_op_rmsnorm_fwd": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I64, _I32, _F, _P]),
    "mt_op_rmsnorm_bwd_ws_floats": (_I64, [_I64, _I32]),
    "mt_op_rmsnorm_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _P]),
    "mt_rope_table": (ctypes.c_int, [_I32, _I32, _F, _P, _P]),
    "mt_op_rope_fwd": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "mt_op_rope_bwd": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "mt_op_attn_fwd": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "mt_op_attn_bwd_ws_bytes": (_I64, [_I32, _I32, _I32, _I32, _I32]),
    "mt_op_attn_bwd": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "mt_op_attn_bwd_rope": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                           _P]),
    "mt_op_attn_bwd_rope_noalloc": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                   _P]),
    "mt_op_swiglu_fwd": (ctypes.c_int, [_I32, _P, _P, _I64, _I32, _P]),
    "mt_op_swiglu_bwd": (ctypes.c_int, [_I32, _P, _P, _P, _I64, _I32, _P]),
    "mt_op_xent": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I64, _I32, _F, _P]),
    "mt_op_cast": (ctypes.c_int, [_I32, _P, _P, _I64, _P]),
    "mt_adamw_host": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_double, _P, _I32]),
    "mt_adamw_host_g16": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_double, ctypes.c_double, _P, _I32]),
}
_lib = None


def lib():
    """The loaded ``libmt.so`` with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def exported_names():
    return list(_SIGS)


def _check(rc, ctx=None):
    if rc != MT_OK:
        msg = lib().mt_last_error(ctx)
        raise MTError(rc, msg.decode() if msg else "")


def _ptr(a) -> int:
    """Address of a numpy array or a torch tensor (anything with data_ptr)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous
    return a.ctypes.data


def make_config(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, max_batch, max_seq,
                dtype=MT_FP32, n_layer_buffers=2, host_threads=0, flags=0, rms_eps=1e-5,
                rope_base=10000.0, lr=1e-3, beta1=0.9, beta2=0.999, adam_eps=1e-8,
                weight_decay=0.01, chunk_rows=0, ckpt_host=0, grad_ring_slots=0,
                wait_timeout_ms=0, micro_batches=0) -> ModelConfig:
    return ModelConfig(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, max_batch,
                       max_seq, dtype, n_layer_buffers, host_threads, flags, rms_eps, rope_base, lr,
                       beta1, beta2, adam_eps, weight_decay, chunk_rows, ckpt_host, grad_ring_slots,
                       wait_timeout_ms, micro_batches)


def host_bytes(cfg: ModelConfig) -> dict:
    """Host memory a context of cfg allocates (no GPU needed)."""
    st, pin, pag, ck = _I64(), _I64(), _I64(), _I64()
    _check(lib().mt_host_bytes(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(pin), ctypes.byref(pag),
                               ctypes.byref(ck)))
    return {"state": st.value, "pinned": pin.value, "pageable": pag.value, "parked_ckpt": ck.value}


def device_plan(cfg: ModelConfig) -> dict:
    """Device memory a context of cfg takes (no GPU needed): the fixed part
    and one residual checkpoint slot."""
    fixed, slot = _I64(), _I64()
    _check(lib().mt_device_plan(ctypes.byref(cfg), ctypes.byref(fixed), ctypes.byref(slot)))
    return {"fixed": fixed.value, "ckpt_slot": slot.value}


def tensor_table(cfg: ModelConfig):
    """[(name, shape)] in the canonical order, as the library reports it."""
    out = []
    name = ctypes.create_string_buffer(96)
    shape = (_I64 * 2)()
    nd = _I32()
    for i in range(lib().mt_tensor_count(ctypes.byref(cfg))):
        _check(lib().mt_tensor_info(ctypes.byref(cfg), i, name, 96, shape, ctypes.byref(nd)))
        out.append((name.value.decode(), (shape[0],) if nd.value == 1 else (shape[0], shape[1])))
    return out


class Context:
    """One training context (mt_create ... mt_destroy)."""

    def __init__(self, cfg: ModelConfig, params=None, streams=None, workspace=None):
        self.cfg = cfg
        self.table = tensor_table(cfg)
        h = _P()
        arr = None
        if params is not None:
            keep = [np.ascontiguousarray(p, dtype=np.float32) for p in params]   # alive during the call
            arr = (_P * len(keep))(*[k.ctypes.data for k in keep])
        env = None
        if streams is not None or workspace is not None:
            st = tuple(streams) if streams is not None else (None, None, None)
            ws_ptr, ws_bytes = (None, 0)
            if workspace is not None:
                ws_ptr, ws_bytes = _ptr(workspace[0]), int(workspace[1])
            env = DeviceEnv(*st, ws_ptr, ws_bytes)
        rc = lib().mt_create(ctypes.byref(cfg), ctypes.cast(arr, _P) if arr is not None else None,
                             ctypes.byref(env) if env is not None else None, ctypes.byref(h))
        _check(rc, None)
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().mt_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def __del__(self):
        self.close()

    def set_param(self, tid: int, value: np.ndarray):
        v = np.ascontiguousarray(value, dtype=np.float32)
        assert v.size == int(np.prod(self.table[tid][1]))
        _check(lib().mt_set_param(self.h, tid, v.ctypes.data), self.h)

    def train_step(self, tokens: np.ndarray, targets: np.ndarray) -> float:
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        tgt = np.ascontiguousarray(targets, dtype=np.int32)
        assert tok.shape == tgt.shape and tok.ndim == 2
        loss = _F()
        _check(lib().mt_train_step(self.h, tok.ctypes.data, tgt.ctypes.data, tok.shape[0], tok.shape[1],
                                   ctypes.byref(loss)), self.h)
        return loss.value

    def _view(self, fn, tid, shape=None):
        p, n = _P(), _I64()
        _check(fn(self.h, tid, ctypes.byref(p), ctypes.byref(n)), self.h)
        a = np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_float)), shape=(n.value,))
        return a.reshape(shape or self.table[tid][1]).copy()

    def params(self, tid: int) -> np.ndarray:
        return self._view(lib().mt_params, tid)

    def grads(self, tid: int) -> np.ndarray:
        return self._view(lib().mt_grads, tid)

    def opt_state(self, tid: int):
        m, v, t = _P(), _P(), _I64()
        _check(lib().mt_opt_state(self.h, tid, ctypes.byref(m), ctypes.byref(v), ctypes.byref(t)), self.h)
        n = int(np.prod(self.table[tid][1]))
        fp = ctypes.POINTER(ctypes.c_float)
        mm = np.ctypeslib.as_array(ctypes.cast(m, fp), shape=(n,)).reshape(self.table[tid][1]).copy()
        vv = np.ctypeslib.as_array(ctypes.cast(v, fp), shape=(n,)).reshape(self.table[tid][1]).copy()
        return mm, vv, t.value

    def sync(self):
        """Wait for every AdamW update submitted so far (overlapped mode)."""
        _check(lib().mt_sync(self.h), self.h)

    def token_losses(self) -> np.ndarray:
        p, n = _P(), _I64()
        _check(lib().mt_token_losses(self.h, ctypes.byref(p), ctypes.byref(n)), self.h)
        if n.value == 0:
            return np.zeros(0, np.float32)
        return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_float)), shape=(n.value,)).copy()

    def stats(self) -> dict:
        s = StepStats()
        _check(lib().mt_stats(self.h, ctypes.byref(s)), self.h)
        return s.as_dict()

    def kernel_stats(self) -> list:
        buf = (KernelStat * 64)()
        n = _I32()
        _check(lib().mt_kernel_stats(self.h, buf, 64, ctypes.byref(n)), self.h)
        return [dict(name=b.name.decode(), launches=b.launches, ms=b.ms, flops=b.flops, bytes=b.bytes)
                for b in buf[:n.value]]

    def schedule(self) -> list:
        n = _I32()
        _check(lib().mt_schedule(self.h, None, 0, ctypes.byref(n)), self.h)
        buf = (SchedEntry * max(1, n.value))()
        _check(lib().mt_schedule(self.h, buf, n.value, ctypes.byref(n)), self.h)
        return [dict(phase=PHASES[e.phase], unit=e.unit, buffer=e.buffer, stream=e.stream, t0=e.t0_ms, t1=e.t1_ms)
                for e in buf[:n.value]]

    def trace_dump(self, path: str):
        _check(lib().mt_trace_dump(self.h, path.encode()), self.h)

    def device_bytes(self) -> int:
        b = _I64()
        _check(lib().mt_device_bytes(self.h, ctypes.byref(b)), self.h)
        return b.value

    def layout_info(self) -> dict:
        """Token rows per chunk, parked (host) checkpoints, device checkpoint slots."""
        ch, kh, kd = _I64(), _I32(), _I32()
        _check(lib().mt_layout_info(self.h, ctypes.byref(ch), ctypes.byref(kh), ctypes.byref(kd)), self.h)
        return {"chunk_rows": ch.value, "ckpt_host": kh.value, "ckpt_device_slots": kd.value}


# ----------------------------------------------------------------- ops ---

def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream


def gemm(dtype, layout, A, lda, B, ldb, C, ldc, M, N, K, R=None, ldr=0, stream=None, variant=0):
    _check(lib().mt_op_gemm_variant(dtype, layout, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(R), ldr, M, N,
                                    K, variant, _stream(stream)))


def gemm_ws_bytes():
    return lib().mt_op_gemm_ws_bytes()


def gemm_ws(dtype, layout, A, lda, B, ldb, C, ldc, M, N, K, ws, ws_bytes, R=None, ldr=0, stream=None):
    _check(lib().mt_op_gemm_ws(dtype, layout, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(R), ldr, M, N, K,
                               _ptr(ws), ws_bytes, _stream(stream)))


def rmsnorm_fwd(out_dtype, x, w, y, rstd, rows, d, eps, stream=None):
    _check(lib().mt_op_rmsnorm_fwd(out_dtype, _ptr(x), _ptr(w), _ptr(y), _ptr(rstd), rows, d, eps,
                                   _stream(stream)))


def rmsnorm_bwd_ws_floats(rows, d):
    return lib().mt_op_rmsnorm_bwd_ws_floats(rows, d)


def rmsnorm_bwd(x, w, rstd, dy, dx, accumulate, dw, ws, rows, d, stream=None):
    _check(lib().mt_op_rmsnorm_bwd(_ptr(x), _ptr(w), _ptr(rstd), _ptr(dy), _ptr(dx), accumulate, _ptr(dw),
                                   _ptr(ws), rows, d, _stream(stream)))


def rope_table(T, hd, base):
    c = np.empty((T, hd // 2), np.float32)
    s = np.empty((T, hd // 2), np.float32)
    _check(lib().mt_rope_table(T, hd, base, c.ctypes.data, s.ctypes.data))
    return c, s


def rope(out_dtype, backward, x, out, cos, sin, B, T, H, Hkv, hd, stream=None):
    f = lib().mt_op_rope_bwd if backward else lib().mt_op_rope_fwd
    _check(f(out_dtype, _ptr(x), _ptr(out), _ptr(cos), _ptr(sin), B, T, H, Hkv, hd, _stream(stream)))


def attn_fwd(dtype, qkv, o, o_cast, lse, B, T, H, Hkv, hd, stream=None):
    _check(lib().mt_op_attn_fwd(dtype, _ptr(qkv), _ptr(o), _ptr(o_cast), _ptr(lse), B, T, H, Hkv, hd,
                                _stream(stream)))


def attn_bwd_ws_bytes(dtype, B, T, H, hd):
    return lib().mt_op_attn_bwd_ws_bytes(dtype, B, T, H, hd)


def attn_bwd(dtype, qkv, o, dout, lse, dqkv, ws, B, T, H, Hkv, hd, stream=None):
    _check(lib().mt_op_attn_bwd(dtype, _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dqkv), _ptr(ws), B, T,
                                H, Hkv, hd, _stream(stream)))


def attn_bwd_rope(dtype, qkv, o, dout, lse, cos, sin, dqkv, ws, B, T, H, Hkv, hd, stream=None):
    _check(lib().mt_op_attn_bwd_rope(dtype, _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(cos), _ptr(sin),
                                     _ptr(dqkv), _ptr(ws), B, T, H, Hkv, hd, _stream(stream)))


def attn_bwd_rope_noalloc(dtype, qkv, o, dout, lse, cos, sin, dqkv, B, T, H, Hkv, hd, stream=None):
    """mt_op_attn_bwd_rope with the library's static scratch (no workspace)."""
    _check(lib().mt_op_attn_bwd_rope_noalloc(dtype, _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(cos),
                                             _ptr(sin), _ptr(dqkv), B, T, H, Hkv, hd, _stream(stream)))


def swiglu_fwd(out_dtype, gu, act, M, F, stream=None):
    _check(lib().mt_op_swiglu_fwd(out_dtype, _ptr(gu), _ptr(act), M, F, _stream(stream)))


def swiglu_bwd(out_dtype, gu, dact, dgu, M, F, stream=None):
    _check(lib().mt_op_swiglu_bwd(out_dtype, _ptr(gu), _ptr(dact), _ptr(dgu), M, F, _stream(stream)))


def xent(out_dtype, logits, targets, loss, dlogits, rows, V, scale, stream=None):
    _check(lib().mt_op_xent(out_dtype, _ptr(logits), _ptr(targets), _ptr(loss), _ptr(dlogits), rows, V, scale,
                            _stream(stream)))


def cast(out_dtype, x, y, n, stream=None):
    _check(lib().mt_op_cast(out_dtype, _ptr(x), _ptr(y), n, _stream(stream)))


def adamw_host(p, m, v, g, t, lr, beta1, beta2, eps, weight_decay, bf16_out=None, threads=0):
    for a in (p, m, v, g):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    _check(lib().mt_adamw_host(_ptr(p), _ptr(m), _ptr(v), _ptr(g), p.size, t, lr, beta1, beta2, eps,
                               weight_decay, _ptr(bf16_out), threads))


def adamw_host_g16(p, m, v, g16, t, lr, beta1, beta2, eps, weight_decay, g32_out=None, bf16_out=None,
                   threads=0):
    """mt_adamw_host with the gradient as bf16 bit patterns (uint16)."""
    for a in (p, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    assert g16.dtype == np.uint16 and g16.flags.c_contiguous
    _check(lib().mt_adamw_host_g16(_ptr(p), _ptr(m), _ptr(v), _ptr(g16), _ptr(g32_out), p.size, t, lr, beta1,
                                   beta2, eps, weight_decay, _ptr(bf16_out), threads))


@dataclass
class Workload:
    """A named synthetic workload: model shape plus batch and sequence."""
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    batch: int
    seq: int


WORKLOADS = {
    "tiny": Workload("tiny", 2, 64, 4, 4, 16, 172, 256, 2, 32),
    "1.3b": Workload("1.3b", 24, 2048, 16, 16, 128, 5632, 32000, 4, 2048),
    "14b": Workload("14b", 48, 5120, 40, 8, 128, 13824, 152064, 1, 4096),
    "7b-512k": Workload("7b-512k", 32, 4096, 32, 32, 128, 11008, 32000, 1, 524288),
    # the same decoder at twice the context (1048576 tokens), past the pages' 512k
    "7b-1m": Workload("7b-1m", 32, 4096, 32, 32, 128, 11008, 32000, 1, 1048576),
    "120b": Workload("120b", 88, 10240, 80, 8, 128, 28672, 128000, 1, 4096),
}
