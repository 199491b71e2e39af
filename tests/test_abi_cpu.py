"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, reports the canonical tensor table, rejects bad configurations before
touching a device, and its host-side AdamW and RoPE table agree with the
oracle."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
from oracle.configs import SHAPES
from host_memory_streamed_amd import mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(mt.LIB_PATH):
        from host_memory_streamed_amd import build
        build.build_mt()


def _declared():
    names = set()
    for h in ("mt.h", "mt_ops.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"\b(mt_\w+)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mt.LIB_PATH)
    declared = _declared()
    assert len(declared) >= 30
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert declared == set(mt.exported_names())


@pytest.mark.parametrize("name", list(SHAPES))
def test_tensor_table_matches_oracle(name):
    cfg, B, T = SHAPES[name]
    c = mt.make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                       cfg.vocab, B, T, dtype=mt.MT_BF16)
    lib_table = mt.tensor_table(c)
    orc = O.tensor_table(cfg)
    assert [n for n, _ in lib_table] == [n for n, _, _ in orc]
    assert [tuple(s) for _, s in lib_table] == [tuple(s) for _, s, _ in orc]


@pytest.mark.parametrize("field,value", [("n_layers", 0), ("n_kv_heads", 3), ("head_dim", 48),
                                         ("compute_dtype", 7), ("n_layer_buffers", 1), ("d_model", 66),
                                         ("max_seq", 0), ("flags", 1 << 10), ("chunk_rows", -1),
                                         ("ckpt_host", -1), ("ckpt_host", 1), ("grad_ring_slots", -1),
                                         ("grad_ring_slots", 65), ("wait_timeout_ms", -5), ("micro_batches", -1),
                                         ("micro_batches", 3)])
def test_create_rejects_bad_config(field, value):
    # two layers: no checkpoint can be parked (x_1..x_k with k <= n_layers - 2)
    c = mt.make_config(2, 64, 4, 4, 16, 172, 256, 2, 32)
    setattr(c, field, value)
    h = ctypes.c_void_p()
    rc = mt.lib().mt_create(ctypes.byref(c), None, None, ctypes.byref(h))
    assert rc == mt.MT_EINVAL and not h.value
    assert mt.lib().mt_last_error(None)


def test_bf16_head_dim_restriction():
    c = mt.make_config(2, 64, 4, 4, 16, 172, 256, 2, 32, dtype=mt.MT_BF16)
    h = ctypes.c_void_p()
    assert mt.lib().mt_create(ctypes.byref(c), None, None, ctypes.byref(h)) == mt.MT_EINVAL


def test_host_adamw_matches_oracle_over_steps():
    # Each step starts both sides from the same fp32 state; the fp32 error of
    # each update is bounded by a few ulps of the terms it sums.
    cfg = O.Config(1, 8, 1, 1, 8, 8, 8)
    rng = np.random.default_rng(5)
    n = 100_003   # ragged against the vector width and the chunking
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bf = np.empty(n, np.uint16)
    u = 2.0 ** -23
    for t in range(1, 5):
        g = (rng.standard_normal(n) * 10.0 ** rng.integers(-9, -1, n)).astype(np.float32)
        p0, m0, v0 = (a.astype(np.float64) for a in (p, m, v))
        g64 = g.astype(np.float64)
        mt.adamw_host(p, m, v, g, t, cfg.lr, cfg.beta1, cfg.beta2, cfg.adam_eps, cfg.weight_decay, bf16_out=bf,
                      threads=4)
        P, Mo, Vo = O.adamw(p0, g64, m0, v0, t, cfg)
        assert np.all(np.abs(m - Mo) <= 4 * u * (0.9 * np.abs(m0) + 0.1 * np.abs(g64)) + 1e-45)
        assert np.all(np.abs(v - Vo) <= 4 * u * (0.999 * v0 + 0.001 * g64 * g64) + 1e-45)
        step = cfg.lr * (Mo / (1 - 0.9 ** t)) / (np.sqrt(Vo / (1 - 0.999 ** t)) + cfg.adam_eps)
        assert np.all(np.abs(p - P) <= 8 * u * (np.abs(p0) + np.abs(step)) + 1e-45)
        # the bf16 image is exactly the rounding of the updated fp32 value
        img = (bf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        np.testing.assert_array_equal(img, O.bf16(p))


def test_host_adamw_with_bf16_gradients():
    """The bf16-gradient form widens each gradient exactly and then takes the
    same update: it equals the fp32 form given the widened gradient, bit for
    bit, and writes the widened gradient out."""
    rng = np.random.default_rng(6)
    n = 70_001
    g32 = (rng.standard_normal(n) * 10.0 ** rng.integers(-8, -1, n)).astype(np.float32)
    g16 = (O.bf16(g32).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wide = (g16.astype(np.uint32) << 16).view(np.float32)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    state = [p, np.zeros(n, np.float32), np.zeros(n, np.float32)]
    ref = [a.copy() for a in state]
    out = np.full(n, np.nan, np.float32)
    bf_a, bf_b = np.empty(n, np.uint16), np.empty(n, np.uint16)
    for t in (1, 2):
        mt.adamw_host_g16(*state, g16, t, 1e-3, 0.9, 0.999, 1e-8, 0.01, g32_out=out, bf16_out=bf_a, threads=3)
        mt.adamw_host(*ref, wide.copy(), t, 1e-3, 0.9, 0.999, 1e-8, 0.01, bf16_out=bf_b, threads=3)
        for a, b in zip(state, ref):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(bf_a, bf_b)
        np.testing.assert_array_equal(out, wide)


def test_host_adamw_rejects_bad_arguments():
    a = np.zeros(4, np.float32)
    with pytest.raises(mt.MTError):
        mt.adamw_host(a, a.copy(), a.copy(), a.copy(), 0, 1e-3, 0.9, 0.999, 1e-8, 0.01)


def test_rope_table_matches_oracle():
    for T, hd in ((33, 16), (4096, 128)):
        c, s = mt.rope_table(T, hd, 10000.0)
        oc, os_ = O.rope_tables(T, hd, 10000.0)
        np.testing.assert_allclose(c, oc, rtol=0, atol=6e-8)
        np.testing.assert_allclose(s, os_, rtol=0, atol=6e-8)
    # far positions: the table is built in double, so the angle stays exact
    c, s = mt.rope_table(524288, 2, 10000.0)
    t = 524287
    assert abs(c[t, 0] - math.cos(t)) < 1e-7 and abs(s[t, 0] - math.sin(t)) < 1e-7


def test_gemm_ws_rejects_bad_workspace():
    # host-side argument checks run before any device call (addresses only)
    L = mt.lib()
    good, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    base = [mt.MT_BF16, mt.MT_GEMM_NT, good, 64, good, 64, good, 64, None, 0, 64, 64, 64]
    assert L.mt_op_gemm_ws(*base, odd, 1 << 20, None) == mt.MT_EINVAL
    assert L.mt_op_gemm_ws(*base, None, 1 << 20, None) == mt.MT_EINVAL
    assert L.mt_op_gemm_ws(*base, good, -1, None) == mt.MT_EINVAL
    assert mt.gemm_ws_bytes() >= 16 * 15 * 256 * 256 * 4


def test_launch_limits_refused_on_the_host():
    """Shapes past the kernels' 32-bit limits are refused before any device
    call: 2^24 token rows for the one-block-per-row kernels, 2^24 elements
    for a row of the packed projection (the attention tiles' copy offsets),
    2^32 work-items per grid dimension for attention."""
    L = mt.lib()
    p = ctypes.c_void_p(4096)
    # one past the largest token count
    c = mt.make_config(2, 64, 4, 4, 16, 172, 256, 1, 1 << 24)
    h = ctypes.c_void_p()
    assert L.mt_create(ctypes.byref(c), None, None, ctypes.byref(h)) == mt.MT_EINVAL and not h.value
    assert b"2^24" in L.mt_last_error(None)
    c = mt.make_config(2, 64, 131072, 1, 128, 172, 256, 1, 32)
    assert L.mt_create(ctypes.byref(c), None, None, ctypes.byref(h)) == mt.MT_EINVAL and not h.value
    assert L.mt_op_xent(mt.MT_BF16, p, p, p, p, 1 << 24, 1000, 1.0, None) == mt.MT_EINVAL
    assert L.mt_op_rope_fwd(mt.MT_BF16, p, p, p, p, 1, 1 << 24, 4, 4, 128, None) == mt.MT_EINVAL
    assert L.mt_op_rope_fwd(mt.MT_BF16, p, p, p, p, 2, 1 << 23, 4, 4, 128, None) == mt.MT_EINVAL
    # packed projection rows of (H + 2 Hkv) hd >= 2^24 elements
    assert L.mt_op_attn_fwd(mt.MT_BF16, p, p, p, p, 1, 64, 65535, 65535, 128, None) == mt.MT_EINVAL
    # (T / 64) * H workgroups of 256 threads past 2^32
    assert L.mt_op_attn_fwd(mt.MT_BF16, p, p, p, p, 1, (1 << 31) - 1, 64, 8, 128, None) == mt.MT_EINVAL
    assert L.mt_op_attn_bwd_rope(mt.MT_BF16, p, p, p, p, p, p, p, p, 1, 64, 65535, 65535, 128, None) \
        == mt.MT_EINVAL


def test_rmsnorm_bwd_rejects_misaligned_operands():
    # host-side argument checks run before any device call (addresses only)
    L = mt.lib()
    good, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    args = [good] * 5 + [1, good, good, 8, 64, None]
    for i in (1, 7):   # w, ws
        a = list(args)
        a[i] = odd
        assert L.mt_op_rmsnorm_bwd(*a) == mt.MT_EINVAL
    for i in (0, 3, 4):   # x, dy, dx
        a = list(args)
        a[i] = odd
        assert L.mt_op_rmsnorm_bwd(*a) == mt.MT_EINVAL
    assert mt.rmsnorm_bwd_ws_floats(4096, 5120) == 1024 * 5120


def test_device_plan_without_a_device():
    """The device memory plan of the 14B-shaped workload, computed on the
    host: the fixed part (layer and gradient buffers, activation workspace)
    and one checkpoint slot of 4096 x 5120 fp32; micro-batches shrink the
    fixed part and leave the slot (the whole batch's residuals) alone."""
    w = mt.WORKLOADS["14b"]
    def plan(batch, mb):
        c = mt.make_config(w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_dim, w.vocab,
                           batch, w.seq, dtype=mt.MT_BF16, micro_batches=mb)
        return mt.device_plan(c)
    p1, p4, p4m = plan(1, 0), plan(4, 0), plan(4, 4)
    assert p1["ckpt_slot"] == 4096 * 5120 * 4
    assert p4["ckpt_slot"] == 4 * p1["ckpt_slot"] == p4m["ckpt_slot"]
    # two bf16 layer buffers (the head, 1.56 GB, is the largest unit) and two
    # fp32 gradient buffers (3.1 GB) at least
    assert p1["fixed"] > 2 * 1.5e9 + 2 * 3.1e9
    assert p4m["fixed"] < p4["fixed"]
    assert p4m["fixed"] - p1["fixed"] < 0.1 * p1["fixed"]   # only the residual gradient and the losses grow
