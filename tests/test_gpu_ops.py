"""Each kernel of the step, called through the C-ABI (mt_op_*), against the
oracle's operation on the same seeded inputs.

Small shapes span several tiles and a ragged tail; the full 14B per-layer
shapes are checked on sampled outputs that the oracle computes one by one.
Tolerances: fp32 results within a few fp32 ulps of the sum of absolute terms;
bf16-mode results within 2e-2 * (|ref| + rms(ref)) of the bf16-emulating
oracle (exact bf16 rounding outcomes are not pinned)."""
import math

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from host_memory_streamed_amd import mt  # noqa: E402

DEV = "cuda"
RNG = np.random.default_rng(42)


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def sync():
    torch.cuda.synchronize()


def bf16_close(gpu, ref, tol=2e-2, floor=0.0):
    scale = np.abs(ref) + np.sqrt(np.mean(ref ** 2)) + floor + 1e-30
    bad = np.abs(gpu - ref) > tol * scale
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside bf16 tolerance; max {np.max(np.abs(gpu - ref) / scale)}"


def fp32_close(gpu, ref, absterm, ulps=64):
    bound = ulps * 2.0 ** -24 * absterm + 1e-30
    bad = np.abs(gpu - ref) > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside fp32 bound; worst ratio {np.max(np.abs(gpu - ref) / bound)}"


# -------------------------------------------------------------------- GEMM ---

def _gemm_case(dtype, layout, M, N, K, residual=False, sample=None, variant=0, ws=None, alias=False):
    # logical operands: X [M, K], Y [K, N]; stored per layout
    X = RNG.standard_normal((M, K)).astype(np.float32)
    Y = RNG.standard_normal((K, N)).astype(np.float32)
    if dtype == mt.MT_BF16:
        X, Y = O.bf16(X).astype(np.float32), O.bf16(Y).astype(np.float32)
    tdt = torch.bfloat16 if dtype == mt.MT_BF16 else torch.float32
    if layout == mt.MT_GEMM_NT:
        A, B, lda, ldb = dev(X, tdt), dev(Y.T, tdt), K, K
    elif layout == mt.MT_GEMM_NN:
        A, B, lda, ldb = dev(X, tdt), dev(Y, tdt), K, N
    else:
        A, B, lda, ldb = dev(X.T, tdt), dev(Y, tdt), M, N
    R = RNG.standard_normal((M, N)).astype(np.float32) if residual else None
    C = torch.full((M, N), float("nan"), device=DEV)
    Rd = dev(R) if residual else None
    if alias:   # C = C + A B: the residual is the output itself
        C.copy_(Rd)
        Rd = C
    if ws is None:
        mt.gemm(dtype, layout, A, lda, B, ldb, C, N, M, N, K, R=Rd, ldr=N, variant=variant)
    else:
        mt.gemm_ws(dtype, layout, A, lda, B, ldb, C, N, M, N, K, ws, ws.numel() * 4, R=Rd, ldr=N)
    got = host(C)
    if ws is not None and not alias:
        # fixed-order sums: a second call gives the same bits
        C2 = torch.full((M, N), float("nan"), device=DEV)
        mt.gemm_ws(dtype, layout, A, lda, B, ldb, C2, N, M, N, K, ws, ws.numel() * 4, R=Rd, ldr=N)
        np.testing.assert_array_equal(host(C2), got)
    X64, Y64 = X.astype(np.float64), Y.astype(np.float64)
    if sample is None:
        ref = X64 @ Y64 + (R if residual else 0)
        absterm = np.abs(X64) @ np.abs(Y64) + (np.abs(R) if residual else 0)
        fp32_close(got, ref, absterm)
    else:
        ii = RNG.integers(0, M, sample)
        jj = RNG.integers(0, N, sample)
        ref = np.einsum("sk,ks->s", X64[ii], Y64[:, jj]) + (R[ii, jj] if residual else 0)
        absterm = np.einsum("sk,ks->s", np.abs(X64[ii]), np.abs(Y64[:, jj])) + (np.abs(R[ii, jj]) if residual else 0)
        fp32_close(got[ii, jj], ref, absterm)


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("layout", [mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN])
@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (256, 384, 96), (200, 72, 40), (1, 3, 5), (300, 172, 64),
                                   (64, 172, 300)])
def test_gemm_small_and_ragged(dtype, layout, M, N, K):
    _gemm_case(dtype, layout, M, N, K, residual=(M % 2 == 0))


@pytest.mark.parametrize("variant", [1, 2])
@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("layout", [mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN])
@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (512, 768, 192), (300, 520, 72), (1, 3, 5), (260, 256, 1000)])
def test_gemm_tile_variants(variant, dtype, layout, M, N, K):
    _gemm_case(dtype, layout, M, N, K, residual=(K % 2 == 0), variant=variant)


@pytest.mark.parametrize("layout,M,N,K", [(mt.MT_GEMM_NT, 4096, 7168, 5120), (mt.MT_GEMM_NN, 4096, 5120, 13824),
                                          (mt.MT_GEMM_TN, 27648, 5120, 4096)])
def test_gemm_full_14b_shapes_sampled(layout, M, N, K):
    _gemm_case(mt.MT_BF16, layout, M, N, K, sample=512)


@pytest.fixture(scope="module")
def gemm_ws_buf():
    return torch.empty(mt.gemm_ws_bytes() // 4, dtype=torch.float32, device=DEV)


# With a workspace, a grid of at most half a wave of 256x256 tiles (16 here)
# and the tiles of a part-filled last wave (64 of 320) are split along K; the
# ragged case puts a K tail in the last block of each split tile.
@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("layout", [mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN])
@pytest.mark.parametrize("M,N,K", [(1024, 1024, 4096), (1000, 904, 3000)])
def test_gemm_split_k(gemm_ws_buf, dtype, layout, M, N, K):
    _gemm_case(dtype, layout, M, N, K, residual=True, ws=gemm_ws_buf)


@pytest.mark.parametrize("layout", [mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN])
def test_gemm_split_k_accumulates_into_output(gemm_ws_buf, layout):
    _gemm_case(mt.MT_BF16, layout, 1000, 904, 3000, residual=True, ws=gemm_ws_buf, alias=True)


@pytest.mark.parametrize("layout,M,N,K", [(mt.MT_GEMM_NT, 4096, 5120, 5120), (mt.MT_GEMM_NN, 4096, 5120, 13824),
                                          (mt.MT_GEMM_TN, 5120, 5120, 4096), (mt.MT_GEMM_TN, 2048, 2048, 16384)])
def test_gemm_split_k_full_shapes_sampled(gemm_ws_buf, layout, M, N, K):
    _gemm_case(mt.MT_BF16, layout, M, N, K, residual=True, sample=4096, ws=gemm_ws_buf)


def test_gemm_k_zero_gives_residual():
    R = dev(RNG.standard_normal((5, 7)))
    C = torch.zeros(5, 7, device=DEV)
    A = torch.zeros(1, device=DEV)
    mt.gemm(mt.MT_FP32, mt.MT_GEMM_NT, A, 1, A, 1, C, 7, 5, 7, 0, R=R, ldr=7)
    np.testing.assert_array_equal(host(C), host(R))


def test_gemm_rejects_bad_leading_dimension():
    A = torch.zeros(64, device=DEV)
    with pytest.raises(mt.MTError):
        mt.gemm(mt.MT_FP32, mt.MT_GEMM_NT, A, 4, A, 8, A, 8, 8, 8, 8)


# ----------------------------------------------------------------- RMSNorm ---

@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("rows,d", [(37, 64), (300, 2048), (5, 5120)])
def test_rmsnorm(dtype, rows, d):
    x = RNG.standard_normal((rows, d)).astype(np.float32) * 3
    w = RNG.standard_normal(d).astype(np.float32)
    dy = RNG.standard_normal((rows, d)).astype(np.float32)
    acc0 = RNG.standard_normal((rows, d)).astype(np.float32)
    tdt = torch.bfloat16 if dtype else torch.float32
    xd, wd = dev(x), dev(w)
    y = torch.empty(rows, d, device=DEV, dtype=tdt)
    rstd = torch.empty(rows, device=DEV)
    mt.rmsnorm_fwd(dtype, xd, wd, y, rstd, rows, d, 1e-5)
    yref, rref = O.rmsnorm_fwd(x.astype(np.float64), w.astype(np.float64), 1e-5)
    np.testing.assert_allclose(host(rstd), rref, rtol=2e-6)
    if dtype:
        assert np.all(np.abs(host(y) - yref) <= 2.0 ** -8 * np.abs(yref) + 1e-30)
    else:
        fp32_close(host(y), yref, np.abs(yref), ulps=8)
    # backward (accumulating into an existing gradient)
    dx = dev(acc0)
    dw = torch.empty(d, device=DEV)
    ws = torch.empty(mt.rmsnorm_bwd_ws_floats(rows, d), device=DEV)
    mt.rmsnorm_bwd(xd, wd, rstd, dev(dy), dx, 1, dw, ws, rows, d)
    dxr, dwr = O.rmsnorm_bwd(x.astype(np.float64), w.astype(np.float64), host(rstd), dy.astype(np.float64))
    gw = np.abs(dy * w)
    np.testing.assert_allclose(host(dx), dxr + acc0, rtol=1e-4, atol=1e-5 * np.sqrt(np.mean(dxr ** 2)))
    fp32_close(host(dw), dwr, np.sum(np.abs(dy * x) * host(rstd)[:, None], axis=0), ulps=512)
    del gw


def test_rmsnorm_bwd_14b_rows_several_per_block():
    """The 14B-shaped step's RMSNorm backward: 4096 rows of d 5120 (more than
    1024 rows, the path that gives each workgroup several rows), dx
    accumulated into an existing gradient and dw summed over all rows."""
    rows, d = 4096, 5120
    x = RNG.standard_normal((rows, d)).astype(np.float32)
    w = (1.0 + 0.1 * RNG.standard_normal(d)).astype(np.float32)
    dy = RNG.standard_normal((rows, d)).astype(np.float32)
    acc0 = RNG.standard_normal((rows, d)).astype(np.float32)
    xd, wd = dev(x), dev(w)
    y = torch.empty(rows, d, device=DEV, dtype=torch.bfloat16)
    rstd = torch.empty(rows, device=DEV)
    mt.rmsnorm_fwd(mt.MT_BF16, xd, wd, y, rstd, rows, d, 1e-5)
    dx = dev(acc0)
    dw = torch.empty(d, device=DEV)
    ws = torch.empty(mt.rmsnorm_bwd_ws_floats(rows, d), device=DEV)
    mt.rmsnorm_bwd(xd, wd, rstd, dev(dy), dx, 1, dw, ws, rows, d)
    x64, w64, dy64 = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    _, r = O.rmsnorm_fwd(x64, w64, 1e-5)
    np.testing.assert_allclose(host(rstd), r, rtol=2e-6)
    dxr, dwr = O.rmsnorm_bwd(x64, w64, host(rstd), dy64)
    np.testing.assert_allclose(host(dx), dxr + acc0, rtol=1e-4, atol=1e-5 * np.sqrt(np.mean(dxr ** 2)))
    fp32_close(host(dw), dwr, np.sum(np.abs(dy64 * x64) * host(rstd)[:, None], axis=0), ulps=512)


# -------------------------------------------------------------------- RoPE ---

@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("B,T,H,Hkv,hd", [(2, 33, 4, 2, 16), (1, 300, 8, 2, 128)])
def test_rope(dtype, B, T, H, Hkv, hd):
    W = (H + 2 * Hkv) * hd
    x = RNG.standard_normal((B * T, W)).astype(np.float32)
    c, s = mt.rope_table(T, hd, 10000.0)
    tdt = torch.bfloat16 if dtype else torch.float32
    out = torch.empty(B * T, W, device=DEV, dtype=tdt)
    cos, sin = O.rope_tables(T, hd, 10000.0)
    for bwd in (0, 1):
        mt.rope(dtype, bwd, dev(x), out, dev(c), dev(s), B, T, H, Hkv, hd)
        xr = x.astype(np.float64).reshape(B, T, H + 2 * Hkv, hd)
        f = O.rope_bwd if bwd else O.rope_fwd
        ref = np.concatenate([f(xr[:, :, :H + Hkv], cos, sin), xr[:, :, H + Hkv:]], axis=2).reshape(B * T, W)
        got = host(out)
        if dtype:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
        else:
            np.testing.assert_allclose(got, ref, rtol=0, atol=3e-6 * np.max(np.abs(ref)))


# --------------------------------------------------------------- attention ---

def _attn_inputs(B, T, H, Hkv, hd, dtype, scale=1.0):
    qkv = (RNG.standard_normal((B * T, (H + 2 * Hkv) * hd)) * scale).astype(np.float32)
    if dtype:
        qkv = O.bf16(qkv).astype(np.float32)
    return qkv


def _split(qkv, B, T, H, Hkv, hd):
    a = qkv.astype(np.float64).reshape(B, T, H + 2 * Hkv, hd)
    return a[:, :, :H], a[:, :, H:H + Hkv], a[:, :, H + Hkv:]


@pytest.mark.parametrize("dtype,hd", [(mt.MT_FP32, 16), (mt.MT_FP32, 32), (mt.MT_FP32, 64), (mt.MT_FP32, 128),
                                      (mt.MT_BF16, 64), (mt.MT_BF16, 128)])
@pytest.mark.parametrize("B,T,H,Hkv", [(2, 100, 4, 2), (1, 130, 4, 4), (1, 1, 2, 1), (1, 257, 8, 1)])
def test_attention_fwd_bwd(dtype, hd, B, T, H, Hkv):
    tdt = torch.bfloat16 if dtype else torch.float32
    qkv = _attn_inputs(B, T, H, Hkv, hd, dtype)
    q, k, v = _split(qkv, B, T, H, Hkv, hd)
    prec = O.decoder._Prec("bf16" if dtype else "fp32")
    oref, lref = O.attention_fwd(q, k, v, prec)
    M = B * T
    qd = dev(qkv, tdt)
    o = torch.full((M, H * hd), float("nan"), device=DEV)
    oc = torch.empty(M, H * hd, device=DEV, dtype=tdt) if dtype else None
    lse = torch.empty(B, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, oc, lse, B, T, H, Hkv, hd)
    got = host(o).reshape(B, T, H, hd)
    np.testing.assert_allclose(host(lse), lref, rtol=1e-5, atol=1e-5)
    if dtype:
        # against the plain reading (the normalised P rounded once): every
        # element within 2e-2 (|ref| + rms(ref)), and 2e-2 normwise
        bf16_close(got, oref)
        assert np.linalg.norm(got - oref) <= 2e-2 * np.linalg.norm(oref)
        assert np.all(np.abs(host(oc).reshape(got.shape) - got) <= 2.0 ** -8 * np.abs(got) + 1e-30)
    else:
        np.testing.assert_allclose(got, oref, rtol=1e-4, atol=1e-5)
    # backward, both sides from the same forward output o and lse
    do = RNG.standard_normal((B, T, H, hd))
    dqr, dkr, dvr = O.attention_bwd(q, k, v, got, host(lse), do, prec)
    dqkv = torch.full((M, (H + 2 * Hkv) * hd), float("nan"), device=DEV)
    ws = torch.empty(mt.attn_bwd_ws_bytes(dtype, B, T, H, hd), device=DEV, dtype=torch.uint8)
    mt.attn_bwd(dtype, qd, o, dev(do.reshape(M, H * hd)), lse, dqkv, ws, B, T, H, Hkv, hd)
    dq, dk, dv = _split(host(dqkv).astype(np.float32), B, T, H, Hkv, hd)
    # magnitude of the terms each gradient sums (dS = P (dP - D) cancels exactly at T = 1)
    rms = lambda a: np.sqrt(np.mean(np.square(a)))
    term_qk = rms(do) * rms(v) * rms(k) * math.sqrt(hd)
    for g, r, term in ((dq, dqr, term_qk), (dk, dkr, term_qk), (dv, dvr, rms(do))):
        if dtype:
            bf16_close(g, r, floor=1e-2 * term)
        else:
            np.testing.assert_allclose(g, r, rtol=1e-4, atol=1e-4 * rms(r) + 1e-5 * term)


@pytest.mark.parametrize("B,T,H,Hkv", [(1, 4096, 40, 8)])
def test_attention_full_14b_shape_sampled_rows(B, T, H, Hkv):
    hd, dtype = 128, mt.MT_BF16
    qkv = _attn_inputs(B, T, H, Hkv, hd, dtype)
    q, k, v = _split(qkv, B, T, H, Hkv, hd)
    M = B * T
    qd = dev(qkv, torch.bfloat16)
    o = torch.empty(M, H * hd, device=DEV)
    lse = torch.empty(B, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, None, lse, B, T, H, Hkv, hd)
    got, gl = host(o).reshape(B, T, H, hd), host(lse)
    for _ in range(48):
        h, t = int(RNG.integers(H)), int(RNG.integers(T))
        s = q[0, t, h] @ k[0, :t + 1, h // (H // Hkv)].T / math.sqrt(hd)
        mx = s.max()
        p = np.exp(s - mx)
        ref = (O.bf16(p / p.sum()) @ v[0, :t + 1, h // (H // Hkv)])
        assert abs(gl[0, h, t] - (mx + math.log(p.sum()))) < 1e-4
        bf16_close(got[0, t, h], ref)


@pytest.mark.parametrize("dtype,hd", [(mt.MT_FP32, 16), (mt.MT_FP32, 32), (mt.MT_FP32, 128), (mt.MT_BF16, 64),
                                      (mt.MT_BF16, 128)])
@pytest.mark.parametrize("B,T,H,Hkv", [(2, 100, 4, 2), (1, 257, 8, 1)])
def test_attention_bwd_with_rope(dtype, hd, B, T, H, Hkv):
    """The fused backward (attention, then the rotation's backward, written in
    the compute dtype) against the oracle's attention backward followed by
    its RoPE backward, and against the two separate GPU passes."""
    tdt = torch.bfloat16 if dtype else torch.float32
    qkv = _attn_inputs(B, T, H, Hkv, hd, dtype)
    q, k, v = _split(qkv, B, T, H, Hkv, hd)
    prec = O.decoder._Prec("bf16" if dtype else "fp32")
    M = B * T
    qd = dev(qkv, tdt)
    o = torch.empty(M, H * hd, device=DEV)
    oc = torch.empty(M, H * hd, device=DEV, dtype=tdt) if dtype else None
    lse = torch.empty(B, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, oc, lse, B, T, H, Hkv, hd)
    do = RNG.standard_normal((B, T, H, hd))
    dod = dev(do.reshape(M, H * hd))
    c32, s32 = mt.rope_table(T, hd, 10000.0)
    cd, sd = dev(c32), dev(s32)
    ws = torch.empty(mt.attn_bwd_ws_bytes(dtype, B, T, H, hd), device=DEV, dtype=torch.uint8)
    W = (H + 2 * Hkv) * hd
    fused = torch.full((M, W), float("nan"), device=DEV, dtype=tdt)
    mt.attn_bwd_rope(dtype, qd, o, dod, lse, cd, sd, fused, ws, B, T, H, Hkv, hd)
    # two passes: fp32 gradients of the rotated operands, then the rotation's backward
    raw = torch.full((M, W), float("nan"), device=DEV)
    mt.attn_bwd(dtype, qd, o, dod, lse, raw, ws, B, T, H, Hkv, hd)
    two = torch.full((M, W), float("nan"), device=DEV, dtype=tdt)
    mt.rope(dtype, 1, raw, two, cd, sd, B, T, H, Hkv, hd)
    got, sep = host(fused), host(two)
    if dtype:
        assert np.all(np.abs(got - sep) <= 2.0 ** -7 * np.abs(sep) + 1e-30)
    else:
        np.testing.assert_allclose(got, sep, rtol=1e-6, atol=1e-7 * np.max(np.abs(sep)))
    # oracle: attention backward from the GPU's forward output, then RoPE backward
    dqr, dkr, dvr = O.attention_bwd(q, k, v, host(o).reshape(B, T, H, hd), host(lse), do, prec)
    cos, sin = O.rope_tables(T, hd, 10000.0)
    dq, dk, dv = _split(got.astype(np.float32), B, T, H, Hkv, hd)
    rms = lambda a: np.sqrt(np.mean(np.square(a)))
    term_qk = rms(do) * rms(v) * rms(k) * math.sqrt(hd)
    for g, r, term in ((dq, O.rope_bwd(dqr, cos, sin), term_qk), (dk, O.rope_bwd(dkr, cos, sin), term_qk),
                       (dv, dvr, rms(do))):
        if dtype:
            bf16_close(g, r, floor=1e-2 * term)
        else:
            np.testing.assert_allclose(g, r, rtol=1e-4, atol=1e-4 * rms(r) + 1e-5 * term)


def test_attention_bwd_14b_shape_sampled():
    """Backward at the 14B-shaped layer's attention (1 x 4096 tokens, 40
    query / 8 kv heads, hd 128, bf16): dq of sampled query rows of every
    head, and dk/dv of two interior 64-key tiles of two kv heads (each summed
    over its 5 query heads), against float64 computed row by row from the
    same operands (exact softmax, the bf16 dO the kernel reads)."""
    B, T, H, Hkv, hd, dtype = 1, 4096, 40, 8, 128, mt.MT_BF16
    rng = np.random.default_rng(4096)
    W = (H + 2 * Hkv) * hd
    qkv = O.bf16(rng.standard_normal((T, W), dtype=np.float32)).astype(np.float32)
    do = rng.standard_normal((T, H * hd), dtype=np.float32)
    qd = dev(qkv, torch.bfloat16)
    o = torch.empty(T, H * hd, device=DEV)
    lse = torch.empty(1, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, None, lse, B, T, H, Hkv, hd)
    dqkv = torch.full((T, W), float("nan"), device=DEV)
    ws = torch.empty(mt.attn_bwd_ws_bytes(dtype, B, T, H, hd), device=DEV, dtype=torch.uint8)
    mt.attn_bwd(dtype, qd, o, dev(do), lse, dqkv, ws, B, T, H, Hkv, hd)
    og = host(o).reshape(T, H, hd)
    g = host(dqkv).reshape(T, H + 2 * Hkv, hd)
    assert np.all(np.isfinite(g))
    Q = qkv[:, :H * hd].reshape(T, H, hd).astype(np.float64)
    K = qkv[:, H * hd:(H + Hkv) * hd].reshape(T, Hkv, hd).astype(np.float64)
    V = qkv[:, (H + Hkv) * hd:].reshape(T, Hkv, hd).astype(np.float64)
    dO = do.reshape(T, H, hd).astype(np.float64)
    dOb = O.bf16(dO)
    sc = 1.0 / math.sqrt(hd)
    grp = H // Hkv
    for t in [0, 63, 64, 127, 128, 2047, 2048, 3001, T - 1] + [int(x) for x in rng.integers(0, T, 3)]:
        for h in range(H):
            kv = h // grp
            s = K[:t + 1, kv] @ Q[t, h] * sc
            P = np.exp(s - s.max())
            P /= P.sum()
            dS = P * (V[:t + 1, kv] @ dOb[t, h] - dO[t, h] @ og[t, h])
            ref = sc * (dS @ K[:t + 1, kv])
            bf16_close(g[t, h], ref, floor=1e-2 * np.sqrt(np.mean(ref ** 2)))
    # interior key tiles: queries q >= k0 reach keys [k0, k0 + 64)
    for kv, k0 in ((1, 1024), (6, 2560)):
        dk = np.zeros((64, hd))
        dv = np.zeros((64, hd))
        for h in range(kv * grp, (kv + 1) * grp):
            S = Q[k0:, h] @ K[:, kv].T * sc                          # [T - k0, T]
            S[(np.arange(T - k0)[:, None] + k0) < np.arange(T)[None, :]] = -np.inf
            Pf = np.exp(S - S.max(axis=1, keepdims=True))
            Pf /= Pf.sum(axis=1, keepdims=True)
            Pt = Pf[:, k0:k0 + 64]
            D = np.sum(dO[k0:, h] * og[k0:, h], axis=1)
            dS = Pt * (dOb[k0:, h] @ V[k0:k0 + 64, kv].T - D[:, None])
            dk += sc * dS.T @ Q[k0:, h]
            dv += Pt.T @ dOb[k0:, h]
        bf16_close(g[k0:k0 + 64, H + kv], dk, floor=1e-2 * np.sqrt(np.mean(dk ** 2)))
        bf16_close(g[k0:k0 + 64, H + Hkv + kv], dv, floor=1e-2 * np.sqrt(np.mean(dv ** 2)))


@pytest.mark.parametrize("T,H,Hkv", [(524288, 2, 2), (1048576, 2, 2), (8192, 4, 2), (8320, 4, 2)])
def test_attention_long_sequence_sampled(T, H, Hkv):
    """Causal attention over one sequence of 524288 tokens (the long-context
    workload's length) and of 1048576 (twice it); 2 heads of dim 128 keep
    the check to seconds: forward rows and the dq rows of sampled queries,
    and dk/dv of the last 64-key tile, against float64 computed row by row;
    plus, over the whole length, sum_t dv[t] = sum_q dO[q] (each probability
    row sums to one). With grouped kv heads, on both sides of the length up
    to which the dK/dV pass takes one query head per work item (8192 tokens:
    per-head partials and their sum; 8320: the whole group per item)."""
    hd, dtype = 128, mt.MT_BF16
    rng = np.random.default_rng(T)
    W = (H + 2 * Hkv) * hd
    qkv = O.bf16(rng.standard_normal((T, W), dtype=np.float32)).astype(np.float32)
    do = rng.standard_normal((T, H * hd), dtype=np.float32)
    qd = dev(qkv, torch.bfloat16)
    o = torch.empty(T, H * hd, device=DEV)
    lse = torch.empty(1, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, None, lse, 1, T, H, Hkv, hd)
    dqkv = torch.empty(T, W, device=DEV)
    ws = torch.empty(mt.attn_bwd_ws_bytes(dtype, 1, T, H, hd), device=DEV, dtype=torch.uint8)
    mt.attn_bwd(dtype, qd, o, dev(do), lse, dqkv, ws, 1, T, H, Hkv, hd)
    og, lg = host(o).reshape(T, H, hd), host(lse)[0]
    g = host(dqkv).reshape(T, H + 2 * Hkv, hd)
    del qd, dqkv, ws
    Q = qkv[:, :H * hd].reshape(T, H, hd).astype(np.float64)
    K = qkv[:, H * hd:(H + Hkv) * hd].reshape(T, Hkv, hd).astype(np.float64)
    V = qkv[:, (H + Hkv) * hd:].reshape(T, Hkv, hd).astype(np.float64)
    dO = do.reshape(T, H, hd).astype(np.float64)
    dOb = O.bf16(dO)
    sc = 1.0 / math.sqrt(hd)
    # sampled query rows: o, lse and dq
    rows = [0, 1, 63, 64, 4095, T // 2 + 17, T - 65, T - 1] + [int(x) for x in rng.integers(0, T, 4)]
    for t in rows:
        for h in range(H):
            kv = h // (H // Hkv)
            s = K[:t + 1, kv] @ Q[t, h] * sc
            m = s.max()
            p = np.exp(s - m)
            P = p / p.sum()
            assert abs(lg[h, t] - (m + math.log(p.sum()))) < 1e-4, (t, h)
            bf16_close(og[t, h], P @ V[:t + 1, kv])
            dP = V[:t + 1, kv] @ dOb[t, h]
            dS = P * (dP - dO[t, h] @ og[t, h])
            ref = sc * (dS @ K[:t + 1, kv])
            bf16_close(g[t, h], ref, floor=1e-2 * np.sqrt(np.mean(ref ** 2)))
    # dk, dv of the last 64 keys: only the last 64 queries reach them
    q0 = T - 64
    for kv in range(Hkv):
        dk = np.zeros((64, hd))
        dv = np.zeros((64, hd))
        for h in range(kv * (H // Hkv), (kv + 1) * (H // Hkv)):
            S = Q[q0:, h] @ K[:, kv].T * sc                       # [64, T]
            S[np.arange(64)[:, None] < (np.arange(T)[None, :] - q0)] = -np.inf
            m = S.max(axis=1, keepdims=True)
            Pf = np.exp(S - m)
            Pf /= Pf.sum(axis=1, keepdims=True)
            P = Pf[:, q0:]                                          # [64 q, 64 k]
            D = np.sum(dO[q0:, h] * og[q0:, h], axis=1)
            dS = P * (dOb[q0:, h] @ V[q0:, kv].T - D[:, None])
            dk += sc * dS.T @ Q[q0:, h]
            dv += P.T @ dOb[q0:, h]
        bf16_close(g[q0:, H + kv], dk, floor=1e-2 * np.sqrt(np.mean(dk ** 2)))
        bf16_close(g[q0:, H + Hkv + kv], dv, floor=1e-2 * np.sqrt(np.mean(dv ** 2)))
    # whole length: sum over keys of dv equals the sum of the (rounded) dO over the group's queries
    for kv in range(Hkv):
        grp = slice(kv * (H // Hkv), (kv + 1) * (H // Hkv))
        lhs = g[:, H + Hkv + kv].sum(axis=0)
        rhs = dOb[:, grp].sum(axis=(0, 1))
        scale = np.sqrt(np.sum(dOb[:, grp] ** 2) / hd)
        assert np.max(np.abs(lhs - rhs)) <= 2e-3 * scale, np.max(np.abs(lhs - rhs)) / scale


# ------------------------------------------------------- SwiGLU / CE / cast ---

# F % 4 == 0: four per thread, row-wise; F = 170: one per thread; the real FFN
# width of the 14B-shaped model
@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("M,F", [(77, 172), (33, 170), (5, 13824)])
def test_swiglu(dtype, M, F):
    gu = (RNG.standard_normal((M, 2 * F)) * 4).astype(np.float32)
    da = RNG.standard_normal((M, F)).astype(np.float32)
    tdt = torch.bfloat16 if dtype else torch.float32
    act = torch.empty(M, F, device=DEV, dtype=tdt)
    dgu = torch.empty(M, 2 * F, device=DEV, dtype=tdt)
    mt.swiglu_fwd(dtype, dev(gu), act, M, F)
    mt.swiglu_bwd(dtype, dev(gu), dev(da), dgu, M, F)
    g, u = gu[:, :F].astype(np.float64), gu[:, F:].astype(np.float64)
    aref = O.swiglu_fwd(g, u)
    dg, du = O.swiglu_bwd(g, u, da.astype(np.float64))
    dref = np.concatenate([dg, du], axis=1)
    rt = 2.0 ** -8 if dtype else 2e-6
    assert np.all(np.abs(host(act) - aref) <= rt * np.abs(aref) + 1e-6)
    assert np.all(np.abs(host(dgu) - dref) <= rt * np.abs(dref) + 1e-6)


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
def test_swiglu_vector_path_is_bitwise_scalar(dtype):
    # the same operands one element off 16-byte alignment take the
    # one-per-thread kernels: identical bits
    M, F = 40, 512
    gu = (RNG.standard_normal((M, 2 * F)) * 4).astype(np.float32)
    da = RNG.standard_normal((M, F)).astype(np.float32)
    tdt = torch.bfloat16 if dtype else torch.float32
    outs = []
    for off in (0, 1):
        gbuf = torch.zeros(M * 2 * F + off, device=DEV)
        gbuf[off:] = dev(gu).reshape(-1)
        dbuf = torch.zeros(M * F + off, device=DEV)
        dbuf[off:] = dev(da).reshape(-1)
        act = torch.empty(M * F + off, device=DEV, dtype=tdt)
        dgu = torch.empty(M * 2 * F + off, device=DEV, dtype=tdt)
        mt.swiglu_fwd(dtype, gbuf[off:], act[off:], M, F)
        mt.swiglu_bwd(dtype, gbuf[off:], dbuf[off:], dgu[off:], M, F)
        outs.append((host(act[off:]), host(dgu[off:])))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
@pytest.mark.parametrize("rows,V", [(9, 256), (3, 152064), (5, 32000)])
def test_cross_entropy(dtype, rows, V):
    z = (RNG.standard_normal((rows, V)) * 3).astype(np.float32)
    tgt = RNG.integers(0, V, rows).astype(np.int32)
    tdt = torch.bfloat16 if dtype else torch.float32
    zd = dev(z)
    loss = torch.empty(rows, device=DEV)
    dz = zd if not dtype else torch.empty(rows, V, device=DEV, dtype=tdt)   # fp32 in place
    mt.xent(dtype, zd, torch.from_numpy(tgt).to(DEV), loss, dz, rows, V, 1.0 / 1000)
    lref, dref = O.cross_entropy(z.astype(np.float64), tgt)
    np.testing.assert_allclose(host(loss), lref, rtol=1e-5, atol=1e-5)
    dref = dref * rows / 1000
    rt = 2.0 ** -8 if dtype else 1e-5
    assert np.all(np.abs(host(dz) - dref) <= rt * np.abs(dref) + 1e-12)


def test_cross_entropy_in_place_repeated():
    # dlogits overwrite the logits: every row's loss must still see its target logit
    rows, V = 64, 256
    for rep in range(20):
        z = (RNG.standard_normal((rows, V)) * 3).astype(np.float32)
        tgt = RNG.integers(0, V, rows).astype(np.int32)
        zd = dev(z)
        loss = torch.empty(rows, device=DEV)
        mt.xent(mt.MT_FP32, zd, torch.from_numpy(tgt).to(DEV), loss, zd, rows, V, 1.0)
        lref, dref = O.cross_entropy(z.astype(np.float64), tgt)
        np.testing.assert_allclose(host(loss), lref, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(host(zd), dref * rows, rtol=1e-5, atol=1e-7)


# 10003 elements: the scalar path; 8 * 4099: eight per thread (16-byte
# loads and stores); the same from an offset of one element: scalar again
@pytest.mark.parametrize("n,off", [(10003, 0), (8 * 4099, 0), (8 * 4099, 1)])
def test_cast_is_round_to_nearest_even(n, off):
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 3.0e38], np.float32)
    x = np.concatenate([RNG.standard_normal(n + off - ties.size).astype(np.float32), ties])
    xd = dev(x)
    y = torch.empty(n + off, device=DEV, dtype=torch.bfloat16)
    mt.cast(mt.MT_BF16, xd[off:], y[off:], n)
    np.testing.assert_array_equal(host(y[off:]), O.bf16(x[off:]))
