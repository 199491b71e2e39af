"""Pins of the CPU oracle to things other than itself: library routines it
must reduce to, closed forms, invariants and finite differences.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong kv-head mapping) fails it.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle as O
from oracle.configs import shape
from host_memory_streamed_amd import synth

RNG = np.random.default_rng(1234)


def _params(cfg, seed=0, std=0.02):
    return [synth.init_tensor(seed, i, shp, gain, std) for i, (_, shp, gain) in
            enumerate(O.tensor_table(cfg))]


def _t(x):
    return torch.tensor(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------- rounding ---

def test_bf16_matches_torch_conversion():
    x = np.concatenate([RNG.standard_normal(10000) * 10.0 ** RNG.integers(-6, 6, 10000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, 65504.0]])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16(x), ref)
    # ties go to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert O.bf16(np.float32(1.0 + 2.0 ** -8)) == 1.0
    assert O.bf16(np.float32(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6


# ----------------------------------------------------------------- RMSNorm ---

def test_rmsnorm_matches_torch_and_unit_rms():
    x = RNG.standard_normal((7, 48))
    w = RNG.standard_normal(48)
    y, r = O.rmsnorm_fwd(x, w, 1e-5)
    ref = F.rms_norm(_t(x), (48,), _t(w), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    y1, _ = O.rmsnorm_fwd(x * 50.0, np.ones(48), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 ** 2, axis=1)), 1.0, rtol=1e-12)


def test_rmsnorm_backward_matches_autograd():
    x = RNG.standard_normal((5, 32))
    w = RNG.standard_normal(32)
    dy = RNG.standard_normal((5, 32))
    _, r = O.rmsnorm_fwd(x, w, 1e-5)
    dx, dw = O.rmsnorm_bwd(x, w, r, dy)
    xt, wt = _t(x).requires_grad_(), _t(w).requires_grad_()
    F.rms_norm(xt, (32,), wt, eps=1e-5).backward(_t(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-13)


# -------------------------------------------------------------------- RoPE ---

def test_rope_frequencies_and_rotation():
    # hd = 4, base 10000: pair 0 turns by 1 rad per position, pair 1 by 0.01 rad.
    cos, sin = O.rope_tables(3, 4, 10000.0)
    x = np.zeros((1, 3, 1, 4))
    x[..., 0] = 1.0   # pair 0 = (x[0], x[2])
    x[..., 1] = 1.0   # pair 1 = (x[1], x[3])
    y = O.rope_fwd(x, cos, sin)
    for t in range(3):
        assert y[0, t, 0, 0] == pytest.approx(math.cos(1.0 * t), abs=1e-7)
        assert y[0, t, 0, 2] == pytest.approx(math.sin(1.0 * t), abs=1e-7)
        assert y[0, t, 0, 1] == pytest.approx(math.cos(0.01 * t), abs=1e-7)
        assert y[0, t, 0, 3] == pytest.approx(math.sin(0.01 * t), abs=1e-7)


def test_rope_norm_relative_position_and_adjoint():
    T, hd = 40, 16
    cos, sin = O.rope_tables(T, hd, 10000.0)
    q = RNG.standard_normal((1, T, 1, hd))
    y = O.rope_fwd(q, cos, sin)
    h = hd // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, q[..., :h] ** 2 + q[..., h:] ** 2,
                               rtol=1e-6)
    # the same q at every position and the same k: q(m).k(n) depends on m - n only
    qs = np.repeat(q[:, :1], T, axis=1)
    ks = np.repeat(RNG.standard_normal((1, 1, 1, hd)), T, axis=1)
    dots = np.einsum("d,nd->n", O.rope_fwd(qs, cos, sin)[0, 10, 0], O.rope_fwd(ks, cos, sin)[0, :, 0])
    dots2 = np.einsum("d,nd->n", O.rope_fwd(qs, cos, sin)[0, 25, 0], O.rope_fwd(ks, cos, sin)[0, :, 0])
    np.testing.assert_allclose(dots[0:11], dots2[15:26], rtol=1e-5, atol=1e-6)
    # backward is the adjoint of forward
    g = RNG.standard_normal((1, T, 1, hd))
    assert np.sum(O.rope_fwd(q, cos, sin) * g) == pytest.approx(np.sum(q * O.rope_bwd(g, cos, sin)),
                                                                rel=1e-12)


# --------------------------------------------------------------- attention ---

@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_attention_matches_torch_sdpa(H, Hkv):
    B, T, hd = 2, 9, 8
    q = RNG.standard_normal((B, T, H, hd))
    k = RNG.standard_normal((B, T, Hkv, hd))
    v = RNG.standard_normal((B, T, Hkv, hd))
    prec = O.decoder._Prec("fp32")
    o, lse = O.attention_fwd(q, k, v, prec)
    qt, kt, vt = (_t(a).permute(0, 2, 1, 3).requires_grad_() for a in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).detach().numpy(), rtol=1e-10, atol=1e-12)
    # lse of row i is logsumexp over j <= i of the scaled scores
    grp = H // Hkv
    S = np.einsum("thd,shd->hts", q[1], np.repeat(k[1], grp, axis=1)) / math.sqrt(hd)
    for i in range(T):
        np.testing.assert_allclose(lse[1, :, i], logsumexp(S[:, i, :i + 1], axis=1), rtol=1e-12)
    do = RNG.standard_normal(o.shape)
    ref.backward(_t(do).permute(0, 2, 1, 3))
    dq, dk, dv = O.attention_bwd(q, k, v, o, lse, do, prec)
    np.testing.assert_allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-9, atol=1e-11)


def test_attention_special_cases():
    prec = O.decoder._Prec("fp32")
    v = RNG.standard_normal((1, 6, 2, 4))
    # T = 1: the only key is itself, o = v
    o1, _ = O.attention_fwd(RNG.standard_normal((1, 1, 2, 4)), RNG.standard_normal((1, 1, 2, 4)),
                            v[:, :1], prec)
    np.testing.assert_allclose(o1, v[:, :1], rtol=0, atol=1e-15)
    # q = 0: uniform weights over the causal prefix, o_t = mean(v_0..v_t)
    o0, lse = O.attention_fwd(np.zeros((1, 6, 2, 4)), RNG.standard_normal((1, 6, 2, 4)), v, prec)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, 7)[None, :, None, None]
    np.testing.assert_allclose(o0, prefix_mean, rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 7)), rtol=1e-12)


# ------------------------------------------------------------- SwiGLU / CE ---

def test_swiglu_matches_torch():
    g = RNG.standard_normal((4, 10)) * 3
    u = RNG.standard_normal((4, 10))
    np.testing.assert_allclose(O.swiglu_fwd(g, u), (F.silu(_t(g)) * _t(u)).numpy(), rtol=1e-13)
    gt, ut = _t(g).requires_grad_(), _t(u).requires_grad_()
    da = RNG.standard_normal((4, 10))
    (F.silu(gt) * ut).backward(_t(da))
    dg, du = O.swiglu_bwd(g, u, da)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-12, atol=1e-14)
    # silu(0) = 0 and silu'(0) = 1/2
    assert O.swiglu_fwd(np.array(0.0), np.array(1.0)) == 0.0
    assert O.swiglu_bwd(np.array(0.0), np.array(1.0), np.array(1.0))[0] == 0.5


def test_cross_entropy_matches_torch():
    z = RNG.standard_normal((12, 37)) * 4
    tgt = RNG.integers(0, 37, 12)
    loss, dz = O.cross_entropy(z, tgt)
    np.testing.assert_allclose(loss, logsumexp(z, axis=1) - z[np.arange(12), tgt], rtol=1e-13)
    zt = _t(z).requires_grad_()
    F.cross_entropy(zt, torch.tensor(tgt)).backward()
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)


# ------------------------------------------------------------------- AdamW ---

def test_adamw_closed_form_first_two_steps():
    cfg = O.Config(1, 8, 1, 1, 8, 8, 8)
    p0 = RNG.standard_normal(1000) * 0.02
    g1 = RNG.standard_normal(1000) * 10.0 ** RNG.integers(-9, -1, 1000)
    g2 = RNG.standard_normal(1000) * 1e-3
    lr, wd, eps = cfg.lr, cfg.weight_decay, cfg.adam_eps
    p1, m1, v1 = O.adamw(p0, g1, np.zeros(1000), np.zeros(1000), 1, cfg)
    # first step: m = 0.1 g, v = 0.001 g^2, the update is g / (|g| + eps)
    np.testing.assert_allclose(m1, 0.1 * g1, rtol=1e-13)
    np.testing.assert_allclose(v1, 0.001 * g1 * g1, rtol=1e-13)
    np.testing.assert_allclose(p1, p0 * (1 - lr * wd) - lr * g1 / (np.abs(g1) + eps), rtol=1e-13)
    # second step, written out with its own bias corrections
    p2, m2, v2 = O.adamw(p1, g2, m1, v1, 2, cfg)
    mm = 0.09 * g1 + 0.1 * g2
    vv = 0.000999 * g1 ** 2 + 0.001 * g2 ** 2
    upd = (mm / 0.19) / (np.sqrt(vv / (1 - 0.999 ** 2)) + eps)
    np.testing.assert_allclose(p2, p1 * (1 - lr * wd) - lr * upd, rtol=1e-12)


def test_adamw_matches_torch_optimizer():
    cfg = O.Config(1, 8, 1, 1, 8, 8, 8)
    p = RNG.standard_normal(257) * 0.02
    pt = _t(p).requires_grad_()
    opt = torch.optim.AdamW([pt], lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.adam_eps,
                            weight_decay=cfg.weight_decay)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for t in range(1, 5):
        g = RNG.standard_normal(257) * 1e-3
        pt.grad = _t(g)
        opt.step()
        p, m, v = O.adamw(p, g, m, v, t, cfg)
    np.testing.assert_allclose(p, pt.detach().numpy(), rtol=1e-13)


# ------------------------------------------------------------- whole step ---

def _fd_check(cfg, B, T, n_coords, seed=0):
    params = _params(cfg, seed, std=0.3)   # larger weights: non-trivial attention patterns
    tokens, targets = synth.token_batch(seed, B, T, cfg.vocab)
    loss, _, grads, _ = O.gradients(params, tokens, targets, cfg)
    P = [p.astype(np.float64) for p in params]
    h = 1e-5
    rng = np.random.default_rng(7)
    worst = 0.0
    for i, (name, shp, gain) in enumerate(O.tensor_table(cfg)):
        n = int(np.prod(shp))
        if name == "tok_emb":   # only rows that occur in the batch have a gradient
            rows = np.unique(tokens)
            idx = [r * shp[1] + c for r in rng.choice(rows, n_coords) for c in [rng.integers(shp[1])]]
        else:
            idx = rng.choice(n, min(n, n_coords), replace=False)
        for j in idx:
            flat = P[i].reshape(-1)
            old = flat[j]
            flat[j] = old + h
            lp, _ = O.forward_loss(P, tokens, targets, cfg)
            flat[j] = old - h
            lm, _ = O.forward_loss(P, tokens, targets, cfg)
            flat[j] = old
            fd = (lp - lm) / (2 * h)
            g = grads[i].reshape(-1)[j]
            err = abs(fd - g) / (abs(g) + 1e-6)
            worst = max(worst, err)
            assert abs(fd - g) <= 1e-8 + 2e-5 * abs(g), (name, j, fd, g)
    return worst


def test_step_gradients_match_finite_differences_tiny():
    cfg, B, T = shape("tiny")
    _fd_check(cfg, B, T, n_coords=24)


def test_step_gradients_match_finite_differences_gqa():
    cfg = O.Config(2, 32, 4, 2, 8, 40, 50)
    _fd_check(cfg, 2, 7, n_coords=24, seed=3)


def test_zero_head_gives_log_vocab_exactly():
    cfg, B, T = shape("tiny")
    params = _params(cfg)
    params[-1] = np.zeros_like(params[-1])
    tokens, targets = synth.token_batch(0, B, T, cfg.vocab)
    loss, tl, grads, _ = O.gradients(params, tokens, targets, cfg)
    np.testing.assert_allclose(tl, math.log(cfg.vocab), rtol=0, atol=1e-14)
    # dz = (1/V - onehot)/M, so d lm_head = dz^T hf; its row sums over targets are known
    assert abs(loss - math.log(cfg.vocab)) < 1e-14


def test_initial_loss_near_log_vocab():
    # logits ~ N(0, s^2) with s = 0.02 sqrt(d) (unit-gain norms): E[loss] ~ ln V + s^2/2
    cfg, B, T = shape("tiny")
    losses = []
    for seed in range(4):
        params = _params(cfg, seed)
        tokens, targets = synth.token_batch(seed, B, T, cfg.vocab)
        losses.append(O.forward_loss(params, tokens, targets, cfg)[0])
    s2 = 0.02 ** 2 * cfg.d_model
    assert abs(np.mean(losses) - (math.log(cfg.vocab) + s2 / 2)) < 0.01


def test_causality_of_whole_model():
    cfg, B, T = shape("tiny")
    params = _params(cfg, 0, std=0.2)
    tokens, targets = synth.token_batch(0, B, T, cfg.vocab)
    _, full = O.forward_loss(params, tokens, targets, cfg)
    _, pre = O.forward_loss(params, tokens[:, :11].copy(), targets[:, :11].copy(), cfg)
    np.testing.assert_allclose(pre, full[:, :11], rtol=1e-13)
    # changing a later token leaves earlier losses untouched
    t2 = tokens.copy()
    t2[:, 20] = (t2[:, 20] + 1) % cfg.vocab
    _, alt = O.forward_loss(params, t2, targets, cfg)
    np.testing.assert_array_equal(alt[:, :20], full[:, :20])
    assert not np.allclose(alt[:, 20:], full[:, 20:])


def test_train_step_applies_adamw_to_every_tensor():
    cfg, B, T = shape("tiny")
    params = _params(cfg)
    tokens, targets = synth.token_batch(0, B, T, cfg.vocab)
    zeros = [np.zeros_like(p) for p in params]
    r = O.train_step(params, zeros, zeros, 0, tokens, targets, cfg)
    for p, g, p1, m1 in zip(params, r.grads, r.params, r.m):
        exp = p.astype(np.float64) * (1 - cfg.lr * cfg.weight_decay) - cfg.lr * g / (np.abs(g) + cfg.adam_eps)
        np.testing.assert_allclose(p1, exp, rtol=2e-7, atol=1e-9)
        np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-6, atol=1e-30)


def test_bf16_mode_stays_near_fp32():
    cfg, B, T = shape("tiny")
    params = _params(cfg, 0, std=0.1)
    tokens, targets = synth.token_batch(0, B, T, cfg.vocab)
    l32, _, g32, _ = O.gradients(params, tokens, targets, cfg, "fp32")
    l16, _, g16, _ = O.gradients(params, tokens, targets, cfg, "bf16")
    assert abs(l16 - l32) < 1e-2 * l32
    for a, b in zip(g32, g16):
        assert np.linalg.norm(a - b) <= 5e-2 * np.linalg.norm(a) + 1e-12
