"""The streamed training step through the C-ABI against the CPU oracle.

fp32 mode: loss, per-token losses, every gradient, updated parameters and
AdamW moments within rtol 1e-4 / atol 1e-5 of the oracle elementwise, and
each tensor within 1e-4 of the oracle normwise (||gpu - ref|| <= 1e-4 ||ref||,
which binds where most elements sit below the absolute tolerance).

bf16-compute mode: against the oracle's plain bf16 reading (``mode="bf16"``:
every matrix-product operand rounded where the definition forms it, the
normalised attention probabilities included), with the fixed tolerances of
``tolerances.py``: per tensor kind and depth class, a normwise bound and an
elementwise guard on each row's own scale, each at least twice the oracle's
own distance between that reading and its float64 step (measured by
``golden/bf16_distance.py``, recorded in ``golden/bf16_distance.json``).

Token order is bit-exact (per-token losses in (b, t) order), streamed equals
fully resident bitwise, and the schedule log follows the layer order."""
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle.configs import shape
from tolerances import bf16_tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from host_memory_streamed_amd import mt, synth  # noqa: E402


def release_on_failure(fn):
    """Run fn; on an assertion failure raise a fresh AssertionError (with the
    original traceback as text) once fn's frames, and the oracle arrays they
    hold, are released: a failed multi-gigabyte comparison must not keep its
    memory for the rest of the session."""
    import functools
    import traceback

    @functools.wraps(fn)
    def wrapper(*a, **kw):
        msg = None
        try:
            return fn(*a, **kw)
        except AssertionError as e:
            msg = "".join(traceback.format_exception(type(e), e, e.__traceback__))[-6000:]
        raise AssertionError(msg)
    return wrapper


def init_params(cfg, seed, std=0.02):
    return [synth.init_tensor(seed, i, shp, gain, std) for i, (_, shp, gain) in enumerate(O.tensor_table(cfg))]


def make_ctx(cfg, B, T, params, dtype=mt.MT_FP32, resident=False, flags=mt.MT_KEEP_GRADS, threads=8,
             chunk_rows=0, ckpt_host=0, buffers=None, ring_slots=0, micro_batches=0):
    if buffers is None:
        buffers = cfg.n_layers + 1 if resident else 2
    c = mt.make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                       cfg.vocab, B, T, dtype=dtype, n_layer_buffers=buffers,
                       host_threads=threads, flags=flags, rms_eps=cfg.rms_eps, rope_base=cfg.rope_base,
                       lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, adam_eps=cfg.adam_eps,
                       weight_decay=cfg.weight_decay, chunk_rows=chunk_rows, ckpt_host=ckpt_host,
                       grad_ring_slots=ring_slots, micro_batches=micro_batches)
    return mt.Context(c, params)


def check_normwise(name, got, ref, tol):
    n = np.linalg.norm(ref)
    err = np.linalg.norm(np.asarray(got, np.float64) - ref)
    assert err <= tol * n + 1e-30, f"{name}: normwise {err / (n + 1e-300):.3g} > {tol}"


def check_fp32(name, got, ref, rtol=1e-4, atol=1e-5):
    np.testing.assert_allclose(got, ref, rtol=rtol, atol=atol, err_msg=name)
    check_normwise(name, got, ref, rtol)


def check_bf16(name, got, ref, tol, spill=1e-3):
    """tol = (tau, gamma, rho): ||got - ref|| <= tau ||ref||; |got - ref| <=
    gamma rms(row of ref) for all but a fraction `spill` of the elements; and
    ||got_row - ref_row|| <= rho ||ref_row|| for every row. A row is one
    output unit (the whole vector for gains and per-token losses)."""
    tau, gamma, rho = tol
    got = np.asarray(got, np.float64)
    r2 = ref.reshape(ref.shape[0], -1) if ref.ndim > 1 else ref.reshape(1, -1)
    diff = got.reshape(r2.shape) - r2
    rn = np.sqrt(np.sum(np.square(r2), axis=1))
    dn = np.sqrt(np.sum(np.square(diff), axis=1))
    rms = (rn / np.sqrt(r2.shape[1]))[:, None]
    if os.environ.get("MT_TEST_REPORT"):
        # the measured distances against their bounds, for the record
        q = float(np.quantile(np.abs(diff) / (rms + 1e-300), 0.999))
        ok = rn > 0
        rmax = float(np.max(dn[ok] / rn[ok])) if ok.any() else 0.0
        print(f"BF16REPORT {name}: norm {np.linalg.norm(diff) / (np.linalg.norm(r2) + 1e-300):.4g}/{tau} "
              f"q999 {q:.4g}/{gamma} row {rmax:.4g}/{rho}", flush=True)
    check_normwise(name, got, ref, tau)
    n_out = int((np.abs(diff) > gamma * rms).sum())
    assert n_out <= spill * r2.size, f"{name}: {n_out} of {r2.size} elements beyond {gamma} rms(row)"
    bad = dn > rho * rn + 1e-30
    if bad.any():
        worst = int(np.argmax(dn / (rn + 1e-300)))
        raise AssertionError(f"{name}: {int(bad.sum())} rows beyond {rho} normwise; row {worst} at "
                             f"{dn[worst] / (rn[worst] + 1e-300):.3g}")


def _kind(name):
    return name.split(".")[-1]


def compare_step(ctx, res, cfg, mode, prev, tokens=None, depth="narrow", sample=None, extra=0.0):
    """Gradients against the oracle's; the update against the oracle's AdamW
    applied to the library's own gradient (fp32 rounding only); and the
    updated state against the oracle's end-to-end step, except (fp32 mode)
    where the first-moment update g/(|g|+eps) is ill-conditioned: |g| < 1e-5,
    where a gradient difference inside the gradient tolerance can move it by
    O(1) (the update of such an element is still checked given the gradient).
    bf16 mode uses the fixed tolerances of its depth class. `sample`: check
    AdamW (an elementwise map) on that many random elements per tensor
    instead of all of them. `extra`: a relative error the gradients carry
    by design (bf16 gradient transfer: 2^-8), added to rtol, tau and rho."""
    P0, M0, V0, t0 = prev
    rng = np.random.default_rng(0)
    keep = bool(ctx.cfg.flags & mt.MT_KEEP_GRADS)
    for i, (name, _, _) in enumerate(O.tensor_table(cfg)):
        kind = _kind(name)
        # without kept gradients, m and v (which the update forms from the
        # gradient) stand in for it below
        g = ctx.grads(i) if keep else None
        def tg(what):
            tau, gamma, rho = bf16_tol(depth, what + " " + kind)
            return tau + extra, gamma, rho + extra
        chk = (lambda n_, a, b, what: check_bf16(n_, a, b, tg(what))) if mode == "bf16" else \
              (lambda n_, a, b, what: check_fp32(n_, a, b, rtol=1e-4 + extra))
        rows = None
        if i == 0 and tokens is not None:
            # embedding: rows outside the batch have an exactly zero gradient;
            # the touched rows are compared on their own scale
            rows = np.unique(tokens)
            if keep:
                other = np.setdiff1d(np.arange(cfg.vocab), rows)
                assert not g[other].any(), "embedding rows outside the batch must have zero gradient"
                chk(f"grad {name}", g[rows], res.grads[i][rows], "grad")
        elif keep:
            chk(f"grad {name}", g, res.grads[i], "grad")
        p = ctx.params(i)
        m, v, t = ctx.opt_state(i)
        assert t == res.t == t0 + 1
        sel = rows if rows is not None else slice(None)
        if sample is not None and p.size > sample and rows is None and p.ndim == 2:
            # whole rows (AdamW is elementwise; the row bounds need whole rows)
            k = max(1, sample // p.shape[1])
            sel = np.sort(rng.choice(p.shape[0], min(k, p.shape[0]), replace=False))
        pick = lambda a: np.asarray(a)[sel]
        ps, ms, vs = pick(p), pick(m), pick(v)
        P0s, M0s, V0s = (np.asarray(pick(a), np.float64) for a in (P0[i], M0[i], V0[i]))
        u = 2.0 ** -24
        if keep:
            # AdamW given the library's gradient
            g64 = pick(g).astype(np.float64)
            pg, mg, vg = O.adamw(P0s, g64, M0s, V0s, t, cfg)
            assert np.all(np.abs(ms - mg) <= 8 * u * (cfg.beta1 * np.abs(M0s) + (1 - cfg.beta1) * np.abs(g64))
                          + 1e-45), f"m(g) {name}"
            assert np.all(np.abs(vs - vg) <= 8 * u * (cfg.beta2 * V0s + (1 - cfg.beta2) * g64 * g64) + 1e-45), \
                f"v(g) {name}"
            # magnitude of the terms the step sums: lr/bc1 (b1|m0| + (1-b1)|g|) / denom
            denom = np.sqrt(vg / (1 - cfg.beta2 ** t)) + cfg.adam_eps
            step_terms = cfg.lr / (1 - cfg.beta1 ** t) * (cfg.beta1 * np.abs(M0s) + (1 - cfg.beta1) * np.abs(g64)) \
                / denom
            assert np.all(np.abs(ps - pg) <= 8 * u * (np.abs(P0s) + step_terms) + 1e-45), f"p(g) {name}"
        # end to end (embedding: the rows of this step's tokens); an oracle
        # result without updated state carries the gradients only, and its
        # update is the oracle's AdamW taken on the compared elements
        rg = pick(res.grads[i])
        if res.params is None:
            rp, rm, rv = (O.decoder.fp32(a) for a in O.adamw(P0s, np.asarray(rg, np.float64), M0s, V0s, t, cfg))
        else:
            rp, rm, rv = pick(res.params[i]), pick(res.m[i]), pick(res.v[i])
        if mode == "bf16":
            chk(f"param {name}", ps, rp, "param")
            chk(f"m {name}", ms, rm, "m")
            # v = (1-b2) g^2: compare on g's scale
            chk(f"sqrt v {name}", np.sqrt(vs), np.sqrt(rv), "sqrt v")
        else:
            ok = np.abs(rg) >= 1e-5
            check_fp32(f"param {name}", ps[ok], rp[ok], rtol=1e-4 + extra)
            # m = b1 m0 + (1 - b1) g with m0 equal on both sides: the
            # gradient's tolerance, scaled by (1 - b1), plus fp32 rounding of
            # the sum (relative to |m| it is unbounded where the terms cancel)
            ga = np.abs(rg.astype(np.float64))
            tol_m = (1 - cfg.beta1) * ((1e-4 + extra) * ga + 1e-5) + \
                8 * u * (cfg.beta1 * np.abs(M0s) + (1 - cfg.beta1) * ga) + 1e-12
            bad = np.abs(ms.astype(np.float64) - rm) > tol_m
            assert not bad.any(), f"m {name}: {int(bad.sum())} elements beyond the gradient-implied bound"
            check_normwise(f"m {name}", ms, rm, 1e-4 + extra)
            # v = b2 v0 + (1 - b2) g^2 with v0 equal on both sides: a gradient
            # inside its own tolerance d = 1e-5 + 1e-4 |g| moves v by up to
            # (1 - b2)(2 |g| d + d^2); fp32 rounding adds a few ulp
            dg = 1e-5 + (1e-4 + extra) * ga
            tol_v = (1 - cfg.beta2) * (2 * ga * dg + dg * dg) + 2e-4 * np.abs(rv) + 1e-12
            bad = np.abs(vs.astype(np.float64) - rv) > tol_v
            assert not bad.any(), f"v {name}: {int(bad.sum())} elements beyond the gradient-implied bound"


def check_losses(mode, loss, tl, res, depth="narrow"):
    if mode == "bf16":
        assert abs(loss - res.loss) <= bf16_tol(depth, "loss")[0] * abs(res.loss), (loss, res.loss)
        check_bf16("token losses", tl, res.token_loss, bf16_tol(depth, "token_loss"))
    else:
        assert abs(loss - res.loss) <= 1e-4 * abs(res.loss) + 1e-5
        check_fp32("token losses", tl, res.token_loss)


@release_on_failure
def run_parity(cfg, B, T, mode, steps=1, seed=0, std=0.02, depth="narrow", sample=None, extra=0.0, **ctx_kw):
    params = init_params(cfg, seed, std)
    zeros = [np.zeros_like(p) for p in params]
    dtype = mt.MT_BF16 if mode == "bf16" else mt.MT_FP32
    ctx_kw.setdefault("flags", mt.MT_KEEP_GRADS)
    with make_ctx(cfg, B, T, params, dtype=dtype, **ctx_kw) as ctx:
        P, Mm, Vv, t = params, zeros, zeros, 0
        for s in range(steps):
            tokens, targets = synth.token_batch(seed + 10 * s, B, T, cfg.vocab)
            print(f"step {s + 1}/{steps}: gpu", flush=True)
            loss = ctx.train_step(tokens, targets)
            ctx.sync()
            print(f"step {s + 1}/{steps}: oracle", flush=True)
            res = O.train_step(P, Mm, Vv, t, tokens, targets, cfg, mode)
            check_losses(mode, loss, ctx.token_losses().reshape(B, T), res, depth)
            compare_step(ctx, res, cfg, mode, (P, Mm, Vv, t), tokens, depth, sample, extra)
            t = res.t
            # continue both sides from the library's state (fp32 master values)
            P = [ctx.params(i).astype(np.float64) for i in range(len(params))]
            Mm = [ctx.opt_state(i)[0].astype(np.float64) for i in range(len(params))]
            Vv = [ctx.opt_state(i)[1].astype(np.float64) for i in range(len(params))]


# Large shapes: the oracle's gradients in full, its AdamW (an elementwise
# map) on 65536 sampled elements per tensor.
@release_on_failure
def run_parity_sampled(cfg, B, T, mode, steps=1, seed=0, std=0.02, depth="narrow", **ctx_kw):
    params = init_params(cfg, seed, std)
    n = len(params)
    dtype = mt.MT_BF16 if mode == "bf16" else mt.MT_FP32
    with make_ctx(cfg, B, T, params, dtype=dtype, flags=mt.MT_KEEP_GRADS, **ctx_kw) as ctx:
        P, M0, V0, t = params, [np.zeros(0)] * n, [np.zeros(0)] * n, 0
        for s in range(steps):
            tokens, targets = synth.token_batch(seed + 10 * s, B, T, cfg.vocab)
            print(f"step {s + 1}/{steps}: gpu", flush=True)
            loss = ctx.train_step(tokens, targets)
            print(f"step {s + 1}/{steps}: oracle", flush=True)
            ref_loss, ref_tl, grads, _ = O.gradients(P, tokens, targets, cfg, mode)
            res = O.StepResult(ref_loss, ref_tl, grads, None, None, None, t + 1)
            print(f"step {s + 1}/{steps}: compare", flush=True)
            check_losses(mode, loss, ctx.token_losses().reshape(B, T), res, depth)
            if t == 0:
                M0 = V0 = [np.zeros_like(p) for p in P]
            compare_step(ctx, res, cfg, mode, (P, M0, V0, t), tokens, depth, sample=1 << 16)
            del res, grads
            t += 1
            if s + 1 < steps:
                P = [ctx.params(i) for i in range(n)]
                M0 = [ctx.opt_state(i)[0] for i in range(n)]
                V0 = [ctx.opt_state(i)[1] for i in range(n)]


def test_tiny_fp32_two_steps():
    cfg, B, T = shape("tiny")
    run_parity(cfg, B, T, "fp32", steps=2)


def test_tiny_fp32_larger_weights():
    cfg, B, T = shape("tiny")
    run_parity(cfg, B, T, "fp32", seed=3, std=0.2)


def test_gqa_ragged_fp32():
    cfg = O.Config(3, 128, 8, 2, 16, 200, 1000)
    run_parity(cfg, 3, 70, "fp32", steps=2, seed=5, std=0.1)


def test_gqa_ragged_bf16():
    cfg = O.Config(2, 256, 4, 2, 64, 344, 1000)
    run_parity(cfg, 2, 100, "bf16", steps=2, seed=7, std=0.05)


def test_bf16_hd128():
    cfg = O.Config(2, 256, 2, 1, 128, 512, 512)
    run_parity(cfg, 1, 200, "bf16", seed=9, std=0.05)


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_1p3b_layer_shape_reduced_depth(mode):
    # per-layer shape of the 1.3B workload, 2 layers, 1 x 256 tokens
    cfg, _, _ = shape("1.3b", n_layers=2)
    run_parity(cfg, 1, 256, mode, seed=11)


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_1p3b_full_depth_short_sequence(mode):
    # all 24 layers of the 1.3B workload (d 2048, FFN 5632, vocab 32000) on
    # 1 x 96 tokens: the streamed schedule's accumulation through the full
    # depth at the real width, against the oracle's whole step; bf16 with the
    # deep class's bounds (the oracle's own bf16 reading lies up to 3.8%
    # normwise from its float64 step on the query/key projection gradients)
    cfg, _, _ = shape("1.3b")
    run_parity_sampled(cfg, 1, 96, mode, seed=31, depth="deep")


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_token_chunks_and_parked_checkpoints(mode):
    # 2 x 48 tokens in chunks of 40 rows (40, 40, 16) for the QKV projection
    # and the MLP; 3 of the 5 layers' input checkpoints parked in host memory
    cfg = O.Config(5, 128, 2, 1, 64, 200, 300)
    run_parity(cfg, 2, 48, mode, steps=2, seed=19, std=0.05, chunk_rows=40, ckpt_host=3)


def _run_steps(cfg, B, T, dtype, steps=2, **kw):
    params = init_params(cfg, 23, 0.05)
    out = []
    with make_ctx(cfg, B, T, params, dtype=dtype, flags=mt.MT_KEEP_GRADS | mt.MT_TRACE, **kw) as ctx:
        for s in range(steps):
            tokens, targets = synth.token_batch(23 + s, B, T, cfg.vocab)
            out.append(ctx.train_step(tokens, targets))
        n = len(params)
        out += [ctx.params(i).copy() for i in range(n)] + [ctx.grads(i).copy() for i in range(n)]
        return out, ctx.layout_info(), ctx.schedule()


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
def test_parked_checkpoints_are_bitwise_neutral(dtype):
    """Where a residual checkpoint waits between forward and backward does not
    change any result: every parking depth gives the same bits as none. The
    schedule shows each parked checkpoint going out once and coming back once,
    x_0 from the gathered embedding rows."""
    L = 6
    cfg = O.Config(L, 128, 2, 1, 64, 200, 300)
    ref, info, _ = _run_steps(cfg, 2, 40, dtype, chunk_rows=32)
    assert info == {"chunk_rows": 32, "ckpt_host": 0, "ckpt_device_slots": L + 1}
    for k in (1, 2, L - 2):
        got, info, sched = _run_steps(cfg, 2, 40, dtype, chunk_rows=32, ckpt_host=k)
        assert info == {"chunk_rows": 32, "ckpt_host": k, "ckpt_device_slots": L - k}
        for a, b in zip(ref, got):
            assert np.array_equal(np.asarray(a), np.asarray(b))
        outs = sorted(e["unit"] for e in sched if e["phase"] == "ckpt_out")
        ins = sorted(e["unit"] for e in sched if e["phase"] == "ckpt_in")
        assert outs == list(range(1, k + 1)) and ins == list(range(0, k + 1))


def test_token_chunks_change_only_rounding():
    """Chunking the projections changes only the order in which the weight
    gradients add up the chunks."""
    cfg = O.Config(3, 128, 2, 1, 64, 200, 300)
    ref, info0, _ = _run_steps(cfg, 2, 40, mt.MT_FP32, steps=1)
    got, info1, _ = _run_steps(cfg, 2, 40, mt.MT_FP32, steps=1, chunk_rows=24)
    assert info0["chunk_rows"] == 80 and info1["chunk_rows"] == 24
    assert abs(ref[0] - got[0]) <= 1e-6 * abs(ref[0])
    n = (len(ref) - 1) // 2
    for i in range(n):
        pa, pb, ga, gb = ref[1 + i], got[1 + i], ref[1 + n + i], got[1 + n + i]
        np.testing.assert_allclose(gb, ga, rtol=1e-5, atol=1e-7 * (np.max(np.abs(ga)) + 1e-30))
        # the first AdamW step moves p by about lr g / (|g| + eps): only where
        # |g| >> eps does a gradient within rounding give an update within rounding
        ok = np.abs(ga) >= 1e-5
        np.testing.assert_allclose(pb[ok], pa[ok], rtol=1e-5, atol=1e-9)


@pytest.mark.parametrize("dtype,keep", [(mt.MT_FP32, True), (mt.MT_BF16, False), (mt.MT_BF16, True)])
def test_overlapped_optimizer_is_bitwise_synchronous(dtype, keep):
    """With MT_OVERLAP_OPT a step returns before its AdamW updates have all
    landed; the next step loads each unit only after its update. Losses of
    every step and the final state match the synchronous mode bit for bit."""
    cfg = O.Config(5, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 29, 0.05)
    base = mt.MT_KEEP_GRADS if keep else 0
    out = []
    for flags in (base, base | mt.MT_OVERLAP_OPT):
        with make_ctx(cfg, 2, 40, params, dtype=dtype, flags=flags) as ctx:
            losses = []
            for s in range(4):
                tokens, targets = synth.token_batch(29 + s, 2, 40, cfg.vocab)
                losses.append(ctx.train_step(tokens, targets))
                tl = ctx.token_losses().copy()
            ctx.sync()
            n = len(params)
            state = [ctx.params(i).copy() for i in range(n)]
            state += [ctx.opt_state(i)[0].copy() for i in range(n)] + [ctx.opt_state(i)[1].copy() for i in range(n)]
            if keep:
                state += [ctx.grads(i).copy() for i in range(n)]
            out.append((losses, tl, state))
    (l0, t0, s0), (l1, t1, s1) = out
    assert l0 == l1
    assert np.array_equal(t0, t1)
    for a, b in zip(s0, s1):
        assert np.array_equal(a, b)


def _run_cached_steps(ctx, n, seed, B, T, vocab, n_params, between=None):
    losses, tls = [], []
    for s in range(n):
        if between:
            between(ctx, s)
        tok, tgt = synth.token_batch(seed + s, B, T, vocab)
        losses.append(ctx.train_step(tok, tgt))
        tls.append(ctx.token_losses().copy())
    ctx.sync()
    state = [ctx.params(i).copy() for i in range(n_params)]
    state += [ctx.opt_state(i)[0].copy() for i in range(n_params)] + [ctx.opt_state(i)[1].copy() for i in range(n_params)]
    if ctx.cfg.flags & mt.MT_KEEP_GRADS:
        state += [ctx.grads(i).copy() for i in range(n_params)]
    return losses, tls, state


# A device cache (more than two layer buffers) changes only where the weights
# wait between uses: every loss and the whole host state after four steps
# equal the streamed schedule's bit for bit. 6 layers: 3 buffers cache the
# head, 4 the head and layer 5, 7 every unit.
@pytest.mark.parametrize("dtype,buffers,flags", [
    (mt.MT_FP32, 7, mt.MT_KEEP_GRADS),
    (mt.MT_BF16, 7, mt.MT_KEEP_GRADS),
    (mt.MT_FP32, 3, mt.MT_OVERLAP_OPT),
    (mt.MT_BF16, 4, mt.MT_KEEP_GRADS | mt.MT_OVERLAP_OPT),
    (mt.MT_BF16, 7, mt.MT_OVERLAP_OPT),
    (mt.MT_BF16, 7, mt.MT_OVERLAP_OPT | mt.MT_CACHE_NO_REFRESH),
])
def test_streamed_equals_device_cache_bitwise(dtype, buffers, flags):
    cfg = O.Config(6, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 21, 0.1)
    out = []
    for nb in (2, buffers):
        with make_ctx(cfg, 2, 64, params, dtype=dtype, buffers=nb, flags=flags) as ctx:
            out.append(_run_cached_steps(ctx, 4, 21, 2, 64, cfg.vocab, len(params)))
    (l0, t0, s0), (l1, t1, s1) = out
    assert l0 == l1
    for a, b in zip(t0 + s0, t1 + s1):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
def test_set_param_reaches_cached_units(dtype):
    """mt_set_param between steps changes a cached unit's host image; its
    stale device copy must not be used by the next forward."""
    cfg = O.Config(4, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 5, 0.1)
    names = [n for n, _, _ in O.tensor_table(cfg)]
    ids = [names.index("layers.3.wq"), names.index("layers.0.w_down"), names.index("lm_head")]
    rng = np.random.default_rng(5)
    fresh = {i: (0.05 * rng.standard_normal(params[i].shape)).astype(np.float32) for i in ids}

    def between(ctx, s):
        if s == 2:
            for i in ids:
                ctx.set_param(i, fresh[i])

    out = []
    for nb in (2, cfg.n_layers + 1):
        with make_ctx(cfg, 2, 48, params, dtype=dtype, buffers=nb, flags=mt.MT_OVERLAP_OPT) as ctx:
            out.append(_run_cached_steps(ctx, 4, 5, 2, 48, cfg.vocab, len(params), between))
    (l0, t0, s0), (l1, t1, s1) = out
    assert l0 == l1
    for a, b in zip(t0 + s0, t1 + s1):
        np.testing.assert_array_equal(a, b)


def test_device_cache_schedule():
    """Every unit cached: the first step fetches each unit once, for its
    forward; each unit's updated image is copied in after its gradients have
    left and its AdamW has landed; the next step fetches only the units not
    refreshed that way. Two of four buffers cached: the streamed layers still
    held by their buffers at the turn are not fetched again."""
    cfg = O.Config(6, 256, 4, 4, 64, 512, 512)
    L = cfg.n_layers
    params = init_params(cfg, 1, 0.05)
    units = list(range(L)) + [mt.UNIT_HEAD]
    with make_ctx(cfg, 2, 128, params, buffers=L + 1, flags=mt.MT_KEEP_GRADS | mt.MT_TRACE) as ctx:
        tok, tgt = synth.token_batch(1, 2, 128, cfg.vocab)
        scheds = []
        for _ in range(3):
            ctx.train_step(tok, tgt)
            scheds.append(ctx.schedule())
    for k, sched in enumerate(scheds):
        for e in sorted(sched, key=lambda e: e["t0"]):   # shown on failure
            print(k, f'{e["phase"]:7s} unit {e["unit"]:3d} stream {e["stream"]} {e["t0"]:9.3f} {e["t1"]:9.3f}')
        comp = [(e["phase"], e["unit"]) for e in sched if e["stream"] == 1]
        assert comp == [("fwd", l) for l in range(L)] + [("head", mt.UNIT_HEAD)] + \
            [("bwd", l) for l in reversed(range(L))]
    head_t0 = {k: [e for e in s if e["phase"] == "head"][0]["t0"] for k, s in enumerate(scheds)}
    loads = [[e["unit"] for e in s if e["phase"] == "load" and e["stream"] == 0] for s in scheds]
    refr = [[e for e in s if e["phase"] == "refresh" and e["stream"] == 0] for s in scheds]
    assert loads[0] == units
    for k in range(3):
        # forward only
        assert all(e["t1"] <= head_t0[k] for e in scheds[k] if e["phase"] == "load" and e["stream"] == 0)
        by = {(e["phase"], e["unit"]): e for e in scheds[k] if e["stream"] in (1, 2, 3)}
        for e in refr[k]:
            assert e["t0"] >= by[("grad", e["unit"])]["t1"] - 1e-3
            assert e["t0"] >= by[("adamw", e["unit"])]["t1"] - 0.5
    for k in (1, 2):
        done = {e["unit"] for e in refr[k - 1]}
        assert sorted(loads[k], key=units.index) == [u for u in units if u not in done]
    # (the first step's updates may all land after its last gradient: fresh
    # host pages make them slow)
    assert min(len(loads[1]), len(loads[2])) < len(units)
    with make_ctx(cfg, 2, 128, params, buffers=4, flags=mt.MT_KEEP_GRADS | mt.MT_TRACE) as ctx:
        ctx.train_step(tok, tgt)
        ctx.train_step(tok, tgt)
        sched = ctx.schedule()
        refreshed = {e["unit"] for e in sched if e["phase"] == "refresh"}
    assert refreshed <= {L - 1, mt.UNIT_HEAD}
    t_head = [e for e in sched if e["phase"] == "head"][0]["t0"]
    bwd_loads = [e["unit"] for e in sched if e["phase"] == "load" and e["stream"] == 0 and e["t0"] >= t_head]
    assert bwd_loads == list(range(L - 4, -1, -1))


def test_token_order_is_exact():
    # swapping two batch rows permutes the per-token losses exactly
    cfg, B, T = shape("tiny")
    params = init_params(cfg, 0, 0.1)
    tok, tgt = synth.token_batch(0, B, T, cfg.vocab)
    res = []
    for order in ([0, 1], [1, 0]):
        with make_ctx(cfg, B, T, params) as ctx:
            ctx.train_step(tok[order].copy(), tgt[order].copy())
            res.append(ctx.token_losses().reshape(B, T))
    np.testing.assert_array_equal(res[0], res[1][[1, 0]])


def test_schedule_order_and_overlap():
    cfg = O.Config(6, 256, 4, 4, 64, 512, 512)
    L = cfg.n_layers
    params = init_params(cfg, 1, 0.05)
    with make_ctx(cfg, 2, 128, params, flags=mt.MT_KEEP_GRADS | mt.MT_TRACE) as ctx:
        tok, tgt = synth.token_batch(1, 2, 128, cfg.vocab)
        ctx.train_step(tok, tgt)
        ctx.train_step(tok, tgt)
        sched = ctx.schedule()
    for e in sorted(sched, key=lambda e: e["t0"]):   # shown on failure
        print(f'{e["phase"]:6s} unit {e["unit"]:3d} stream {e["stream"]} {e["t0"]:9.3f} {e["t1"]:9.3f}')
    comp = [(e["phase"], e["unit"]) for e in sched if e["stream"] == 1]
    exp = [("fwd", l) for l in range(L)] + [("head", mt.UNIT_HEAD)] + [("bwd", l) for l in reversed(range(L))]
    assert comp == exp
    loads = [e for e in sched if e["phase"] == "load" and e["stream"] == 0]
    # every layer is fetched once forward, and every layer but the last again for backward
    assert [e["unit"] for e in loads] == list(range(L)) + [mt.UNIT_HEAD] + list(range(L - 2, -1, -1))
    by = {(e["phase"], e["unit"]): e for e in sched if e["stream"] in (1, 2)}
    fwd_load = {e["unit"]: e for e in loads[:L]}
    for l in range(1, L - 1):
        # layer l+1 is being fetched while layer l computes
        assert fwd_load[l + 1]["t0"] <= by[("fwd", l)]["t1"]
        assert fwd_load[l + 1]["buffer"] != by[("fwd", l)]["buffer"]
    for l in range(L - 1, 1, -1):
        # gradients of layer l have been copied out before layer l-2 finishes
        assert by[("grad", l)]["t1"] <= by[("bwd", l - 2)]["t1"]
    adam = {e["unit"]: e for e in sched if e["phase"] == "adamw"}
    # the submitting thread never waits on the device inside an enqueue call
    host = [e for e in sched if e["stream"] == 4]
    assert host and max(e["t1"] - e["t0"] for e in host) < 2.0
    for l in range(L):
        assert adam[l]["t0"] >= by[("grad", l)]["t1"] - 0.5


def test_device_memory_independent_of_depth():
    sizes = {}
    for L in (2, 8):
        cfg = O.Config(L, 256, 4, 4, 64, 512, 512)
        with make_ctx(cfg, 1, 128, init_params(cfg, 0)) as ctx:
            sizes[L] = ctx.device_bytes()
            free0 = torch.cuda.mem_get_info()[0]
            tok, tgt = synth.token_batch(0, 1, 128, cfg.vocab)
            ctx.train_step(tok, tgt)
            assert torch.cuda.mem_get_info()[0] == free0   # nothing allocated by the step
    # only the residual checkpoints grow with depth
    assert sizes[8] - sizes[2] == 6 * 128 * 256 * 4


def test_bad_token_is_rejected_before_any_work():
    cfg, B, T = shape("tiny")
    params = init_params(cfg, 0)
    with make_ctx(cfg, B, T, params) as ctx:
        tok, tgt = synth.token_batch(0, B, T, cfg.vocab)
        tok[1, 5] = cfg.vocab
        with pytest.raises(mt.MTError) as e:
            ctx.train_step(tok, tgt)
        assert e.value.code == mt.MT_EINVAL
        assert ctx.opt_state(0)[2] == 0
        with pytest.raises(mt.MTError):
            ctx.train_step(np.zeros((B + 1, T), np.int32), np.zeros((B + 1, T), np.int32))
        # empty batches and sequences are rejected, not run
        for shp in ((0, T), (B, 0)):
            with pytest.raises(mt.MTError) as e:
                ctx.train_step(np.zeros(shp, np.int32), np.zeros(shp, np.int32))
            assert e.value.code == mt.MT_EINVAL
        assert ctx.opt_state(0)[2] == 0


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_step_smaller_than_allocated(mode):
    """A context sized for 3 x 70 tokens runs a 2 x 45 step: every kernel
    sees the actual, ragged sizes, not the allocated ones."""
    cfg = O.Config(2, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 31, 0.05)
    zeros = [np.zeros_like(p) for p in params]
    dtype = mt.MT_BF16 if mode == "bf16" else mt.MT_FP32
    c = mt.make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                       cfg.vocab, 3, 70, dtype=dtype, flags=mt.MT_KEEP_GRADS, host_threads=8)
    with mt.Context(c, params) as ctx:
        tokens, targets = synth.token_batch(31, 2, 45, cfg.vocab)
        loss = ctx.train_step(tokens, targets)
        res = O.train_step(params, zeros, zeros, 0, tokens, targets, cfg, mode)
        assert ctx.token_losses().shape == (2 * 45,)
        check_losses(mode, loss, ctx.token_losses().reshape(2, 45), res)
        compare_step(ctx, res, cfg, mode, (params, zeros, zeros, 0), tokens)


def test_nonfinite_loss_applies_no_update():
    cfg, B, T = shape("tiny")
    params = init_params(cfg, 0)
    params[-1] = params[-1].copy()
    params[-1][3, 7] = np.inf
    with make_ctx(cfg, B, T, params) as ctx:
        tok, tgt = synth.token_batch(0, B, T, cfg.vocab)
        before = [ctx.params(i) for i in range(len(params))]
        with pytest.raises(mt.MTError) as e:
            ctx.train_step(tok, tgt)
        assert e.value.code == mt.MT_ENONFINITE
        for i, b in enumerate(before):
            np.testing.assert_array_equal(ctx.params(i), b)
            assert not ctx.opt_state(i)[0].any()
        assert ctx.opt_state(0)[2] == 0
        # a finite weight restores normal operation
        ctx.set_param(len(params) - 1, init_params(cfg, 0)[-1])
        assert math.isfinite(ctx.train_step(tok, tgt))


def test_gradients_not_kept_without_flag():
    cfg, B, T = shape("tiny")
    params = init_params(cfg, 0)
    with make_ctx(cfg, B, T, params, flags=0) as a, make_ctx(cfg, B, T, params) as b:
        tok, tgt = synth.token_batch(0, B, T, cfg.vocab)
        la, lb = a.train_step(tok, tgt), b.train_step(tok, tgt)
        assert la == lb
        with pytest.raises(mt.MTError) as e:
            a.grads(0)
        assert e.value.code == mt.MT_ENOGRADS
        # the staging ring gives the same update as kept gradients
        for i in range(len(params)):
            np.testing.assert_array_equal(a.params(i), b.params(i))


# ---------------------------------------------------------------------------
# The launch configuration bench.py times: overlapped optimizer, no kept
# gradients (pinned staging ring), kernel timing and trace on. Two staging
# slots for six layers make every step recycle slots while earlier updates
# still hold them; three steps carry the moments forward.

BENCH_FLAGS = mt.MT_OVERLAP_OPT | mt.MT_KERNEL_TIMING | mt.MT_TRACE


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_bench_flag_set_recycled_ring(mode):
    cfg = O.Config(6, 128, 2, 1, 64, 200, 300)
    run_parity(cfg, 2, 32, mode, steps=3, seed=37, std=0.05, flags=BENCH_FLAGS, ring_slots=2)


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_bench_flag_set_every_unit_cached(mode):
    cfg = O.Config(6, 128, 2, 1, 64, 200, 300)
    run_parity(cfg, 2, 32, mode, steps=3, seed=37, std=0.05, flags=BENCH_FLAGS, buffers=cfg.n_layers + 1)


# ---------------------------------------------------------------------------
# Micro-batch gradient accumulation inside each streamed unit: 5 sequences in
# micro-batches of 2, 2 and 1 (the workspace holds 2), weight gradients summed
# on the device over them, against the oracle's whole-batch step; plus the
# same split with token chunks and parked checkpoints, and the bench flag set.

@pytest.mark.parametrize("mode,kw", [("fp32", {}), ("bf16", {}),
                                     ("fp32", dict(chunk_rows=24, ckpt_host=2)),
                                     ("bf16", dict(flags=BENCH_FLAGS, ring_slots=2))])
def test_micro_batch_accumulation(mode, kw):
    cfg = O.Config(4, 128, 2, 1, 64, 200, 300)
    run_parity(cfg, 5, 20, mode, steps=2, seed=47, std=0.05, micro_batches=3, **kw)


def test_micro_batches_change_only_rounding():
    """Micro-batches change only the order in which the weight gradients
    add up: losses within fp32 rounding, gradients within a few ulp of their
    terms' magnitude, of the whole-batch step."""
    cfg = O.Config(3, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 49, 0.05)
    tok, tgt = synth.token_batch(49, 4, 24, cfg.vocab)
    out = []
    for k in (0, 4):
        with make_ctx(cfg, 4, 24, params, micro_batches=k) as ctx:
            loss = ctx.train_step(tok, tgt)
            out.append((loss, ctx.token_losses().copy(), [ctx.grads(i) for i in range(len(params))]))
    (l0, t0, g0), (l1, t1, g1) = out
    assert abs(l0 - l1) <= 1e-6 * abs(l0)
    np.testing.assert_allclose(t1, t0, rtol=1e-6, atol=1e-7)
    for a, b in zip(g0, g1):
        np.testing.assert_allclose(b, a, rtol=1e-5, atol=1e-7 * (np.max(np.abs(a)) + 1e-30))


# ---------------------------------------------------------------------------
# Gradients over the link in bf16 (MT_BF16_GRADS): each gradient is the
# oracle's within its own rounding (2^-8 relative at most) on top of the mode's
# tolerance, with kept gradients (widened on the host) and through the
# recycled staging ring in the bench's flag set.

@pytest.mark.parametrize("mode,flags", [("fp32", mt.MT_KEEP_GRADS | mt.MT_BF16_GRADS),
                                        ("bf16", mt.MT_KEEP_GRADS | mt.MT_BF16_GRADS),
                                        ("bf16", BENCH_FLAGS | mt.MT_BF16_GRADS)])
def test_bf16_gradient_transfer(mode, flags):
    cfg = O.Config(6, 128, 2, 1, 64, 200, 300)
    run_parity(cfg, 2, 32, mode, steps=3, seed=37, std=0.05, flags=flags, ring_slots=2, extra=2.0 ** -8)


# ---------------------------------------------------------------------------
# Schedule robustness: host delays injected into loads, gradient copies and
# every AdamW, and NaN written over each released layer and gradient buffer,
# leave every result bit for bit unchanged.

class _env:
    def __init__(self, **kv):
        self.kv = {k: str(v) for k, v in kv.items()}

    def __enter__(self):
        import os
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update(self.kv)

    def __exit__(self, *a):
        import os
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("dtype,flags,slots", [(mt.MT_BF16, mt.MT_OVERLAP_OPT, 2),
                                               (mt.MT_FP32, mt.MT_KEEP_GRADS, 0),
                                               (mt.MT_BF16, 0, 1)])
def test_host_delays_and_poisoned_buffers_change_nothing(dtype, flags, slots):
    cfg = O.Config(6, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 41, 0.05)
    out = []
    hooks = (dict(), dict(MT_TEST_DELAY_H2D_US=1500, MT_TEST_DELAY_D2H_US=1500, MT_TEST_DELAY_ADAMW_US=20000,
                          MT_TEST_POISON=1))
    for env in hooks:
        with _env(**env):
            ctx = make_ctx(cfg, 2, 40, params, dtype=dtype, flags=flags, ring_slots=slots)
        with ctx:
            out.append(_run_cached_steps(ctx, 3, 41, 2, 40, cfg.vocab, len(params)))
    (l0, t0, s0), (l1, t1, s1) = out
    assert l0 == l1
    for a, b in zip(t0 + s0, t1 + s1):
        np.testing.assert_array_equal(a, b)
    assert all(np.isfinite(x).all() for x in s1)


# ---------------------------------------------------------------------------
# A host wait beyond cfg.wait_timeout_ms: every AdamW held for 1.5 s against
# a 250 ms limit. The step returns MT_ETIMEOUT naming what it waited for, the
# context refuses further steps, and its state can still be read and freed.

@pytest.mark.parametrize("flags,slots,steps,expect", [
    (mt.MT_KEEP_GRADS, 0, 1, "AdamW updates still running"),
    (0, 1, 1, "no free staging slot"),
    (mt.MT_OVERLAP_OPT | mt.MT_KEEP_GRADS, 0, 2, "AdamW update"),
])
def test_wait_timeout(flags, slots, steps, expect):
    cfg = O.Config(4, 128, 2, 1, 64, 200, 300)
    params = init_params(cfg, 43, 0.05)
    with _env(MT_TEST_DELAY_ADAMW_US=1500000):
        c = mt.make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                           cfg.vocab, 2, 40, dtype=mt.MT_BF16, flags=flags, host_threads=4,
                           grad_ring_slots=slots, wait_timeout_ms=250)
        ctx = mt.Context(c, params)
    with ctx:
        tok, tgt = synth.token_batch(43, 2, 40, cfg.vocab)
        for _ in range(steps - 1):
            ctx.train_step(tok, tgt)
        with pytest.raises(mt.MTError) as e:
            ctx.train_step(tok, tgt)
        assert e.value.code == mt.MT_ETIMEOUT
        assert expect in str(e.value), str(e.value)
        with pytest.raises(mt.MTError) as e2:
            ctx.train_step(tok, tgt)
        assert e2.value.code == mt.MT_ESTATE
        assert np.all(np.isfinite(ctx.params(1)))


def test_trace_dump_is_chrome_json_in_schedule_order(tmp_path):
    import json
    cfg = O.Config(4, 128, 2, 1, 64, 200, 300)
    L = cfg.n_layers
    with make_ctx(cfg, 2, 40, init_params(cfg, 3, 0.05), flags=mt.MT_KEEP_GRADS | mt.MT_TRACE) as ctx:
        tok, tgt = synth.token_batch(3, 2, 40, cfg.vocab)
        ctx.train_step(tok, tgt)
        path = str(tmp_path / "trace.json")
        ctx.trace_dump(path)
        sched = ctx.schedule()
    with open(path) as f:
        ev = json.load(f)["traceEvents"]
    names = {e["tid"]: e["args"]["name"] for e in ev if e["ph"] == "M"}
    assert names[0] == "copy-in" and names[1] == "compute" and names[2] == "copy-out"
    spans = [e for e in ev if e["ph"] == "X"]
    assert len(spans) == len(sched)
    comp = [e["name"] for e in sorted((e for e in spans if e["tid"] == 1), key=lambda e: e["ts"])]
    assert comp == [f"fwd layer {l}" for l in range(L)] + ["head head"] + \
        [f"bwd layer {l}" for l in reversed(range(L))]
    for e in spans:
        assert e["dur"] >= 0
    grads = [e["name"] for e in sorted((e for e in spans if e["tid"] == 2), key=lambda e: e["ts"])]
    assert grads == ["grad head"] + [f"grad layer {l}" for l in reversed(range(L))]


# ---------------------------------------------------------------------------
# A caller-supplied device workspace (mt_device_env.workspace, here a torch
# tensor): every device buffer is carved from it; with room for all
# checkpoints nothing is parked, with room for two plus one the rest are
# parked in host memory; results equal a context that allocates its own.

def test_caller_workspace():
    cfg = O.Config(5, 128, 2, 1, 64, 200, 300)
    L = cfg.n_layers
    params = init_params(cfg, 53, 0.05)
    c = mt.make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                       cfg.vocab, 2, 40, dtype=mt.MT_BF16, flags=mt.MT_KEEP_GRADS, host_threads=8)
    plan = mt.device_plan(c)
    runs = []
    with mt.Context(c, params) as ctx:
        runs.append(_run_cached_steps(ctx, 2, 53, 2, 40, cfg.vocab, len(params)))
        assert ctx.device_bytes() == plan["fixed"] + (L + 1) * plan["ckpt_slot"]
    for slots, parked in ((L + 1, 0), (3, L - 3)):
        nbytes = plan["fixed"] + slots * plan["ckpt_slot"]
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        with mt.Context(c, params, workspace=(ws, nbytes)) as ctx:
            assert ctx.device_bytes() == nbytes
            assert ctx.layout_info()["ckpt_host"] == parked
            runs.append(_run_cached_steps(ctx, 2, 53, 2, 40, cfg.vocab, len(params)))
        del ws
    (l0, t0, s0) = runs[0]
    for (l1, t1, s1) in runs[1:]:
        assert l0 == l1
        for a, b in zip(t0 + s0, t1 + s1):
            np.testing.assert_array_equal(a, b)
    # too small for two checkpoint slots next to the rest
    ws = torch.empty(plan["fixed"] + plan["ckpt_slot"], dtype=torch.uint8, device="cuda")
    with pytest.raises(mt.MTError) as e:
        mt.Context(c, params, workspace=(ws, ws.numel()))
    assert e.value.code == mt.MT_EDEVOOM
