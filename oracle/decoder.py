"""CPU oracle of one layer-streamed training step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
``oracle/``. The GPU library never routes through it, and it shares no code,
table or constant with the GPU library: the only thing both sides use is the
seeded input generator (``host_memory_streamed_amd.synth``), which draws
numbers and computes nothing of the method.

What is computed
----------------
Streaming, double buffering and recompute change where and when the math
runs, not what it computes ("MegaTrain: Full Precision Training of 100B+
Parameter LLMs on a Single GPU", abstract: parameters stream in per layer,
gradients stream out, autograd graphs are replaced by stateless templates;
"Technical Brief: MegaTrain's Single-GPU 120B-Parameter Training
Breakthrough", section "Checkpointing, Manual Gradients, and CPU-Side
Optimizer Steps": activations are recomputed in backward and the optimizer
step runs on the CPU over fp32 master weights and moments). So this oracle is
the plain definition of one training step of the decoder, in float64, with no
streaming and no recompute: every intermediate is simply kept.

The pages do not describe the model. The model is a Llama-style decoder:
RMSNorm (eps inside the square root, gain after normalising), half-split
rotary embeddings, causal grouped-query attention with scale 1/sqrt(head_dim),
SwiGLU MLP ``down(silu(gate(h)) * up(h))``, no biases, final RMSNorm and an
untied LM head, mean next-token cross-entropy over all B*T positions, and
AdamW with decoupled weight decay on every tensor (the Adam paper is listed as
a foundation on the abstract's page, section "Builds on").

Precision modes
---------------
``mode="fp32"``: the GPU computes in fp32; the oracle computes every step in
float64 from the fp32 master values.

``mode="bf16"``: the GPU feeds bf16 operands (round-to-nearest-even) to its
matrix cores and accumulates in fp32 ("Mixed Precision Training" is listed on
the abstract's page under "Builds on"). The oracle rounds to bf16 at exactly
the same points and accumulates in float64:

* weights that enter a matrix product: ``bf16(p)`` of the fp32 master;
* activation operands of products: the RMSNorm outputs, the rotated q and k,
  v, the attention probabilities P (for P.V and for dV), the attention output
  o, the SwiGLU output, and every incoming gradient of a product (dz, the
  residual gradients before the down and out projections, dgate/dup, dO,
  dS, dq/dk/dv after the inverse rotation);
* everything else (residual stream, norms, softmax statistics, rotations, the
  loss, ``D = rowsum(dO * O)``, the weight gradients, AdamW) stays full
  precision.

The attention probabilities are rounded where the definition forms them:
the normalised P = softmax(S), once, before the product with V (and the
same P, recomputed from the logsumexp, before the product that gives dV).
This is the plain reading of "bf16 operands into the matrix product"; no
implementation's blocking or running maximum enters it.

The exact rounding outcomes in bf16 mode are parity unpinned: a bf16
implementation is held to this reading within tolerances derived from the
distance of this reading itself from the float64 step (``mode="fp32"``).

Master state is stored in fp32 (the method's "full precision" state), so
``train_step`` rounds p, m and v to fp32 after each update.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
from threadpoolctl import threadpool_limits

# attention heads run on a thread pool (False: one after another)
PARALLEL_HEADS = True

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


@dataclass
class Config:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    weight_decay: float = 0.01


def tensor_table(cfg: Config):
    """Canonical tensor order: ``tok_emb``; per layer the nine LAYER_TENSORS;
    ``final_norm``; ``lm_head``. Linear weights are ``[out, in]`` (y = x W^T).
    Returns a list of ``(name, shape, is_gain)``."""
    d, hd, F, V = cfg.d_model, cfg.head_dim, cfg.ffn_dim, cfg.vocab
    qd, kvd = cfg.n_heads * hd, cfg.n_kv_heads * hd
    out = [("tok_emb", (V, d), False)]
    for l in range(cfg.n_layers):
        shapes = {"attn_norm": (d,), "wq": (qd, d), "wk": (kvd, d), "wv": (kvd, d),
                  "wo": (d, qd), "mlp_norm": (d,), "w_gate": (F, d), "w_up": (F, d),
                  "w_down": (d, F)}
        for n in LAYER_TENSORS:
            out.append((f"layers.{l}.{n}", shapes[n], n.endswith("norm")))
    out.append(("final_norm", (d,), True))
    out.append(("lm_head", (V, d), False))
    return out


# ----------------------------------------------------------------------------
# Rounding
# ----------------------------------------------------------------------------

def bf16(x) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even) through fp32, and
    return the value as float64. Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f.view(np.uint32)
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32).astype(np.float64)


def fp32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


class _Prec:
    def __init__(self, mode: str):
        if mode not in ("fp32", "bf16"):
            raise ValueError(mode)
        self.mode = mode

    def op(self, x):
        """Operand of a matrix product."""
        return bf16(x) if self.mode != "fp32" else x


# ----------------------------------------------------------------------------
# Layer pieces (each is the textbook definition; backward is the analytic one)
# ----------------------------------------------------------------------------

def rmsnorm_fwd(x, w, eps):
    """y = x * (mean(x^2) + eps)^(-1/2) * w over the last axis. Returns (y, r)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None] * w, r


def rmsnorm_bwd(x, w, r, dy):
    """With gw = dy*w: dx = r*(gw - x*r^2*mean(gw*x)), dw = sum_tokens dy*x*r."""
    gw = dy * w
    dx = r[..., None] * (gw - x * (r * r)[..., None] * np.mean(gw * x, axis=-1)[..., None])
    dw = np.sum(dy * x * r[..., None], axis=tuple(range(x.ndim - 1)))
    return dx, dw


def rope_tables(T, hd, base):
    """cos and sin of angle t*base^(-2i/hd), t < T, i < hd/2: built in float64
    and stored in fp32 (positions reach 524287, where an fp32 angle would be off
    by up to ~1.6e-2 rad)."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / hd)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    return fp32(np.cos(ang)), fp32(np.sin(ang))


def rope_fwd(x, cos, sin):
    """Half-split rotation. x: [B, T, heads, hd]; cos/sin: [T, hd/2]."""
    h = x.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_bwd(dy, cos, sin):
    """Adjoint of the rotation: rotate by the negative angle."""
    h = dy.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    d1, d2 = dy[..., :h], dy[..., h:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def _threads():
    """Worker threads: the CPUs this process may run on, at most
    OMP_NUM_THREADS when that is set, and at most 16."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(16, n))


def _per_head(fn, B, H):
    """[fn(b, h) for b < B, h < H] in that order. Heads are independent, so
    they run on a thread pool (one BLAS thread each); the results, and every
    sum formed from them, are exactly those of the plain loop."""
    pairs = [(b, h) for b in range(B) for h in range(H)]
    workers = min(len(pairs), _threads())
    if workers <= 1 or not PARALLEL_HEADS:
        return [fn(b, h) for b, h in pairs]
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda bh: fn(*bh), pairs))


def attention_fwd(q, k, v, prec: _Prec):
    """Causal GQA attention. q: [B,T,H,hd], k/v: [B,T,Hkv,hd] (already the
    matrix-product operands). Query head h reads kv head h // (H/Hkv).
    Returns o [B,T,H,hd] and lse [B,H,T] (natural-log logsumexp of the scaled,
    masked scores)."""
    B, T, H, hd = q.shape
    Hkv = k.shape[2]
    grp = H // Hkv
    scale = 1.0 / np.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    o = np.empty_like(q)
    lse = np.empty((B, H, T))

    def head(b, h):
        kv = h // grp
        S = (q[b, :, h, :] @ k[b, :, kv, :].T) * scale
        S[mask] = -np.inf
        m = S.max(axis=1, keepdims=True)
        e = np.exp(S - m)
        l = e.sum(axis=1, keepdims=True)
        P = e / l
        lse[b, h] = (m + np.log(l))[:, 0]
        o[b, :, h, :] = prec.op(P) @ v[b, :, kv, :]

    _per_head(head, B, H)
    return o, lse


def attention_bwd(q, k, v, o, lse, do, prec: _Prec):
    """Backward of attention_fwd given dO (full precision). With P recomputed
    from lse: dP = dO V^T, D = rowsum(dO*O), dS = P*(dP - D),
    dq = scale dS k, dk = scale dS^T q, dv = P^T dO; dk and dv are summed over
    the query heads of each kv group, in head order."""
    B, T, H, hd = q.shape
    Hkv = k.shape[2]
    grp = H // Hkv
    scale = 1.0 / np.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dob = prec.op(do)

    def head(b, h):
        kv = h // grp
        S = (q[b, :, h, :] @ k[b, :, kv, :].T) * scale
        S[mask] = -np.inf
        P = np.exp(S - lse[b, h][:, None])
        dP = dob[b, :, h, :] @ v[b, :, kv, :].T
        D = np.sum(do[b, :, h, :] * o[b, :, h, :], axis=1)
        dS = prec.op(P * (dP - D[:, None]))
        dq[b, :, h, :] = (dS @ k[b, :, kv, :]) * scale
        return (dS.T @ q[b, :, h, :]) * scale, prec.op(P).T @ dob[b, :, h, :]

    parts = _per_head(head, B, H)
    for (b, h), (dkh, dvh) in zip([(b, h) for b in range(B) for h in range(H)], parts):
        dk[b, :, h // grp, :] += dkh
        dv[b, :, h // grp, :] += dvh
    return dq, dk, dv


def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def swiglu_fwd(g, u):
    return g * sigmoid(g) * u


def swiglu_bwd(g, u, da):
    """d/dg [g*sig(g)*u] = u*sig(g)*(1 + g*(1 - sig(g))); d/du = g*sig(g)."""
    s = sigmoid(g)
    return da * u * s * (1.0 + g * (1.0 - s)), da * g * s


def cross_entropy(z, targets):
    """Per-token loss = logsumexp(z) - z[target]; dz = (softmax(z) - onehot)/M
    for the mean over the M rows."""
    M = z.shape[0]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    rows = np.arange(M)
    loss = lse - z[rows, targets]
    dz = e / s
    dz[rows, targets] -= 1.0
    return loss, dz / M


def adamw(p, g, m, v, t, cfg: Config):
    """One decoupled-weight-decay Adam step at step count t >= 1:
    p <- p(1 - lr wd); m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
    p <- p - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)."""
    p = p * (1.0 - cfg.lr * cfg.weight_decay)
    m = cfg.beta1 * m + (1.0 - cfg.beta1) * g
    v = cfg.beta2 * v + (1.0 - cfg.beta2) * g * g
    mhat = m / (1.0 - cfg.beta1 ** t)
    vhat = v / (1.0 - cfg.beta2 ** t)
    p = p - cfg.lr * mhat / (np.sqrt(vhat) + cfg.adam_eps)
    return p, m, v


# ----------------------------------------------------------------------------
# Decoder block, head, full step
# ----------------------------------------------------------------------------

def _layer_weights(params, cfg, l):
    base = 1 + 9 * l
    return {n: params[base + i] for i, n in enumerate(LAYER_TENSORS)}


def layer_fwd(x, W, cfg: Config, prec: _Prec, rope, B, T):
    """One decoder block on x [M, d] (M = B*T tokens in (b, t) order)."""
    H, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    c = {"x": x}
    hn, c["r1"] = rmsnorm_fwd(x, W["attn_norm"], cfg.rms_eps)
    h = prec.op(hn)
    c["h"] = h
    q = (h @ prec.op(W["wq"]).T).reshape(B, T, H, hd)
    k = (h @ prec.op(W["wk"]).T).reshape(B, T, Hkv, hd)
    v = (h @ prec.op(W["wv"]).T).reshape(B, T, Hkv, hd)
    q = prec.op(rope_fwd(q, *rope))
    k = prec.op(rope_fwd(k, *rope))
    v = prec.op(v)
    c["q"], c["k"], c["v"] = q, k, v
    o, c["lse"] = attention_fwd(q, k, v, prec)
    c["o"] = o
    ob = prec.op(o.reshape(B * T, H * hd))
    c["ob"] = ob
    x1 = x + ob @ prec.op(W["wo"]).T
    c["x1"] = x1
    h2n, c["r2"] = rmsnorm_fwd(x1, W["mlp_norm"], cfg.rms_eps)
    h2 = prec.op(h2n)
    c["h2"] = h2
    gt = h2 @ prec.op(W["w_gate"]).T
    up = h2 @ prec.op(W["w_up"]).T
    c["gt"], c["up"] = gt, up
    a = prec.op(swiglu_fwd(gt, up))
    c["a"] = a
    return x1 + a @ prec.op(W["w_down"]).T, c


def layer_bwd(g, c, W, cfg: Config, prec: _Prec, rope, B, T):
    """Backward of layer_fwd: g = dL/d(block output). Returns dL/dx and the
    nine weight gradients."""
    H, Hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    dW = {}
    gb = prec.op(g)
    da = gb @ prec.op(W["w_down"])
    dW["w_down"] = gb.T @ c["a"]
    dgt, dup = swiglu_bwd(c["gt"], c["up"], da)
    dgt, dup = prec.op(dgt), prec.op(dup)
    dh2 = dgt @ prec.op(W["w_gate"]) + dup @ prec.op(W["w_up"])
    dW["w_gate"] = dgt.T @ c["h2"]
    dW["w_up"] = dup.T @ c["h2"]
    dx1, dW["mlp_norm"] = rmsnorm_bwd(c["x1"], W["mlp_norm"], c["r2"], dh2)
    g1 = g + dx1
    g1b = prec.op(g1)
    do = g1b @ prec.op(W["wo"])
    dW["wo"] = g1b.T @ c["ob"]
    dq, dk, dv = attention_bwd(c["q"], c["k"], c["v"], c["o"], c["lse"],
                               do.reshape(B, T, H, hd), prec)
    dq = prec.op(rope_bwd(dq, *rope).reshape(B * T, H * hd))
    dk = prec.op(rope_bwd(dk, *rope).reshape(B * T, Hkv * hd))
    dv = prec.op(dv.reshape(B * T, Hkv * hd))
    dh = dq @ prec.op(W["wq"]) + dk @ prec.op(W["wk"]) + dv @ prec.op(W["wv"])
    dW["wq"] = dq.T @ c["h"]
    dW["wk"] = dk.T @ c["h"]
    dW["wv"] = dv.T @ c["h"]
    dx, dW["attn_norm"] = rmsnorm_bwd(c["x"], W["attn_norm"], c["r1"], dh)
    return g1 + dx, dW


def head_fwd_bwd(x, w_norm, w_head, targets, cfg: Config, prec: _Prec):
    """Final RMSNorm, logits, mean cross-entropy and its backward.
    Returns (per-token loss [M], dL/dx, d final_norm, d lm_head)."""
    hn, r = rmsnorm_fwd(x, w_norm, cfg.rms_eps)
    hf = prec.op(hn)
    z = hf @ prec.op(w_head).T
    loss, dz = cross_entropy(z, targets)
    dzb = prec.op(dz)
    d_head = dzb.T @ hf
    dhf = dzb @ prec.op(w_head)
    dx, d_norm = rmsnorm_bwd(x, w_norm, r, dhf)
    return loss, dx, d_norm, d_head


def forward_loss(params, tokens, targets, cfg: Config, mode: str = "fp32"):
    """Mean loss and per-token loss [B, T] of the forward pass only."""
    prec = _Prec(mode)
    B, T = tokens.shape
    P = [np.asarray(p, dtype=np.float64) for p in params]
    rope = rope_tables(T, cfg.head_dim, cfg.rope_base)
    x = P[0][tokens.reshape(-1)]
    for l in range(cfg.n_layers):
        x, _ = layer_fwd(x, _layer_weights(P, cfg, l), cfg, prec, rope, B, T)
    hn, _ = rmsnorm_fwd(x, P[-2], cfg.rms_eps)
    z = prec.op(hn) @ prec.op(P[-1]).T
    loss, _ = cross_entropy(z, targets.reshape(-1))
    return float(loss.mean()), loss.reshape(B, T)


@dataclass
class StepResult:
    loss: float
    token_loss: np.ndarray           # [B, T], (b, t) order
    grads: list                      # raw dL/dp per tensor (float64)
    params: list                     # updated master values (fp32 values as float64)
    m: list
    v: list
    t: int
    checkpoints: list = field(default_factory=list)   # residual stream x_0..x_L


def gradients(params, tokens, targets, cfg: Config, mode: str = "fp32", progress=None):
    """Loss, per-token loss, gradients of every tensor, and the residual-stream
    checkpoints x_0..x_L, by the plain forward and analytic backward.
    progress: optional callable given a short text after each layer's
    forward and backward and after the head (for runs that take minutes)."""
    say = progress or (lambda text: None)
    prec = _Prec(mode)
    B, T = tokens.shape
    M = B * T
    P = [np.asarray(p, dtype=np.float64) for p in params]
    rope = rope_tables(T, cfg.head_dim, cfg.rope_base)
    tok = tokens.reshape(-1)
    x = P[0][tok]
    ckpts = [x]
    caches = []
    for l in range(cfg.n_layers):
        x, c = layer_fwd(x, _layer_weights(P, cfg, l), cfg, prec, rope, B, T)
        caches.append(c)
        ckpts.append(x)
        say(f"oracle {mode}: layer {l} forward")
    loss, g, d_fn, d_head = head_fwd_bwd(x, P[-2], P[-1], targets.reshape(-1), cfg, prec)
    say(f"oracle {mode}: head")
    grads = [None] * len(P)
    grads[-2], grads[-1] = d_fn, d_head
    for l in reversed(range(cfg.n_layers)):
        g, dW = layer_bwd(g, caches[l], _layer_weights(P, cfg, l), cfg, prec, rope, B, T)
        for i, n in enumerate(LAYER_TENSORS):
            grads[1 + 9 * l + i] = dW[n]
        say(f"oracle {mode}: layer {l} backward")
    dE = np.zeros_like(P[0])
    np.add.at(dE, tok, g)
    grads[0] = dE
    assert M == loss.shape[0]
    return float(loss.mean()), loss.reshape(B, T), grads, ckpts


def train_step(params, m, v, t, tokens, targets, cfg: Config, mode: str = "fp32") -> StepResult:
    """One full training step: forward, backward, then AdamW at step count
    t + 1 on every tensor. params/m/v are fp32 master values; the updated
    state is rounded back to fp32 (its storage precision)."""
    loss, tl, grads, ckpts = gradients(params, tokens, targets, cfg, mode)
    t1 = t + 1
    newp, newm, newv = [], [], []
    for p, g, mm, vv in zip(params, grads, m, v):
        p2, m2, v2 = adamw(np.asarray(p, np.float64), g, np.asarray(mm, np.float64),
                           np.asarray(vv, np.float64), t1, cfg)
        newp.append(fp32(p2))
        newm.append(fp32(m2))
        newv.append(fp32(v2))
    return StepResult(loss, tl, grads, newp, newm, newv, t1, ckpts)
