"""Distance of the oracle's bf16 reading from its own float64 step.

Writes ``tests/golden/bf16_distance.json``. Calls only ``oracle`` and the
seeded input generator (``host_memory_streamed_amd.synth``); nothing here
comes from the HIP library.

Why: the bf16 tolerances of the GPU step tests are fixed numbers derived from
this measurement. A bf16 step (GPU) and the oracle's bf16 reading are two
implementations of the same rounded arithmetic, each some distance delta from
the exact (float64) step; by the triangle inequality they lie within about
2 delta of each other. For every case, tensor by tensor, this script records

* ``norm``: ||bf16 - exact|| / ||exact||;
* ``row_max``: the largest ||bf16 - exact|| / ||exact|| over the rows (a row
  is one output unit of a weight; the whole vector for gains and the
  per-token losses);
* ``elem_q999`` and ``elem_max``: the 99.9th-percentile and the largest
  elementwise |bf16 - exact| / rms(row of exact);

reduced to the maximum over the layers for each tensor kind. The embedding
is measured on the rows of the step's tokens (the other rows are exactly 0).

Cases are the shapes of the GPU step tests, in three classes: "narrow" (1-6
layers, d_model up to 2048), "wide" (2-3 layers at the 7B, 14B and 120B
widths, d_model 4096 to 10240: the oracle's own bf16 reading lies about
twice as far from float64 there) and "deep" (24 layers).

Usage: ``python tests/golden/bf16_distance.py [case ...]`` (default: every
case whose result is missing); ``--all`` re-measures every case; ``--out
PATH`` records into another file (merged by hand into the record). The
14B- and 120B-shaped cases need about 100 and 200 GB of host memory.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from oracle.configs import shape  # noqa: E402
from host_memory_streamed_amd import synth  # noqa: E402

OUT = os.path.join(HERE, "bf16_distance.json")


def _cfg(name, n_layers=None, **over):
    cfg, _, _ = shape(name, n_layers)
    return O.Config(**{**cfg.__dict__, **over})


# name: (class, config, B, T, seed, std, steps)
CASES = {
    "gqa_ragged": ("narrow", O.Config(2, 256, 4, 2, 64, 344, 1000), 2, 100, 7, 0.05, 2),
    "hd128": ("narrow", O.Config(2, 256, 2, 1, 128, 512, 512), 1, 200, 9, 0.05, 1),
    "chunks_parked": ("narrow", O.Config(5, 128, 2, 1, 64, 200, 300), 2, 48, 19, 0.05, 2),
    "smaller_than_alloc": ("narrow", O.Config(2, 128, 2, 1, 64, 200, 300), 2, 45, 31, 0.05, 1),
    "ring_recycle": ("narrow", O.Config(6, 128, 2, 1, 64, 200, 300), 2, 32, 37, 0.05, 3),
    "1.3b_2l_256": ("narrow", _cfg("1.3b", 2), 1, 256, 11, 0.02, 1),
    "1.3b_2l_4x2048": ("narrow", _cfg("1.3b", 2), 4, 2048, 41, 0.02, 2),
    "7b_3l_8192": ("wide", _cfg("7b-512k", 3), 1, 8192, 43, 0.02, 1),
    "14b_2l_4096": ("wide", _cfg("14b", 2), 1, 4096, 13, 0.02, 1),
    "120b_2l_512": ("wide", _cfg("120b", 2), 1, 512, 17, 0.02, 1),
    "1.3b_24l_96": ("deep", _cfg("1.3b"), 1, 96, 31, 0.02, 1),
}


# measured through measure_grads (host memory)
BIG = {"1.3b_24l_96", "7b_3l_8192", "14b_2l_4096", "120b_2l_512"}


def _params(cfg, seed, std):
    return [synth.init_tensor(seed, i, shp, gain, std) for i, (_, shp, gain) in enumerate(O.tensor_table(cfg))]


def _dist(b, e):
    """(norm, elem_max, elem_q999, row_max) of b against e, rows of e."""
    b = np.asarray(b, np.float64)
    e = np.asarray(e, np.float64)
    n = float(np.linalg.norm(b - e) / (np.linalg.norm(e) + 1e-300))
    e2 = e.reshape(e.shape[0], -1) if e.ndim > 1 else e.reshape(1, -1)
    diff = b.reshape(e2.shape) - e2
    rn = np.sqrt(np.sum(np.square(e2), axis=1))
    dn = np.sqrt(np.sum(np.square(diff), axis=1))
    row = float(np.max(dn[rn > 0] / rn[rn > 0])) if np.any(rn > 0) else 0.0
    rms = (rn / np.sqrt(e2.shape[1]))[:, None] + 1e-300
    r = (np.abs(diff) / rms).reshape(-1)
    return n, float(r.max()), float(np.quantile(r, 0.999)), row


def _kind(name):
    return name.split(".")[-1]


def _merge(acc, key, d):
    old = acc.get(key)
    acc[key] = list(d) if old is None else [max(a, b) for a, b in zip(old, d)]


def measure_grads(case):
    """Single-step cases too large for two whole oracle steps side by side:
    the exact gradients are kept in fp32 (ample for distances of order 1e-2)
    while the bf16 reading runs, and the first AdamW step is then taken one
    tensor at a time on both sides (from zero moments, as train_step does)."""
    cls, cfg, B, T, seed, std, steps = CASES[case]
    assert steps == 1
    params = _params(cfg, seed, std)
    table = O.tensor_table(cfg)
    tokens, targets = synth.token_batch(seed, B, T, cfg.vocab)
    rows = np.unique(tokens)
    say = lambda text: print(f"  {case}: {text}", flush=True)
    loss, tl, grads, _ = O.gradients(params, tokens, targets, cfg, "fp32", progress=say)
    ex = [(g[rows] if i == 0 else g).astype(np.float32) for i, g in enumerate(grads)]
    del grads
    bl, btl, grads, _ = O.gradients(params, tokens, targets, cfg, "bf16", progress=say)
    acc = {}
    _merge(acc, "loss", (abs(bl - loss) / abs(loss), 0.0, 0.0, 0.0))
    _merge(acc, "token_loss", _dist(btl.reshape(-1), tl.reshape(-1)))
    for i, (name, _, _) in enumerate(table):
        k = _kind(name)
        g = grads[i][rows] if i == 0 else grads[i]
        p0 = np.asarray(params[i][rows] if i == 0 else params[i], np.float64)
        _merge(acc, "grad " + k, _dist(g, ex[i]))
        z = np.zeros_like(p0)
        pb, mb, vb = (O.decoder.fp32(a) for a in O.adamw(p0, g, z, z, 1, cfg))
        pe, me, ve = (O.decoder.fp32(a) for a in O.adamw(p0, ex[i].astype(np.float64), z, z, 1, cfg))
        _merge(acc, "param " + k, _dist(pb, pe))
        _merge(acc, "m " + k, _dist(mb, me))
        _merge(acc, "sqrt v " + k, _dist(np.sqrt(vb), np.sqrt(ve)))
        grads[i] = ex[i] = None
        say(f"compared {name}")
    return acc


def measure(case):
    cls, cfg, B, T, seed, std, steps = CASES[case]
    if case in BIG:
        acc = measure_grads(case)
        return {"class": cls, "layers": cfg.n_layers, "d_model": cfg.d_model, "B": B, "T": T, "seed": seed,
                "std": std, "steps": steps, "grads_only": True,
                "kinds": {k: {"norm": v[0], "elem_max": v[1], "elem_q999": v[2], "row_max": v[3]}
                      for k, v in sorted(acc.items())}}
    params = _params(cfg, seed, std)
    zeros = [np.zeros_like(p) for p in params]
    table = O.tensor_table(cfg)
    acc = {}
    P, Mm, Vv, t = params, zeros, zeros, 0
    for s in range(steps):
        tokens, targets = synth.token_batch(seed + 10 * s, B, T, cfg.vocab)
        ex = O.train_step(P, Mm, Vv, t, tokens, targets, cfg, "fp32")
        bf = O.train_step(P, Mm, Vv, t, tokens, targets, cfg, "bf16")
        _merge(acc, "loss", (abs(bf.loss - ex.loss) / abs(ex.loss), 0.0, 0.0, 0.0))
        _merge(acc, "token_loss", _dist(bf.token_loss.reshape(-1), ex.token_loss.reshape(-1)))
        rows = np.unique(tokens)
        for i, (name, _, _) in enumerate(table):
            sel = rows if i == 0 else slice(None)
            k = _kind(name)
            _merge(acc, "grad " + k, _dist(bf.grads[i][sel], ex.grads[i][sel]))
            _merge(acc, "param " + k, _dist(bf.params[i][sel], ex.params[i][sel]))
            _merge(acc, "m " + k, _dist(bf.m[i][sel], ex.m[i][sel]))
            _merge(acc, "sqrt v " + k, _dist(np.sqrt(bf.v[i][sel]), np.sqrt(ex.v[i][sel])))
        # the next step starts both readings from the exact step's state
        P, Mm, Vv, t = ex.params, ex.m, ex.v, ex.t
    return {"class": cls, "layers": cfg.n_layers, "d_model": cfg.d_model, "B": B, "T": T, "seed": seed,
            "std": std, "steps": steps,
            "kinds": {k: {"norm": v[0], "elem_max": v[1], "elem_q999": v[2], "row_max": v[3]}
                      for k, v in sorted(acc.items())}}


def _load():
    return json.load(open(OUT)) if os.path.exists(OUT) else {}


def main(argv):
    global OUT
    if "--out" in argv:
        i = argv.index("--out")
        OUT = os.path.abspath(argv[i + 1])
        argv = argv[:i] + argv[i + 2:]
    names = [a for a in argv if not a.startswith("--")]
    if not names:
        done = _load()
        names = list(CASES) if "--all" in argv else [c for c in CASES if c not in done]
    for c in names:
        t0 = time.time()
        r = measure(c)
        r["seconds"] = round(time.time() - t0, 1)
        print(f"{c}: {r['seconds']} s", flush=True)
        # re-read before writing: other runs may have recorded other cases meanwhile
        data = _load()
        data[c] = r
        data = {k: v for k, v in data.items() if k in CASES}
        with open(OUT + ".tmp", "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        os.replace(OUT + ".tmp", OUT)


if __name__ == "__main__":
    main(sys.argv[1:])
