"""Fixed bf16-mode tolerances of the GPU step tests, derived from the oracle alone.

A bf16 step on the GPU and the oracle's plain bf16 reading are two
implementations of the same rounded arithmetic. Each lies some distance
delta from the exact step (the oracle in float64), so by the triangle
inequality they lie within about 2 delta of each other. The bounds below are
at least twice the largest distance the oracle itself shows between its bf16
reading and its float64 step on the cases of each depth class
(``golden/bf16_distance.py`` measures them; ``golden/bf16_distance.json``
holds the record; ``test_bf16_tolerances.py`` checks that every bound still
covers twice the record).

For each quantity a triple (tau, gamma, rho), a row being one output unit
(one row of a weight; the whole vector for gains and the per-token losses):

* normwise over the tensor: ||gpu - ref|| <= tau ||ref||;
* elementwise, on each row's own scale: |gpu - ref| <= gamma rms(row) for
  all but 0.1% of the elements;
* normwise over each row: ||gpu_row - ref_row|| <= rho ||ref_row||.

No bound is put on the single largest elementwise deviation: over millions
of elements it is an extreme value of the rounding noise (the largest of two
implementations' deviations land on different elements), so it grows with
the tensor's size, while a wrong row or tile shows in the row bound.

Quantities: "grad <kind>", "m <kind>" and "sqrt v <kind>" (the moments are
linear in the gradient at a first step, so they share the gradient's
bounds), "param <kind>" (the updated parameters) for the nine layer kinds
and tok_emb, final_norm, lm_head; "loss" (relative, tau only) and
"token_loss".

Classes: "narrow" (1-6 layers, d_model up to 2048), "wide" (2-3 layers at
d_model 4096 to 10240: the 7B, 14B and 120B layer shapes, where the oracle's
own bf16 reading lies about twice as far from float64 as at the narrow
shapes) and "deep" (24 layers).
"""
from __future__ import annotations

import math

# kind groups sharing one bound
ATTN_IN = ("wq", "wk")                       # gradients through the attention scores
MATS = ("wv", "wo", "w_gate", "w_up", "w_down")
GAINS = ("attn_norm", "mlp_norm")
HEAD = ("final_norm", "lm_head")
EMB = ("tok_emb",)

# (tau, gamma, rho) per group and class: tolerances.derive() of the record,
# written out
BF16 = {
    "narrow": {
        "loss": (0.0002, 0.0, 0.0),
        "token_loss": (0.003, 0.01, 0.003),
        "grad attn_in": (0.059, 0.75, 0.488),
        "grad mats": (0.027, 0.31, 0.211),
        "grad gains": (0.029, 0.16, 0.029),
        "grad head": (0.021, 0.07, 0.028),
        "grad emb": (0.026, 0.09, 0.031),
        "param mats": (0.016, 0.21, 0.032),
        "param gains": (0.001, 0.01, 0.001),
        "param head": (0.008, 0.16, 0.018),
        "param emb": (0.013, 0.21, 0.02),
    },
    "wide": {
        "loss": (0.0003, 0.0, 0.0),
        "token_loss": (0.006, 0.02, 0.006),
        "grad attn_in": (0.117, 0.4, 0.169),
        "grad mats": (0.087, 0.3, 0.132),
        "grad gains": (0.113, 0.37, 0.113),
        "grad head": (0.042, 0.39, 0.341),
        "grad emb": (0.081, 0.27, 0.124),
        "param mats": (0.028, 0.21, 0.033),
        "param gains": (0.001, 0.01, 0.001),
        "param head": (0.016, 0.2, 0.034),
        "param emb": (0.023, 0.21, 0.027),
    },
    "deep": {
        "loss": (0.0003, 0.0, 0.0),
        "token_loss": (0.004, 0.01, 0.004),
        "grad attn_in": (0.076, 0.38, 0.328),
        "grad mats": (0.063, 0.76, 1.002),
        "grad gains": (0.065, 0.34, 0.065),
        "grad head": (0.04, 0.14, 0.061),
        "grad emb": (0.064, 0.22, 0.077),
        "param mats": (0.022, 0.21, 0.077),
        "param gains": (0.001, 0.01, 0.001),
        "param head": (0.01, 0.19, 0.022),
        "param emb": (0.021, 0.21, 0.027),
    },
}


def group_of(kind: str) -> str:
    for name, members in (("attn_in", ATTN_IN), ("mats", MATS), ("gains", GAINS), ("head", HEAD),
                          ("emb", EMB)):
        if kind in members:
            return name
    raise KeyError(kind)


def key_of(quantity: str) -> str:
    """Table key of a quantity name ("grad wq", "sqrt v lm_head", "loss", ...)."""
    if quantity in ("loss", "token_loss"):
        return quantity
    what, kind = quantity.rsplit(" ", 1)
    what = "grad" if what in ("grad", "m", "sqrt v") else what
    if what == "param" and group_of(kind) == "attn_in":
        return "param mats"
    return f"{what} {group_of(kind)}"


def bf16_tol(depth: str, quantity: str):
    return BF16[depth][key_of(quantity)]


def derive(record: dict) -> dict:
    """Twice the largest recorded distance per table key and depth class,
    rounded up (tau and rho to 3 decimals, the loss to 1e-4, gamma to 2)."""
    out: dict = {}
    for case in record.values():
        cls = case["class"]
        for q, d in case["kinds"].items():
            k = key_of(q)
            cur = out.setdefault(cls, {}).setdefault(k, [0.0, 0.0, 0.0])
            cur[0] = max(cur[0], 2 * d["norm"])
            cur[1] = max(cur[1], 2 * d["elem_q999"])
            cur[2] = max(cur[2], 2 * d["row_max"])
    for cls in out.values():
        for k, v in cls.items():
            step = 1e-4 if k == "loss" else 1e-3
            cls[k] = (round(math.ceil(v[0] / step - 1e-9) * step, 6), math.ceil(v[1] * 100 - 1e-9) / 100,
                      round(math.ceil(v[2] / step - 1e-9) * step, 6))
    return out
