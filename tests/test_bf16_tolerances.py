"""The fixed bf16 tolerances of the GPU step tests (``tolerances.py``) cover
twice the oracle's own distance between its bf16 reading and its float64
step on every recorded case of their depth class (the record is written by
``golden/bf16_distance.py``, which calls only the oracle)."""
import json
import os

import pytest

import tolerances as T

HERE = os.path.dirname(os.path.abspath(__file__))
RECORD = os.path.join(HERE, "golden", "bf16_distance.json")


def _record():
    with open(RECORD) as f:
        return json.load(f)


def test_record_covers_every_case_and_class():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bf16_distance", os.path.join(HERE, "golden", "bf16_distance.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    rec = _record()
    assert set(rec) == set(mod.CASES)
    for name, (cls, cfg, B, T_, seed, std, steps) in mod.CASES.items():
        r = rec[name]
        assert (r["class"], r["layers"], r["d_model"], r["B"], r["T"], r["seed"], r["std"], r["steps"]) == \
            (cls, cfg.n_layers, cfg.d_model, B, T_, seed, std, steps), name
    assert {r["class"] for r in rec.values()} == set(T.BF16)


@pytest.mark.parametrize("case", sorted(_record()))
def test_tolerance_is_twice_the_oracle_distance(case):
    r = _record()[case]
    table = T.BF16[r["class"]]
    for q, d in r["kinds"].items():
        tau, gamma, rho = table[T.key_of(q)]
        assert tau >= 2 * d["norm"] - 1e-12, (q, tau, d["norm"])
        if q != "loss":
            assert gamma >= 2 * d["elem_q999"] - 1e-12, (q, gamma, d["elem_q999"])
            assert rho >= 2 * d["row_max"] - 1e-12, (q, rho, d["row_max"])


def test_table_is_the_derivation():
    """No bound is looser than the derivation rounds to (the table is the
    derivation, written out once)."""
    derived = T.derive(_record())
    for cls, rows in derived.items():
        for k, v in rows.items():
            got = T.BF16[cls][k]
            assert all(abs(a - b) <= 1e-9 for a, b in zip(got, v)), (cls, k, got, v)


def test_every_tensor_kind_has_a_bound():
    kinds = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down", "tok_emb",
             "final_norm", "lm_head")
    for cls in T.BF16:
        for k in kinds:
            for what in ("grad", "m", "sqrt v", "param"):
                assert len(T.bf16_tol(cls, f"{what} {k}")) == 3
        T.bf16_tol(cls, "loss")
        T.bf16_tol(cls, "token_loss")
