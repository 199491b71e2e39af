"""The host store's size against the figures the pages print
(tests/golden/host_memory_pages.txt): about 12 GB of host RAM per billion
parameters for the fp32 master weights and the two AdamW moments, and a
120B-parameter model trained within 1.5 TB of host RAM. CPU only: the library
sizes a configuration without allocating it."""
import os

import numpy as np
import pytest

from host_memory_streamed_amd import mt

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "host_memory_pages.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = float(v)
    return out


def _cfg(w, n_layers=None, dtype=mt.MT_BF16, flags=0):
    return mt.make_config(n_layers or w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_dim,
                          w.vocab, w.batch, w.seq, dtype=dtype, flags=flags)


def _params(cfg):
    return sum(int(np.prod(s)) for _, s in mt.tensor_table(cfg))


@pytest.mark.parametrize("name", ["1.3b", "14b", "7b-512k", "120b"])
def test_state_is_about_12_gb_per_billion_params(name):
    g = _golden()
    cfg = _cfg(mt.WORKLOADS[name])
    hb = mt.host_bytes(cfg)
    per_billion = hb["state"] / (_params(cfg) / 1e9) / 1e9
    # slabs pad each matrix group to 64 elements: a few parts per million
    assert abs(per_billion - g["gb_per_billion_params"]) <= 1e-3 * g["gb_per_billion_params"]


def test_headline_model_fits_the_headline_host_ram():
    # a 120B-parameter model's fp32 state at the same rate fits 1.5 TB; so
    # does the 120B-shaped workload at its full 88 layers (100.4B parameters)
    g = _golden()
    assert g["headline_params"] * g["gb_per_billion_params"] <= g["headline_host_ram_bytes"]
    cfg = _cfg(mt.WORKLOADS["120b"])
    hb = mt.host_bytes(cfg)
    assert hb["state"] <= g["headline_host_ram_bytes"]
    # everything the library holds in host memory for it, at the full depth
    assert hb["state"] <= hb["pinned"] + hb["pageable"] <= 1.2 * g["headline_host_ram_bytes"]


@pytest.mark.parametrize("dtype,flags", [(mt.MT_BF16, 0), (mt.MT_BF16, mt.MT_OVERLAP_OPT),
                                         (mt.MT_FP32, mt.MT_KEEP_GRADS)])
def test_host_bytes_accounts_every_array(dtype, flags):
    # the sum over arrays the host store keeps, from the tensor table alone:
    # p, m, v in fp32; the image (bf16 matrices, fp32 gains) of every layer
    # and the head in bf16 mode; kept gradients or the staging slots
    w = mt.WORKLOADS["1.3b"]
    cfg = _cfg(w, 3, dtype, flags)
    hb = mt.host_bytes(cfg)
    n = _params(cfg)
    n_emb = w.vocab * w.d_model
    assert hb["state"] >= 12 * n and hb["state"] - 12 * n <= 12 * 64 * (9 * 3 + 3)
    total = hb["pinned"] + hb["pageable"]
    image = 0 if dtype == mt.MT_FP32 else 2 * (n - n_emb)
    grads = 4 * n   # kept gradients, or the embedding's plus slots (checked below)
    assert total >= 12 * n + image + 4 * n_emb
    if flags & mt.MT_KEEP_GRADS:
        assert total >= 12 * n + image + grads
    M = w.batch * w.seq
    assert hb["parked_ckpt"] == M * w.d_model * 4


def test_host_bytes_rejects_bad_config():
    w = mt.WORKLOADS["1.3b"]
    cfg = _cfg(w)
    cfg.n_layer_buffers = 1
    with pytest.raises(mt.MTError):
        mt.host_bytes(cfg)
