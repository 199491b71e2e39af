"""The streamed step at each workload's own layer shape and sequence length,
against the CPU oracle (float64; bf16 operands rounded where the oracle's
plain reading rounds them).

The oracle computes the whole step's gradients at these sizes; every
gradient tensor is compared in full. AdamW is an elementwise map, so the
updated parameters and moments are compared on 65536 sampled elements per
tensor (all of them below that), with the oracle's own AdamW taken on those
elements. Depth is reduced to two or three layers where a full-depth oracle step is
out of reach (the per-layer shape, the vocabulary and the sequence length
are the workload's):

* 1.3B: 2 layers, 4 x 2048 tokens, 3 AdamW steps, fp32 and bf16; plus the
  full 24 layers streamed against fully resident, bitwise, at 4 x 2048;
* 14B-shaped: 2 layers, 1 x 4096 tokens, vocabulary 152064, bf16;
* 7B long-context: 3 layers (the fewest with a checkpoint that can be
  parked), 1 x 8192 tokens, bf16, with the QKV projection and the MLP in
  token chunks and a residual checkpoint parked in host memory, so those
  paths run at d 4096;
* 120B-shaped: 2 layers of d 10240 / 80 q heads / 8 kv heads / FFN 28672,
  vocabulary 128000, 1 x 512 tokens.
"""
import numpy as np
import pytest

from oracle.configs import shape
from test_gpu_step import init_params, make_ctx, run_parity_sampled

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from host_memory_streamed_amd import mt, synth  # noqa: E402

@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_1p3b_two_layers_4x2048_three_steps(mode):
    cfg, B, T = shape("1.3b", n_layers=2)
    run_parity_sampled(cfg, B, T, mode, steps=3, seed=41)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
def test_1p3b_full_depth_streamed_equals_resident(dtype):
    """All 24 layers at 4 x 2048 tokens: two steps streamed through two
    buffers and with every unit resident give the same bits."""
    cfg, B, T = shape("1.3b")
    params = init_params(cfg, 5)
    out = []
    for buffers in (2, cfg.n_layers + 1):
        with make_ctx(cfg, B, T, params, dtype=dtype, flags=mt.MT_OVERLAP_OPT, buffers=buffers) as ctx:
            losses = []
            for s in range(2):
                tok, tgt = synth.token_batch(5 + s, B, T, cfg.vocab)
                losses.append(ctx.train_step(tok, tgt))
            ctx.sync()
            tl = ctx.token_losses().copy()
            # every tensor of the first and last layers, the head and the embedding
            ids = [0] + list(range(1, 10)) + list(range(1 + 9 * (cfg.n_layers - 1), 3 + 9 * cfg.n_layers))
            state = [ctx.params(i) for i in ids] + [ctx.opt_state(i)[1] for i in ids]
            out.append((losses, tl, state))
    (l0, t0, s0), (l1, t1, s1) = out
    assert l0 == l1
    np.testing.assert_array_equal(t0, t1)
    for a, b in zip(s0, s1):
        np.testing.assert_array_equal(a, b)


@pytest.mark.timeout(600)
def test_14b_two_layers_4096_full_vocab_bf16():
    cfg, B, T = shape("14b", n_layers=2)
    run_parity_sampled(cfg, B, T, "bf16", seed=13, depth="wide")


@pytest.mark.timeout(600)
def test_7b_three_layers_8192_chunked_parked_bf16():
    cfg, _, _ = shape("7b-512k", n_layers=3)
    # three layers so that one residual checkpoint can be parked (x_1); the
    # QKV projection and the MLP run in chunks of 3000 rows (3000, 3000, 2192)
    run_parity_sampled(cfg, 1, 8192, "bf16", seed=43, depth="wide", chunk_rows=3000, ckpt_host=1)


@pytest.mark.timeout(600)
def test_120b_layer_shape_two_layers_bf16():
    cfg, _, _ = shape("120b", n_layers=2)
    run_parity_sampled(cfg, 1, 512, "bf16", seed=17, depth="wide")
