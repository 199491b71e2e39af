"""CPU oracle of the layer-streamed training step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. See ``decoder.py`` for what it computes.
"""
from .decoder import (Config, LAYER_TENSORS, StepResult, adamw, attention_bwd, attention_fwd,
                      bf16, cross_entropy, forward_loss, gradients, head_fwd_bwd, layer_bwd,
                      layer_fwd, rmsnorm_bwd, rmsnorm_fwd, rope_bwd, rope_fwd, rope_tables,
                      swiglu_bwd, swiglu_fwd, tensor_table, train_step)

__all__ = ["Config", "LAYER_TENSORS", "StepResult", "adamw", "attention_bwd", "attention_fwd",
           "bf16", "cross_entropy", "forward_loss", "gradients", "head_fwd_bwd", "layer_bwd",
           "layer_fwd", "rmsnorm_bwd", "rmsnorm_fwd", "rope_bwd", "rope_fwd", "rope_tables",
           "swiglu_bwd", "swiglu_fwd", "tensor_table", "train_step"]
