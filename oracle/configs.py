"""The five workload shapes, as oracle Configs plus batch/sequence sizes
(test infrastructure only).

tiny    : 2 layers, d 64, 4 heads (hd 16), FFN 172, vocab 256, batch 2 x 32, fp32.
1.3B    : 24 layers, d 2048, 16 heads (hd 128), FFN 5632, vocab 32000, 4 x 2048.
14B     : 48 layers, d 5120, 40 q / 8 kv heads (hd 128), FFN 13824, vocab 152064, 1 x 4096.
7B-512k : 32 layers, d 4096, 32 heads (hd 128), FFN 11008, vocab 32000, 1 x 524288.
120B    : 88 layers (cut to fit host RAM), d 10240, 80 q / 8 kv heads (hd 128),
          FFN 28672, vocab 128000, 1 x 4096.
All: RMSNorm eps 1e-5, RoPE base 10000, AdamW lr 1e-3, betas (0.9, 0.999),
eps 1e-8, weight decay 0.01.
"""
from .decoder import Config

SHAPES = {
    "tiny": (Config(2, 64, 4, 4, 16, 172, 256), 2, 32),
    "1.3b": (Config(24, 2048, 16, 16, 128, 5632, 32000), 4, 2048),
    "14b": (Config(48, 5120, 40, 8, 128, 13824, 152064), 1, 4096),
    "7b-512k": (Config(32, 4096, 32, 32, 128, 11008, 32000), 1, 524288),
    "120b": (Config(88, 10240, 80, 8, 128, 28672, 128000), 1, 4096),
}


def shape(name: str, n_layers: int | None = None):
    """(Config, batch, seq) of a named workload, optionally with fewer layers."""
    cfg, B, T = SHAPES[name]
    if n_layers is not None:
        cfg = Config(**{**cfg.__dict__, "n_layers": n_layers})
    return cfg, B, T
