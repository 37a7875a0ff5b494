"""The five workload configurations (sizes, thresholds, input recipe).

Shapes follow the video latents the pages measure on: a tiny fp32 case, a
small bf16 case, a Wan2.1-scale case (81 frames at 720p -> 21 latent frames
of 32x48 tokens) and two HunyuanVideo-scale cases (129 frames -> 33 latent
frames of 48x80 tokens), one of them with the static sliding-tile window
unioned into the adaptive mask (NABLA page, Metodologia item 3).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    heads: int
    T: int
    H: int
    W: int
    head_dim: int
    patch: int            # P: fractal patch side
    block: int            # N: tokens per block (N = P*P in every config)
    thr: float
    window: Optional[Tuple[int, int, int]]   # (win_t, win_h, win_w) in tiles, or None
    pos_amp: float        # a: amplitude multiplier of the positional term
    local_heads: Optional[int] = None        # heads [0, local_heads) carry the term; rest pure N(0,1)
    seed: int = 0

    @property
    def L(self) -> int:
        return self.T * self.H * self.W

    @property
    def S(self) -> int:
        return self.L // self.block

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.S

    @property
    def dense_flops(self) -> float:
        return 4.0 * self.batch * self.heads * float(self.L) ** 2 * self.head_dim

    def n_local_heads(self) -> int:
        return self.heads if self.local_heads is None else self.local_heads


_BASE_SEED = 20261203

CONFIGS = [
    Config(0, "tiny-fp32", "f32", 1, 4, 4, 16, 16, 64, 8, 64, 0.1, None, 1.0,
           seed=_BASE_SEED + 0),
    Config(1, "small-bf16", "bf16", 1, 8, 8, 32, 32, 128, 8, 64, 0.2, None, 3.0,
           seed=_BASE_SEED + 1),
    Config(2, "wan21-bf16", "bf16", 1, 40, 21, 32, 48, 128, 8, 64, 0.1, None, 3.0,
           seed=_BASE_SEED + 2),
    Config(3, "hunyuan-bf16", "bf16", 1, 24, 33, 48, 80, 128, 8, 64, 0.05, None, 4.0,
           local_heads=17, seed=_BASE_SEED + 3),
    Config(4, "hunyuan-hybrid-bf16", "bf16", 2, 24, 33, 48, 80, 128, 8, 64, 0.1, (1, 1, 1), 4.0,
           local_heads=17, seed=_BASE_SEED + 4),
]


def get_config(i: int) -> Config:
    return CONFIGS[i]
