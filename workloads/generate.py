"""Seeded Q/K/V generation.

Recipe (the same for every configuration):
  * numpy Generator(PCG64(seed)); draw standard-normal float32 arrays in the
    order Q, K, V, each of shape [batch, heads, L, D] with tokens in original
    (t, h, w) row-major order.
  * For Q and K only, in heads that carry it, add to every channel the
    positional term  a * 2 * sum_{f in {1,2}} sin(f*pi*s + phi_head)  with
    s = t/T + h/H + w/W and phi_head = 2*pi*head/heads.
  * bf16 configurations round the float32 values to bf16 (round to nearest,
    ties to even).  Both the oracle and the GPU read exactly these values.

Nothing here computes any part of the attention method.
"""
import numpy as np

from .configs import Config


def positional_term(T: int, H: int, W: int, head: int, heads: int, amp: float) -> np.ndarray:
    """Positional term per token, shape [T*H*W], float64, original token order."""
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    h = np.arange(H, dtype=np.float64)[None, :, None] / H
    w = np.arange(W, dtype=np.float64)[None, None, :] / W
    s = (t + h + w).reshape(-1)
    phi = 2.0 * np.pi * head / heads
    return amp * 2.0 * (np.sin(np.pi * s + phi) + np.sin(2.0 * np.pi * s + phi))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE); returns the bf16 bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(cfg: Config, seed: int = None, batch: int = None, heads: int = None):
    """Return dict with 'q', 'k', 'v' as float32 arrays holding the exact input values
    (already bf16-rounded for bf16 configs) and, for bf16 configs, 'q_bits', 'k_bits',
    'v_bits' (uint16 bf16 patterns).  Shapes [batch, heads, L, D], original order.

    `batch`/`heads` may shrink the draw for quick tests; the head-class rule
    (local vs diffuse heads) and the phase phi_head keep using cfg.heads."""
    seed = cfg.seed if seed is None else seed
    B = cfg.batch if batch is None else batch
    nh = cfg.heads if heads is None else heads
    L, D = cfg.L, cfg.head_dim
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal((B, nh, L, D), dtype=np.float32)
        if name in ("q", "k"):
            for h in range(min(nh, cfg.n_local_heads())):
                pos = positional_term(cfg.T, cfg.H, cfg.W, h, cfg.heads, cfg.pos_amp)
                x[:, h] += pos.astype(np.float32)[None, :, None]
        if cfg.dtype == "bf16":
            bits = bf16_round(x)
            out[name + "_bits"] = bits
            x = bf16_bits_to_f32(bits)
        out[name] = x
    return out
