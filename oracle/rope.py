"""Rotary position embedding in float64 (oracle; test infrastructure only).

The pages apply RoPE [RoFormer] to queries and keys ("MiniPIC: Flexible
Position-Independent Caching in <100LOC", §3.2.1 score equation, and §3.2.2
where each K element costs two fused multiply-adds after a cos/sin lookup).
They do not fix the pairing or the frequencies. The reading used here (the
Llama / NeoX convention, the one the 8B and 70B shapes use):

* frequencies theta_i = base^(-2 i / d) for i in [0, d/2);
* rotate-half pairing: element i is paired with element i + d/2, and the pair
  (a, b) at position p becomes (a cos(p theta_i) - b sin(p theta_i),
  b cos(p theta_i) + a sin(p theta_i)).

No rope scaling is applied: the workloads name only the base.
"""
import numpy as np


def inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i = 0 .. d/2-1, in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """Angle matrix p * theta_i, shape [len(pos), d/2], float64."""
    return np.asarray(pos, np.float64)[:, None] * inv_freq(head_dim, base)[None, :]


def rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Apply R_p to each row of x.

    x:   [n, ..., d] float64 (any number of middle axes, e.g. heads)
    pos: [n] positions
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = rope_angles(pos, d, base)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    a = x[..., :half]
    b = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = a * c - b * s
    out[..., half:] = b * c + a * s
    return out
