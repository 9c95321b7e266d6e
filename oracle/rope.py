"""Rotary position embedding in float64.

Summary, "前置知识 / RoPE": RoPE rotates queries and keys by an angle that
depends on absolute position, so the logit q_i k_j^T / sqrt(d) carries the
relative position; the pre-RoPE query is the unrotated vector.  Paper text,
§4.3 "Query Construction and Alignment": beacon queries are rotated to the
current decoding step t, recent queries to their own generation positions.

The pages fix neither the pairing of coordinates nor the frequencies.  The
reading taken here is the rotate-half convention of the Qwen models the
workloads are shaped after: coordinate i pairs with i + d/2, and pair i
turns at omega_i = theta ** (-2 i / d) radians per position.
"""

import numpy as np


def rope_freqs(d, theta):
    """omega_i = theta ** (-2 i / d) for i in [0, d/2), float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope(x, pos, theta):
    """Rotate x[..., d] to position(s) pos (broadcast over x's leading axes).

    For pair i with angle a = pos * omega_i:
        x'_i       = x_i cos a - x_{i+d/2} sin a
        x'_{i+d/2} = x_{i+d/2} cos a + x_i sin a
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    omega = rope_freqs(d, theta)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * omega
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
