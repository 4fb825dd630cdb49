"""3D rotary position embedding on video tokens, in float64.

Source: "Hy-Nomas: Towards Free-Form Interactive World Generation",
architecture table, position-encoding row (3D RoPE; 16, 56 and 56 of the
128 dimensions for t, h and w; theta 256) and section "Segment-Autoregressive
Diffusion Transformer" (3D RoPE encodes video positions); "Hy-Nomas Explained
...", Step 2 "Segment-wise causal joint attention" (RoPE rotates query and key
vectors by position; reference [16], RoFormer).

Readings (the pages print no formula):
* The 128 dimensions of a head are split into contiguous slices in the order
  t, h, w with widths (16, 56, 56), i.e. offsets (0, 16, 72).
* Inside a slice of width d, element pairs (2i, 2i+1), i < d/2, are rotated by
  the angle pos_axis * theta**(-2i/d), as in RoFormer's adjacent-pair form.
* Positions are integer, 0-based latent-grid coordinates; t is the global
  latent-frame index, so cached frames sit at earlier t.
* Text rows take no rotation (the pages say RoPE encodes video positions).
The convention itself is "parity unpinned": no rotated values are printed.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16


def rope_frequencies(width, theta):
    """theta**(-2i/width) for i = 0 .. width/2 - 1, in float64."""
    i = np.arange(width // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(width))


def rope3d(x, pos, theta=256.0, dims=(16, 56, 56)):
    """Rotate every head of every video row; exact float64 result.

    x   : float64 [n, H, D] (D = sum(dims))
    pos : int [n, 3] = (t, h, w)
    Returns float64 [n, H, D], not rounded.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n, nh, d = x.shape
    if sum(dims) != d or any(w % 2 for w in dims):
        raise ValueError("axis widths must be even and sum to the head dim")
    if pos.shape != (n, 3):
        raise ValueError("pos must be [n, 3]")
    out = np.array(x, copy=True)
    off = 0
    for axis, width in enumerate(dims):
        freq = rope_frequencies(width, theta)                  # [width/2]
        ang = pos[:, axis].astype(np.float64)[:, None] * freq[None, :]
        c = np.cos(ang)[:, None, :]                            # [n, 1, width/2]
        s = np.sin(ang)[:, None, :]
        x0 = x[:, :, off + 0:off + width:2]
        x1 = x[:, :, off + 1:off + width:2]
        out[:, :, off + 0:off + width:2] = x0 * c - x1 * s
        out[:, :, off + 1:off + width:2] = x0 * s + x1 * c
        off += width
    return out


def rope3d_bf16(x_bits, pos, theta=256.0, dims=(16, 56, 56)):
    """bf16 in, bf16 out: the exact rotation rounded once to bf16 (as float64)."""
    return round_to_bf16(rope3d(bf16_bits_to_f64(x_bits), pos, theta, dims))
