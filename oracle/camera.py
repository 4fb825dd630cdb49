"""Per-latent-frame camera cross-attention.

Source: model card, section "Text and Camera Conditioning" (the camera
extrinsics of four video frames form one 64-dimensional input per latent
frame; in each double-stream block, following its video MLP, the video tokens
cross-attend to the projected camera features, chunk by chunk, and a chunk of
one latent frame ties each frame's tokens to that frame's camera) and the
Explainer's camera-conditioning section.

Reading: video rows are grouped into chunks of `tokens_per_chunk` consecutive
rows (the latent frames of one camera chunk, raster order); chunk c owns
`t_cam` camera tokens, rows [c * t_cam, (c + 1) * t_cam) of the camera
keys/values (the pages' configuration: one token per latent frame, t_cam = 1).
Per head:
    o_i = sum_j softmax_j(sm_scale * q_i . k_j) v_j   over the chunk's tokens.
With t_cam = 1 the weight is exactly 1 and o_i = v of the row's chunk.

Pinned by brute-force loops, the t_cam = 1 closed form and identical keys
giving the mean of the values (tests/test_oracle_basic.py).
"""

import numpy as np


def camera_cross_attn(q, k_cam, v_cam, tokens_per_chunk, t_cam, sm_scale):
    """float64 [n, H, D] for q [n, H, D] and camera k/v [n_chunks * t_cam, H, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_cam, dtype=np.float64)
    v = np.asarray(v_cam, dtype=np.float64)
    n, h, d = q.shape
    out = np.empty_like(q)
    for c0 in range(0, n, tokens_per_chunk):
        c = c0 // tokens_per_chunk
        rows = slice(c0, min(n, c0 + tokens_per_chunk))
        kc, vc = k[c * t_cam:(c + 1) * t_cam], v[c * t_cam:(c + 1) * t_cam]   # [t_cam, H, D]
        s = sm_scale * np.einsum("nhd,thd->nht", q[rows], kc)
        s = s - s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=2, keepdims=True)
        out[rows] = np.einsum("nht,thd->nhd", p, vc)
    return out
