"""Gradients of segment-wise causal joint attention in the packed training form.

Source: "Hy-Nomas Explained: How Tencent's Open World Model Runs Steerable Video
on an RTX 4090", section "The training recipe" (fine-tuning trains the
autoregressive model with a segment-forcing pipeline on sequences packed
offline, up to 360,000 tokens); the attention it differentiates is the one of
`attention.py` (model card, section "Segment-Autoregressive Diffusion
Transformer"). Reading: in the packed form every segment of the sequence is
present, so there is no cache; the mask is the same segment-causal mask.

For a scalar loss L with upstream gradient do = dL/do, per head (plain
calculus of o_i = sum_j p_ij v_j, p_i = softmax_j(s_ij), s_ij = sm_scale q_i.k_j
over visible j):

    dv_j  = sum_i p_ij do_i
    dp_ij = do_i . v_j
    ds_ij = p_ij (dp_ij - D_i),          D_i = sum_j p_ij dp_ij = do_i . o_i
    dq_i  = sm_scale sum_j ds_ij k_j
    dk_j  = sm_scale sum_i ds_ij q_i

Pinned by central finite differences of L = sum(do * o) on tiny inputs and by
the invariants sum_j dv_j = sum_i do_i and dq = 0 when every visible key is the
same vector (tests/test_oracle_backward.py). `joint_attn_dq_rows` (dq of
selected query rows only, for sequences too long for the full gradient) is
pinned by finite differences on its own.
"""

import numpy as np

from .attention import Segment, visible_mask   # noqa: F401  (Segment re-exported for callers)


def joint_attn_backward(q, k, v, segments, do, sm_scale=1.0, chunk=512):
    """(dq, dk, dv), float64 [n, H, D], of L = sum(do * o) for the packed form.

    q, k, v, do : float64 [n, H, D] (post-RoPE q and k; no history)
    segments    : list of Segment covering rows [0, n)
    """
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    n, h, d = q.shape
    mask = visible_mask(0, segments, n)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for hd in range(h):
        qh, kh, vh, doh = q[:, hd], k[:, hd], v[:, hd], do[:, hd]
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            s = sm_scale * (qh[a:b] @ kh.T)
            s = np.where(mask[a:b], s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / np.sum(e, axis=1, keepdims=True)
            o = p @ vh
            dp = doh[a:b] @ vh.T
            big_d = np.sum(doh[a:b] * o, axis=1, keepdims=True)
            ds = p * (dp - big_d)
            dq[a:b, hd] = sm_scale * (ds @ kh)
            dk[:, hd] += sm_scale * (ds.T @ qh[a:b])
            dv[:, hd] += p.T @ doh[a:b]
    return dq, dk, dv


def joint_attn_dq_rows(q, k, v, segments, do, rows, sm_scale=1.0):
    """dq of the selected query rows, float64 [len(rows), H, D].

    Row i needs only its own softmax row: p_i over visible keys, o_i = p_i v,
    D_i = do_i . o_i, ds_i = p_i (v do_i - D_i), dq_i = sm_scale ds_i k.
    """
    q, do = np.asarray(q, dtype=np.float64), np.asarray(do, dtype=np.float64)
    k, v = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    n, h, d = q.shape
    mask = visible_mask(0, segments, n, rows=rows)
    out = np.zeros((len(rows), h, d))
    for hd in range(h):
        s = sm_scale * (q[rows, hd] @ k[:, hd].T)
        s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / np.sum(e, axis=1, keepdims=True)
        o = p @ v[:, hd]
        big_d = np.sum(do[rows, hd] * o, axis=1, keepdims=True)
        ds = p * (do[rows, hd] @ v[:, hd].T - big_d)
        out[:, hd] = sm_scale * (ds @ k[:, hd])
    return out
