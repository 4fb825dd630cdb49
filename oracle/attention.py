"""Segment-wise causal joint attention over a KV cache plus the current segment.

Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
"Segment-Autoregressive Diffusion Transformer": one joint attention mixes the
text and video tokens of a block; each layer keeps the keys and values of the
segments already generated and reuses them; a segment's tokens see the
earlier segments (through that cache) and their own segment, and never a
later one. Architecture table: 16 heads of 128 dimensions. "Hy-Nomas Explained
...", Step 2 "Segment-wise causal joint attention": the same visibility rule,
earlier and current segments only.

The method computes exactly (up to rounding order) masked softmax attention,
so this is that definition in float64:

    s_ij  = sm_scale * q_i . k_j            for visible (i, j)
    p_ij  = exp(s_ij - m_i) / sum_j exp(s_ij - m_i),  m_i = max_j s_ij
    o_i   = sum_j p_ij v_j
    lse_i = m_i + ln sum_j exp(s_ij - m_i)

Keys are the selected history rows (video only, earlier than every segment)
followed by the current rows. Current rows are packed segments, each laid out
as [text (text_len rows) | video rows]. Readings where the pages are silent:

* inside a segment, text and video see each other fully (joint attention);
* the cache holds video tokens only: a query sees an earlier segment's video
  rows but not its text rows;
* every current query (text or video) sees every selected history row;
* text rows at index >= text_valid inside their segment are padding: no query
  sees them as keys (padded query rows are computed like any other row);
* a query never sees rows of a later segment.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np


@dataclass(frozen=True)
class Segment:
    start: int        # first row of the segment in the current sequence
    text_len: int     # text rows at the front of the segment
    text_valid: int   # text rows that are real tokens (<= text_len)


def _key_tags(n_hist, segments, n_cur):
    """Per key: segment (-1 = history), is_text, is_pad."""
    n_keys = n_hist + n_cur
    seg = np.full(n_keys, -1, dtype=np.int64)
    is_text = np.zeros(n_keys, dtype=bool)
    is_pad = np.zeros(n_keys, dtype=bool)
    bounds = [s.start for s in segments] + [n_cur]
    for si, s in enumerate(segments):
        a, b = n_hist + s.start, n_hist + bounds[si + 1]
        seg[a:b] = si
        is_text[a:a + s.text_len] = True
        is_pad[a + s.text_valid:a + s.text_len] = True
    return seg, is_text, is_pad


def _query_segments(segments, n_cur):
    qseg = np.empty(n_cur, dtype=np.int64)
    bounds = [s.start for s in segments] + [n_cur]
    for si in range(len(segments)):
        qseg[bounds[si]:bounds[si + 1]] = si
    return qseg


def _check_segments(segments, n_cur):
    if not segments or segments[0].start != 0:
        raise ValueError("segments must start at row 0")
    bounds = [s.start for s in segments] + [n_cur]
    for si, s in enumerate(segments):
        if not (0 <= s.text_valid <= s.text_len <= bounds[si + 1] - s.start):
            raise ValueError("bad segment %d" % si)


def visible_mask(n_hist, segments, n_cur, rows=None):
    """Boolean [len(rows), n_hist + n_cur]: may query row i see key j."""
    _check_segments(segments, n_cur)
    kseg, ktext, kpad = _key_tags(n_hist, segments, n_cur)
    qseg = _query_segments(segments, n_cur)
    if rows is not None:
        qseg = qseg[np.asarray(rows)]
    qs = qseg[:, None]
    hist = (kseg == -1)[None, :]
    same = (kseg[None, :] == qs) & ~kpad[None, :]
    earlier = (kseg[None, :] >= 0) & (kseg[None, :] < qs) & ~ktext[None, :]
    return hist | same | earlier


def history_keys(cache_k, cache_v, slots, k_scale=None, v_scale=None):
    """Gather the selected frames of a per-layer cache into key rows.

    cache_k/v : [n_slots, H, G, D] float64 values (BF16 cache) or int8 codes
                (INT8 cache, then k_scale/v_scale are [n_slots, H, G])
    slots     : selected slot indices, ascending in t
    Returns float64 (k, v), each [len(slots) * G, H, D]; INT8 entries are
    dequantised as code * scale.
    """
    slots = np.asarray(slots, dtype=np.int64)
    k = np.asarray(cache_k)[slots]
    v = np.asarray(cache_v)[slots]
    if k_scale is not None:
        k = k.astype(np.float64) * np.asarray(k_scale, np.float64)[slots][..., None]
        v = v.astype(np.float64) * np.asarray(v_scale, np.float64)[slots][..., None]
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, h, g, d = k.shape
    k = k.transpose(0, 2, 1, 3).reshape(n * g, h, d)
    v = v.transpose(0, 2, 1, 3).reshape(n * g, h, d)
    return k, v


def _one_head(qh, kh, vh, mask, sm_scale):
    s = sm_scale * (qh @ kh.T)
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    o = (e @ vh) / l
    return o, (m + np.log(l))[:, 0]


def joint_attn_rows(q, k, v, segments, rows, hist_k=None, hist_v=None,
                    sm_scale=1.0, chunk=1024, workers=None):
    """Attention for the listed query rows only.

    q, k, v     : float64 [n_cur, H, D] (current segment rows)
    hist_k/v    : float64 [n_hist, H, D] or None
    Returns (o float64 [len(rows), H, D], lse float64 [H, len(rows)]).
    """
    q = np.asarray(q, np.float64)
    n_cur, nh, d = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    if hist_k is not None and len(hist_k):
        keys = np.concatenate([hist_k, k], axis=0)
        vals = np.concatenate([hist_v, v], axis=0)
        n_hist = hist_k.shape[0]
    else:
        keys, vals, n_hist = np.asarray(k, np.float64), np.asarray(v, np.float64), 0
    o = np.empty((len(rows), nh, d))
    lse = np.empty((nh, len(rows)))
    jobs = [(h, c0) for h in range(nh) for c0 in range(0, len(rows), chunk)]
    kT = [np.ascontiguousarray(keys[:, h, :]) for h in range(nh)]
    vT = [np.ascontiguousarray(vals[:, h, :]) for h in range(nh)]

    def run(job):
        h, c0 = job
        r = rows[c0:c0 + chunk]
        mask = visible_mask(n_hist, segments, n_cur, rows=r)
        oh, lh = _one_head(q[r, h, :], kT[h], vT[h], mask, sm_scale)
        o[c0:c0 + len(r), h, :] = oh
        lse[h, c0:c0 + len(r)] = lh

    workers = workers or min(len(jobs), os.cpu_count() or 1)
    if workers <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, jobs))
    return o, lse


def joint_attn(q, k, v, segments, hist_k=None, hist_v=None, sm_scale=1.0,
               chunk=1024, workers=None):
    """Attention for every current query row: (o [n_cur, H, D], lse [H, n_cur])."""
    n_cur = np.asarray(q).shape[0]
    return joint_attn_rows(q, k, v, segments, np.arange(n_cur), hist_k, hist_v,
                           sm_scale, chunk, workers)
