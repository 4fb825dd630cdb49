"""Pins for the oracle's segment-causal joint attention (CPU only).

Brute force with explicit per-(i, j) Python loops on tiny inputs, closed
forms, invariants (rows sum to 1, causality, cache == recompute, INT8
round-trip bound) and a library special case (torch SDPA in float64).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import Segment
import workloads
from workloads import HEAD_DIM

TINY = ["c0", "c0_int8", "c0_win3", "c0_pad", "c0_packed3"]


def _f(b):
    return oracle.bf16_bits_to_f64(b)


def oracle_chain(inp):
    """Oracle end-to-end chain from pre-RoPE inputs (the reference result)."""
    cfg = inp.cfg
    q = _f(inp.q)
    k = _f(inp.k)
    v = _f(inp.v)
    k[inp.video_rows] = oracle.rope3d_bf16(inp.k[inp.video_rows], inp.pos)
    q[inp.video_rows] = oracle.rope3d_bf16(inp.q[inp.video_rows], inp.pos)
    segs = [Segment(*s) for s in inp.segments]
    hk = hv = None
    if len(cfg.hist_t):
        g = cfg.tokens_per_frame
        kr = oracle.rope3d_bf16(inp.hist_k, inp.hist_pos)            # [F*G, H, D]
        vr = _f(inp.hist_v)
        nf = len(cfg.hist_t)
        ck = kr.reshape(nf, g, cfg.n_heads, HEAD_DIM).transpose(0, 2, 1, 3)
        cv = vr.reshape(nf, g, cfg.n_heads, HEAD_DIM).transpose(0, 2, 1, 3)
        slots = oracle.window_select(inp.slot_t, cfg.window)
        if cfg.cache_dtype == "int8":
            kc, ks = oracle.quantise_int8(ck)
            vc, vs = oracle.quantise_int8(cv)
            hk, hv = oracle.history_keys(kc, vc, slots, ks, vs)
        else:
            hk, hv = oracle.history_keys(ck, cv, slots)
    return q, k, v, segs, hk, hv


# ----------------------------------------------------- brute force loops ----

def _brute(q, k, v, segs, hk, hv, sm_scale):
    """Per-(head, i, j) Python loops, written from the definition."""
    n_cur, nh, d = q.shape
    n_hist = 0 if hk is None else hk.shape[0]
    bounds = [s.start for s in segs] + [n_cur]

    def seg_of(r):
        for si in range(len(segs)):
            if bounds[si] <= r < bounds[si + 1]:
                return si
        raise AssertionError

    def visible(i, j):
        if j < n_hist:
            return True
        jc = j - n_hist
        si, sj = seg_of(i), seg_of(jc)
        text_idx = jc - segs[sj].start
        is_text = text_idx < segs[sj].text_len
        if sj > si:
            return False
        if sj == si:
            return (not is_text) or text_idx < segs[sj].text_valid
        return not is_text

    keys = [hk[j] for j in range(n_hist)] + [k[j] for j in range(n_cur)]
    vals = [hv[j] for j in range(n_hist)] + [v[j] for j in range(n_cur)]
    o = np.zeros_like(q)
    lse = np.zeros((nh, n_cur))
    for h in range(nh):
        for i in range(n_cur):
            js = [j for j in range(len(keys)) if visible(i, j)]
            s = [sm_scale * sum(q[i, h, e] * keys[j][h, e] for e in range(d)) for j in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for e in range(d):
                o[i, h, e] = sum(wj * vals[j][h, e] for wj, j in zip(w, js)) / tot
            lse[h, i] = m + math.log(tot)
    return o, lse


@pytest.mark.parametrize("name", ["c0", "c0_pad", "c0_packed3", "c0_int8"])
def test_brute_force_tiny(name):
    inp = workloads.make_inputs(name)
    q, k, v, segs, hk, hv = oracle_chain(inp)
    # brute force over a subset of heads/rows keeps the pure-Python loops short
    o, lse = oracle.joint_attn(q, k, v, segs, hk, hv, inp.cfg.sm_scale)
    rows = np.arange(0, q.shape[0], 7)
    qs = q[:, :1]
    ob, lb = _brute(qs, k[:, :1], v[:, :1], segs,
                    None if hk is None else hk[:, :1], None if hv is None else hv[:, :1],
                    inp.cfg.sm_scale)
    assert np.max(np.abs(ob[rows] - o[rows, :1])) < 1e-12
    assert np.max(np.abs(lb[0, rows] - lse[0, rows])) < 1e-12


def test_brute_force_window3():
    inp = workloads.make_inputs("c0_win3")
    q, k, v, segs, hk, hv = oracle_chain(inp)
    assert hk.shape[0] == 3 * inp.cfg.tokens_per_frame
    o, lse = oracle.joint_attn(q, k, v, segs, hk, hv, inp.cfg.sm_scale)
    ob, lb = _brute(q[:, 1:], k[:, 1:], v[:, 1:], segs, hk[:, 1:], hv[:, 1:], inp.cfg.sm_scale)
    assert np.max(np.abs(ob - o[:, 1:])) < 1e-12


# ---------------------------------------------------------- invariants ----

def _small_case(seed, segs_spec, n_hist, nh=2):
    rng = np.random.default_rng(seed)
    n_cur = segs_spec[-1][0] + segs_spec[-1][3]
    q = rng.standard_normal((n_cur, nh, HEAD_DIM)) / math.sqrt(HEAD_DIM)
    k = rng.standard_normal((n_cur, nh, HEAD_DIM))
    v = rng.standard_normal((n_cur, nh, HEAD_DIM))
    hk = rng.standard_normal((n_hist, nh, HEAD_DIM)) if n_hist else None
    hv = rng.standard_normal((n_hist, nh, HEAD_DIM)) if n_hist else None
    segs = [Segment(a, b, c) for a, b, c, _ in segs_spec]
    return q, k, v, segs, hk, hv


def test_rows_sum_to_one_via_one_hot_values():
    # with one-hot values v_j = e_j the output row is the weight vector itself
    segs_spec = [(0, 5, 4, 30), (30, 6, 6, 40)]        # (start, text_len, text_valid, rows)
    q, k, _, segs, hk, _ = _small_case(11, segs_spec, n_hist=20)
    n_keys = 20 + 70
    eye = np.eye(HEAD_DIM)[:n_keys]
    hv = np.repeat(eye[:20, None, :], 2, axis=1)
    v = np.repeat(eye[20:, None, :], 2, axis=1)
    o, _ = oracle.joint_attn(q, k, v, segs, hk, hv, 1.0)
    assert np.max(np.abs(o.sum(axis=2) - 1.0)) < 1e-12
    mask = oracle.visible_mask(20, segs, 70)
    assert np.all(o[:, :, :n_keys][~np.broadcast_to(mask[:, None, :], o[:, :, :n_keys].shape)] == 0.0)
    assert np.all(o[:, :, :n_keys][np.broadcast_to(mask[:, None, :], o[:, :, :n_keys].shape)] > 0.0)


def test_causality_future_segment_perturbation():
    inp = workloads.make_inputs("c0_packed3")
    q, k, v, segs, hk, hv = oracle_chain(inp)
    o1, l1 = oracle.joint_attn(q, k, v, segs, hk, hv, inp.cfg.sm_scale)
    s2 = segs[2].start
    rng = np.random.default_rng(99)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[s2:] = rng.standard_normal(a[s2:].shape) * 5
    o2, l2 = oracle.joint_attn(q2, k2, v2, segs, hk, hv, inp.cfg.sm_scale)
    assert np.array_equal(o1[:s2], o2[:s2]) and np.array_equal(l1[:, :s2], l2[:, :s2])
    assert not np.array_equal(o1[s2:], o2[s2:])


def _packed_vs_cache(int8):
    """Segment 2 of the packed 3-segment form against the cache form."""
    inp = workloads.make_inputs("c0_packed3")
    q, k, v, segs, _, _ = oracle_chain(inp)
    cfg = inp.cfg
    o_full, l_full = oracle.joint_attn(q, k, v, segs, None, None, cfg.sm_scale)
    s2 = segs[2].start
    # cache = the (RoPE'd) video K/V of segments 0 and 1
    vid = np.concatenate([np.arange(s.start + s.text_len, b) for s, b in
                          zip(segs[:2], [segs[1].start, segs[2].start])])
    hk, hv = k[vid], v[vid]
    if int8:
        kc, ks = oracle.quantise_int8(hk)
        vc, vs = oracle.quantise_int8(hv)
        hk, hv = oracle.dequantise_int8(kc, ks), oracle.dequantise_int8(vc, vs)
    o_c, l_c = oracle.joint_attn(q[s2:], k[s2:], v[s2:], [Segment(0, segs[2].text_len,
                                 segs[2].text_valid)], hk, hv, cfg.sm_scale)
    return q[s2:], k[vid], v[vid], hk, hv, o_full[s2:], o_c, l_full[:, s2:], l_c, cfg.sm_scale


def test_cache_equals_recompute_bf16():
    _, _, _, _, _, o_full, o_c, l_full, l_c, _ = _packed_vs_cache(False)
    assert np.max(np.abs(o_full - o_c)) < 1e-12
    assert np.max(np.abs(l_full - l_c)) < 1e-12


def test_cache_int8_within_roundtrip_bound():
    q, k_ex, v_ex, hk, hv, o_full, o_c, _, _, sm = _packed_vs_cache(True)
    # key error per element <= s_k/2 (+ fp32 quotient rounding), so each logit
    # moves by at most eps_ij = sm * sum_d |q_id| * max|dk_jd|; the weights then
    # move by a factor within exp(+-2 eps), and values by at most max|dv|.
    dk = np.max(np.abs(hk - k_ex), axis=2)                 # [n_hist, H]
    dv = np.max(np.abs(hv - v_ex))
    qa = np.sum(np.abs(q), axis=2)                           # [n_q, H]
    eps = sm * qa[:, None, :] * dk[None, :, :]               # [n_q, n_hist, H]
    e_max = eps.max(axis=1)                                  # [n_q, H]
    vmax = max(np.max(np.abs(v_ex)), np.max(np.abs(hv)))
    bound = (np.exp(2 * e_max) - 1.0) * vmax + dv           # [n_q, H]
    err = np.max(np.abs(o_full - o_c), axis=2)
    assert np.all(err <= bound + 1e-12)
    assert np.max(err) > 0


# -------------------------------------------------------- closed forms ----

def test_zero_query_gives_mean_of_visible_values_and_log_count():
    for name in TINY + ["mid_packed", "mid_bf16"]:
        inp = workloads.make_inputs(name)
        q, k, v, segs, hk, hv = oracle_chain(inp)
        q = np.zeros_like(q)
        o, lse = oracle.joint_attn(q, k, v, segs, hk, hv, inp.cfg.sm_scale)
        n_hist = 0 if hk is None else hk.shape[0]
        mask = oracle.visible_mask(n_hist, segs, q.shape[0])
        keys_v = v if hk is None else np.concatenate([hv, v])
        cnt = mask.sum(axis=1)
        want = np.einsum("ij,jhd->ihd", mask.astype(np.float64), keys_v) / cnt[:, None, None]
        assert np.max(np.abs(o - want)) < 1e-12, name
        assert np.max(np.abs(lse - np.log(cnt)[None, :])) < 1e-12, name
        # the counts themselves, from the segment layout
        g = inp.cfg.tokens_per_frame
        earlier = 0
        for si, s in enumerate(inp.cfg.segments):
            r0 = segs[si].start
            assert cnt[r0] == n_hist + earlier + s.text_valid + s.n_frames * g, name
            earlier += s.n_frames * g


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 2, HEAD_DIM))
    k = rng.standard_normal((3, 2, HEAD_DIM))
    v = rng.standard_normal((3, 2, HEAD_DIM))
    o, lse = oracle.joint_attn(q, k, v, [Segment(0, 3, 1)], sm_scale=0.3)
    assert np.array_equal(o, np.broadcast_to(v[0], o.shape))
    assert np.allclose(lse, 0.3 * np.einsum("ihd,hd->hi", q, k[0]), atol=1e-14)


def test_matches_torch_sdpa_without_masks_or_rope():
    rng = np.random.default_rng(6)
    n, nh = 300, 3
    q = rng.standard_normal((n, nh, HEAD_DIM))
    k = rng.standard_normal((n, nh, HEAD_DIM))
    v = rng.standard_normal((n, nh, HEAD_DIM))
    o, _ = oracle.joint_attn(q, k, v, [Segment(0, 0, 0)], sm_scale=0.05)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.05)
    assert np.max(np.abs(ref[0].numpy().transpose(1, 0, 2) - o)) < 1e-12


def test_visible_pairs_count_matches_mask():
    for name, cfg in workloads.ALL.items():
        if cfg.n_cur > 2000:
            continue
        segs = [Segment(*s) for s in cfg.segment_rows()]
        mask = oracle.visible_mask(cfg.n_hist_rows, segs, cfg.n_cur)
        assert mask.sum() == cfg.visible_pairs(), name


def test_mask_rejects_bad_segments():
    with pytest.raises(ValueError):
        oracle.visible_mask(0, [Segment(0, 5, 6)], 10)
    with pytest.raises(ValueError):
        oracle.visible_mask(0, [Segment(1, 0, 0)], 10)


def test_history_keys_layout_and_dequant():
    # cache[slot, h, g, d] = a unique code per index: the gather must return
    # row f*G + g of frame slots[f], head h, element d
    ns, nh, g, d = 5, 3, 7, HEAD_DIM
    idx = np.indices((ns, nh, g, d))
    code = ((idx[0] * 1000 + idx[1] * 100 + idx[2]) * 1000 + idx[3]).astype(np.float64)
    slots = np.array([4, 1, 2])
    k, v = oracle.history_keys(code, -code, slots)
    for f, s in enumerate(slots):
        for gi in range(g):
            for h in range(nh):
                assert np.array_equal(k[f * g + gi, h], code[s, h, gi])
                assert np.array_equal(v[f * g + gi, h], -code[s, h, gi])
    rng = np.random.default_rng(3)
    kc = rng.integers(-127, 128, size=(ns, nh, g, d)).astype(np.int8)
    ks = rng.random((ns, nh, g)).astype(np.float32)
    k8, v8 = oracle.history_keys(kc, kc, slots, ks, 2 * ks)
    assert k8[2 * g + 3, 1, 5] == float(kc[2, 1, 3, 5]) * float(ks[2, 1, 3])
    assert v8[0 * g + 6, 2, 9] == float(kc[4, 2, 6, 9]) * float(2 * ks[4, 2, 6])
