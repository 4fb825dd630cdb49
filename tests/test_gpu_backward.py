"""GPU parity of the attention gradients (packed training form) against the
fp64 oracle, through the C ABI.

Inputs: the seeded workload draws; q and k are rotated by the library's RoPE
(bit-exact with the oracle's) and the forward's o and lse come from the
library's forward, as in training. The oracle recomputes everything from the
same bf16 q, k, v and do.

Bar (derived from the arithmetic; no tolerance is printed for gradients):
every gradient row is a sum of products with one bf16-rounded factor (p or
ds, relative error <= 2^-9) and is itself rounded to bf16 (another 2^-9);
with independent rounding errors the per-element error is about
2^-9 * sqrt(2/3) ~ 1.6e-3 of the size of that row's terms. The size of a
gradient row varies about tenfold between rows that see few keys and rows
that see many, so the errors are measured against the rms of each
(row, head) of the fp64 gradient: max <= 2^-4 (the largest over 10^5..10^9
elements of a 1.6e-3-wide error, whose tail grows with |g| / rms_row, stays
below about 2.5e-2) and mean <= 2^-8 (2.4x the expected 1.6e-3). Keys no
query sees have dk = dv = 0 exactly, and are left out of the ratios. The
random packed forms also hold rows that see only a few keys, whose dq (and
the dk of their keys) can be much smaller than the terms that cancel in it:
there each element may instead stay within the error that delta, formed from
the forward's bf16 output, carries into it (_delta_bounds).
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from chain import bits, gpu_chain, oracle_inputs, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
sc = pytest.importorskip("segment_causal_dit_amd._lib")

MAX_REL, MEAN_REL = 2.0 ** -4, 2.0 ** -8


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def _invisible_keys(cfg):
    rows = []
    for (start, tl, tv) in cfg.segment_rows():
        rows.extend(range(start + tv, start + tl))
    return np.asarray(rows, dtype=np.int64)


def _check(name, got, want, bound=None):
    """Errors relative to the rms of each (row, head) of the fp64 gradient.
    With `bound` (per element, from _delta_bounds), an element whose derived
    rounding bound exceeds the rms bar is held to that bound instead."""
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    live = np.broadcast_to(rms > 0, want.shape)
    err = np.abs(got - want)
    rel = err[live] / np.broadcast_to(rms, want.shape)[live]
    mx, mean = float(rel.max()), float(rel.mean())
    _say("  %s: max %.4f, mean %.5f of the row rms" % (name, mx, mean))
    assert mean <= MEAN_REL, name
    if bound is None:
        assert mx <= MAX_REL, name
    else:
        allowed = np.maximum(MAX_REL * np.broadcast_to(rms, want.shape), bound)
        worst = float((err[live] / allowed[live]).max())
        _say("  %s: max %.3f of max(rms bar, derived bound)" % (name, worst))
        assert worst <= 1.0, name


def _delta_bounds(q, k, v, do, segs, sm_scale):
    """Per-element bounds on the dq and dk errors that come from delta.
    The kernel forms delta_i = do_i . o_i from the forward's bf16 output
    (relative error <= 2^-8 per element of o, the forward's error included),
    so |delta' - delta| <= eps_i = 2^-8 sum_d |do_id o_id|; with p_ij rounded
    to bf16 inside ds_ij = p_ij (dp_ij - delta_i) that gives
    |ds' - ds| <= p_ij (eps_i + 2^-8 |dp_ij - delta_i|), and
    dq_i = sm_scale sum_j ds_ij k_j, dk_j = sm_scale sum_i ds_ij q_i carry it
    with |k| and |q|. Rows that see few keys can have a dq far smaller than
    these terms (ds nearly cancels across the keys), where an rms-relative bar
    cannot hold."""
    n, nh, _ = q.shape
    vis = oracle.visible_mask(0, segs, n)
    o, lse = oracle.joint_attn(q, k, v, segs, sm_scale=sm_scale)
    bq, bk = np.zeros_like(q), np.zeros_like(k)
    for h in range(nh):
        s = sm_scale * q[:, h] @ k[:, h].T
        p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[h][:, None]), 0.0)
        eps = 2.0 ** -8 * np.abs(do[:, h] * o[:, h]).sum(-1)
        dp = do[:, h] @ v[:, h].T
        delta = (do[:, h] * o[:, h]).sum(-1)
        t = p * (eps[:, None] + 2.0 ** -8 * np.abs(dp - delta[:, None]))
        bq[:, h] = sm_scale * t @ np.abs(k[:, h])
        bk[:, h] = sm_scale * t.T @ np.abs(q[:, h])
    return bq, bk


def _gpu_backward(inp, do_bits, sm_scale=None):
    r = gpu_chain(inp)
    do = _bf(do_bits)
    scale = inp.cfg.sm_scale if sm_scale is None else sm_scale
    dq, dk, dv = sc.segcausal_joint_attn_bwd(r.q, r.k, r.v, r.o, do, r.lse, inp.segments, scale)
    torch.cuda.synchronize()
    return r, dq, dk, dv


@pytest.mark.parametrize("name", ["bwd_small", "bwd_one", "bwd_text", "c0_packed3", "mid_nocache",
                                  "bwd_mid", "bwd_seg16"])
def test_gradients_match_oracle(name):
    _say("bwd", name)
    inp = workloads.make_inputs(name)
    do_bits = workloads.upstream_grad(inp.cfg)
    _, dq, dk, dv = _gpu_backward(inp, do_bits)
    q, k, v = oracle_inputs(inp)
    segs = [oracle.Segment(*s) for s in inp.segments]
    want = oracle.joint_attn_backward(q, k, v, segs, oracle.bf16_bits_to_f64(do_bits),
                                      sm_scale=inp.cfg.sm_scale)
    for nm, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(nm, to_f64(g), w)
    dead = _invisible_keys(inp.cfg)
    if len(dead):
        assert not bits(dk)[dead].any() and not bits(dv)[dead].any()


@pytest.mark.parametrize("i", range(12))
def test_gradients_random_packed_configs(i):
    # seeded random packed forms (no cache): 1-16 segments, text padding,
    # text-only and text-free segments, frame sizes on and off 16 tokens
    cfg = workloads.random_config(i, history=False)
    _say("bwd", cfg)
    inp = workloads.make_inputs(cfg)
    do_bits = workloads.upstream_grad(cfg)
    _, dq, dk, dv = _gpu_backward(inp, do_bits)
    q, k, v = oracle_inputs(inp)
    segs = [oracle.Segment(*s) for s in inp.segments]
    do = oracle.bf16_bits_to_f64(do_bits)
    want = oracle.joint_attn_backward(q, k, v, segs, do, sm_scale=cfg.sm_scale)
    bq, bk = _delta_bounds(q, k, v, do, segs, cfg.sm_scale)
    for nm, g, w, b in zip(("dq", "dk", "dv"), (dq, dk, dv), want, (bq, bk, None)):
        _check(nm, to_f64(g), w, b)
    dead = _invisible_keys(cfg)
    if len(dead):
        assert not bits(dk)[dead].any() and not bits(dv)[dead].any()


def test_deterministic_strided_and_aliased_outputs():
    # strided views (rows of a [n, 3, H, 128] buffer), the same bits on a rerun
    inp = workloads.make_inputs("bwd_small")
    cfg = inp.cfg
    do_bits = workloads.upstream_grad(cfg)
    r, dq, dk, dv = _gpu_backward(inp, do_bits)
    buf = torch.full((cfg.n_cur, 3, cfg.n_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    do = _bf(do_bits)
    delta = torch.empty((cfg.n_heads, cfg.n_cur), dtype=torch.float32, device="cuda")
    sc.segcausal_joint_attn_bwd(r.q, r.k, r.v, r.o, do, r.lse, inp.segments, cfg.sm_scale,
                                dq=buf[:, 0], dk=buf[:, 1], dv=buf[:, 2], delta=delta)
    torch.cuda.synchronize()
    for a, b in ((dq, buf[:, 0]), (dk, buf[:, 1]), (dv, buf[:, 2])):
        assert np.array_equal(bits(a), bits(b))
    # delta is rowsum(do * o) of the bf16 values
    want = (to_f64(do) * to_f64(r.o)).sum(axis=2).T
    assert np.max(np.abs(delta.cpu().numpy() - want)) <= 1e-5 * (1 + np.abs(want).max())


def test_other_scale():
    # sm_scale is a free parameter of the gradient: check a second value
    inp = workloads.make_inputs("bwd_text")
    do_bits = workloads.upstream_grad(inp.cfg)
    r = gpu_chain(inp, with_lse=False)
    lse = torch.empty((inp.cfg.n_heads, inp.cfg.n_cur), dtype=torch.float32, device="cuda")
    o = sc.segcausal_joint_attn(r.q, r.k, r.v, inp.segments, 0.37, lse=lse)
    dq, dk, dv = sc.segcausal_joint_attn_bwd(r.q, r.k, r.v, o, _bf(do_bits), lse, inp.segments, 0.37)
    torch.cuda.synchronize()
    q, k, v = oracle_inputs(inp)
    segs = [oracle.Segment(*s) for s in inp.segments]
    want = oracle.joint_attn_backward(q, k, v, segs, oracle.bf16_bits_to_f64(do_bits), sm_scale=0.37)
    for nm, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(nm, to_f64(g), w)


def test_training_scale_sampled_rows_and_sums():
    # 13 packed segments, 346,528 rows, 16 heads, in the launch configuration
    # of the timed run: dq of sampled rows against the oracle (rows from every
    # segment, text and video, first and last), exact zeros for the keys no
    # query sees, finite outputs, and the identities sum_j dv_j = sum_i do_i
    # and sum_j dk_j = 0 per head and column. The exact dk and dv of a key
    # need every query's full softmax row (about 2 minutes of fp64 per head
    # here), so their element-wise check is the full comparison of the
    # smaller cases above, which run the same kernels over many tiles.
    name = "train13"
    _say("bwd", name)
    inp = workloads.make_inputs(name)
    cfg = inp.cfg
    do_bits = workloads.upstream_grad(cfg)
    r, dq, dk, dv = _gpu_backward(inp, do_bits)
    rng = np.random.default_rng(5)
    rows = [0, cfg.n_cur - 1]
    for (start, tl, tv) in cfg.segment_rows():
        rows += [start, start + tl - 1, start + tl, start + tl + 880 * 29]
    rows = np.unique(np.asarray(rows + list(rng.integers(0, cfg.n_cur, 24)), dtype=np.int64))
    q, k, v = oracle_inputs(inp)
    segs = [oracle.Segment(*s) for s in inp.segments]
    do = oracle.bf16_bits_to_f64(do_bits)
    want = oracle.joint_attn_dq_rows(q, k, v, segs, do, rows, sm_scale=cfg.sm_scale)
    _check("dq rows", to_f64(dq[torch.from_numpy(rows).cuda()]), want)
    # column sums (fp64 over the bf16 outputs)
    sdv = dv.to(torch.float64).sum(dim=0).cpu().numpy()
    sdk = dk.to(torch.float64).sum(dim=0).cpu().numpy()
    sdo = do.sum(axis=0)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    # each summed row carries an error of about 1.2 * 2^-9 of its size (the
    # small cases measure a mean of 1.8e-3 of the row rms), partly correlated
    # across rows through each query's shared lse and delta: the bar is
    # 16 * 2^-9 * sqrt(n) * rms(g), a coarse check (a dropped head, a wrong
    # scale or a lost segment moves a sum by far more)
    rms_dv = float(dv.to(torch.float64).pow(2).mean().sqrt())
    rms_dk = float(dk.to(torch.float64).pow(2).mean().sqrt())
    tol_v = 16 * 2.0 ** -9 * np.sqrt(cfg.n_cur) * rms_dv
    tol_k = 16 * 2.0 ** -9 * np.sqrt(cfg.n_cur) * rms_dk
    _say("  sum dv err %.4g (tol %.4g), sum dk %.4g (tol %.4g)" %
         (np.abs(sdv - sdo).max(), tol_v, np.abs(sdk).max(), tol_k))
    assert np.abs(sdv - sdo).max() <= tol_v
    assert np.abs(sdk).max() <= tol_k
    dead = _invisible_keys(cfg)
    assert not bits(dk[torch.from_numpy(dead).cuda()]).any()
    assert not bits(dv[torch.from_numpy(dead).cuda()]).any()


@pytest.mark.parametrize("n,h,segs", [
    (1, 1, [(0, 0, 0)]),                         # one row: p = 1, dq = dk = 0, dv = do
    (65, 2, [(0, 0, 0)]),                        # one row past a 64-row tile
    (129, 1, [(0, 1, 1), (2, 0, 0), (3, 3, 2), (9, 0, 0)]),   # tiny segments, padded text
    (300, 3, [(0, 300, 300)]),                   # all rows text
])
def test_edge_shapes(n, h, segs):
    _say("bwd edge", n, h, segs)
    q = workloads.normal_bf16(30, (n, h, 128), 1.0 / np.sqrt(128))
    k, v, do = (workloads.normal_bf16(31 + i, (n, h, 128)) for i in range(3))
    qt, kt, vt = _bf(q), _bf(k), _bf(v)
    lse = torch.empty((h, n), dtype=torch.float32, device="cuda")
    o = sc.segcausal_joint_attn(qt, kt, vt, segs, 1.0, lse=lse)
    dq, dk, dv = sc.segcausal_joint_attn_bwd(qt, kt, vt, o, _bf(do), lse, segs, 1.0)
    torch.cuda.synchronize()
    f = oracle.bf16_bits_to_f64
    osegs = [oracle.Segment(*s) for s in segs]
    want = oracle.joint_attn_backward(f(q), f(k), f(v), osegs, f(do), sm_scale=1.0)
    vis = oracle.visible_mask(0, osegs, n)                       # [query, key]
    for nm, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        got = to_f64(g)
        zero = np.sqrt(np.mean(w * w, axis=-1)) == 0             # [row, head]
        # keys no query sees: p is exactly 0, so dk and dv are exactly 0
        if nm != "dq":
            unseen = ~vis.any(axis=0)
            assert not got[unseen].any(), nm
        # rows that are zero only by cancellation (a query seeing one key: ds =
        # do.v - do.o with o = v): the kernel forms do.v and do.o in two fp32
        # summation orders, so |ds| <= 2^-18 sum_t |do_t v_t| and
        # |dq| <= |ds| max |k|
        # (and dk_j = sm_scale sum_i ds_ij q_i likewise with |q|)
        if nm in ("dq", "dk") and zero.any():
            fq, fk, fv, fdo = f(q), f(k), f(v), f(do)
            for r, hd in zip(*np.nonzero(zero)):
                if nm == "dq":
                    qs, ks_, other = np.array([r]), np.nonzero(vis[r])[0], fk
                else:
                    qs, ks_, other = np.nonzero(vis[:, r])[0], np.array([r]), fq
                    if not len(qs):
                        continue                          # unseen key: exact zero, checked above
                terms = np.abs(fdo[qs, hd][:, None, :] * fv[ks_, hd][None, :, :]).sum(axis=-1).max()
                big = np.abs(other[ks_ if nm == "dq" else qs, hd]).max()
                bound = 2.0 ** -18 * terms * big
                assert np.abs(got[r, hd]).max() <= bound, (nm, r, hd, np.abs(got[r, hd]).max(), bound)
        if (~zero).any():
            _check(nm, np.where(zero[..., None], w, got), w)
