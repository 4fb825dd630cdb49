"""Pins of the oracle's attention gradients (packed training form): central
finite differences of L = sum(do * o) on tiny inputs, and invariants."""

import numpy as np
import pytest

import oracle

SEGS = [oracle.Segment(0, 3, 3), oracle.Segment(7, 2, 1), oracle.Segment(12, 0, 0)]
N, H, D = 17, 2, 6


def _inputs(seed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((N, H, D)) for _ in range(4))
    return q, k, v, do


def _loss(q, k, v, do, scale):
    o, _ = oracle.joint_attn(q, k, v, SEGS, sm_scale=scale)
    return float(np.sum(do * o))


@pytest.mark.parametrize("scale", [1.0, 0.37])
def test_gradients_match_central_differences(scale):
    q, k, v, do = _inputs(3)
    grads = oracle.joint_attn_backward(q, k, v, SEGS, do, sm_scale=scale)
    eps = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v]
        for idx in np.ndindex(N, H, D):
            xp = [a.copy() for a in base]
            xm = [a.copy() for a in base]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            fd = (_loss(*xp, do, scale) - _loss(*xm, do, scale)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(fd)), (which, idx, fd, g[idx])


def test_value_gradient_sums_to_upstream_sum():
    # every query row's weights sum to 1, so the dv rows add up to the do rows
    q, k, v, do = _inputs(4)
    _, _, dv = oracle.joint_attn_backward(q, k, v, SEGS, do)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_query_gradient_vanishes_for_identical_keys():
    # ds sums to zero over each row, so with one key vector dq = scale * k * 0
    q, k, v, do = _inputs(5)
    k[:] = k[0:1]
    dq, _, _ = oracle.joint_attn_backward(q, k, v, SEGS, do, sm_scale=0.5)
    assert np.max(np.abs(dq)) <= 1e-12


def test_invisible_keys_get_no_gradient():
    # segment 1's padded text row (row 8) is visible to nobody
    q, k, v, do = _inputs(6)
    _, dk, dv = oracle.joint_attn_backward(q, k, v, SEGS, do)
    assert not np.any(dk[8]) and not np.any(dv[8])


def test_key_gradient_sums_to_zero():
    # ds sums to zero over each query row, so sum_j dk_j = scale sum_i q_i * 0
    q, k, v, do = _inputs(7)
    _, dk, _ = oracle.joint_attn_backward(q, k, v, SEGS, do, sm_scale=0.8)
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12


def test_chunking_does_not_change_gradients():
    q, k, v, do = _inputs(8)
    a = oracle.joint_attn_backward(q, k, v, SEGS, do, chunk=512)
    b = oracle.joint_attn_backward(q, k, v, SEGS, do, chunk=3)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-13)


def test_dq_rows_match_central_differences():
    # the sampled-row form, pinned on its own: perturb q of the chosen rows
    q, k, v, do = _inputs(9)
    rows = [0, 4, 8, 11, 16]
    got = oracle.joint_attn_dq_rows(q, k, v, SEGS, do, rows, sm_scale=0.6)
    eps = 1e-6
    for ri, r in enumerate(rows):
        for hd in range(H):
            for c in range(D):
                qp, qm = q.copy(), q.copy()
                qp[r, hd, c] += eps
                qm[r, hd, c] -= eps
                fd = (_loss(qp, k, v, do, 0.6) - _loss(qm, k, v, do, 0.6)) / (2 * eps)
                assert abs(fd - got[ri, hd, c]) <= 1e-6 * (1 + abs(fd)), (r, hd, c)
