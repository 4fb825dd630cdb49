"""Pins for the oracle's bf16, RoPE, INT8 and window functions (CPU only).

Each test ties an oracle function to something other than itself: a
hand-worked fixture, a library special case, a closed form or an invariant.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ bf16 ----

def test_bf16_hand_cases():
    for xs, ys in _golden("bf16_rounding_cases.json")["cases"]:
        env = {"__builtins__": {}, "inf": math.inf}
        x, y = eval(xs, env), eval(ys, env)  # fixture expressions are plain arithmetic
        got = oracle.round_to_bf16(np.array([x]))[0]
        assert got == y, (xs, got, y)


def test_bf16_matches_torch_on_fp32_inputs():
    # library special case: torch's float32 -> bfloat16 cast rounds to nearest
    # even; on fp32 inputs the oracle must agree bit for bit.
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want)
    back = oracle.bf16_bits_to_f64(got)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_input_rounding_agrees_with_oracle_rounding():
    # the generator's bit trick and the oracle's definition are separate code;
    # they must agree on fp32 draws
    d = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    assert np.array_equal(workloads.f32_to_bf16_bits(d), oracle.f64_to_bf16_bits(d.astype(np.float64)))


# ------------------------------------------------------------------ RoPE ----

def test_rope_frequencies_closed_form():
    # theta = 256 and a 16-wide temporal slice give theta**(-2i/16) = 2**-i
    f = oracle.rope_frequencies(16, 256.0)
    assert np.array_equal(f, 2.0 ** -np.arange(8))
    g = oracle.rope_frequencies(56, 256.0)
    assert np.allclose(g, 2.0 ** (-2.0 * np.arange(28) / 7.0), rtol=0, atol=1e-16)


def test_rope_pos_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 3, 128))
    assert np.array_equal(oracle.rope3d(x, np.zeros((5, 3), np.int32)), x)


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 2, 128))
    pos = rng.integers(0, 400, size=(40, 3))
    y = oracle.rope3d(x, pos)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = np.concatenate([
        pos[:, 0:1] * 256.0 ** (-np.arange(8) / 8.0),
        pos[:, 1:2] * 256.0 ** (-np.arange(28) / 28.0),
        pos[:, 2:3] * 256.0 ** (-np.arange(28) / 28.0)], axis=1)
    w = z * np.exp(1j * ang)[:, None, :]
    assert np.max(np.abs(y[..., 0::2] - w.real)) < 1e-12
    assert np.max(np.abs(y[..., 1::2] - w.imag)) < 1e-12


def test_rope_preserves_pair_norms_and_axis_slices():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((30, 4, 128))
    pos = rng.integers(0, 300, size=(30, 3))
    y = oracle.rope3d(x, pos)
    assert np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]),
                       np.hypot(x[..., 0::2], x[..., 1::2]), atol=1e-12)
    # moving only h touches only dims 16..71
    p2 = pos.copy()
    p2[:, 1] += 5
    y2 = oracle.rope3d(x, p2)
    diff = np.any(y2 != y, axis=(0, 1))
    assert not diff[:16].any() and diff[16:72].all() and not diff[72:].any()


def test_rope_scores_depend_only_on_position_differences():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((20, 2, 128))
    k = rng.standard_normal((25, 2, 128))
    pq = rng.integers(0, 50, size=(20, 3))
    pk = rng.integers(0, 50, size=(25, 3))
    shift = np.array([37, -3, 11])
    s0 = np.einsum("ihd,jhd->hij", oracle.rope3d(q, pq), oracle.rope3d(k, pk))
    s1 = np.einsum("ihd,jhd->hij", oracle.rope3d(q, pq + shift), oracle.rope3d(k, pk + shift))
    assert np.max(np.abs(s0 - s1)) < 1e-11


def test_rope_bf16_is_exact_rotation_rounded_once():
    cfg = workloads.ALL["c0"]
    inp = workloads.make_inputs(cfg)
    kv = inp.k[inp.video_rows]
    y = oracle.rope3d_bf16(kv, inp.pos)
    exact = oracle.rope3d(oracle.bf16_bits_to_f64(kv), inp.pos)
    # each output is a bf16 value within half a bf16 ulp of the exact rotation
    assert np.array_equal(y, oracle.round_to_bf16(y))
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    assert np.all(np.abs(y - exact) <= 0.5 * ulp + 1e-300)


# ------------------------------------------------------------------ INT8 ----

def test_quant_hand_example():
    g = _golden("quant_hand_example.json")
    x = np.array([g["x_head"] + [0.0] * (128 - len(g["x_head"]))])
    codes, scale = oracle.quantise_int8(x)
    assert scale[0] == np.float32(g["scale"])
    assert list(codes[0, :len(g["codes_head"])]) == g["codes_head"]
    assert not codes[0, len(g["codes_head"]):].any()
    c0, s0 = oracle.quantise_int8(np.zeros((1, 128)))
    assert s0[0] == g["x_zero_row_scale"] and not c0.any()


def _bf16_rows(n, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    if spread:
        x *= (2.0 ** rng.integers(-20, 20, size=(n, 1))).astype(np.float32)
    return oracle.bf16_bits_to_f64(workloads.f32_to_bf16_bits(x))


def test_quant_matches_torch_fp32_division():
    # the float64-then-round emulation must equal IEEE fp32 division done by
    # another library (torch float32 tensors)
    x = _bf16_rows(4000, 5)
    codes, scale = oracle.quantise_int8(x)
    xt = torch.from_numpy(x.astype(np.float32))
    a = xt.abs().amax(dim=1)
    st = a / torch.tensor(127.0, dtype=torch.float32)
    assert np.array_equal(st.numpy(), scale)
    qt = xt / st[:, None]
    ct = torch.clamp(torch.round(qt), -127, 127).to(torch.int8)   # torch.round: half to even
    assert np.array_equal(ct.numpy(), codes)


def test_quant_roundtrip_bound_and_symmetry():
    x = _bf16_rows(5000, 6)
    codes, scale = oracle.quantise_int8(x)
    s = scale.astype(np.float64)[:, None]
    err = np.abs(x - codes.astype(np.float64) * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -18))
    amax_idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(codes[np.arange(len(x)), amax_idx]) == 127)
    cn, sn = oracle.quantise_int8(-x)
    assert np.array_equal(cn, -codes) and np.array_equal(sn, scale)
    assert codes.min() >= -127


def test_quant_ties_round_to_even():
    # x/scale lands exactly on k + 1/2 when scale is a power of two
    x = np.zeros((4, 128))
    x[:, 0] = 127.0 * 2.0 ** -3           # scale = 2**-3 exactly
    x[0, 1:4] = np.array([0.5, 1.5, 2.5]) * 2.0 ** -3
    x[1, 1:4] = -np.array([0.5, 1.5, 2.5]) * 2.0 ** -3
    codes, scale = oracle.quantise_int8(x)
    assert scale[0] == 2.0 ** -3
    assert list(codes[0, 1:4]) == [0, 2, 2]
    assert list(codes[1, 1:4]) == [0, -2, -2]


# ---------------------------------------------------------------- window ----

def _window_brute(slot_t, budget):
    valid = sorted((t, i) for i, t in enumerate(slot_t) if t >= 0)
    chosen = valid[max(0, len(valid) - budget):] if budget > 0 else []
    return [i for _, i in chosen]


def test_window_brute_force():
    rng = np.random.default_rng(8)
    for trial in range(300):
        n = int(rng.integers(0, 30))
        ts = rng.permutation(100)[:n]
        ts[rng.random(n) < 0.3] = -1
        for b in (0, 1, 3, 18, 40):
            assert list(oracle.window_select(ts, b)) == _window_brute(list(ts), b)


def test_window_errors():
    with pytest.raises(oracle.WindowError):
        oracle.window_select([3, 5, 3], 2)
    with pytest.raises(oracle.WindowError):
        oracle.window_select([1, 2], -1)
    assert list(oracle.window_select([-1, -1], 5)) == []


# ------------------------------------------------------------ page sizes ----

def test_workload_geometry_matches_pages():
    g = _golden("page_sizes.json")
    c4 = workloads.CONFIGS["c4"]
    assert c4.tokens_per_frame == g["tokens_per_latent_frame_704x1280"]["value"]
    assert c4.n_heads == g["heads"]["value"]
    assert workloads.HEAD_DIM == g["head_dim"]["value"]
    assert workloads.CONFIGS["c2"].window == g["history_budget_frames"]["value"]
    # 12-s turns at 6 latent frames per second = 72 frames
    assert c4.segments[0].n_frames == 12 * g["latent_frames_per_second"]["value"]
    per_tok = 2 * c4.n_heads * workloads.HEAD_DIM   # K and V INT8 codes
    assert per_tok == g["int8_kv_bytes_per_token_per_layer"]["value"]
    assert per_tok * g["dit_layers"]["value"] * c4.tokens_per_frame == \
        g["int8_kv_bytes_per_frame_54_layers"]["value"]
    assert c4.n_hist_rows == 253440 and c4.n_cur == 63616


# ---------------------------------------- dequantisation to the BF16 operand ----

def _f32_mul_then_bf16_bits(codes, scales):
    """Independent path: IEEE fp32 multiply in numpy float32, then bf16
    round-to-nearest-even done on the integer bit pattern."""
    prod = codes.astype(np.float32) * scales.astype(np.float32)[..., None]
    b = prod.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def test_dequant_bf16_matches_fp32_product_rounded_to_bf16():
    rng = np.random.default_rng(31)
    codes = rng.integers(-127, 128, size=(64, 128)).astype(np.int8)
    scales = (rng.random(64) * 10.0 ** rng.uniform(-6, 2, 64)).astype(np.float32)
    got = oracle.f64_to_bf16_bits(oracle.dequantise_int8_bf16(codes, scales))
    assert np.array_equal(got, _f32_mul_then_bf16_bits(codes, scales))


def test_dequant_bf16_closed_forms():
    codes = np.arange(-127, 128, dtype=np.int8)[None, :]
    # power-of-two scale: the product has <= 7 significant bits, exact in bf16
    for k in (-20, -3, 0, 5):
        s = np.array([2.0 ** k], dtype=np.float32)
        assert np.array_equal(oracle.dequantise_int8_bf16(codes, s), codes.astype(np.float64) * 2.0 ** k)
    # zero scale -> zeros; sign symmetry; error within the two roundings
    assert not np.any(oracle.dequantise_int8_bf16(codes, np.zeros(1, np.float32)))
    s = np.array([0.0123456], dtype=np.float32)
    d = oracle.dequantise_int8_bf16(codes, s)
    assert np.array_equal(d, -oracle.dequantise_int8_bf16((-codes.astype(np.int16)).astype(np.int8), s))
    exact = oracle.dequantise_int8(codes, s)
    assert np.all(np.abs(d - exact) <= np.abs(exact) * (2.0 ** -8 + 2.0 ** -24))


# ------------------------------------------------------------ archive ----

def test_move_frames_matches_elementwise_loop():
    rng = np.random.default_rng(31)
    src = rng.integers(-127, 128, size=(9, 2, 3, 4)).astype(np.int8)
    dst = rng.integers(-127, 128, size=(6, 2, 3, 4)).astype(np.int8)
    src_idx, dst_idx = [8, 0, 3, 4], [5, 1, 2, 3]
    got = oracle.move_frames(src, src_idx, dst, dst_idx)
    want = dst.copy()
    for s_, d_ in zip(src_idx, dst_idx):
        for idx in np.ndindex(*src.shape[1:]):
            want[(d_,) + idx] = src[(s_,) + idx]
    assert np.array_equal(got, want)
    assert np.array_equal(dst[[0, 4]], got[[0, 4]])          # untouched frames
    back = oracle.move_frames(got, dst_idx, np.zeros_like(src), src_idx)
    assert np.array_equal(back[src_idx], src[src_idx])       # round trip


def test_move_frames_rejects_duplicate_destinations():
    a = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.move_frames(a, [0, 1], a, [2, 2])


# -------------------------------------------------------- W8A16 linear ----

def test_w8a16_linear_matches_triple_loop():
    rng = np.random.default_rng(41)
    m, n, k = 3, 5, 7
    x = rng.standard_normal((m, k))
    codes = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    scale = rng.random(n) / 64
    bias = rng.standard_normal(n)
    got = oracle.w8a16_linear(x, codes, scale, bias)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += x[i, t] * (int(codes[j, t]) * scale[j])
            assert abs(got[i, j] - (acc + bias[j])) <= 1e-12 * (1 + abs(acc))


def test_w8a16_linear_special_cases():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((4, 6))
    # one-hot codes pick a column of x, scaled
    codes = np.zeros((3, 6), np.int8)
    codes[0, 2], codes[1, 5], codes[2, 0] = 1, -127, 64
    scale = np.array([0.5, 2.0 ** -7, 0.25])
    y = oracle.w8a16_linear(x, codes, scale)
    assert np.array_equal(y[:, 0], 0.5 * x[:, 2])
    assert np.array_equal(y[:, 1], -127 * 2.0 ** -7 * x[:, 5])
    assert np.array_equal(y[:, 2], 16.0 * x[:, 0])
    # no bias equals zero bias; a bias shifts every row
    assert np.array_equal(y, oracle.w8a16_linear(x, codes, scale, np.zeros(3)))
    assert np.allclose(oracle.w8a16_linear(x, codes, scale, [1, 2, 3]) - y, [[1, 2, 3]] * 4, atol=0)


# ------------------------------------------------ camera cross-attention ----

def test_camera_cross_attn_matches_loops():
    rng = np.random.default_rng(51)
    n, h, d, tpc, tc = 11, 2, 5, 4, 3            # a ragged last chunk of 3 rows
    q = rng.standard_normal((n, h, d))
    nch = (n + tpc - 1) // tpc
    k = rng.standard_normal((nch * tc, h, d))
    v = rng.standard_normal((nch * tc, h, d))
    got = oracle.camera_cross_attn(q, k, v, tpc, tc, 0.7)
    for i in range(n):
        c = i // tpc
        for hd in range(h):
            s = [0.7 * sum(q[i, hd, t] * k[c * tc + j, hd, t] for t in range(d)) for j in range(tc)]
            e = [math.exp(x - max(s)) for x in s]
            for t in range(d):
                want = sum(e[j] * v[c * tc + j, hd, t] for j in range(tc)) / sum(e)
                assert abs(got[i, hd, t] - want) <= 1e-12


def test_camera_cross_attn_closed_forms():
    rng = np.random.default_rng(52)
    n, h, d, tpc = 10, 3, 4, 5
    q = rng.standard_normal((n, h, d)) * 10
    v = rng.standard_normal((2, h, d))
    # one camera token per chunk: every row gets its chunk's value exactly
    o = oracle.camera_cross_attn(q, rng.standard_normal((2, h, d)), v, tpc, 1, 0.088)
    assert np.array_equal(o[:5], np.broadcast_to(v[0], (5, h, d)))
    assert np.array_equal(o[5:], np.broadcast_to(v[1], (5, h, d)))
    # identical keys: the plain mean of the chunk's values
    k = np.broadcast_to(rng.standard_normal((1, h, d)), (6, h, d))
    v3 = rng.standard_normal((6, h, d))
    o = oracle.camera_cross_attn(q, k, v3, tpc, 3, 0.5)
    assert np.allclose(o[:5], v3[:3].mean(axis=0), atol=1e-14)
    assert np.allclose(o[5:], v3[3:].mean(axis=0), atol=1e-14)
