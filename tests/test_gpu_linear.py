"""GPU parity of the INT8-weight linear (w8a16_linear) against the fp64 oracle.

Bar (derived): the products of bf16 activations and codes are exact in fp32,
the k-sum accumulates in fp32 (error well under 2^-16 of sum_t |x_t c_t|
for k <= 8192) and the result is scaled, biased and rounded once to bf16
(2^-9 relative). Element-wise:
    |y - y_ref| <= 2^-8 |y_ref| + 2^-14 (scale_n sum_t |x_t c_nt| + |bias_n|)
with the second term from the fp64 absolute sums.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
sc = pytest.importorskip("segment_causal_dit_amd._lib")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _check(got, x_bits, codes, scale, bias, rows=None):
    x = oracle.bf16_bits_to_f64(x_bits if rows is None else x_bits[rows])
    want = oracle.w8a16_linear(x, codes, scale, bias)
    mag = np.abs(x) @ np.abs(codes.astype(np.float64)).T * scale.astype(np.float64)[None, :]
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))[None, :]
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -14 * mag
    _say("  max |err| %.3g, max err/bound %.3f" % (err.max(), (err / bound).max()))
    assert np.all(err <= bound)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k,with_bias", [
    (300, 256, 128, True),       # ragged row tile, one channel tile
    (1, 512, 64, False),         # a single row, one k step
    (513, 768, 320, True),       # three channel tiles, five k steps
    (256, 2048, 2048, False),    # the projection's width
])
def test_linear_matches_oracle(m, n, k, with_bias):
    _say("linear", m, n, k, with_bias)
    x, codes, scale, bias = workloads.linear_inputs(m, n, k, seed=m + n)
    bias = bias if with_bias else None
    y = sc.w8a16_linear(_bf(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(),
                        torch.from_numpy(bias).cuda() if bias is not None else None)
    torch.cuda.synchronize()
    _check(_f64(y), x, codes, scale, bias)


def test_strided_operands_and_determinism():
    m, n, k = 200, 512, 192
    x, codes, scale, bias = workloads.linear_inputs(m, n, k, seed=5)
    xbuf = torch.zeros((m, k + 64), dtype=torch.bfloat16, device="cuda")
    xbuf[:, 32:32 + k] = _bf(x)
    wbuf = torch.zeros((n, k + 48), dtype=torch.int8, device="cuda")
    wbuf[:, 16:16 + k] = torch.from_numpy(codes).cuda()
    ybuf = torch.full((m, n + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    s_t, b_t = torch.from_numpy(scale).cuda(), torch.from_numpy(bias).cuda()
    y1 = sc.w8a16_linear(xbuf[:, 32:32 + k], wbuf[:, 16:16 + k], s_t, b_t, out=ybuf[:, :n])
    y2 = sc.w8a16_linear(_bf(x), torch.from_numpy(codes).cuda(), s_t, b_t)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert bool((ybuf[:, n:] == 7.0).all())            # columns past n untouched
    _check(_f64(y2), x, codes, scale, bias)


@pytest.mark.parametrize("name", ["qkv", "mlp_down"])
def test_full_size_sampled_rows(name):
    # the benchmark shapes at c4's 63,360 rows, in the timed configuration:
    # every output of 96 sampled rows (first, last, random) against the oracle
    m, n, k = workloads.LINEARS[name]
    _say("linear", name, m, n, k)
    x, codes, scale, bias = workloads.linear_inputs(m, n, k)
    y = sc.w8a16_linear(_bf(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(),
                        torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 255, 256, m - 1], rng.integers(0, m, 92)]))
    _check(_f64(y[torch.from_numpy(rows).cuda()]), x, codes, scale, bias, rows=rows)
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("i", range(8))
def test_random_shapes(i):
    # seeded random shapes inside the kernel's tiling rules (n a multiple of
    # 256, k of 64): ragged row tiles, several k steps, with and without bias
    rng = np.random.default_rng(1000 + i)
    m, n, k = int(rng.integers(1, 700)), 256 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 17))
    with_bias = bool(rng.integers(2))
    _say("linear random", m, n, k, with_bias)
    x, codes, scale, bias = workloads.linear_inputs(m, n, k, seed=2000 + i)
    bias = bias if with_bias else None
    y = sc.w8a16_linear(_bf(x), torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda(),
                        torch.from_numpy(bias).cuda() if bias is not None else None)
    torch.cuda.synchronize()
    _check(_f64(y), x, codes, scale, bias)
