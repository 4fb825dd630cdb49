"""Linear layer with INT8 weights and BF16 activations (W8A16).

Source: model card, assets table (the quantized distilled DiT stores weights
in INT8 while the DiT's linear computation stays BF16) and section
"Single-GPU Low-Memory Inference" (INT8 DiT storage, BF16 linear compute);
Explainer, architecture notes (hidden size 2,048, feed-forward 8,192).
Reading: each output channel n has one fp32 scale, weight value =
code[n, k] * scale[n] (codes in [-127, 127]); the linear is
    y[m, n] = sum_k x[m, k] * code[n, k] * scale[n] (+ bias[n]),
evaluated here exactly in float64 from the bf16 activations.

Pinned by a pure-Python triple loop on tiny shapes and by special cases
(one-hot rows, unit codes) in tests/test_oracle_basic.py.
"""

import numpy as np


def w8a16_linear(x, codes, scale, bias=None):
    """float64 [M, N] = x [M, K] @ (codes [N, K] * scale [N, None]).T (+ bias [N])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
