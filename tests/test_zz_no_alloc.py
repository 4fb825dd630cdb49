"""The allocation-free backward entry point against the one that takes a
workspace, through the C ABI, on the GPU.

segcausal_joint_attn_bwd_noalloc runs the same kernels as
segcausal_joint_attn_bwd with delta in the library's device scratch instead
of a caller-owned buffer, so its gradients must equal the workspace form's
bit for bit. Two calls in a row, the second on a smaller problem, check that
the scratch left by the first call does not leak into the second; a third
form checks the size limit, refused on the host.
"""

import ctypes
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
sc = pytest.importorskip("segment_causal_dit_amd._lib")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def _problem(name):
    cfg = workloads.ALL[name]
    inp = workloads.make_inputs(cfg)
    q, k, v = _bf(inp.q), _bf(inp.k), _bf(inp.v)
    do = _bf(workloads.upstream_grad(cfg))
    lse = torch.empty((cfg.n_heads, cfg.n_cur), dtype=torch.float32, device="cuda")
    o = sc.segcausal_joint_attn(q, k, v, inp.segments, cfg.sm_scale, lse=lse)
    return cfg, inp, q, k, v, o, do, lse


@pytest.mark.parametrize("first,second", [("bwd_mid", "bwd_small")])
def test_noalloc_backward_equals_workspace_form_on_two_calls(first, second):
    for name in (first, second):
        _say("no-alloc backward", name)
        cfg, inp, q, k, v, o, do, lse = _problem(name)
        want = sc.segcausal_joint_attn_bwd(q, k, v, o, do, lse, inp.segments, cfg.sm_scale)
        # outputs pre-filled with garbage: every element must be written
        outs = [torch.full_like(q, 7.0) for _ in range(3)]
        got = sc.segcausal_joint_attn_bwd_noalloc(q, k, v, o, do, lse, inp.segments, cfg.sm_scale,
                                                  dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        for nm, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.isfinite(g.float()).all(), (name, nm)
            assert torch.equal(g, w), (name, nm, (g.float() - w.float()).abs().max().item())


def test_noalloc_backward_refuses_more_than_the_scratch_holds():
    lib = sc.raw_library()
    x = torch.zeros((8, 2, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    args = sc.SegcAttnBwdArgs(*([x.data_ptr()] * 8 + [2 * 128, 128] * 8 +
                                [lse.data_ptr(), None, (1 << 22) + 1, 2, 128, 1, 0,
                                 (ctypes.c_int32 * 2)(0, (1 << 22) + 1), (ctypes.c_int32 * 1)(0),
                                 (ctypes.c_int32 * 1)(0), 0.088]))
    assert lib.segcausal_joint_attn_bwd_noalloc(ctypes.byref(args), None) == sc.SEGC_EINVAL
    assert "2^23" in lib.segcausal_last_error().decode()
