"""GPU tests of the CPU history archive (kv_archive_store / kv_archive_fetch):
frames moved between device caches and a pinned host archive must equal the
oracle's indexed copy byte for byte, also while an attention runs on another
stream."""

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


def _tensors(c):
    return [t for t in (c.k, c.v, c.k_scale, c.v_scale) if t is not None]


def _np(t):
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy()


def _filled_cache(cfg, n_slots, dtype, seed):
    """A device cache whose slots hold seeded frames (codes + scales, or bf16)."""
    c = sc.KVCache(n_slots, cfg.n_heads, cfg.tokens_per_frame, dtype, "cuda")
    if dtype == "int8":
        kc, vc, ks, vs = workloads.direct_int8_cache(cfg, n_slots)
        for t, a in zip(_tensors(c), (kc, vc, ks, vs)):
            t.copy_(torch.from_numpy(a))
    else:
        shape = (n_slots, cfg.n_heads, cfg.tokens_per_frame, 128)
        for t, k in ((c.k, seed), (c.v, seed + 1)):
            bits = workloads.normal_bf16(k, shape)
            t.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    return c


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_store_then_fetch_bit_exact(dtype):
    _say("archive", dtype)
    cfg = workloads.ALL["mid_int8"]
    src = _filled_cache(cfg, 8, dtype, 11)
    arch = sc.KVCache.archive(12, cfg.n_heads, cfg.tokens_per_frame, dtype)
    dst = sc.KVCache(6, cfg.n_heads, cfg.tokens_per_frame, dtype, "cuda")
    # a run (3, 4 -> 8, 9) merges into one copy per tensor; the rest are single frames
    store_slots, store_frames = [5, 2, 3, 4], [0, 7, 8, 9]
    fetch_frames, fetch_slots = [9, 0, 7, 8], [1, 2, 3, 4]
    sc.kv_archive_store(src, store_slots, arch, store_frames)
    sc.kv_archive_fetch(arch, fetch_frames, dst, fetch_slots)
    torch.cuda.synchronize()
    for ts, ta, td in zip(_tensors(src), _tensors(arch), _tensors(dst)):
        s_np = _np(ts)
        want_arch = oracle.move_frames(s_np, store_slots, np.zeros((12,) + s_np.shape[1:], s_np.dtype),
                                       store_frames)
        assert np.array_equal(_np(ta), want_arch)
        want_dst = oracle.move_frames(want_arch, fetch_frames, np.zeros((6,) + s_np.shape[1:], s_np.dtype),
                                      fetch_slots)
        assert np.array_equal(_np(td), want_dst)


def test_fetch_on_a_copy_stream_during_attention():
    # the next window's frames arrive on a copy stream while the attention
    # reads other slots of the same cache: both results stay exact
    cfg = workloads.ALL["mid_int8"]
    inp = workloads.make_inputs(cfg)
    cache = _filled_cache(cfg, 10, "int8", 0)
    arch = sc.KVCache.archive(20, cfg.n_heads, cfg.tokens_per_frame, "int8")
    src = _filled_cache(cfg, 20, "int8", 0)
    sc.kv_archive_store(src, list(range(20)), arch, list(range(20)))
    torch.cuda.synchronize()

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    hist = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    ref = sc.segcausal_joint_attn(q, k, v, inp.segments, cfg.sm_scale, cache=cache, hist_slots=hist)
    torch.cuda.synchronize()
    copy_stream = torch.cuda.Stream()
    frames, slots = [13, 14, 15, 2, 19], [5, 6, 7, 8, 9]
    for _ in range(3):
        for t in _tensors(cache):
            t[5:].zero_()
        copy_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(copy_stream):
            sc.kv_archive_fetch(arch, frames, cache, slots, stream=copy_stream)
        out = sc.segcausal_joint_attn(q, k, v, inp.segments, cfg.sm_scale, cache=cache, hist_slots=hist)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        for tc, ta in zip(_tensors(cache), _tensors(arch)):
            assert np.array_equal(_np(tc)[slots], _np(ta)[frames])


def test_unpinned_or_device_archive_is_rejected():
    cfg = workloads.ALL["mid_int8"]
    cache = sc.KVCache(4, cfg.n_heads, cfg.tokens_per_frame, "int8", "cuda")
    pageable = sc.KVCache(4, cfg.n_heads, cfg.tokens_per_frame, "int8", "cpu")
    on_device = sc.KVCache(4, cfg.n_heads, cfg.tokens_per_frame, "int8", "cuda")
    for bad in (pageable, on_device):
        with pytest.raises(sc.SegcError) as e:
            sc.kv_archive_fetch(bad, [0], cache, [1])
        assert e.value.code == sc.SEGC_EINVAL
    pinned = sc.KVCache.archive(4, cfg.n_heads, cfg.tokens_per_frame, "int8")
    with pytest.raises(sc.SegcError):                 # the cache side must be device memory
        sc.kv_archive_store(pinned, [0], pinned, [1])
