"""Shared test plumbing: run one workload through the HIP library (GPU chain)
and through the fp64 oracle (oracle chain) from the same seeded inputs."""

import numpy as np

import oracle
import workloads
from workloads import HEAD_DIM


def f64(bits):
    return oracle.bf16_bits_to_f64(bits)


# --------------------------------------------------------------- oracle ----

def oracle_inputs(inp):
    """Oracle's own RoPE of the current video rows: (q, k, v) float64."""
    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    if len(inp.video_rows):
        k[inp.video_rows] = oracle.rope3d_bf16(inp.k[inp.video_rows], inp.pos)
        q[inp.video_rows] = oracle.rope3d_bf16(inp.q[inp.video_rows], inp.pos)
    return q, k, v


def oracle_cache(inp):
    """Oracle's cache contents for the history frames, slot-major.

    Returns (k, v, k_scale, v_scale): INT8 codes + fp32 scales, or float64
    bf16 values with scales None.
    """
    cfg = inp.cfg
    g, h, nf = cfg.tokens_per_frame, cfg.n_heads, len(cfg.hist_t)
    kr = oracle.rope3d_bf16(inp.hist_k, inp.hist_pos)
    ck = kr.reshape(nf, g, h, HEAD_DIM).transpose(0, 2, 1, 3)
    cv = f64(inp.hist_v).reshape(nf, g, h, HEAD_DIM).transpose(0, 2, 1, 3)
    if cfg.cache_dtype == "int8":
        kc, ks = oracle.quantise_int8(ck)
        vc, vs = oracle.quantise_int8(cv)
        return kc, vc, ks, vs
    return ck, cv, None, None


def oracle_chain(inp, rows=None, cache=None):
    """Reference attention output (o, lse) from pre-RoPE inputs."""
    cfg = inp.cfg
    q, k, v = oracle_inputs(inp)
    segs = [oracle.Segment(*s) for s in inp.segments]
    hk = hv = None
    if len(cfg.hist_t):
        ck, cv, ks, vs = cache if cache is not None else oracle_cache(inp)
        slots = oracle.window_select(inp.slot_t, cfg.window)
        hk, hv = oracle.history_keys(ck, cv, slots, ks, vs)
    if rows is None:
        return oracle.joint_attn(q, k, v, segs, hk, hv, cfg.sm_scale)
    return oracle.joint_attn_rows(q, k, v, segs, rows, hk, hv, cfg.sm_scale)


# ------------------------------------------------------------------ GPU ----

class GpuRun:
    pass


def gpu_chain(inp, with_lse=True):
    """The hot path through the C ABI: RoPE (current video Q/K and history K),
    INT8/BF16 append of the history, window select, attention, then the
    append of the current video K/V when the workload does so."""
    import torch
    import segment_causal_dit_amd as sc

    cfg = inp.cfg
    dev = torch.device("cuda")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    r = GpuRun()
    r.q, r.k, r.v = bf(inp.q), bf(inp.k), bf(inp.v)
    pos = torch.from_numpy(inp.pos).to(dev)
    pr = 0
    for (start, tl, _), s in zip(inp.segments, cfg.segments):
        n = s.n_frames * cfg.tokens_per_frame
        if n:
            a, b = start + tl, start + tl + n
            sc.rope3d_apply(r.q[a:b], pos[pr:pr + n])
            sc.rope3d_apply(r.k[a:b], pos[pr:pr + n])
        pr += n
    r.cache = None
    r.slots = np.zeros(0, np.int32)
    hist = None
    nf = len(cfg.hist_t)
    if nf:
        r.cache = sc.KVCache(cfg.n_slots, cfg.n_heads, cfg.tokens_per_frame, cfg.cache_dtype, dev)
        hk = bf(inp.hist_k)
        sc.rope3d_apply(hk, torch.from_numpy(inp.hist_pos).to(dev))
        sc.kv_cache_append(r.cache, 0, hk, bf(inp.hist_v))
        r.cache.slot_t[:] = inp.slot_t
        r.slots = sc.window_select(r.cache.slot_t, cfg.window)
        hist = torch.from_numpy(r.slots).to(dev)
    r.lse = torch.empty((cfg.n_heads, cfg.n_cur), dtype=torch.float32, device=dev) if with_lse else None
    r.o = sc.segcausal_joint_attn(r.q, r.k, r.v, inp.segments, cfg.sm_scale, cache=r.cache,
                                  hist_slots=hist, lse=r.lse)
    if cfg.append:
        # the current segment's video K/V, after RoPE, into the next free slots
        (start, tl, _), s = inp.segments[0], cfg.segments[0]
        n = s.n_frames * cfg.tokens_per_frame
        sc.kv_cache_append(r.cache, nf, r.k[start + tl:start + tl + n], r.v[start + tl:start + tl + n],
                           t_first=s.t0)
    torch.cuda.synchronize()
    return r


def to_f64(t):
    import torch
    return t.to(torch.float32).cpu().numpy().astype(np.float64)


def bits(t):
    """bf16 device tensor -> uint16 numpy bit patterns."""
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# Attention bars. The stated tolerance for unit-variance inputs is absolute:
# max |err| <= 1e-2, mean |err| <= 1e-3. At long contexts the output itself
# shrinks (|o| ~ sqrt(e / keys): rms 2.9e-3 over 317,056 keys), so an absolute
# mean bar of 1e-3 would pass a kernel that dropped a tenth of the keys. The
# derived bar therefore also holds each (row, head) to its own size, the rms of
# its 128 reference values. Error sources: every product p_j v_j carries the
# bf16 rounding of p (relative 2^-9), dequantised INT8 keys and values carry
# relative 2^-9 each, and the output is rounded to bf16 once; each shifts an
# output element by a fraction of its row's rms that does not shrink with the
# key count. Exact arithmetic with just these roundings, over c4's 253,440
# INT8 history keys (test_parity_bars.py), errs by mean 2^-8.5 and max 2^-6.0
# of the row rms; bars: mean 2^-7 and max 2^-4 (2.8x and 4x that), which one
# missing 64-key tile of 3,960 already exceeds (mean 2^-6.4).
MAX_ERR, MEAN_ERR = 1e-2, 1e-3
REL_MAX, REL_MEAN = 2.0 ** -4, 2.0 ** -7


class AttnErr:
    """Absolute and row-relative error of an attention output against the oracle."""

    def __init__(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        d = np.abs(got - ref)
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        rel = d / np.maximum(rms, 1e-300)
        self.max, self.mean = float(d.max()), float(d.mean())
        self.rel_max, self.rel_mean = float(rel.max()), float(rel.mean())

    def ok(self):
        return (self.max <= MAX_ERR and self.mean <= MEAN_ERR
                and self.rel_max <= REL_MAX and self.rel_mean <= REL_MEAN)

    def __repr__(self):
        return ("max %.3e mean %.3e | of row rms: max %.3e (2^%.1f) mean %.3e (2^%.1f)"
                % (self.max, self.mean, self.rel_max, np.log2(max(self.rel_max, 1e-300)),
                   self.rel_mean, np.log2(max(self.rel_mean, 1e-300))))


def attn_errors(got, ref):
    return AttnErr(got, ref)
