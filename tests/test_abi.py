"""C-ABI tests that need no GPU: exports, host-only window selection, and
every argument check (each fails on the host before anything is launched)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "segcausal.h")

sc = pytest.importorskip("segment_causal_dit_amd._lib",
                         reason="libsegcausal.so not built (run __graft_entry__.build())")
lib = sc.raw_library()
FAKE = 0x10000000          # a 16-byte aligned stand-in pointer: never dereferenced


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|int64_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(sc.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    m = re.search(r"#define SEGC_ABI_VERSION \(\(1 << 16\) \| (\d+)\)", open(HEADER).read())
    assert m and lib.segcausal_abi_version() == (1 << 16) | int(m.group(1))
    assert sc.ABI_VERSION == (1 << 16) | int(m.group(1))     # the binding checks it at import


def test_window_select_matches_oracle():
    rng = np.random.default_rng(12)
    for _ in range(200):
        n = int(rng.integers(0, 40))
        ts = rng.permutation(500)[:n].astype(np.int32)
        ts[rng.random(n) < 0.25] = -1
        for b in (0, 1, 5, 18, 64):
            assert list(sc.window_select(ts, b)) == list(oracle.window_select(ts, b))


def test_window_select_errors():
    with pytest.raises(sc.SegcError) as e:
        sc.window_select(np.array([4, 1, 4], np.int32), 2)
    assert e.value.code == sc.SEGC_EINVAL and "t = 4" in str(e.value)
    with pytest.raises(sc.SegcError):
        sc.window_select(np.array([1], np.int32), -1)
    assert list(sc.window_select(np.array([], np.int32), 3)) == []


# ------------------------------------------------------------- rope ----

def _rope(**kw):
    a = dict(x_in=FAKE, x_out=FAKE, n_tok=10, n_heads=16, head_dim=128, st=2048, sh=128,
             pos=FAKE, theta=256.0, dt=16, dh=56, dw=56)
    a.update(kw)
    return lib.rope3d_apply(a["x_in"], a["x_out"], a["n_tok"], a["n_heads"], a["head_dim"],
                            a["st"], a["sh"], a["pos"], a["theta"], a["dt"], a["dh"], a["dw"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(dt=15, dh=57), 2), (dict(dt=16, dh=56, dw=58), 2),
    (dict(dt=0, dh=72), 2), (dict(n_tok=-1), 1), (dict(n_heads=0), 1), (dict(theta=0.0), 1),
    (dict(theta=float("nan")), 1), (dict(st=2047), 1), (dict(sh=-8), 1), (dict(x_in=None), 1),
    (dict(pos=None), 1), (dict(x_out=FAKE + 8), 1), (dict(pos=FAKE + 2), 1),
])
def test_rope_rejects(kw, code):
    assert _rope(**kw) == code
    assert lib.segcausal_last_error().decode()


def test_rope_zero_tokens_is_noop():
    assert _rope(n_tok=0, x_in=None, x_out=None, pos=None) == 0


# ----------------------------------------------------------- append ----

def _cache(**kw):
    c = sc.SegcCache(sc.SEGC_INT8, 16, 128, 880, 8, 0, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _append(cache=None, first=0, n=2, k=FAKE, v=FAKE, kst=2048, ksh=128):
    c = cache if cache is not None else _cache()
    return lib.kv_cache_append(ctypes.byref(c), first, n, k, kst, ksh, v, 2048, 128, None)


@pytest.mark.parametrize("args,code", [
    (dict(cache=_cache(dtype=5)), 1), (dict(cache=_cache(head_dim=64)), 2),
    (dict(cache=_cache(n_slots=0)), 1), (dict(cache=_cache(k=None)), 1),
    (dict(cache=_cache(k_scale=None)), 1), (dict(cache=_cache(v=FAKE + 4)), 1),
    (dict(first=8), 1), (dict(first=-1), 1), (dict(n=9), 1), (dict(n=-1), 1),
    (dict(k=None), 1), (dict(kst=100), 1), (dict(k=FAKE + 2), 1),
])
def test_append_rejects(args, code):
    assert _append(**args) == code


def test_append_null_cache_and_noop():
    assert lib.kv_cache_append(None, 0, 1, FAKE, 2048, 128, FAKE, 2048, 128, None) == 1
    assert _append(n=0, k=None, v=None) == 0
    # a BF16 cache needs no scales
    assert _append(cache=_cache(dtype=sc.SEGC_BF16, k_scale=None, v_scale=None), n=0) == 0


# ------------------------------------------------ window dequantise ----

def _bf16_cache(**kw):
    c = sc.SegcCache(sc.SEGC_BF16, 16, 128, 880, 8, 0, FAKE, FAKE, None, None)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _dequant(src=None, slots=FAKE, n=3, out=None):
    s = src if src is not None else _cache()
    o = out if out is not None else _bf16_cache()
    return lib.kv_window_dequant(ctypes.byref(s), slots, n, ctypes.byref(o), None)


@pytest.mark.parametrize("args,code", [
    (dict(src=_cache(dtype=sc.SEGC_BF16, k_scale=None, v_scale=None)), 1),   # source not INT8
    (dict(out=_cache()), 1),                                                 # output not BF16
    (dict(out=_bf16_cache(n_heads=8)), 1), (dict(out=_bf16_cache(tokens_per_frame=24)), 1),
    (dict(out=_bf16_cache(head_dim=64)), 2), (dict(src=_cache(k_scale=None)), 1),
    (dict(out=_bf16_cache(v=FAKE + 8)), 1), (dict(n=9), 1), (dict(n=-1), 1),
    (dict(slots=None), 1), (dict(slots=FAKE + 2), 1),
    (dict(out=_bf16_cache(n_slots=200000), src=_cache(n_slots=200000), n=200000), 1),  # > 2^31 rows
])
def test_window_dequant_rejects(args, code):
    assert _dequant(**args) == code


def test_window_dequant_null_descriptors_and_noop():
    o = _bf16_cache()
    assert lib.kv_window_dequant(None, FAKE, 1, ctypes.byref(o), None) == 1
    assert lib.kv_window_dequant(ctypes.byref(_cache()), FAKE, 1, None, None) == 1
    assert _dequant(n=0, slots=None) == 0


# -------------------------------------------------------- attention ----

def _attn(segs=((0, 16, 16),), n_cur=None, **kw):
    n_cur = n_cur if n_cur is not None else 64
    starts = [s[0] for s in segs] + [n_cur]
    ss = (ctypes.c_int32 * len(starts))(*starts)
    tl = (ctypes.c_int32 * len(segs))(*[s[1] for s in segs])
    tv = (ctypes.c_int32 * len(segs))(*[s[2] for s in segs])
    a = sc.SegcAttnArgs(FAKE, FAKE, FAKE, FAKE, 256, 128, 256, 128, 256, 128, 256, 128,
                        None, n_cur, 2, 128, len(segs), 0, ss, tl, tv, None, None, 0, 0.088)
    cache = kw.pop("cache", None)
    if cache is not None:
        a.cache = ctypes.pointer(cache)
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.segcausal_joint_attn(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(n_seg=0), 2), (dict(n_seg=17), 2),
    (dict(n_cur=-1), 1), (dict(n_heads=0), 1), (dict(sm_scale=0.0), 1),
    (dict(sm_scale=float("inf")), 1), (dict(q_stride_tok=100), 1), (dict(o_stride_head=-8), 1),
    (dict(q=None), 1), (dict(o=FAKE + 8), 1), (dict(lse=FAKE + 2), 1),
    (dict(n_hist=-1), 1), (dict(n_hist=2), 1),                       # history without a cache
    (dict(n_hist=2, cache=_cache(n_heads=2)), 1),                   # hist_slots missing
    (dict(n_hist=9, cache=_cache(n_heads=2), hist_slots=FAKE), 1),  # more frames than slots
    (dict(n_hist=2, cache=_cache(), hist_slots=FAKE), 1),           # head count mismatch
    (dict(n_hist=2, cache=_cache(n_heads=2, head_dim=64), hist_slots=FAKE), 2),
    (dict(reserved=1), 1), (dict(reserved2=1), 1), (dict(workspace_bytes=-1), 1),
    (dict(workspace=FAKE + 8, workspace_bytes=1 << 20), 1),         # workspace not 16-byte aligned
])
def test_attn_rejects(kw, code):
    assert _attn(**kw) == code
    assert lib.segcausal_last_error().decode()


@pytest.mark.parametrize("segs,n_cur", [
    (((1, 0, 0),), 64),                   # does not start at 0
    (((0, 16, 16),), 70),                 # n_cur disagrees with seg_start[n_seg] below
    (((0, 16, 17),), 64),                 # text_valid > text_len
    (((0, 65, 10),), 64),                 # text longer than the segment
    (((0, 4, 4), (50, 2, 2), (40, 0, 0)), 64),   # not ascending
    (((0, 8, 0),), 8),                    # only padded text: no visible key
])
def test_attn_rejects_bad_segments(segs, n_cur):
    if n_cur == 70:
        starts = (ctypes.c_int32 * 2)(0, 64)
        a = sc.SegcAttnArgs(FAKE, FAKE, FAKE, FAKE, 256, 128, 256, 128, 256, 128, 256, 128,
                            None, 70, 2, 128, 1, 0, starts, (ctypes.c_int32 * 1)(16),
                            (ctypes.c_int32 * 1)(16), None, None, 0, 0.088)
        assert lib.segcausal_joint_attn(ctypes.byref(a), None) == 1
        return
    assert _attn(segs=segs, n_cur=n_cur) == 1


def _ws_bytes(n_cur, n_heads, segs, n_hist=0, cache=None, n_cu=256):
    starts = [sg[0] for sg in segs] + [n_cur]
    a = sc.SegcAttnArgs()
    a.n_cur, a.n_heads, a.head_dim, a.n_seg = n_cur, n_heads, 128, len(segs)
    a.seg_start = (ctypes.c_int32 * len(starts))(*starts)
    a.seg_text_len = (ctypes.c_int32 * len(segs))(*[sg[1] for sg in segs])
    a.seg_text_valid = (ctypes.c_int32 * len(segs))(*[sg[2] for sg in segs])
    a.n_hist = n_hist
    if cache is not None:
        a.cache = ctypes.pointer(cache)
    return lib.segcausal_joint_attn_workspace_bytes(ctypes.byref(a), n_cu)


def test_attn_workspace_bytes_split_plan():
    # c4: 249 query tiles x 16 heads = 3,984 workgroups on 256 compute units:
    # the last 144 tiles split 7 ways (the cost model's pick), each split
    # keeping an fp32 256 x 128 O and 256 (max, sum) pairs
    seg = [(0, 256, 256)]
    bf16_360 = _cache(dtype=0, n_slots=360, tokens_per_frame=880)
    c4 = dict(n_cur=63616, n_heads=16, segs=seg, n_hist=288)
    assert _ws_bytes(cache=bf16_360, **c4) == 144 * 7 * 256 * 130 * 4
    # the same history held as INT8 (one-tile schedule) and a segment structure never split
    assert _ws_bytes(cache=_cache(dtype=1, n_slots=360, tokens_per_frame=880), **c4) == 0
    assert _ws_bytes(63616, 16, [(0, 256, 200)], 288, bf16_360) == 0
    assert _ws_bytes(63616, 16, [(0, 256, 256), (32000, 256, 256)], 288, bf16_360) == 0
    # a whole number of rounds, or fewer than 4 whole rounds (c1, c2: they measured slower split)
    assert _ws_bytes(256 * 16, 16, seg, 288, bf16_360) == 0
    assert _ws_bytes(7296, 16, seg) == 0
    assert _ws_bytes(7296, 16, seg, 18, bf16_360) == 0
    # 65 query tiles x 16 heads: 4 rounds + 16 tiles, split 8 ways
    assert _ws_bytes(65 * 256, 16, seg, 20, bf16_360) == 16 * 8 * 256 * 130 * 4
    assert _ws_bytes(65 * 256, 16, seg, 20, bf16_360, n_cu=1040) == 0
    # the GPU split tests' shapes: 96, 188 and 56 remaining tiles in 5, 4 and 4 ranges
    assert _ws_bytes(70 * 256 - 100, 16, seg) == 96 * 5 * 256 * 130 * 4
    assert _ws_bytes(100 * 256 + 37, 12, seg, 4, _cache(dtype=0, n_slots=6, tokens_per_frame=880)) == 188 * 4 * 256 * 130 * 4
    assert _ws_bytes(135 * 256, 8, seg, 10, _cache(dtype=0, n_slots=12, tokens_per_frame=880)) == 56 * 4 * 256 * 130 * 4
    assert lib.segcausal_joint_attn_workspace_bytes(None, 256) == -1


def test_attn_noop_and_null_args():
    assert lib.segcausal_joint_attn(None, None) == 1
    assert _attn(segs=((0, 0, 0),), n_cur=0, q=None, k=None, v=None, o=None) == 0


# ----------------------------------------------------- attention backward ----

FAKE2 = 0x20000000        # more aligned stand-ins, spaced so the spans never meet
_BWD_PTRS = ("q", "k", "v", "o", "dout", "dq", "dk", "dv")


def _attn_bwd(segs=((0, 16, 16),), n=64, **kw):
    starts = [s[0] for s in segs] + [n]
    ss = (ctypes.c_int32 * len(starts))(*starts)
    tl = (ctypes.c_int32 * max(1, len(segs)))(*[s[1] for s in segs])
    tv = (ctypes.c_int32 * max(1, len(segs)))(*[s[2] for s in segs])
    ptrs = [FAKE2 + i * 0x1000000 for i in range(len(_BWD_PTRS))]
    a = sc.SegcAttnBwdArgs(*(ptrs + [256, 128] * 8 +
                             [FAKE2 + 8 * 0x1000000, FAKE2 + 9 * 0x1000000, n, 2, 128, len(segs), 0,
                              ss, tl, tv, 0.088]))
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.segcausal_joint_attn_bwd(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(n_seg=0), 2), (dict(n_seg=17), 2),
    (dict(n=-1), 1), (dict(n=1 << 30), 1), (dict(n_heads=0), 1), (dict(sm_scale=0.0), 1),
    (dict(sm_scale=float("nan")), 1), (dict(q_stride_tok=100), 1), (dict(dv_stride_head=-8), 1),
    (dict(do_stride_tok=4), 1), (dict(q=None), 1), (dict(dout=None), 1), (dict(dk=FAKE2 + 8), 1),
    (dict(lse=None), 1), (dict(delta=None), 1), (dict(lse=FAKE2 + 2), 1),
    (dict(delta=FAKE2 + 9 * 0x1000000 + 1), 1),
    (dict(dq=FAKE2), 1),                         # dq in place of q
    (dict(dv=FAKE2 + 6 * 0x1000000), 1),         # dv and dk the same buffer
    (dict(delta=FAKE2 + 3 * 0x1000000), 1),      # delta in place of o
    (dict(dk=FAKE2 + 8 * 0x1000000), 1),         # dk in place of lse
])
def test_attn_bwd_rejects(kw, code):
    assert _attn_bwd(**kw) == code
    assert lib.segcausal_last_error().decode()


@pytest.mark.parametrize("segs,n", [
    (((1, 0, 0),), 64), (((0, 16, 17),), 64), (((0, 65, 10),), 64),
    (((0, 4, 4), (50, 2, 2), (40, 0, 0)), 64),
    (((0, 8, 0),), 8),                           # only padded text: no visible key
    (((0, 8, 8), (8, 8, 0)), 16),                # second segment: only padded text
])
def test_attn_bwd_rejects_bad_segments(segs, n):
    assert _attn_bwd(segs=segs, n=n) == 1


def test_attn_bwd_noop_and_null_args():
    assert lib.segcausal_joint_attn_bwd(None, None) == 1
    assert _attn_bwd(segs=((0, 0, 0),), n=0, q=None, k=None, v=None, o=None, dout=None,
                     dq=None, dk=None, dv=None, lse=None, delta=None) == 0
    # the binding checks shapes before the library is reached
    import torch
    x = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    lse = torch.zeros(2, 4)
    with pytest.raises(ValueError):
        sc.segcausal_joint_attn_bwd(x, x, x[:3], x, x, lse, [(0, 0, 0)], 0.088)


# ------------------------------------------------------------ archive ----

def _frames(*xs):
    return (ctypes.c_int32 * max(1, len(xs)))(*xs)


def _fetch(archive=None, af=(0, 1), cache=None, slots=(2, 3), n=None):
    a = archive if archive is not None else _cache(n_slots=40)
    c = cache if cache is not None else _cache()
    return lib.kv_archive_fetch(ctypes.byref(a) if a != "null" else None, _frames(*af),
                                ctypes.byref(c) if c != "null" else None, _frames(*slots),
                                len(af) if n is None else n, None)


@pytest.mark.parametrize("kw", [
    dict(archive="null"), dict(cache="null"),
    dict(archive=_cache(n_slots=40, dtype=sc.SEGC_BF16, k_scale=None, v_scale=None)),   # dtype differs
    dict(archive=_cache(n_slots=40, n_heads=8)), dict(archive=_cache(n_slots=40, tokens_per_frame=100)),
    dict(n=-1),
    dict(af=(0, 40)), dict(af=(-1, 0)), dict(slots=(2, 8)), dict(slots=(3, 3)),   # range, duplicate
    dict(af=(0, 1), slots=(2, 3)),      # stand-in pointers are neither pinned host nor device memory
])
def test_archive_rejects(kw):
    assert _fetch(**kw) == sc.SEGC_EINVAL
    assert lib.segcausal_last_error().decode()


def test_archive_store_checks_and_noop():
    a, c = _cache(n_slots=40), _cache()
    assert lib.kv_archive_store(ctypes.byref(c), _frames(9), ctypes.byref(a), _frames(0), 1, None) == 1
    assert lib.kv_archive_store(ctypes.byref(c), _frames(1, 2), ctypes.byref(a), _frames(5, 5), 2, None) == 1
    assert lib.kv_archive_store(ctypes.byref(c), None, ctypes.byref(a), None, 0, None) == 0
    assert _fetch(af=(), slots=(), n=0) == 0
    with pytest.raises(ValueError):
        sc.kv_archive_fetch(sc.KVCache.__new__(sc.KVCache), [0, 1], None, [0])


# -------------------------------------------------------- W8A16 linear ----

def _lin(**kw):
    a = dict(x=FAKE, ldx=2048, w=FAKE, ldw=2048, s=FAKE, b=None, y=FAKE2, ldy=6144, m=100, n=6144, k=2048,
             ws=FAKE2 + 0x4000000)
    a.update(kw)
    return lib.w8a16_linear(a["x"], a["ldx"], a["w"], a["ldw"], a["s"], a["b"], a["y"], a["ldy"], a["m"],
                            a["n"], a["k"], a["ws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(m=-1), 1), (dict(m=1 << 31), 1), (dict(n=-256), 1), (dict(k=-64), 1),
    (dict(n=300), 2), (dict(k=100), 2), (dict(k=0), 2),
    (dict(ldx=2040), 1), (dict(ldx=2052), 1), (dict(ldw=2056), 1), (dict(ldy=6146), 1), (dict(ldy=100), 1),
    (dict(x=None), 1), (dict(w=None), 1), (dict(s=None), 1), (dict(y=None), 1),
    (dict(x=FAKE + 8), 1), (dict(s=FAKE + 4), 1), (dict(b=FAKE + 4), 1), (dict(y=FAKE2 + 4), 1),
    (dict(y=FAKE), 1),                                   # in place over x
    (dict(ws=None), 1), (dict(ws=FAKE2 + 0x4000000 + 8), 1),
    (dict(ws=FAKE2 + 4096), 1),                          # workspace overlaps y
])
def test_w8a16_rejects(kw, code):
    assert _lin(**kw) == code
    assert lib.segcausal_last_error().decode()


def test_w8a16_noop():
    assert _lin(m=0, x=None, w=None, s=None, y=None) == 0
    assert _lin(n=0, ldy=0, x=None, w=None, s=None, y=None) == 0


# ------------------------------------------------ camera cross-attention ----

def _cam(**kw):
    a = sc.SegcCameraArgs(FAKE, FAKE2, FAKE2 + 0x1000000, FAKE2 + 0x2000000, 2048, 128, 2048, 128, 2048, 128,
                          1760, 16, 128, 880, 1, 0.088)
    for k, v in kw.items():
        setattr(a, k, v)
    return lib.camera_cross_attn(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(n_tok=-1), 1), (dict(n_tok=1 << 31), 1), (dict(n_heads=0), 1),
    (dict(tokens_per_chunk=0), 1), (dict(t_cam=0), 1), (dict(t_cam=5000), 1), (dict(sm_scale=0.0), 1),
    (dict(q_stride_tok=100), 1), (dict(kv_stride_head=-8), 1), (dict(k=None), 1), (dict(o=None), 1),
    (dict(t_cam=2, q=None), 1), (dict(v=FAKE2 + 8), 1), (dict(o=FAKE2), 1),
])
def test_camera_rejects(kw, code):
    assert _cam(**kw) == code
    assert lib.segcausal_last_error().decode()


def test_camera_noop():
    assert _cam(n_tok=0, q=None, k=None, v=None, o=None) == 0
    assert lib.camera_cross_attn(None, None) == 1


# ---------------------------------------------- binding matches the header ----

_C_TYPES = {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "float": ctypes.c_float,
            "double": ctypes.c_double}


def _header_structs():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"typedef struct (\w+) \{(.*?)\} \w+;", src, flags=re.S):
        fields = []
        for decl in m.group(2).split(";"):
            decl = decl.strip()
            if not decl:
                continue
            typ, names = re.match(r"(.*?)(\**\s*\w+(?:\s*,\s*\**\s*\w+)*)$", decl).groups()
            for nm in names.split(","):
                ptr = "*" in typ or "*" in nm
                fields.append((nm.replace("*", "").strip(), "ptr" if ptr else typ.replace("const", "").strip()))
        out[m.group(1)] = fields
    return out


@pytest.mark.parametrize("cname,py", [
    ("segc_cache", "SegcCache"), ("segc_attn_args", "SegcAttnArgs"),
    ("segc_attn_bwd_args", "SegcAttnBwdArgs"), ("segc_camera_args", "SegcCameraArgs"),
])
def test_binding_structs_match_header(cname, py):
    want = _header_structs()[cname]
    got = getattr(sc, py)._fields_
    assert [n for n, _ in got] == [n for n, _ in want], cname
    for (n, t), (_, ct) in zip(got, want):
        if ct == "ptr":
            assert ctypes.sizeof(t) == ctypes.sizeof(ctypes.c_void_p), n
        else:
            assert t is _C_TYPES[ct], (n, ct, t)


def test_binding_argtypes_match_header_arity():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for m in re.finditer(r"^(?:int|const char\*)\s+(\w+)\s*\((.*?)\);", src, flags=re.M | re.S):
        name, params = m.group(1), m.group(2).strip()
        n_params = 0 if params in ("", "void") else params.count(",") + 1
        argtypes = getattr(lib, name).argtypes
        assert len(argtypes or []) == n_params, (name, n_params, argtypes)


@pytest.mark.parametrize("call", [
    lambda: _attn(n_cur=1 << 30, n_heads=2),        # 2^31 (row, head) pairs
    lambda: _attn(n_cur=(1 << 28) + 1, n_heads=8),
    lambda: _attn_bwd(n=1 << 29, n_heads=4),
    lambda: _cam(n_tok=1 << 28, n_heads=8),
])
def test_pair_count_beyond_32_bit_grid_rejected(call):
    # every size is inside its own range; the product of rows and heads is not
    assert call() == 1
    assert "2^31" in lib.segcausal_last_error().decode()


# ------------------------------------------- binding shape/device checks ----

def _bf16(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_attention_refuses_mismatched_rows_or_heads():
    # the C ABI sees only pointers and strides: the binding is the one place
    # that knows tensor extents, so k, v and out must match q's [n, H]
    x = _bf16(4, 2, 128)
    cases = [dict(k=x[:3]), dict(v=_bf16(4, 3, 128)), dict(out=x[:2]), dict(out=_bf16(4, 1, 128))]
    for bad in cases:
        a = dict(q=x, k=x, v=x, out=None)
        a.update(bad)
        with pytest.raises(ValueError, match="like q"):
            sc.segcausal_joint_attn(a["q"], a["k"], a["v"], [(0, 0, 0)], 1.0, out=a["out"])


def test_binding_refuses_host_tensors():
    # a host pointer handed to a kernel would fault the GPU: refused before the call
    import torch
    x = _bf16(4, 2, 128)
    with pytest.raises(ValueError, match="GPU"):
        sc.segcausal_joint_attn(x, x, x, [(0, 0, 0)], 1.0)
    with pytest.raises(ValueError, match="GPU"):
        sc.segcausal_joint_attn_bwd(x, x, x, x, x, torch.zeros(2, 4), [(0, 0, 0)], 0.088)
    with pytest.raises(ValueError, match="GPU"):
        sc.rope3d_apply(x, torch.zeros(4, 3, dtype=torch.int32))
    cache = sc.KVCache(2, 2, 4, "int8", device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        sc.kv_cache_append(cache, 0, x, x)
    win = sc.KVCache(2, 2, 4, "bf16", device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        sc.kv_window_dequant(cache, torch.zeros(2, dtype=torch.int32), win)
    with pytest.raises(ValueError, match="GPU"):
        sc.w8a16_linear(_bf16(4, 64), torch.zeros(256, 64, dtype=torch.int8), torch.ones(256))
    with pytest.raises(ValueError, match="GPU"):
        sc.camera_cross_attn(x, x[:1], x[:1], 4, 1.0)


def test_binding_append_refuses_other_head_counts():
    cache = sc.KVCache(2, 2, 4, "int8", device="cpu")
    with pytest.raises(ValueError, match="heads"):
        sc.kv_cache_append(cache, 0, _bf16(4, 3, 128), _bf16(4, 3, 128))
    with pytest.raises(ValueError, match="heads"):
        sc.kv_cache_append(cache, 0, _bf16(4, 2, 128), _bf16(4, 1, 128))


def test_binding_camera_refuses_other_head_counts():
    x = _bf16(8, 2, 128)
    with pytest.raises(ValueError, match="like q"):
        sc.camera_cross_attn(x, _bf16(2, 3, 128), _bf16(2, 3, 128), 4, 1.0)
    with pytest.raises(ValueError, match="like q"):
        sc.camera_cross_attn(x, x[:2], x[:2], 4, 1.0, out=_bf16(8, 1, 128))


def test_binding_hist_slots_without_cache_refused():
    import torch
    x = _bf16(4, 2, 128)
    with pytest.raises(ValueError, match="cache"):
        sc.segcausal_joint_attn(x, x, x, [(0, 0, 0)], 1.0, hist_slots=torch.zeros(1, dtype=torch.int32))


# --------------------------------------- 32-bit offsets, alignment, EHIP ----

MAX_STRIDE = 1 << 26


def test_header_stride_bound():
    m = re.search(r"#define SEGC_MAX_STRIDE \(\(int64_t\)1 << (\d+)\)", open(HEADER).read())
    assert m and (1 << int(m.group(1))) == MAX_STRIDE


@pytest.mark.parametrize("call", [
    lambda: _attn(k_stride_tok=MAX_STRIDE), lambda: _attn(v_stride_tok=MAX_STRIDE),
    lambda: _attn(q_stride_head=MAX_STRIDE), lambda: _attn(o_stride_tok=MAX_STRIDE),
    lambda: _attn_bwd(q_stride_tok=MAX_STRIDE), lambda: _attn_bwd(do_stride_tok=MAX_STRIDE),
    lambda: _attn_bwd(k_stride_tok=MAX_STRIDE), lambda: _attn_bwd(dv_stride_head=MAX_STRIDE),
    lambda: _rope(st=MAX_STRIDE), lambda: _append(kst=MAX_STRIDE), lambda: _append(ksh=MAX_STRIDE),
    lambda: _cam(kv_stride_tok=MAX_STRIDE), lambda: _cam(o_stride_head=MAX_STRIDE),
    lambda: _lin(ldx=MAX_STRIDE), lambda: _lin(ldw=MAX_STRIDE), lambda: _lin(ldy=MAX_STRIDE),
])
def test_strides_that_would_wrap_32_bit_offsets_rejected(call):
    # the kernels form row offsets inside a staged group of up to 16 rows in
    # 32 bits; 15 * 2 bytes * 2^26 stays below 2^31, 2^26 itself is refused
    assert call() == sc.SEGC_EINVAL
    assert "2^26" in lib.segcausal_last_error().decode()


def test_attn_rejects_misaligned_hist_slots():
    # the kernel reads the slot list with 4-byte scalar loads
    assert _attn(n_hist=2, cache=_cache(n_heads=2), hist_slots=FAKE + 2) == sc.SEGC_EINVAL
    assert "hist_slots" in lib.segcausal_last_error().decode()


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_gpu_present(), reason="with a GPU these stand-in pointers would reach a kernel")
def test_launch_without_a_device_reports_hip_error():
    # well-formed calls (the largest accepted strides among them) pass every
    # host check; with no device the launch fails and the status is SEGC_EHIP
    # with HIP's own message
    calls = [
        lambda: _rope(st=MAX_STRIDE - 8, sh=MAX_STRIDE - 8),
        lambda: _append(kst=MAX_STRIDE - 8),
        lambda: _dequant(),
        lambda: _attn(k_stride_tok=MAX_STRIDE - 8),
        lambda: _attn_bwd(),
        lambda: _lin(ldx=MAX_STRIDE - 8, ws=0x100000000000),   # x then spans 13 GB
        lambda: _cam(),
    ]
    for call in calls:
        assert call() == sc.SEGC_EHIP
        msg = lib.segcausal_last_error().decode()
        assert "launch" in msg and len(msg) > len("launch: ")


def test_noalloc_backward_refuses_beyond_its_scratch_on_the_host():
    # n x n_heads above the 2^23 delta entries of the device scratch: refused
    # before any device access (stand-in pointers are never touched)
    starts = (ctypes.c_int32 * 2)(0, (1 << 22) + 1)
    ptrs = [FAKE2 + i * 0x1000000 for i in range(len(_BWD_PTRS))]
    a = sc.SegcAttnBwdArgs(*(ptrs + [256, 128] * 8 +
                             [FAKE2 + 8 * 0x1000000, None, (1 << 22) + 1, 2, 128, 1, 0,
                              starts, (ctypes.c_int32 * 1)(0), (ctypes.c_int32 * 1)(0), 0.088]))
    assert lib.segcausal_joint_attn_bwd_noalloc(ctypes.byref(a), None) == sc.SEGC_EINVAL
    assert "2^23" in lib.segcausal_last_error().decode()
    assert lib.segcausal_joint_attn_bwd_noalloc(None, None) == sc.SEGC_EINVAL
    # n == 0 is a no-op, and n < 0 is refused, both without a device
    a.n, a.seg_start = 0, (ctypes.c_int32 * 2)(0, 0)
    assert lib.segcausal_joint_attn_bwd_noalloc(ctypes.byref(a), None) == sc.SEGC_OK
    a.n = -1
    assert lib.segcausal_joint_attn_bwd_noalloc(ctypes.byref(a), None) == sc.SEGC_EINVAL
