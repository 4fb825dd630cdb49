"""Thin ctypes binding of libsegcausal.so (the C ABI in include/segcausal.h).

Argument marshalling only: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the library's
HIP kernels. The names match the C entry points. If the library has not been
built this module raises ImportError: there is no fallback.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SEGCAUSAL_LIB names another build of the same library (e.g. one with
# host-side sanitizers); by default the in-tree build is loaded
LIB_PATH = os.environ.get("SEGCAUSAL_LIB") or os.path.join(_HERE, "libsegcausal.so")

SEGC_OK, SEGC_EINVAL, SEGC_EUNSUPPORTED, SEGC_EHIP = 0, 1, 2, 3
SEGC_BF16, SEGC_INT8 = 0, 1
HEAD_DIM = 128
MAX_SEG = 16
ABI_VERSION = (1 << 16) | 9      # SEGC_ABI_VERSION of the header these bindings mirror

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsegcausal.so is not built; run `python -m segment_causal_dit_amd.build` "
        "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)
_lib.segcausal_abi_version.restype = ctypes.c_int
if _lib.segcausal_abi_version() != ABI_VERSION:
    raise ImportError("%s has ABI version 0x%x, these bindings expect 0x%x; rebuild it"
                      % (LIB_PATH, _lib.segcausal_abi_version(), ABI_VERSION))

_i32, _i64, _f32, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)


class SegcCache(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("n_heads", _i32), ("head_dim", _i32),
                ("tokens_per_frame", _i32), ("n_slots", _i32), ("reserved", _i32),
                ("k", _vp), ("v", _vp), ("k_scale", _vp), ("v_scale", _vp)]


class SegcAttnArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp),
                ("q_stride_tok", _i64), ("q_stride_head", _i64),
                ("k_stride_tok", _i64), ("k_stride_head", _i64),
                ("v_stride_tok", _i64), ("v_stride_head", _i64),
                ("o_stride_tok", _i64), ("o_stride_head", _i64),
                ("lse", _vp), ("n_cur", _i64), ("n_heads", _i32), ("head_dim", _i32),
                ("n_seg", _i32), ("reserved", _i32),
                ("seg_start", _pi32), ("seg_text_len", _pi32), ("seg_text_valid", _pi32),
                ("cache", ctypes.POINTER(SegcCache)), ("hist_slots", _vp),
                ("n_hist", _i32), ("sm_scale", _f32), ("reserved2", _i32),
                ("workspace", _vp), ("workspace_bytes", _i64)]


class SegcAttnBwdArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("dout", _vp),
                ("dq", _vp), ("dk", _vp), ("dv", _vp)] + \
               [(nm + suf, _i64) for nm in ("q", "k", "v", "o", "do", "dq", "dk", "dv")
                for suf in ("_stride_tok", "_stride_head")] + \
               [("lse", _vp), ("delta", _vp), ("n", _i64), ("n_heads", _i32), ("head_dim", _i32),
                ("n_seg", _i32), ("reserved", _i32),
                ("seg_start", _pi32), ("seg_text_len", _pi32), ("seg_text_valid", _pi32),
                ("sm_scale", _f32)]


class SegcCameraArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp),
                ("q_stride_tok", _i64), ("q_stride_head", _i64),
                ("kv_stride_tok", _i64), ("kv_stride_head", _i64),
                ("o_stride_tok", _i64), ("o_stride_head", _i64),
                ("n_tok", _i64), ("n_heads", _i32), ("head_dim", _i32),
                ("tokens_per_chunk", _i32), ("t_cam", _i32), ("sm_scale", _f32)]


_lib.rope3d_apply.argtypes = [_vp, _vp, _i64, _i32, _i32, _i64, _i64, _vp, _f64, _i32, _i32, _i32, _vp]
_lib.kv_cache_append.argtypes = [ctypes.POINTER(SegcCache), _i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp]
_lib.kv_window_dequant.argtypes = [ctypes.POINTER(SegcCache), _vp, _i32, ctypes.POINTER(SegcCache), _vp]
_lib.window_select.argtypes = [_pi32, _i32, _i32, _pi32, _pi32]
_lib.w8a16_linear.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp]
_lib.camera_cross_attn.argtypes = [ctypes.POINTER(SegcCameraArgs), _vp]
_lib.kv_archive_fetch.argtypes = [ctypes.POINTER(SegcCache), _pi32, ctypes.POINTER(SegcCache), _pi32, _i32, _vp]
_lib.kv_archive_store.argtypes = [ctypes.POINTER(SegcCache), _pi32, ctypes.POINTER(SegcCache), _pi32, _i32, _vp]
_lib.segcausal_joint_attn.argtypes = [ctypes.POINTER(SegcAttnArgs), _vp]
_lib.segcausal_joint_attn_workspace_bytes.argtypes = [ctypes.POINTER(SegcAttnArgs), _i32]
_lib.segcausal_joint_attn_workspace_bytes.restype = _i64
_lib.segcausal_joint_attn_bwd.argtypes = [ctypes.POINTER(SegcAttnBwdArgs), _vp]
_lib.segcausal_joint_attn_bwd_noalloc.argtypes = [ctypes.POINTER(SegcAttnBwdArgs), _vp]
_lib.segcausal_last_error.restype = ctypes.c_char_p
_lib.segcausal_abi_version.restype = ctypes.c_int
for _f in ("rope3d_apply", "kv_cache_append", "kv_window_dequant", "window_select",
           "segcausal_joint_attn", "segcausal_joint_attn_bwd", "segcausal_joint_attn_bwd_noalloc",
           "kv_archive_fetch", "kv_archive_store", "w8a16_linear", "camera_cross_attn"):
    getattr(_lib, _f).restype = ctypes.c_int

EXPORTS = ("rope3d_apply", "kv_cache_append", "kv_window_dequant", "window_select",
           "segcausal_joint_attn", "segcausal_joint_attn_workspace_bytes", "segcausal_joint_attn_bwd",
           "segcausal_joint_attn_bwd_noalloc", "kv_archive_fetch", "kv_archive_store",
           "w8a16_linear", "camera_cross_attn", "segcausal_last_error", "segcausal_abi_version")


class SegcError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("segcausal status %d: %s" % (code, msg))
        self.code = code


def _check(rc):
    if rc != SEGC_OK:
        raise SegcError(rc, _lib.segcausal_last_error().decode())


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(stream)


def _rows(t, name):
    """(pointer, token stride, head stride) of a [rows, heads, 128] bf16 tensor."""
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.shape[2] != HEAD_DIM or t.stride(2) != 1:
        raise ValueError("%s must be bf16 [rows, heads, 128] with contiguous last dim" % name)
    return t.data_ptr(), t.stride(0), t.stride(1)


def _on_gpu(dev, **named):
    """Every named tensor (None skipped) must live on GPU device `dev`: the
    library receives bare pointers, and a host pointer or another device's
    memory handed to a kernel faults the GPU."""
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU, got %s" % dev)
    for name, t in named.items():
        if t is not None and t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))


def abi_version():
    return _lib.segcausal_abi_version()


def rope3d_apply(x_in, pos, x_out=None, theta=256.0, dims=(16, 56, 56), stream=None):
    """Rotate video rows in place (x_out None) or into x_out (same layout)."""
    if x_out is None:
        x_out = x_in
    pi, st, sh = _rows(x_in, "x_in")
    po, st2, sh2 = _rows(x_out, "x_out")
    if (st, sh) != (st2, sh2) or x_out.shape != x_in.shape:
        raise ValueError("x_in and x_out must share shape and strides")
    if pos.dtype != torch.int32 or not pos.is_contiguous() or tuple(pos.shape) != (x_in.shape[0], 3):
        raise ValueError("pos must be contiguous int32 [rows, 3]")
    _on_gpu(x_in.device, x_out=x_out, pos=pos)
    _check(_lib.rope3d_apply(pi, po, x_in.shape[0], x_in.shape[1], HEAD_DIM, st, sh,
                             pos.data_ptr(), float(theta), dims[0], dims[1], dims[2],
                             _stream(stream)))
    return x_out


class KVCache:
    """Device memory of one layer's cache plus its C descriptor.

    k, v   : [n_slots, n_heads, G, 128] int8 or bf16
    k_scale, v_scale : [n_slots, n_heads, G] fp32 (INT8 only)
    slot_t : host numpy int32 [n_slots], latent-frame index held by each slot
    """

    def __init__(self, n_slots, n_heads, tokens_per_frame, dtype="int8", device="cuda", pinned=False):
        shape = (n_slots, n_heads, tokens_per_frame, HEAD_DIM)
        self.int8 = dtype == "int8"
        tdt = torch.int8 if self.int8 else torch.bfloat16
        kw = dict(device=device, pin_memory=True) if pinned else dict(device=device)
        self.k = torch.zeros(shape, dtype=tdt, **kw)
        self.v = torch.zeros(shape, dtype=tdt, **kw)
        if self.int8:
            self.k_scale = torch.zeros(shape[:3], dtype=torch.float32, **kw)
            self.v_scale = torch.zeros(shape[:3], dtype=torch.float32, **kw)
        else:
            self.k_scale = self.v_scale = None
        self.slot_t = np.full(n_slots, -1, dtype=np.int32)
        self.desc = SegcCache(SEGC_INT8 if self.int8 else SEGC_BF16, n_heads, HEAD_DIM,
                              tokens_per_frame, n_slots, 0, self.k.data_ptr(), self.v.data_ptr(),
                              self.k_scale.data_ptr() if self.int8 else None,
                              self.v_scale.data_ptr() if self.int8 else None)

    @classmethod
    def archive(cls, n_frames, n_heads, tokens_per_frame, dtype="int8"):
        """A history archive: the cache layout in pinned host memory."""
        return cls(n_frames, n_heads, tokens_per_frame, dtype, device="cpu", pinned=True)

    @property
    def n_slots(self):
        return self.desc.n_slots

    @property
    def tokens_per_frame(self):
        return self.desc.tokens_per_frame


def kv_cache_append(cache, first_slot, k, v, t_first=None, stream=None):
    """Append n_frames * G rows of post-RoPE K and of V into slots
    first_slot, first_slot + 1, ... (mod n_slots). If t_first is given the
    host slot table records frames t_first, t_first + 1, ..."""
    pk, kst, ksh = _rows(k, "k")
    pv, vst, vsh = _rows(v, "v")
    g = cache.tokens_per_frame
    if k.shape[0] != v.shape[0] or k.shape[0] % g:
        raise ValueError("k and v must hold the same whole number of frames")
    if k.shape[1] != cache.desc.n_heads or v.shape[1] != cache.desc.n_heads:
        raise ValueError("k and v must have the cache's %d heads" % cache.desc.n_heads)
    _on_gpu(cache.k.device, k=k, v=v)
    n_frames = k.shape[0] // g
    _check(_lib.kv_cache_append(ctypes.byref(cache.desc), first_slot, n_frames,
                                pk, kst, ksh, pv, vst, vsh, _stream(stream)))
    if t_first is not None:
        for f in range(n_frames):
            cache.slot_t[(first_slot + f) % cache.n_slots] = t_first + f
    return n_frames


def kv_window_dequant(cache, slots, out, stream=None):
    """Expand INT8 cache slots `slots` (device int32 tensor, window order)
    into slots 0..len(slots)-1 of the BF16 KVCache `out`; attention over the
    window then reads `out` with hist_slots = 0, 1, ... ."""
    if slots.dtype != torch.int32 or slots.dim() != 1 or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous 1-D int32 tensor")
    _on_gpu(cache.k.device, slots=slots, out=out.k)
    _check(_lib.kv_window_dequant(ctypes.byref(cache.desc), slots.data_ptr(), slots.shape[0],
                                  ctypes.byref(out.desc), _stream(stream)))
    return slots.shape[0]


def _frame_list(x, name):
    a = np.ascontiguousarray(x, dtype=np.int32)
    if a.ndim != 1:
        raise ValueError("%s must be 1-D" % name)
    return a


def kv_archive_fetch(archive, archive_frames, cache, slots, stream=None):
    """Copy archive frames archive_frames[i] (pinned host) into cache slots
    slots[i] (device), asynchronously on `stream`."""
    af, sl = _frame_list(archive_frames, "archive_frames"), _frame_list(slots, "slots")
    if len(af) != len(sl):
        raise ValueError("archive_frames and slots differ in length")
    _check(_lib.kv_archive_fetch(ctypes.byref(archive.desc), af.ctypes.data_as(_pi32), ctypes.byref(cache.desc),
                                 sl.ctypes.data_as(_pi32), len(af), _stream(stream)))


def kv_archive_store(cache, slots, archive, archive_frames, stream=None):
    """Copy cache slots slots[i] (device) into archive frames archive_frames[i]
    (pinned host), asynchronously on `stream`."""
    af, sl = _frame_list(archive_frames, "archive_frames"), _frame_list(slots, "slots")
    if len(af) != len(sl):
        raise ValueError("archive_frames and slots differ in length")
    _check(_lib.kv_archive_store(ctypes.byref(cache.desc), sl.ctypes.data_as(_pi32), ctypes.byref(archive.desc),
                                 af.ctypes.data_as(_pi32), len(af), _stream(stream)))


def w8a16_linear(x, w_codes, w_scale, bias=None, out=None, workspace=None, stream=None):
    """y = bf16(x @ (w_codes * w_scale[:, None]).T + bias).

    x : bf16 [m, k] (row stride a multiple of 8, unit column stride)
    w_codes : int8 [n, k]; w_scale, bias : fp32 [n]; out : optional bf16 [m, n]
    workspace : optional bf16 tensor of >= n * k elements (the expanded codes)
    """
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be bf16 [m, k] with contiguous rows")
    if w_codes.dtype != torch.int8 or w_codes.dim() != 2 or w_codes.stride(1) != 1:
        raise ValueError("w_codes must be int8 [n, k] with contiguous rows")
    m, k = x.shape
    n = w_codes.shape[0]
    if w_codes.shape[1] != k:
        raise ValueError("w_codes must have k = %d columns" % k)
    for name, t in (("w_scale", w_scale), ("bias", bias)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (n,) or not t.is_contiguous()):
            raise ValueError("%s must be contiguous fp32 [n]" % name)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (m, n) or out.stride(1) != 1:
        raise ValueError("out must be bf16 [m, n] with contiguous rows")
    if workspace is None:
        workspace = torch.empty(n * k, dtype=torch.bfloat16, device=x.device)
    if workspace.dtype != torch.bfloat16 or not workspace.is_contiguous() or workspace.numel() < n * k:
        raise ValueError("workspace must be a contiguous bf16 tensor of >= n * k elements")
    _on_gpu(x.device, w_codes=w_codes, w_scale=w_scale, bias=bias, out=out, workspace=workspace)
    _check(_lib.w8a16_linear(x.data_ptr(), x.stride(0), w_codes.data_ptr(), w_codes.stride(0),
                             w_scale.data_ptr(), bias.data_ptr() if bias is not None else None,
                             out.data_ptr(), out.stride(0), m, n, k, workspace.data_ptr(), _stream(stream)))
    return out


def camera_cross_attn(q, k_cam, v_cam, tokens_per_chunk, sm_scale, out=None, stream=None):
    """Each row of q [n, H, 128] attends to the camera rows of its chunk:
    k_cam, v_cam [n_chunks * t_cam, H, 128] with t_cam = rows / n_chunks."""
    n, nh = q.shape[0], q.shape[1]
    n_chunks = (n + tokens_per_chunk - 1) // tokens_per_chunk
    if n_chunks == 0 or k_cam.shape[0] % n_chunks:
        raise ValueError("camera rows must be a whole number per chunk")
    t_cam = k_cam.shape[0] // n_chunks
    if k_cam.shape != v_cam.shape or k_cam.stride() != v_cam.stride():
        raise ValueError("k_cam and v_cam must share shape and strides")
    if k_cam.dim() != 3 or k_cam.shape[1] != nh:
        raise ValueError("k_cam and v_cam must be [rows, %d, 128] like q" % nh)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if tuple(out.shape[:2]) != (n, nh):
        raise ValueError("out must be [%d, %d, 128] like q" % (n, nh))
    _on_gpu(q.device, k_cam=k_cam, v_cam=v_cam, out=out)
    pq, qst, qsh = _rows(q, "q")
    pk, kst, ksh = _rows(k_cam, "k_cam")
    pv, _, _ = _rows(v_cam, "v_cam")
    po, ost, osh = _rows(out, "out")
    args = SegcCameraArgs(pq, pk, pv, po, qst, qsh, kst, ksh, ost, osh, n, nh, HEAD_DIM,
                          int(tokens_per_chunk), t_cam, float(sm_scale))
    _check(_lib.camera_cross_attn(ctypes.byref(args), _stream(stream)))
    return out


def window_select(slot_t, budget):
    """Host-side window: slot indices of the `budget` most recent frames."""
    st = np.ascontiguousarray(slot_t, dtype=np.int32)
    out = np.zeros(max(1, min(budget, len(st))) if budget >= 0 else 1, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(_lib.window_select(st.ctypes.data_as(_pi32), len(st), int(budget),
                              out.ctypes.data_as(_pi32), ctypes.byref(n)))
    return out[:n.value].copy()


def segcausal_joint_attn(q, k, v, segments, sm_scale, cache=None, hist_slots=None, out=None,
                         lse=None, stream=None, workspace="auto"):
    """Segment-wise causal joint attention.

    q, k, v    : bf16 [n_cur, H, 128] (video rows already rotated)
    segments   : list of (start, text_len, text_valid)
    cache      : KVCache or None; hist_slots: device int32 tensor [n_hist]
    out        : optional bf16 [n_cur, H, 128]; lse: optional fp32 [H, n_cur]
    workspace  : device tensor for splitting the launch's last partial round
                 (attn_workspace_bytes gives its size); "auto" allocates one
                 when the call would split, None never splits
    """
    pq, qst, qsh = _rows(q, "q")
    pk, kst, ksh = _rows(k, "k")
    pv, vst, vsh = _rows(v, "v")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    po, ost, osh = _rows(out, "out")
    n_cur, nh = q.shape[0], q.shape[1]
    for t, nm in ((k, "k"), (v, "v"), (out, "out")):
        if tuple(t.shape[:2]) != (n_cur, nh):
            raise ValueError("%s must be [%d, %d, 128] like q" % (nm, n_cur, nh))
    if hist_slots is not None and hist_slots.numel() > 0 and cache is None:
        raise ValueError("hist_slots needs a cache")
    _on_gpu(q.device, k=k, v=v, out=out, lse=lse, hist_slots=hist_slots,
            cache=cache.k if cache is not None else None)
    seg_start, tl, tv = _segment_tables(segments, n_cur)
    n_hist = 0
    hs_ptr = None
    cache_ptr = None
    if hist_slots is not None and hist_slots.numel() > 0:
        if hist_slots.dtype != torch.int32 or not hist_slots.is_contiguous():
            raise ValueError("hist_slots must be a contiguous int32 device tensor")
        n_hist = hist_slots.numel()
        hs_ptr = hist_slots.data_ptr()
    if cache is not None:
        cache_ptr = ctypes.pointer(cache.desc)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (nh, n_cur)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [H, n_cur]")
    args = SegcAttnArgs(pq, pk, pv, po, qst, qsh, kst, ksh, vst, vsh, ost, osh,
                        lse.data_ptr() if lse is not None else None, n_cur, nh, HEAD_DIM,
                        len(segments), 0, seg_start, tl, tv, cache_ptr, hs_ptr, n_hist,
                        float(sm_scale), 0, None, 0)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        need = _lib.segcausal_joint_attn_workspace_bytes(ctypes.byref(args), 0)
        if need < 0:
            raise SegcError(SEGC_EHIP, "segcausal_joint_attn_workspace_bytes failed")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need > 0 else None
    if workspace is not None:
        _on_gpu(q.device, workspace=workspace)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.segcausal_joint_attn(ctypes.byref(args), _stream(stream)))
    return out


def attn_workspace_bytes(n_cur, n_heads, segments, n_hist=0, cache=None, n_cu=0):
    """Bytes of workspace with which segcausal_joint_attn splits its last
    partial round for this shape (0: it would not split); n_cu = 0 asks the
    current device for its compute-unit count."""
    seg_start, tl, tv = _segment_tables(segments, n_cur)
    args = SegcAttnArgs()
    args.n_cur, args.n_heads, args.head_dim, args.n_seg = n_cur, n_heads, HEAD_DIM, len(segments)
    args.seg_start, args.seg_text_len, args.seg_text_valid = seg_start, tl, tv
    args.n_hist = n_hist
    if cache is not None:
        args.cache = ctypes.pointer(cache.desc)
    return _lib.segcausal_joint_attn_workspace_bytes(ctypes.byref(args), n_cu)


def _segment_tables(segments, n):
    starts = [int(s[0]) for s in segments] + [n]
    seg_start = (ctypes.c_int32 * len(starts))(*starts)
    tl = (ctypes.c_int32 * max(1, len(segments)))(*[int(s[1]) for s in segments])
    tv = (ctypes.c_int32 * max(1, len(segments)))(*[int(s[2]) for s in segments])
    return seg_start, tl, tv


def segcausal_joint_attn_bwd(q, k, v, o, dout, lse, segments, sm_scale, dq=None, dk=None,
                             dv=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of the packed-form attention (no history).

    q, k, v, o, dout : bf16 [n, H, 128]; lse: fp32 [H, n] from the forward
    segments         : list of (start, text_len, text_valid)
    dq, dk, dv       : optional bf16 [n, H, 128] outputs; delta: optional fp32
                       [H, n] workspace (receives rowsum(dout * o))
    """
    return _attn_bwd(_lib.segcausal_joint_attn_bwd, q, k, v, o, dout, lse, segments, sm_scale,
                     dq, dk, dv, delta, stream, True)


def segcausal_joint_attn_bwd_noalloc(q, k, v, o, dout, lse, segments, sm_scale, dq=None, dk=None,
                                     dv=None, stream=None):
    """segcausal_joint_attn_bwd through the entry point that allocates nothing:
    delta lives in the library's device scratch (n x H <= 2^23); calls that
    overlap on one GPU race. Pass dq, dk, dv to keep this call free of torch
    allocations too."""
    return _attn_bwd(_lib.segcausal_joint_attn_bwd_noalloc, q, k, v, o, dout, lse, segments, sm_scale,
                     dq, dk, dv, None, stream, False)


def _attn_bwd(fn, q, k, v, o, dout, lse, segments, sm_scale, dq, dk, dv, delta, stream, workspace):
    n, nh = q.shape[0], q.shape[1]
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty_like(q, memory_format=torch.contiguous_format) if t is None else t)
    dq, dk, dv = outs
    if workspace and delta is None:
        delta = torch.empty((nh, n), dtype=torch.float32, device=q.device)
    for name, t in (("lse", lse), ("delta", delta)):
        if t is None:
            continue
        if t.dtype != torch.float32 or tuple(t.shape) != (nh, n) or not t.is_contiguous():
            raise ValueError("%s must be contiguous fp32 [H, n]" % name)
    rows = [_rows(t, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"),
                                        (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    for t, nm in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if tuple(t.shape[:2]) != (n, nh):
            raise ValueError("%s must be [%d, %d, 128] like q" % (nm, n, nh))
    _on_gpu(q.device, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv, lse=lse, delta=delta)
    strides = [x for r in rows for x in r[1:]]
    seg_start, tl, tv = _segment_tables(segments, n)
    args = SegcAttnBwdArgs(*([r[0] for r in rows] + strides +
                             [lse.data_ptr(), delta.data_ptr() if delta is not None else None, n, nh,
                              HEAD_DIM, len(segments), 0, seg_start, tl, tv, float(sm_scale)]))
    _check(fn(ctypes.byref(args), _stream(stream)))
    return dq, dk, dv


def raw_library():
    """The loaded ctypes library (for ABI-level tests)."""
    return _lib
