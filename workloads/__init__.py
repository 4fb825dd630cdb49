"""Seeded synthetic inputs at the shapes of the Hy-Nomas pages' workloads.

Shared by the tests, the oracle checks and bench.py. This module holds only
shapes, positions, seeds and random draws: none of the method's arithmetic
(no RoPE, no quantiser, no attention) lives here.

Geometry from the pages: 16 heads x 128 ("Hy-Nomas: Towards Free-Form
Interactive World Generation", architecture table); 32x spatial and 4x
temporal latent compression with a 1x1x1 patch, so a 704x1280 frame is a
22x40 = 880-token latent frame and 24 FPS is 6 latent frames per second
("Hy-Nomas Explained ...", Step 3 "The Video Latent and PixelUMM Decoder
Math"); an 18-latent-frame history budget (model card, section "Single-GPU
Low-Memory Inference"); 12-second turns, i.e. 72 latent frames (ComfyUI-Wiki
news page, the five-turn gallery clip). Seed 42 is the pages' default seed
(model card, standard settings table).

Recipe: numpy PCG64 seeded with 42 + k (k = 0 q, 1 k, 2 v, 3 history k,
4 history v, 5 and 6 INT8 cache draws, 7 upstream gradient), float32 N(0, 1) draws rounded to bf16 (nearest,
ties to even). Q is multiplied by `q_scale` before rounding. Trained
activations do not exist here, so unit-variance draws stand in for them.
"""

from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 128
SEED = 42
_CHUNK = 1 << 22          # draws are always made in chunks of this size


@dataclass(frozen=True)
class SegSpec:
    text_len: int
    text_valid: int
    n_frames: int
    t0: int               # latent-frame index of the segment's first frame


@dataclass(frozen=True)
class Config:
    name: str
    n_heads: int
    grid: tuple                   # (grid_h, grid_w): tokens per frame = h*w
    segments: tuple               # SegSpec per packed current segment
    hist_t: tuple = ()            # t of each cached frame, stored at slot f
    cache_dtype: str = "none"     # "none" | "bf16" | "int8"
    extra_slots: int = 0          # free slots after the history (for append)
    budget: int = -1              # window budget; -1 = every cached frame
    q_scale: float = 1.0
    sm_scale: float = 1.0
    append: bool = False          # the run also appends the current video K/V

    @property
    def tokens_per_frame(self):
        return self.grid[0] * self.grid[1]

    @property
    def n_slots(self):
        return len(self.hist_t) + self.extra_slots

    @property
    def n_cur(self):
        g = self.tokens_per_frame
        return sum(s.text_len + s.n_frames * g for s in self.segments)

    @property
    def n_video(self):
        return sum(s.n_frames for s in self.segments) * self.tokens_per_frame

    @property
    def window(self):
        return len(self.hist_t) if self.budget < 0 else min(self.budget, len(self.hist_t))

    @property
    def n_hist_rows(self):
        return self.window * self.tokens_per_frame

    def segment_rows(self):
        """(start, text_len, text_valid) of each packed segment."""
        out, r, g = [], 0, self.tokens_per_frame
        for s in self.segments:
            out.append((r, s.text_len, s.text_valid))
            r += s.text_len + s.n_frames * g
        return out

    def visible_pairs(self):
        """Number of visible (query, key) pairs per head."""
        rows = self.segment_rows() + [(self.n_cur, 0, 0)]
        g = self.tokens_per_frame
        total = 0
        earlier_video = 0
        for si, s in enumerate(self.segments):
            n_rows = rows[si + 1][0] - rows[si][0]
            own = s.text_valid + s.n_frames * g
            total += n_rows * (self.n_hist_rows + earlier_video + own)
            earlier_video += s.n_frames * g
        return total

    def flops(self):
        """Algorithmic FLOPs of one attention call: QK^T and PV, 2*D each."""
        return 4 * HEAD_DIM * self.n_heads * self.visible_pairs()


_INV_SQRT_D = 1.0 / math.sqrt(HEAD_DIM)
_FULL = (22, 40)

# (text_len, text_valid, n_frames) of 16 packed segments, for the cases at
# the segment limit of one call
_SEG16 = ((8, 8, 1), (0, 0, 2), (5, 3, 1), (12, 12, 0), (7, 7, 1), (3, 1, 2), (0, 0, 1), (16, 9, 1),
          (9, 9, 1), (1, 1, 1), (4, 4, 0), (6, 2, 2), (0, 0, 1), (11, 11, 1), (2, 2, 1), (10, 6, 1))


def _seg_list(t0):
    out, t = [], t0
    for tl, tv, nf in _SEG16:
        out.append(SegSpec(tl, tv, nf, t))
        t += nf
    return tuple(out)

CONFIGS = {
    # 2 heads, 16 text tokens, 4x6 grid; two cached segments of 2 frames each
    # (t = 0..3) and a current segment of 2 frames (t = 4, 5); BF16 cache.
    "c0": Config("c0", 2, (4, 6), (SegSpec(16, 16, 2, 4),), hist_t=(0, 1, 2, 3),
                 cache_dtype="bf16", sm_scale=_INV_SQRT_D),
    # First segment, no cache: 256 text + 8 frames of 22x40.
    "c1": Config("c1", 16, _FULL, (SegSpec(256, 256, 8, 0),),
                 q_scale=_INV_SQRT_D),
    # Same current segment at t = 18..25 over an 18-frame BF16 history.
    "c2": Config("c2", 16, _FULL, (SegSpec(256, 256, 8, 18),), hist_t=tuple(range(18)),
                 cache_dtype="bf16", q_scale=_INV_SQRT_D),
    # As c2 with an INT8 history; the current K/V is appended in the same run.
    "c3": Config("c3", 16, _FULL, (SegSpec(256, 256, 8, 18),), hist_t=tuple(range(18)),
                 cache_dtype="int8", extra_slots=8, q_scale=_INV_SQRT_D, append=True),
    # Five 12-s turns: 4 cached turns of 72 frames (t = 0..287, INT8) and the
    # current turn of 72 frames (t = 288..359) plus 256 text tokens.
    "c4": Config("c4", 16, _FULL, (SegSpec(256, 256, 72, 288),),
                 hist_t=tuple(range(288)), cache_dtype="int8", extra_slots=72,
                 q_scale=_INV_SQRT_D, append=True),
}

# Small variants for parity and edge cases (not bench workloads).
VARIANTS = {
    "c0_int8": Config("c0_int8", 2, (4, 6), (SegSpec(16, 16, 2, 4),), hist_t=(0, 1, 2, 3),
                      cache_dtype="int8", extra_slots=2, sm_scale=_INV_SQRT_D, append=True),
    "c0_win3": Config("c0_win3", 2, (4, 6), (SegSpec(16, 16, 2, 4),), hist_t=(0, 1, 2, 3),
                      cache_dtype="bf16", budget=3, sm_scale=_INV_SQRT_D),
    "c0_pad": Config("c0_pad", 2, (4, 6), (SegSpec(16, 11, 2, 4),), hist_t=(0, 1, 2, 3),
                     cache_dtype="bf16", sm_scale=_INV_SQRT_D),
    "c0_packed3": Config("c0_packed3", 2, (4, 6),
                         (SegSpec(16, 16, 2, 0), SegSpec(16, 16, 2, 2), SegSpec(16, 16, 2, 4)),
                         sm_scale=_INV_SQRT_D),
    # mid-size: several key tiles, frames of 100 tokens, ragged tails
    "mid_int8": Config("mid_int8", 4, (10, 10), (SegSpec(37, 37, 3, 5),), hist_t=(0, 1, 2, 3, 4),
                       cache_dtype="int8", extra_slots=3, budget=4, q_scale=_INV_SQRT_D,
                       append=True),
    "mid_bf16": Config("mid_bf16", 4, (10, 10), (SegSpec(37, 30, 3, 5),), hist_t=(0, 1, 2, 3, 4),
                       cache_dtype="bf16", q_scale=_INV_SQRT_D),
    "mid_packed": Config("mid_packed", 3, (8, 9),
                         (SegSpec(20, 17, 2, 3), SegSpec(5, 5, 3, 5), SegSpec(0, 0, 2, 8)),
                         hist_t=(0, 1, 2), cache_dtype="bf16", q_scale=_INV_SQRT_D),
    "mid_nocache": Config("mid_nocache", 2, (7, 13), (SegSpec(45, 45, 4, 0),),
                          q_scale=_INV_SQRT_D),
    # the most segments one call takes (16), over an INT8 history that the
    # run appends to: text-only segments, segments without text, padded text
    "max_seg16": Config("max_seg16", 2, (4, 8), _seg_list(2), hist_t=(0, 1), cache_dtype="int8",
                        extra_slots=17, q_scale=_INV_SQRT_D, append=True),
}

# Packed training form (segment forcing): every segment present, no cache.
# A segment is 256 text rows + 30 latent frames of 22x40 ("Hy-Nomas Explained
# ...", the section on the latent math: 30 frames of 880 tokens per segment);
# 13 of them (346,528 rows) fill the 360,000-row packing limit of the
# fine-tuning recipe ("The training recipe"). The valid text lengths are
# synthetic: prompts are padded to 256 rows.
_TRAIN_VALID = (256, 201, 256, 143, 256, 256, 77, 256, 230, 256, 256, 164, 256)
TRAIN = {
    "train13": Config("train13", 16, _FULL,
                      tuple(SegSpec(256, tv, 30, 30 * i) for i, tv in enumerate(_TRAIN_VALID)),
                      q_scale=_INV_SQRT_D),
    # small packed forms for gradient parity: ragged tails, padded text, a
    # segment without text and one that is text only
    "bwd_small": Config("bwd_small", 2, (8, 9),
                        (SegSpec(37, 30, 2, 0), SegSpec(20, 20, 3, 2), SegSpec(0, 0, 2, 5),
                         SegSpec(16, 5, 1, 7)), sm_scale=_INV_SQRT_D),
    # full-size frames, four short segments: dozens of workgroups per head
    "bwd_mid": Config("bwd_mid", 2, _FULL,
                      (SegSpec(64, 64, 2, 0), SegSpec(64, 40, 2, 2), SegSpec(64, 7, 2, 4),
                       SegSpec(64, 64, 2, 6)), q_scale=_INV_SQRT_D),
    "bwd_one": Config("bwd_one", 3, (10, 13), (SegSpec(0, 0, 5, 0),), sm_scale=_INV_SQRT_D),
    "bwd_text": Config("bwd_text", 2, (6, 7), (SegSpec(64, 64, 4, 0), SegSpec(64, 33, 0, 4),
                                               SegSpec(1, 1, 3, 4)), q_scale=_INV_SQRT_D),
    "bwd_seg16": Config("bwd_seg16", 2, (4, 8), _seg_list(0), q_scale=_INV_SQRT_D),
}

ALL = dict(CONFIGS, **VARIANTS, **TRAIN)

_RANDOM_GRIDS = ((2, 8), (4, 4), (3, 5), (4, 6), (5, 7), (8, 8))   # 16, 16, 15, 24, 35, 64 tokens


def random_config(i, history=True):
    """A small seeded configuration for parity sweeps (PCG64(42 + 100 + i)).
    Every segment holds at least one frame or two valid text rows, so every
    query row sees at least two keys (a query with one visible key has
    gradients that vanish only by cancellation); history frames precede the
    segments in time."""
    rng = np.random.Generator(np.random.PCG64(SEED + 100 + i))
    grid = _RANDOM_GRIDS[int(rng.integers(len(_RANDOM_GRIDS)))]
    g = grid[0] * grid[1]
    n_hist = int(rng.integers(0, 5)) if history else 0
    segs, t = [], n_hist
    for _ in range(int(rng.integers(1, 17))):
        nf = int(rng.integers(0, 3))
        tl = int(rng.integers(0, 41))
        tv = int(rng.integers(0, tl + 1)) if tl else 0
        if nf == 0 and tv < 2:
            tl, tv = max(tl, 2), 2
        segs.append(SegSpec(tl, tv, nf, t))
        t += nf
    cache = "none" if n_hist == 0 else ("int8" if rng.integers(2) else "bf16")
    append = cache != "none" and segs[0].n_frames > 0 and bool(rng.integers(2))
    budget = -1 if n_hist == 0 or rng.integers(2) else int(rng.integers(1, n_hist + 1))
    unscaled = bool(rng.integers(2))
    return Config("random%d" % i, int(rng.integers(1, 4)), grid, tuple(segs),
                  hist_t=tuple(range(n_hist)), cache_dtype=cache,
                  extra_slots=segs[0].n_frames if append else 0, budget=budget,
                  q_scale=1.0 if unscaled else _INV_SQRT_D,
                  sm_scale=_INV_SQRT_D if unscaled else 1.0, append=append)


# ---------------------------------------------------------------- draws ----

def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(k, shape, scale=1.0):
    """bf16 bits of N(0,1)*scale drawn from PCG64(42 + k), in fixed-size chunks."""
    rng = np.random.Generator(np.random.PCG64(SEED + k))
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        d = rng.standard_normal(b - a, dtype=np.float32)
        if scale != 1.0:
            d = (d * np.float32(scale)).astype(np.float32)
        out[a:b] = f32_to_bf16_bits(d)
    return out.reshape(shape)


def frame_positions(t_list, grid):
    """int32 [len(t_list) * gh * gw, 3] raster (t, h, w) positions."""
    gh, gw = grid
    t = np.repeat(np.asarray(t_list, dtype=np.int32), gh * gw)
    h = np.tile(np.repeat(np.arange(gh, dtype=np.int32), gw), len(t_list))
    w = np.tile(np.arange(gw, dtype=np.int32), gh * len(t_list))
    return np.stack([t, h, w], axis=1)


@dataclass
class Inputs:
    cfg: Config
    q: np.ndarray            # bf16 bits [n_cur, H, D]
    k: np.ndarray            # bf16 bits [n_cur, H, D], before RoPE
    v: np.ndarray            # bf16 bits [n_cur, H, D]
    video_rows: np.ndarray   # int64 indices of the current video rows
    pos: np.ndarray          # int32 [n_video, 3], aligned with video_rows
    hist_k: np.ndarray       # bf16 bits [n_hist_frames * G, H, D], before RoPE
    hist_v: np.ndarray       # bf16 bits [n_hist_frames * G, H, D]
    hist_pos: np.ndarray     # int32 [n_hist_frames * G, 3]
    slot_t: np.ndarray       # int32 [n_slots]: t of the frame in each slot, -1 empty
    segments: list = field(default_factory=list)   # (start, text_len, text_valid)


def make_inputs(cfg):
    if isinstance(cfg, str):
        cfg = ALL[cfg]
    h, g = cfg.n_heads, cfg.tokens_per_frame
    n_cur = cfg.n_cur
    q = normal_bf16(0, (n_cur, h, HEAD_DIM), cfg.q_scale)
    k = normal_bf16(1, (n_cur, h, HEAD_DIM))
    v = normal_bf16(2, (n_cur, h, HEAD_DIM))
    rows, pos = [], []
    for (start, tl, _), s in zip(cfg.segment_rows(), cfg.segments):
        rows.append(np.arange(start + tl, start + tl + s.n_frames * g))
        pos.append(frame_positions(range(s.t0, s.t0 + s.n_frames), cfg.grid))
    video_rows = np.concatenate(rows).astype(np.int64)
    pos = np.concatenate(pos).astype(np.int32)
    nh = len(cfg.hist_t)
    hist_k = normal_bf16(3, (nh * g, h, HEAD_DIM))
    hist_v = normal_bf16(4, (nh * g, h, HEAD_DIM))
    hist_pos = frame_positions(cfg.hist_t, cfg.grid) if nh else np.zeros((0, 3), np.int32)
    slot_t = np.full(cfg.n_slots, -1, dtype=np.int32)
    slot_t[:nh] = np.asarray(cfg.hist_t, dtype=np.int32)
    return Inputs(cfg, q, k, v, video_rows, pos, hist_k, hist_v, hist_pos, slot_t,
                  cfg.segment_rows())


def upstream_grad(cfg):
    """bf16 bits [n_cur, H, D] of an upstream gradient dL/do: N(0, 1) draws
    from PCG64(42 + 7)."""
    if isinstance(cfg, str):
        cfg = ALL[cfg]
    return normal_bf16(7, (cfg.n_cur, cfg.n_heads, HEAD_DIM))


# Linear layers of one double-stream block's video stream at c4's 63,360
# video rows (Explainer, architecture notes: hidden 2,048, feed-forward
# 8,192; model card: INT8 DiT weights with BF16 linear compute):
# (rows m, output channels n, input features k).
LINEARS = {
    "qkv": (63360, 3 * 2048, 2048),
    "proj": (63360, 2048, 2048),
    "mlp_up": (63360, 8192, 2048),
    "mlp_down": (63360, 2048, 8192),
}


def linear_inputs(m, n, k, seed=0):
    """Seeded W8A16 linear inputs: x bf16 bits [m, k] ~ N(0, 1); codes int8
    [n, k] = round(48 N(0, 1)) clipped to [-127, 127]; per-channel scales fp32
    [n] uniform in [1, 2) / (64 sqrt(k)) (outputs of order one); bias fp32 [n]
    ~ N(0, 1). Draws from PCG64(42 + 8 + seed)."""
    rng = np.random.Generator(np.random.PCG64(SEED + 8 + seed))
    x = np.empty((m, k), dtype=np.uint16)
    for a in range(0, m, max(1, _CHUNK // k)):
        b = min(m, a + max(1, _CHUNK // k))
        x[a:b] = f32_to_bf16_bits(rng.standard_normal((b - a, k), dtype=np.float32))
    codes = np.clip(np.rint(rng.standard_normal((n, k), dtype=np.float32) * 48.0), -127, 127).astype(np.int8)
    scale = ((1.0 + rng.random(n)) / (64.0 * math.sqrt(k))).astype(np.float32)
    bias = rng.standard_normal(n).astype(np.float32)
    return x, codes, scale, bias


def direct_int8_cache(cfg, frames):
    """Seeded INT8 codes and fp32 scales for `frames` cache slots, drawn
    directly (for attention-only checks on identical cache bytes).

    Returns (k_codes, v_codes, k_scale, v_scale): codes int8 [frames, H, G, D]
    in [-127, 127] (round(48 * N(0,1)), clipped); scales float32 [frames, H, G]
    uniform in [1/64, 1/32).
    """
    rng = np.random.Generator(np.random.PCG64(SEED + 5))
    shape = (frames, cfg.n_heads, cfg.tokens_per_frame, HEAD_DIM)

    def codes():
        return np.clip(np.rint(rng.standard_normal(shape) * 48.0), -127, 127).astype(np.int8)

    def scales():
        return ((1.0 + rng.random(shape[:3])) / 64.0).astype(np.float32)

    kc = codes()
    vc = codes()
    return kc, vc, scales(), scales()


def uniform_int8_cache(cfg, frames):
    """Like direct_int8_cache but with codes uniform in [-127, 127] (a fast
    draw for timing runs). Returns (k_codes, v_codes, k_scale, v_scale)."""
    rng = np.random.Generator(np.random.PCG64(SEED + 6))
    shape = (frames, cfg.n_heads, cfg.tokens_per_frame, HEAD_DIM)
    kc = rng.integers(-127, 128, size=shape, dtype=np.int8)
    vc = rng.integers(-127, 128, size=shape, dtype=np.int8)
    ks = ((1.0 + rng.random(shape[:3])) / 64.0).astype(np.float32)
    vs = ((1.0 + rng.random(shape[:3])) / 64.0).astype(np.float32)
    return kc, vc, ks, vs
