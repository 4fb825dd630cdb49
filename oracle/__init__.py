"""Plain fp64 CPU oracle for segment-causal joint attention over a KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything in this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constants or
tables with the HIP library and imports nothing from it.

Every function is the plain definition of what the method computes, written
in numpy float64 (no blocking, fusion or reordering beyond chunking over query
rows, which changes no value beyond fp64 rounding). The sources are the pages
describing Hy-Nomas:

* "Hy-Nomas: Towards Free-Form Interactive World Generation" (model card),
  sections "Segment-Autoregressive Diffusion Transformer" (joint attention,
  3D RoPE, per-layer KV cache, causal across segments, bounded history) and
  "Single-GPU Low-Memory Inference" (INT8 KV storage with BF16 compute,
  18-frame history budget), plus its architecture table (16 heads x 128,
  RoPE split [16, 56, 56], theta 256).
* "Hy-Nomas Explained: How Tencent's Open World Model Runs Steerable Video on
  an RTX 4090", Step 2 "Segment-wise causal joint attention".
* "Tencent Opens Hy-Nomas, an Interactive Video World Model Running on One
  RTX 4090", section "How the RTX 4090 configuration saves memory".
* The Explainer's section "The training recipe" (segment forcing on packed
  sequences) for the gradients of the packed form (attention_bwd.py).
* The model card's "Single-GPU Low-Memory Inference" for the CPU history
  archive (archive.py) and, with its assets table, for the INT8-weight
  linear layer (linear.py).
* The model card's "Text and Camera Conditioning" for the per-latent-frame
  camera cross-attention (camera.py).

Readings where the pages leave a step open are listed in each module.

Pins (tests/test_oracle_*.py): brute-force loops on tiny inputs, closed forms,
invariants and library special cases. ``rope3d``'s pairing/axis-order
convention is a reading, not a printed value: its convention is
"parity unpinned" (its invariants are pinned).
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16
from .rope import rope3d, rope3d_bf16, rope_frequencies
from .quant import quantise_int8, dequantise_int8, dequantise_int8_bf16
from .window import window_select, WindowError
from .attention_bwd import joint_attn_backward, joint_attn_dq_rows
from .archive import move_frames
from .linear import w8a16_linear
from .camera import camera_cross_attn
from .attention import (Segment, visible_mask, history_keys, joint_attn,
                        joint_attn_rows)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_bf16",
    "rope3d", "rope3d_bf16", "rope_frequencies",
    "quantise_int8", "dequantise_int8",
    "window_select", "WindowError",
    "Segment", "visible_mask", "history_keys", "joint_attn", "joint_attn_rows",
    "dequantise_int8_bf16", "joint_attn_backward", "joint_attn_dq_rows", "move_frames",
    "w8a16_linear", "camera_cross_attn",
]
