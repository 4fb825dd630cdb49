"""Frame moves between a device cache and a host history archive.

Source: model card, section "Single-GPU Low-Memory Inference" (a bounded set
of historical frames stays on the GPU while older history is archived on the
CPU). Reading: an archived frame is the cache frame byte for byte (codes and
scales of an INT8 cache, values of a BF16 one), so moving frames is an
indexed copy; a destination listed twice is an error.

Pinned by an element-by-element loop on small caches
(tests/test_oracle_basic.py).
"""

import numpy as np


def move_frames(src, src_idx, dst, dst_idx):
    """A copy of `dst` whose frame dst_idx[i] is src[src_idx[i]] for every i.

    src, dst : arrays whose first axis is the frame (any trailing shape, same
               trailing shape and dtype)
    """
    src_idx = np.asarray(src_idx, dtype=np.int64)
    dst_idx = np.asarray(dst_idx, dtype=np.int64)
    if len(src_idx) != len(dst_idx):
        raise ValueError("frame lists differ in length")
    if len(np.unique(dst_idx)) != len(dst_idx):
        raise ValueError("a destination frame appears twice")
    out = np.array(dst, copy=True)
    out[dst_idx] = np.asarray(src)[src_idx]
    return out
