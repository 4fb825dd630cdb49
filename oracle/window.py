"""Bounded GPU history: which cached latent frames the attention reads.

Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
"Segment-Autoregressive Diffusion Transformer" (on one GPU only a limited
number of past latent frames is attended, 18 by default and not counting the
current segment; the standard configuration attends to the whole history) and section "Single-GPU Low-Memory Inference" (up to 18 historical
frames chosen by temporal_context sampling, older ones archived on CPU);
"Tencent Opens Hy-Nomas ...", section "How the RTX 4090 configuration saves
memory" (a sliding, fixed context window bounds KV-cache growth).

Reading: the window is the `budget` most recent valid frames by latent-frame
index t (fewer if fewer exist), returned in ascending t. Empty slots carry
t = -1. Two valid slots with the same t are an error.
"""

import numpy as np


class WindowError(ValueError):
    pass


def window_select(slot_t, budget):
    """Return the slot indices of the selected frames, ascending in t."""
    t = np.asarray(slot_t, dtype=np.int64)
    if budget < 0:
        raise WindowError("budget must be >= 0")
    valid = np.nonzero(t >= 0)[0]
    tv = t[valid]
    if len(np.unique(tv)) != len(tv):
        raise WindowError("duplicate latent-frame index among valid slots")
    order = valid[np.argsort(tv, kind="stable")]     # ascending t
    keep = min(int(budget), len(order))
    return order[len(order) - keep:].astype(np.int32)
