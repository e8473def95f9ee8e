"""Reference for the per-owner contiguous buffer (pack / unpack).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Z2 vs Z3 Modes", "The two packed-buffer lifecycles": the Muon-target
parameters that share an owner are packed into one contiguous buffer, which is
what the owner broadcasts.  The pages do not give the layout; the reading
taken here: matrix i occupies ``numel_i`` consecutive elements starting at
``offset_i`` in row-major order, the bytes copied bit for bit.  The gaps
between matrices (alignment padding) have no defined contents.

Both functions work on raw element bits (``uint16`` for bf16, ``uint32`` or
``float32`` for fp32) with explicit Python index loops over rows, so that a
reader can check them against the definition by eye.
"""

from __future__ import annotations

import numpy as np


def pack(mats, offsets, total: int, fill=0) -> np.ndarray:
    """``packed[offset_i + row*cols + col] = mats[i][row, col]``.

    Elements of ``packed`` that no matrix covers are set to ``fill``."""
    dtype = mats[0].dtype
    packed = np.full(total, fill, dtype=dtype)
    for m, off in zip(mats, offsets):
        rows, cols = m.shape
        for row in range(rows):
            start = off + row * cols
            packed[start:start + cols] = m[row, :]
    return packed


def unpack(packed: np.ndarray, shapes, offsets):
    """Inverse of ``pack``: ``mats[i][row, col] = packed[offset_i + row*cols + col]``."""
    out = []
    for (rows, cols), off in zip(shapes, offsets):
        m = np.empty((rows, cols), dtype=packed.dtype)
        for row in range(rows):
            start = off + row * cols
            m[row, :] = packed[start:start + cols]
        out.append(m)
    return out
