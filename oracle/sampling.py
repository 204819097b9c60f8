"""Seeded choice of the output tiles and bias-gradient columns checked on large shapes.

Test infrastructure.  Tiles are 128 x 128 at offsets that are multiples of 32 (so a
tile's columns start on a relu_aux word boundary), deliberately not aligned to any
kernel tile, plus the four corner tiles.
"""
import numpy as np


def sample_tiles(m, n, count=32, tile=128, align=32, seed=0):
    """Return a list of (r0, r1, c0, c1) half-open tile bounds inside an m x n output."""
    rng = np.random.default_rng(seed)
    th, tw = min(tile, m), min(tile, n)
    out = []

    def clip(r0, c0):
        r0 = max(0, min(r0, m - th))
        c0 = max(0, min(c0, n - tw))
        c0 -= c0 % align
        return (r0, r0 + th, c0, min(c0 + tw, n))

    for _ in range(count):
        r0 = int(rng.integers(0, max(1, (m - th) // align + 1))) * align
        c0 = int(rng.integers(0, max(1, (n - tw) // align + 1))) * align
        out.append(clip(r0, c0))
    for r0, c0 in ((0, 0), (0, n - tw), (m - th, 0), (m - th, n - tw)):
        # corner tiles; a right-hand corner that starts off a word boundary is widened
        # leftwards to the boundary and still ends at column n
        c1 = c0 + tw
        c0 -= c0 % align
        out.append((r0, r0 + th, c0, c1))
    return sorted(set(out))


def sample_columns(n, count=64, seed=0):
    """Sorted unique column indices: `count` seeded ones plus the first and last."""
    rng = np.random.default_rng(seed)
    cols = set(int(c) for c in rng.integers(0, n, size=count)) | {0, n - 1}
    return np.array(sorted(cols), dtype=np.int64)
