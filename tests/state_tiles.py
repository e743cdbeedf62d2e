"""Host-side conversion between separate fp32 master/m/v arrays and the tiled
state layout that include/zero.h documents (tiles of ZERO_STATE_TILE
elements, each holding master, then m, then v of its elements; the last tile
compact). Written for the tests from that description; shares nothing with
the library."""

import os
import re

import numpy as np

_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "zero.h")
TILE = int(re.search(r"#define\s+ZERO_STATE_TILE\s+(\d+)", open(_HEADER, encoding="utf-8").read()).group(1))


def to_tiles(master, m, v):
    master, m, v = (np.asarray(x, np.float32) for x in (master, m, v))
    n = master.size
    out = np.empty(3 * n, np.float32)
    for lo in range(0, n, TILE):
        L = min(TILE, n - lo)
        base = 3 * lo
        out[base:base + L] = master[lo:lo + L]
        out[base + L:base + 2 * L] = m[lo:lo + L]
        out[base + 2 * L:base + 3 * L] = v[lo:lo + L]
    return out


def from_tiles(state, n):
    state = np.asarray(state, np.float32)
    assert state.size == 3 * n
    master = np.empty(n, np.float32)
    m = np.empty(n, np.float32)
    v = np.empty(n, np.float32)
    for lo in range(0, n, TILE):
        L = min(TILE, n - lo)
        base = 3 * lo
        master[lo:lo + L] = state[base:base + L]
        m[lo:lo + L] = state[base + L:base + 2 * L]
        v[lo:lo + L] = state[base + 2 * L:base + 3 * L]
    return master, m, v


def tile_span(n, begin, count):
    """Element span [lo, hi) of the whole tiles that cover [begin, begin+count);
    the sub-buffer state[3*lo:3*hi] has the same tile structure as an
    (hi - lo)-element state, because lo is a tile boundary."""
    lo = (begin // TILE) * TILE
    hi = min(n, -(-(begin + count) // TILE) * TILE)
    return lo, hi


def state_range(state_slice_fn, n, begin, count):
    """master, m, v of elements [begin, begin+count) of an n-element tiled
    state; ``state_slice_fn(a, b)`` returns floats [a, b) of the buffer."""
    lo, hi = tile_span(n, begin, count)
    sub = np.asarray(state_slice_fn(3 * lo, 3 * hi), np.float32)
    master, m, v = from_tiles(sub, hi - lo)
    sl = slice(begin - lo, begin - lo + count)
    return master[sl], m[sl], v[sl]
