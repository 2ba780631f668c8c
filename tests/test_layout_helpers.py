"""The host-side tiled-layout helpers used by the GPU tests, checked element
by element against the layout's definition in include/fp4q.h (written out
here as a plain per-element address formula)."""
import numpy as np
import pytest

from gpu_helpers import tile_codes, tile_scales, untile_codes, untile_scales


def code_addr(r, b, K):
    # block (16-row group, 128-column step), then chunk c of the step's 64
    # bytes and row within the group, then the byte within the chunk
    G, rr = divmod(r, 16)
    k, bb = divmod(b, 64)
    c, e = divmod(bb, 16)
    return (G * (K // 128) + k) * 1024 + (c * 16 + rr) * 16 + e


def scale_addr(r, j, K, fmt):
    H, rr = divmod(r, 64)
    sps = 8 if fmt == 0 else 4
    k, jj = divmod(j, sps)
    base = (H * (K // 128) + k) * 64 * sps
    if fmt == 0:
        d, e = divmod(jj, 4)
        return base + (d * 64 + rr) * 4 + e
    return base + rr * 4 + jj


@pytest.mark.parametrize("rows,K", [(1, 128), (37, 256), (64, 384), (130, 512)])
def test_codes_match_definition(rows, K):
    rng = np.random.default_rng(rows + K)
    q = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    t = tile_codes(q)
    assert t.size == -(-rows // 16) * 16 * K // 2
    for r in range(rows):
        for b in range(K // 2):
            assert t[code_addr(r, b, K)] == q[r, b]
    assert np.array_equal(untile_codes(t, rows, K), q)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,K", [(1, 128), (37, 256), (64, 384), (130, 512)])
def test_scales_match_definition(fmt, rows, K):
    blk = 16 if fmt == 0 else 32
    rng = np.random.default_rng(rows * K + fmt)
    s = rng.integers(0, 256, (rows, K // blk), dtype=np.uint8)
    t = tile_scales(s, fmt)
    assert t.size == -(-rows // 64) * 64 * K // blk
    for r in range(rows):
        for j in range(K // blk):
            assert t[scale_addr(r, j, K, fmt)] == s[r, j]
    assert np.array_equal(untile_scales(t, rows, K, fmt), s)
