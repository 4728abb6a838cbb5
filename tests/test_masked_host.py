"""Host-side check of the masked kernel's bias addressing.

Each wave of the masked forward reads its bias rows through a buffer resource
that starts at row q0 (the wave's first query row) and spans
min(31, N - 1 - q0) row strides plus N elements; a wave whose rows all lie
past the end of the sequence (possible in the last 128-row block when N is
ragged) gets an empty resource.  This test walks every wave of the launch
grid for ragged lengths and broadcast strides and checks that the resource
never extends past the bias tensor the strides describe, so no load can leave
the caller's allocation.
"""
import pytest

ROWS_PER_BLOCK, WAVES = 128, 4


def wave_bias_range(bh, H, q0, N, sb, sh, si):
    """(first element, element count) of one wave's bias resource, or None
    for an empty resource, as the kernel forms them."""
    if q0 >= N:
        return None
    b, h = divmod(bh, H)
    base = b * sb + h * sh + q0 * si
    rows = min(31, N - 1 - q0)
    return base, rows * si + N


@pytest.mark.parametrize("N", [1, 17, 31, 32, 33, 96, 97, 127, 128, 129, 200, 257, 8200])
@pytest.mark.parametrize("shape", ["full", "per_head", "per_batch", "one"])
def test_every_wave_stays_inside_the_bias(N, shape):
    B, H = 2, 3
    strides = {"full": (H * N * N, N * N, N), "per_head": (0, N * N, N),
               "per_batch": (H * N * N, 0, N), "one": (0, 0, N)}[shape]
    sb, sh, si = strides
    extent = (B - 1) * sb + (H - 1) * sh + (N - 1) * si + N  # elements of the bias tensor
    nqb = (N + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    empty = 0
    for bh in range(B * H):
        for qb in range(nqb):
            for w in range(WAVES):
                r = wave_bias_range(bh, H, qb * ROWS_PER_BLOCK + 32 * w, N, sb, sh, si)
                if r is None:
                    empty += 1
                    continue
                lo, count = r
                assert 0 <= lo and lo + count <= extent, (bh, qb, w, lo, count, extent)
    ragged_waves = WAVES - (-(-(N - (nqb - 1) * ROWS_PER_BLOCK) // 32))
    assert empty == B * H * ragged_waves
