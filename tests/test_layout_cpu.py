"""The packed-weight layout helpers (workloads.qweight_to_blocked / qweight_from_blocked) the GPU tests,
smoke() and the CPU baseline use to move between the oracle's row-major
qweight and the library's blocked one (include/paro.h, "Packed weights"): pinned here against
the definition's byte formula, on ragged row counts."""
from __future__ import annotations

import numpy as np
import pytest

from tests import gpu_common as C


def _offset(n: int, t: int, N: int, D: int) -> int:
    """Byte offset of byte t of row n: 16 b D/2 + g R_b 64 + r 64 + t % 64 (b = n // 16,
    r = n % 16, g = t // 64, R_b = min(16, N - 16 b))."""
    b, r, g = n // 16, n % 16, t // 64
    R = min(16, N - 16 * b)
    return 16 * b * (D // 2) + g * R * 64 + r * 64 + t % 64


@pytest.mark.parametrize("N,D", [(1, 128), (15, 256), (16, 128), (17, 256), (20, 256), (33, 384), (64, 512)])
def test_blocked_layout_matches_definition(N, D):
    rng = np.random.default_rng(N * 1000 + D)
    q = rng.integers(0, 256, size=(N, D // 2), dtype=np.uint8)
    qb = C.to_blocked(q)
    assert qb.shape == q.shape
    flat = qb.reshape(-1)
    for n in range(N):
        for t in range(D // 2):
            assert flat[_offset(n, t, N, D)] == q[n, t], (n, t)
    assert np.array_equal(C.from_blocked(qb), q)


def test_blocked_layout_worked_example():
    # N = 20, D = 256: rows 16..19 form a 4-row tail block starting at byte 16 * 128 = 2048; byte
    # 69 of row 17 (group 1, byte 5 of it) sits at 2048 + 1 * 4 * 64 + 1 * 64 + 5 = 2373
    q = np.arange(20 * 128, dtype=np.int64).reshape(20, 128) % 251
    q = q.astype(np.uint8)
    assert C.to_blocked(q).reshape(-1)[2373] == q[17, 69]
    # a full block: byte 0 of row 1 directly follows the 64 bytes of row 0's group 0
    assert C.to_blocked(q).reshape(-1)[64] == q[1, 0]
