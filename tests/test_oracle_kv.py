"""Pins for the KV-append oracle (CPU only)."""
import numpy as np
import pytest

from oracle import kv_cache as OK


def test_append_copies_oldest_block_bytes():
    rng = np.random.default_rng(0)
    nb, hkv, cap, w, d, B = 2, 3, 20, 8, 5, 4
    kc, vc = rng.standard_normal((nb, hkv, cap, d)), rng.standard_normal((nb, hkv, cap, d))
    kw, vw = rng.standard_normal((nb, hkv, w, d)), rng.standard_normal((nb, hkv, w, d))
    k2, v2, p2 = OK.kv_commit(kc, vc, kw, vw, [5, 9], 1, B)
    assert p2 == [5, 13]
    assert k2[1, :, 9:13].tobytes() == kw[1, :, 0:4].tobytes()
    assert v2[1, :, 9:13].tobytes() == vw[1, :, 0:4].tobytes()
    # nothing else moved
    mask = np.ones(k2.shape, bool)
    mask[1, :, 9:13] = False
    assert (k2[mask] == kc[mask]).all() and (v2[mask] == vc[mask]).all()


def test_capacity_is_enforced():
    z = np.zeros((1, 1, 6, 2))
    with pytest.raises(ValueError):
        OK.kv_commit(z, z, np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)), [3], 0, 4)


def test_drop_oldest_block_shifts_window():
    x = np.arange(2 * 1 * 6 * 1, dtype=float).reshape(2, 1, 6, 1)
    y = OK.drop_oldest_block(x, 0, 2)
    assert list(y[0, 0, :4, 0]) == [2, 3, 4, 5] and np.isnan(y[0, 0, 4:]).all()
    assert (y[1] == x[1]).all()
