"""CPU checks of the full-size golden files (tests/golden/full_c<n>.npz):
they were written from the current oracle and input generator, hold one
entry per row and request of their workload, and their q digest separates
rows that differ in one count or one id."""
import hashlib
import os
import sys

import numpy as np
import pytest

from oracle import dyadic24 as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import make_full_parity as G  # noqa: E402

SIZES = {1: 1, 2: 4, 3: 64, 4: 256, 5: 1024}


@pytest.mark.parametrize("cfg", sorted(SIZES))
def test_golden_is_current(cfg):
    g = np.load(os.path.join(GOLDEN, f"full_c{cfg}.npz"))
    assert str(g["meta_sources_sha256"]) == G.sources_hash(), "rerun tests/golden/make_full_parity.py"
    R = SIZES[cfg]
    assert g["d_status"].shape == (5 * R,) and g["t_argmax"].shape == (6 * R,) and g["r_accept"].shape == (R,)
    assert ((g["r_accept"] >= 0) & (g["r_accept"] <= 5)).all()
    ok = g["d_status"] == 0
    assert ((g["d_conf"][ok] > 0) & (g["d_conf"][ok] <= 1)).all()


def test_digest_is_sensitive():
    V = 129280
    c = np.zeros(V, np.uint32)
    c[5] = O.M
    c2 = c.copy()
    c2[5] -= 1
    c2[6] = 1
    assert G.q_digest(None, c, True, V) != G.q_digest(None, c2, True, V)
    assert G.q_digest([3, 9], [1, O.M - 1], False, V) != G.q_digest([3, 10], [1, O.M - 1], False, V)
    assert hashlib.sha256(b"").digest()[:8] == G.q_digest([], [], False, V).to_bytes(8, "little")
