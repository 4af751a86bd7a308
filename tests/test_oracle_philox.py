"""Pins of the oracle's counter-based generator and of the mapping from
(seed, step, request, slot) to the uniforms the verifier draws for itself."""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox4x32_known_answers():
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in g["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        assert [int(x) for x in O.philox4x32_10(ctr, key)] == [int(x, 16) for x in v["out"]]


@pytest.mark.parametrize("key", [(0, 0), (1234, 5678), (2**64 - 1, 2**63 + 12345)])
def test_philox4x64_round_structure_matches_numpy(key):
    """The 64-bit member of the family shares the round structure; NumPy's
    Philox bit generator (which advances its counter before each block) must
    agree with it block for block."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.zeros(4, np.uint64))
    raw = bg.random_raw(4 * 6)
    for j in range(6):
        ours = O.philox4x64_10([j + 1, 0, 0, 0], list(key))
        assert np.array_equal(ours, raw[4 * j: 4 * j + 4]), j


def test_step_uniform_mapping():
    u_acc, u_smp = O.step_uniforms(5, 15, seed=0x0123456789ABCDEF, offset=(7 << 32) + 42)
    for r in (0, 4):
        words = np.concatenate([O.philox4x32_10([j, r, 42, 7], [0x89ABCDEF, 0x01234567]) for j in range(9)])
        u = (words >> 8).astype(np.float64) / 2**24
        assert np.array_equal(u_acc[r], u[:15].astype(np.float32)) and u_smp[r] == np.float32(u[32])
    assert ((u_acc >= 0) & (u_acc < 1)).all()


def test_step_uniforms_are_uniform_and_independent():
    u_acc, u_smp = O.step_uniforms(4000, 32, seed=99, offset=1)
    u = np.concatenate([u_acc.ravel(), u_smp])
    hist = np.bincount((u * 64).astype(int), minlength=64)
    e = len(u) / 64
    chi2 = ((hist - e) ** 2 / e).sum()
    assert chi2 < 120          # 63 degrees of freedom: p ~ 1e-5 at 110
    # neighbouring steps and requests do not repeat each other
    a, _ = O.step_uniforms(64, 8, seed=99, offset=2)
    b, _ = O.step_uniforms(64, 8, seed=99, offset=3)
    assert abs(np.corrcoef(a.ravel(), b.ravel())[0, 1]) < 0.1
    assert len(np.unique(u_acc[:, 0])) > 3990
