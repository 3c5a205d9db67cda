"""Pins for the oracle's E8 nearest-point quantizer.

The checks do not retype the quantizer: they enumerate lattice points by
brute force (numpy), use lattice invariants, and compare the normalized
second moment with Conway & Sloane's closed form for E8.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e8_constants.json")))


def in_e8(v2):
    """v2 = 2*y; y in E8 = D8 u (D8 + 1/2)."""
    v2 = np.asarray(v2, dtype=np.int64)
    par = v2 & 1
    if par.min() != par.max():
        return False
    y_int = (v2 - par) // 2          # integer part (for the half coset: y - 1/2)
    return int(y_int.sum()) % 2 == 0


def brute_force_nearest(U):
    """Minimum squared distance from each row of U to E8, enumerating every
    point whose coordinates lie within 1 of the input (the covering radius is
    1, so the nearest point is among them)."""
    best = np.full(U.shape[0], np.inf)
    argbest = np.zeros((U.shape[0], 8))
    for shift in (0.0, 0.5):
        base = np.floor(U - shift) + shift             # candidate values per coordinate: base-1 .. base+2
        offs = np.array(list(itertools.product(range(-1, 3), repeat=8)), dtype=np.float64)  # 65536 x 8
        for b0 in range(0, offs.shape[0], 8192):
            o = offs[b0:b0 + 8192]
            P = base[:, None, :] + o[None, :, :]        # n x k x 8
            ok = np.abs(P - U[:, None, :]) <= 1.0 + 1e-12
            ok = ok.all(axis=2)
            ints = P - shift
            even = (np.rint(ints).sum(axis=2).astype(np.int64) % 2) == 0
            ok &= even
            d = ((P - U[:, None, :]) ** 2).sum(axis=2)
            d = np.where(ok, d, np.inf)
            k = d.argmin(axis=1)
            dm = d[np.arange(U.shape[0]), k]
            better = dm < best
            best = np.where(better, dm, best)
            argbest[better] = P[np.arange(U.shape[0]), k][better]
    return best, argbest


def q(u):
    return oracle.e8_nearest(np.asarray(u, dtype=np.float64))


def dist2(u, v2):
    return float(((np.asarray(u) - np.asarray(v2) / 2.0) ** 2).sum())


def test_brute_force_random():
    rng = np.random.default_rng(11)
    U = rng.uniform(-3.0, 3.0, size=(240, 8))
    best, _ = brute_force_nearest(U)
    for i in range(U.shape[0]):
        v = q(U[i])
        assert in_e8(v)
        assert abs(dist2(U[i], v) - best[i]) <= 1e-12, (U[i], v, best[i])


def test_brute_force_near_ties():
    """Points within 1e-9 of Voronoi faces: midpoints of neighbouring E8
    points, nudged to either side; the oracle must land on a nearest point."""
    rng = np.random.default_rng(12)
    pts = []
    for _ in range(120):
        a = q(rng.uniform(-2, 2, 8)) / 2.0
        mv = minimal_vectors()[rng.integers(240)]
        mid = a + mv / 2.0
        pts.append(mid + rng.choice([-1e-9, 1e-9], size=8) * rng.integers(0, 2, 8))
        pts.append(mid)
    U = np.array(pts)
    best, _ = brute_force_nearest(U)
    for i in range(U.shape[0]):
        v = q(U[i])
        assert in_e8(v)
        assert abs(dist2(U[i], v) - best[i]) <= 1e-12


def minimal_vectors():
    vs = []
    for i, j in itertools.combinations(range(8), 2):
        for si in (-1, 1):
            for sj in (-1, 1):
                v = np.zeros(8)
                v[i], v[j] = si, sj
                vs.append(v)
    for signs in itertools.product((-0.5, 0.5), repeat=8):
        if sum(1 for s in signs if s < 0) % 2 == 0:
            vs.append(np.array(signs))
    return np.array(vs)


def test_minimal_vectors():
    mv = minimal_vectors()
    assert mv.shape[0] == GOLDEN["kissing_number"]
    assert np.allclose((mv ** 2).sum(1), GOLDEN["min_norm_squared"])
    rng = np.random.default_rng(13)
    for lam in mv:
        assert in_e8(2 * lam)
        u = lam + rng.uniform(-0.1, 0.1, 8)
        assert np.array_equal(q(u), (2 * lam).astype(np.int32))


def test_invariants():
    rng = np.random.default_rng(14)
    mv = minimal_vectors()
    for _ in range(2000):
        u = rng.normal(0, 4, 8)
        v = q(u)
        assert in_e8(v)
        assert dist2(u, v) <= GOLDEN["covering_radius_squared"] + 1e-12
        assert np.array_equal(q(v / 2.0), v)                    # idempotent
        lam = mv[rng.integers(240)] * 2 + mv[rng.integers(240)]  # a lattice vector
        assert np.array_equal(q(u + lam), v + (2 * lam).astype(np.int32))  # translation invariance


def test_normalized_second_moment():
    """E||u - Q(u)||^2 / 8 over u uniform on a large box equals G(E8) for a
    unit-covolume lattice; Z8 (1/12) and D8 (~0.0766) are far outside."""
    rng = np.random.default_rng(15)
    n = 30000
    U = rng.uniform(0, 64, size=(n, 8))
    e = np.empty(n)
    for i in range(n):
        e[i] = dist2(U[i], q(U[i])) / 8.0
    G = GOLDEN["normalized_second_moment_num"] / GOLDEN["normalized_second_moment_den"]
    se = e.std() / np.sqrt(n)
    assert abs(e.mean() - G) < 4 * se + 1e-4, (e.mean(), G, se)
    assert abs(e.mean() - GOLDEN["z8_normalized_second_moment"]) > 0.005
    assert abs(e.mean() - GOLDEN["d8_normalized_second_moment_approx"]) > 0.002


def test_half_integer_ties_follow_readings():
    """Exact ties resolve by the stated readings: round half to even in D8,
    lowest index for the parity fix, D8 coset on an exact coset tie."""
    # all coordinates 0.25: D8 gives 0 (dist 0.5), D8+1/2 gives 0.5 (dist 0.5) -> D8 wins the tie
    assert np.array_equal(q(np.full(8, 0.25)), np.zeros(8, np.int32))
    # rounding 0.5 -> 0 (even); odd-sum fix moves coordinate 0 (largest error ties -> lowest index)
    u = np.array([0.5, 0.0, 0, 0, 0, 0, 0, 1.0])
    v = q(u)
    assert in_e8(v)
    assert abs(dist2(u, v) - brute_force_nearest(u[None, :])[0][0]) < 1e-12
