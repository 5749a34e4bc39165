"""The seeded input generators: determinism, layout, and the distributions
they claim (uniform cube, lognormal masses, Plummer sphere and its
distribution function, two colliding spheres)."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

import workloads


def test_seeded_and_float32():
    a, va = workloads.uniform_cube(1000, seed=0)
    b, vb = workloads.uniform_cube(1000, seed=0)
    c, _ = workloads.uniform_cube(1000, seed=1)
    assert a.dtype == np.float32 and a.shape == (1000, 4)
    assert va.dtype == np.float32 and va.shape == (1000, 4)
    assert np.array_equal(a, b) and np.array_equal(va, vb)
    assert not np.array_equal(a, c)
    assert a.flags["C_CONTIGUOUS"]


def test_uniform_cube_ranges():
    pm, v = workloads.make("uniform1k")
    assert pm.shape == (1024, 4)
    assert np.all(np.abs(pm[:, :3]) <= 1.0)
    m = pm[:, 3].astype(np.float64) * 1024
    assert m.min() >= 0.5 - 1e-6 and m.max() <= 1.5 + 1e-6
    assert np.all(v == 0)
    # roughly uniform: each octant holds about 1/8
    counts = np.histogramdd(pm[:, :3], bins=2, range=[[-1, 1]] * 3)[0]
    assert counts.min() > 90 and counts.max() < 170


def test_lognormal_masses():
    pm, _ = workloads.uniform_cube(131072, seed=0, masses="lognormal")
    m = pm[:, 3].astype(np.float64)
    assert abs(m.sum() - 1.0) < 1e-5
    logm = np.log(m)
    assert abs(logm.std() - 0.5) < 0.01


def _plummer_radii(pm):
    pos = pm[:, :3].astype(np.float64)
    return np.linalg.norm(pos - pos.mean(axis=0), axis=1)


def test_plummer_mass_profile_ks():
    """M(<r)/M = r^3 / (1 + r^2)^{3/2} for a = 1."""
    pm, _ = workloads.plummer(20000, seed=2)
    r = _plummer_radii(pm)
    cdf = lambda x: x ** 3 / (1 + x * x) ** 1.5
    res = stats.kstest(r, cdf)
    assert res.pvalue > 1e-3
    # half-mass radius 1 / sqrt(2^{2/3} - 1) = 1.3048
    assert abs(np.median(r) - 1.0 / math.sqrt(2 ** (2 / 3) - 1)) < 0.04


def test_plummer_speed_distribution_ks():
    """q = v / v_esc(r) follows g(q) ~ q^2 (1 - q^2)^{7/2}."""
    pm, v = workloads.plummer(20000, seed=3)
    r = _plummer_radii(pm)
    speed = np.linalg.norm(v[:, :3].astype(np.float64), axis=1)
    q = speed / (math.sqrt(2.0) * (1 + r * r) ** -0.25)
    g = lambda x: x * x * (1 - x * x) ** 3.5
    norm = integrate.quad(g, 0, 1)[0]
    cdf = np.vectorize(lambda x: integrate.quad(g, 0, min(max(x, 0.0), 1.0))[0] / norm)
    res = stats.kstest(q[:4000], cdf)
    assert res.pvalue > 1e-3
    assert q.max() < 1.0 + 1e-3


def test_plummer_centred_equal_masses():
    pm, v = workloads.make("plummer16k")
    assert pm.shape == (16384, 4)
    assert np.all(pm[:, 3] == np.float32(1.0 / 16384))
    assert np.abs(pm[:, :3].astype(np.float64).mean(axis=0)).max() < 1e-6
    assert np.abs(v[:, :3].astype(np.float64).mean(axis=0)).max() < 1e-6
    assert np.all(v[:, 3] == 0)


@pytest.mark.slow
def test_two_plummer_layout():
    pm, v = workloads.make("collision1m")
    n = 1000003
    assert pm.shape == (n, 4)
    a, b = slice(0, 500001), slice(500001, n)
    xa = pm[a, :3].astype(np.float64).mean(axis=0)
    xb = pm[b, :3].astype(np.float64).mean(axis=0)
    assert abs(xa[0] - 4.0) < 1e-5 and abs(xb[0] + 4.0) < 1e-5
    assert np.abs(xa[1:]).max() < 1e-5 and np.abs(xb[1:]).max() < 1e-5
    va = v[a, :3].astype(np.float64).mean(axis=0)
    vb = v[b, :3].astype(np.float64).mean(axis=0)
    assert abs(va[0] + 0.3) < 1e-5 and abs(vb[0] - 0.3) < 1e-5
    assert np.all(pm[:, 3] == np.float32(1.0 / n))


def test_workload_table():
    names = set(workloads.WORKLOADS)
    assert names == {"uniform1k", "plummer16k", "lognormal128k", "plummer1m", "collision1m"}
    assert workloads.WORKLOADS["plummer1m"].n == 1 << 20
    assert workloads.WORKLOADS["collision1m"].n == 1000003
    assert workloads.WORKLOADS["lognormal128k"].eps2 == 1e-6
