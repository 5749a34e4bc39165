"""Pins for the double-precision oracle, checked against mathematics rather
than against the oracle's own formula.

Each test names the mistake it is there to catch.  Closed forms are evaluated
with Python's decimal module at 40 digits; invariants (Newton's third law,
translation invariance, power-of-two homogeneity, force = -grad W) hold for
any correct implementation; the integrator pins use exactness under constant
acceleration, second-order convergence and time reversibility, which the
kick-drift-kick scheme has and a mis-weighted kick does not.

Sources: force law and softening -- "CUDA N-Body Simulation" README,
sections 1.1-1.2; leapfrog -- section 1.3 of the same README (closed by a
second half-kick); pair flop count -- "Cuda Nbody Notes".
"""
import decimal
import math
import os

import numpy as np
import pytest

import oracle
import workloads

D = decimal.Decimal
decimal.getcontext().prec = 40


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# Pair term
# --------------------------------------------------------------------------

def test_unsoftened_inverse_square_law():
    """eps2 = 0 reduces to Newton: |a_1| = G m_2 / r^2 toward body 2.
    Catches a wrong exponent, a wrong sign of r_ij and m_i used for m_j."""
    pos = np.array([[0.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    mass = np.array([3.0, 0.5])
    a = oracle.accel(pos, mass, G=1.0, eps2=0.0)
    assert a[0].tolist() == [0.0, 0.5 / 4.0, 0.0]     # pulled toward +y by m_2
    assert a[1].tolist() == [0.0, -3.0 / 4.0, 0.0]    # pulled toward -y by m_1


def test_two_body_softened_unit_distance():
    """x1 = 0, x2 = e_x, m = 1, eps^2 = 1e-4: a_1 = (1.0001^{-3/2}, 0, 0).
    Catches a dropped or mis-squared softening term."""
    pos = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
    mass = np.array([1.0, 1.0])
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    expect = float(D("1.0001") ** D("-1.5"))   # 0.99985001874781...
    assert abs(a[0, 0] - expect) <= 1e-15 * expect
    assert a[0, 1] == 0.0 and a[0, 2] == 0.0
    assert a[1].tolist() == (-a[0]).tolist()


def test_two_body_softened_closed_form_random():
    """Random pair, unequal masses, G = 3: a_1 = G m_2 d / (|d|^2+eps^2)^{3/2},
    a_2 = -G m_1 d / (...)^{3/2}, evaluated in 40-digit decimal."""
    g = np.random.default_rng(11)
    for _ in range(5):
        pos = g.uniform(-2, 2, (2, 3))
        mass = g.uniform(0.1, 5.0, 2)
        eps2, G = 0.37, 3.0
        a = oracle.accel(pos, mass, G=G, eps2=eps2)
        d = [D(float(pos[1, k])) - D(float(pos[0, k])) for k in range(3)]
        den = (sum(x * x for x in d) + D(eps2)) ** D("1.5")
        a1 = [float(D(G) * D(float(mass[1])) * x / den) for x in d]
        a2 = [float(-D(G) * D(float(mass[0])) * x / den) for x in d]
        assert _rel(a[0], a1) <= 1e-14
        assert _rel(a[1], a2) <= 1e-14


def test_equilateral_triangle():
    """Side 1, equal unit masses, eps^2 = 1e-4: each body feels
    sqrt(3) / 1.0001^{3/2} toward the centroid (two edges 60 degrees apart)."""
    s3 = math.sqrt(3.0)
    pos = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0], [0.5, s3 / 2.0, 0.0]])
    mass = np.ones(3)
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    mag = float(D(3).sqrt() / D("1.0001") ** D("1.5"))   # 1.7317910324199...
    centroid = pos.mean(axis=0)
    for i in range(3):
        u = (centroid - pos[i]) / np.linalg.norm(centroid - pos[i])
        assert abs(np.linalg.norm(a[i]) - mag) <= 1e-14 * mag
        assert np.dot(a[i], u) / np.linalg.norm(a[i]) > 1 - 1e-14


def test_octahedron_centre_is_exactly_zero():
    """A body at the centre of six equal masses at +-e_x, +-e_y, +-e_z."""
    pos = np.array([[0, 0, 0], [1, 0, 0], [-1, 0, 0], [0, 1, 0], [0, -1, 0],
                    [0, 0, 1], [0, 0, -1]], dtype=np.float64)
    mass = np.array([2.0] + [0.75] * 6)
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    assert a[0].tolist() == [0.0, 0.0, 0.0]


def test_self_term_and_coincident_bodies_contribute_nothing():
    a = oracle.accel(np.array([[0.3, -0.2, 0.9]]), np.array([5.0]), G=1.0, eps2=1e-4)
    assert a.tolist() == [[0.0, 0.0, 0.0]]
    pos = np.array([[0.5, 0.5, 0.5], [0.5, 0.5, 0.5]])
    a = oracle.accel(pos, np.array([1.0, 2.0]), G=1.0, eps2=1e-4)
    assert a.tolist() == [[0.0, 0.0, 0.0], [0.0, 0.0, 0.0]]


def test_decimal_brute_force_small():
    """N = 7 random bodies: every component against a 40-digit evaluation."""
    g = np.random.default_rng(5)
    pos = g.uniform(-1, 1, (7, 3))
    mass = g.uniform(0.5, 1.5, 7)
    eps2, G = 1e-3, 1.25
    a = oracle.accel(pos, mass, G=G, eps2=eps2)
    for i in range(7):
        acc = [D(0)] * 3
        for j in range(7):
            if j == i:
                continue
            d = [D(float(pos[j, k])) - D(float(pos[i, k])) for k in range(3)]
            den = (sum(x * x for x in d) + D(eps2)) ** D("1.5")
            acc = [acc[k] + D(float(mass[j])) * d[k] / den for k in range(3)]
        ref = [float(D(G) * x) for x in acc]
        assert _rel(a[i], ref) <= 1e-14


def test_summation_rounding_is_small():
    """The oracle's running double sums against an exactly rounded sum
    (math.fsum) of double-precision terms, over all 16384 bodies of the
    Plummer workload for 48 sampled rows: a sum that lost digits (float
    accumulation, a term dropped or doubled) would show far above 1e-12."""
    pm, _ = workloads.make("plummer16k")
    pos, mass = oracle.split_posmass(pm)
    eps2 = float(np.float32(1e-4))
    rows = np.random.default_rng(11).choice(pos.shape[0], 48, replace=False)
    a = oracle.accel_rows(pos, mass, 1.0, eps2, rows.astype(np.int64))
    for r, i in enumerate(rows):
        d = pos - pos[i]
        d2 = (d * d).sum(axis=1) + eps2
        w = mass / (d2 * np.sqrt(d2))
        w[i] = 0.0
        exact = [math.fsum(w * d[:, k]) for k in range(3)]
        assert _rel(a[r], exact) <= 1e-12, i


# --------------------------------------------------------------------------
# Invariants on the project's workloads
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def uniform1k():
    pm, _ = workloads.make("uniform1k")
    return oracle.split_posmass(pm)


def test_newton_third_law(uniform1k):
    """sum_i m_i a_i = 0.  Catches m_i in place of m_j and any asymmetric index bug."""
    pos, mass = uniform1k
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    net = np.linalg.norm((mass[:, None] * a).sum(axis=0))
    scale = (mass * np.linalg.norm(a, axis=1)).sum()
    assert net / scale <= 1e-13


def test_translation_invariance_is_exact(uniform1k):
    """Shifting float32-derived positions by (0.25, -0.5, 0.125) is exact in
    double, and so is every x_j - x_i; the result must be bit-identical."""
    pos, mass = uniform1k
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    b = oracle.accel(pos + np.array([0.25, -0.5, 0.125]), mass, G=1.0, eps2=1e-4)
    assert np.array_equal(a, b)


def test_power_of_two_homogeneity(uniform1k):
    """G -> 2G and m -> 2m double a exactly; x -> 2x with eps -> 2 eps
    divides a by 4 exactly.  Catches a missing G, a mass used twice, or a
    distance power other than -2 overall."""
    pos, mass = uniform1k
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    assert np.array_equal(oracle.accel(pos, mass, G=2.0, eps2=1e-4), 2 * a)
    assert np.array_equal(oracle.accel(pos, 2 * mass, G=1.0, eps2=1e-4), 2 * a)
    assert np.array_equal(oracle.accel(2 * pos, mass, G=1.0, eps2=4e-4), a / 4)


def test_rows_match_full(uniform1k):
    pos, mass = uniform1k
    a = oracle.accel(pos, mass, G=1.0, eps2=1e-4)
    rows = np.array([0, 5, 1023, 512, 5])
    assert np.array_equal(oracle.accel_rows(pos, mass, 1.0, 1e-4, rows), a[rows])


def test_readme_default_scale(golden_dir):
    """The README's own workload (section 6.1 constants: positions in
    [-1e5, 1e5]^3, masses in [1e5, 1e9], EPS2 = 0.002), cut to 512 bodies:
    Newton's third law still holds to rounding."""
    consts = {}
    with open(os.path.join(golden_dir, "readme_constants.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                consts[k] = float(v)
    g = np.random.default_rng(3)
    n = 512
    pos = g.uniform(-consts["MAX_X"], consts["MAX_X"], (n, 3))
    mass = g.uniform(consts["MIN_W"], consts["MAX_W"], n)
    a = oracle.accel(pos, mass, G=1.0, eps2=consts["EPS2"])
    net = np.linalg.norm((mass[:, None] * a).sum(axis=0))
    assert net / (mass * np.linalg.norm(a, axis=1)).sum() <= 1e-13


# --------------------------------------------------------------------------
# Energy
# --------------------------------------------------------------------------

def test_two_body_energy_closed_form():
    """|d| = 5 (3-4-5), eps^2 = 11 -> sqrt(25 + 11) = 6: W = -G m1 m2 / 6.
    v1 = (1,0,0), v2 = (0,2,0), unit masses: K = 1/2 + 2.  Catches a missing
    1/2 in K, a pair counted twice in W, and a sign error."""
    pos = np.array([[0.0, 0.0, 0.0], [3.0, 4.0, 0.0]])
    vel = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    mass = np.array([1.0, 1.0])
    e = oracle.energy(pos, vel, mass, G=1.0, eps2=11.0)
    assert e["K"] == 2.5
    assert abs(e["W"] + 1.0 / 6.0) <= 1e-16
    assert abs(e["E"] - (2.5 - 1.0 / 6.0)) <= 1e-15
    assert (e["Px"], e["Py"], e["Pz"], e["M"]) == (1.0, 2.0, 0.0, 2.0)
    e2 = oracle.energy(pos, vel, np.array([2.0, 3.0]), G=2.0, eps2=11.0)
    assert abs(e2["W"] + 2.0 * 6.0 / 6.0) <= 1e-15


def test_force_is_minus_gradient_of_potential_energy():
    """m_i a_i = -dW/dx_i by central differences: ties the energy's pair
    potential to the force law (exponent, eps placement, G, masses)."""
    g = np.random.default_rng(2)
    n = 48
    pos = g.uniform(-1, 1, (n, 3))
    mass = g.uniform(0.5, 1.5, n) / n
    vel = np.zeros((n, 3))
    G, eps2, h = 1.7, 3e-3, 1e-5
    a = oracle.accel(pos, mass, G=G, eps2=eps2)
    for i in (0, 17, 47):
        for k in range(3):
            p = pos.copy()
            p[i, k] += h
            wp = oracle.energy(p, vel, mass, G, eps2)["W"]
            p[i, k] -= 2 * h
            wm = oracle.energy(p, vel, mass, G, eps2)["W"]
            grad = (wp - wm) / (2 * h)
            assert abs(-grad - mass[i] * a[i, k]) <= 1e-6 * np.abs(mass[i] * a[i]).max()


def test_potential_rows_sum_to_twice_pair_energy(uniform1k):
    """sum_i m_i phi_i counts every pair twice: it equals 2 W."""
    pos, mass = uniform1k
    phi = oracle.potential_rows(pos, mass, 1.0, 1e-4, np.arange(pos.shape[0]))
    w = oracle.energy(pos, np.zeros_like(pos), mass, 1.0, 1e-4)["W"]
    assert abs(0.5 * (mass * phi).sum() - w) <= 1e-13 * abs(w)


def test_plummer_virial_equilibrium():
    """A Plummer sphere (a = 1, M = 1, G = 1) has W -> -3 pi / 32 and
    K -> 3 pi / 64 as N grows.  At N = 16384 sampling noise is ~1/sqrt(N)
    and softening (eps = 0.01) shifts W by well under 1 %.  Catches W counted
    twice (factor 2), K without its 1/2, and a wrong velocity scale in the
    generator."""
    pm, v = workloads.make("plummer16k")
    pos, mass = oracle.split_posmass(pm)
    e = oracle.energy(pos, v, mass, 1.0, 1e-4)
    assert abs(e["W"] / (-3 * math.pi / 32) - 1) < 0.04
    assert abs(e["K"] / (3 * math.pi / 64) - 1) < 0.04
    assert abs(2 * e["K"] / abs(e["W"]) - 1) < 0.06


# --------------------------------------------------------------------------
# Integrator
# --------------------------------------------------------------------------

def test_kick_drift_kick_exact_under_constant_acceleration():
    """With a fixed a, KDK gives x = x0 + v0 T + a T^2 / 2 and v = v0 + a T.
    A scheme with one half-kick per step (the README's as printed) would
    reach only a T^2 / 4 and v0 + a T / 2."""
    g = np.random.default_rng(9)
    x0 = g.uniform(-1, 1, (16, 3))
    v0 = g.uniform(-1, 1, (16, 3))
    a = g.uniform(-1, 1, (16, 3))
    dt, steps = 0.125, 8
    x, v = x0.copy(), v0.copy()
    for _ in range(steps):
        v = oracle.kick(v, a, 0.5 * dt)
        x = oracle.drift(x, v, dt)
        v = oracle.kick(v, a, 0.5 * dt)
    T = dt * steps
    assert np.abs(x - (x0 + v0 * T + 0.5 * a * T * T)).max() <= 1e-14
    assert np.abs(v - (v0 + a * T)).max() <= 1e-14


def _circular_binary(eps2):
    m = np.array([0.5, 0.5])
    d = 1.0
    omega = math.sqrt((m[0] + m[1]) / (d * d + eps2) ** 1.5)
    pos = np.array([[-d / 2, 0, 0], [d / 2, 0, 0]], dtype=np.float64)
    vel = np.array([[0, -omega * d / 2, 0], [0, omega * d / 2, 0]], dtype=np.float64)
    return pos, vel, m, omega


def test_kdk_circular_binary():
    """Equal-mass circular binary with the softened force: omega^2 =
    G (m1 + m2) / (d^2 + eps^2)^{3/2}.  After one period at dt = T/1000 the
    separation stays within (omega dt)^2 of d and the bodies are back near
    their start (leapfrog phase error is O((omega dt)^2) per orbit)."""
    eps2 = 1e-4
    pos, vel, m, omega = _circular_binary(eps2)
    period = 2 * math.pi / omega
    steps = 1000
    dt = period / steps
    x, v = pos, vel
    worst = 0.0
    for _ in range(20):
        x, v, _ = oracle.kdk(x, v, m, 1.0, eps2, dt, steps // 20)
        worst = max(worst, abs(np.linalg.norm(x[1] - x[0]) - 1.0))
    assert worst <= (omega * dt) ** 2
    assert np.abs(x - pos).max() <= 2e-3


def test_kdk_is_second_order():
    """Max energy error over one binary orbit drops ~4x when dt halves
    (first-order schemes: ~2x)."""
    eps2 = 1e-4
    pos, vel, m, omega = _circular_binary(eps2)
    # eccentric orbit: slow the bodies down so energy errors are visible
    vel = vel * 0.6
    e0 = oracle.energy(pos, vel, m, 1.0, eps2)["E"]
    period = 2 * math.pi / omega

    def max_err(steps):
        dt = period / steps
        x, v, worst = pos, vel, 0.0
        for _ in range(50):
            x, v, _ = oracle.kdk(x, v, m, 1.0, eps2, dt, steps // 50)
            worst = max(worst, abs(oracle.energy(x, v, m, 1.0, eps2)["E"] - e0))
        return worst

    ratio = max_err(2000) / max_err(4000)
    assert 3.3 < ratio < 4.7


def test_kdk_time_reversible():
    pm, vel = workloads.plummer(256, seed=4)
    pos, mass = oracle.split_posmass(pm)
    v0 = vel[:, :3].astype(np.float64)
    x, v, _ = oracle.kdk(pos, v0, mass, 1.0, 1e-4, 1e-3, 20)
    x, v, _ = oracle.kdk(x, -v, mass, 1.0, 1e-4, 1e-3, 20)
    assert np.abs(x - pos).max() <= 1e-12
    assert np.abs(-v - v0).max() <= 1e-12


def test_kdk_conserves_momentum_and_energy():
    """Plummer N = 4096, 10 steps of dt = 1e-3 (the 16k workload's step):
    total momentum stays at rounding level, energy drift far below 1e-4."""
    pm, vel = workloads.plummer(4096, seed=1)
    pos, mass = oracle.split_posmass(pm)
    v0 = vel[:, :3].astype(np.float64)
    e0 = oracle.energy(pos, v0, mass, 1.0, 1e-4)
    x, v, _ = oracle.kdk(pos, v0, mass, 1.0, 1e-4, 1e-3, 10)
    e1 = oracle.energy(x, v, mass, 1.0, 1e-4)
    dp = math.sqrt(sum((e1[k] - e0[k]) ** 2 for k in ("Px", "Py", "Pz")))
    assert dp <= 1e-15
    assert abs(e1["E"] - e0["E"]) / abs(e0["E"]) <= 1e-5
