"""Seeded synthetic N-body initial conditions.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It only draws bodies (positions, masses, velocities); it holds none of the
force, integrator or energy arithmetic.  Every generator works in float64 with
one ``numpy.random.Generator(PCG64(seed))`` and rounds the result to float32
(round-to-nearest-even).  The rounded float32 arrays are the canonical inputs:
the GPU consumes them as-is and the oracle promotes them exactly to float64.

Layouts
-------
``posmass``: float32 [N, 4] = (x, y, z, m), the body record of the tiled
CUDA kernels on "Cuda Nbody Notes" and of section 2.2 ("Data Structures and
Memory Alignment") of the LienoPC N-BodySimulation README.
``vel``: float32 [N, 4] = (vx, vy, vz, 0); w is unused.

Workloads
---------
The five named workloads of this project (see ``WORKLOADS``) mix three body
distributions:

* uniform cube: positions uniform in [-1, 1]^3 (the README's utils.cpp draws
  uniform positions in [-MAX, MAX]^3, section 2.3);
* Plummer sphere of scale radius a and mass M, velocities drawn from its
  isotropic distribution function (Aarseth, Henon & Wielen 1974, A&A 37, 183);
* two Plummer spheres set on a collision course.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make",
    "uniform_cube",
    "plummer",
    "two_plummer",
    "lognormal_masses",
    "rng",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_f32(pos: np.ndarray, mass: np.ndarray, vel: np.ndarray | None):
    n = pos.shape[0]
    pm = np.empty((n, 4), dtype=np.float32)
    pm[:, :3] = pos.astype(np.float32)
    pm[:, 3] = mass.astype(np.float32)
    v = np.zeros((n, 4), dtype=np.float32)
    if vel is not None:
        v[:, :3] = vel.astype(np.float32)
    return pm, v


def _isotropic(g: np.random.Generator, n: int) -> np.ndarray:
    """Unit vectors uniform on the sphere (cos(theta) uniform in [-1, 1])."""
    cos_t = g.uniform(-1.0, 1.0, n)
    phi = g.uniform(0.0, 2.0 * math.pi, n)
    sin_t = np.sqrt(np.maximum(0.0, 1.0 - cos_t * cos_t))
    return np.stack([sin_t * np.cos(phi), sin_t * np.sin(phi), cos_t], axis=1)


def uniform_cube(n: int, seed: int = 0, masses: str = "uniform_0.5_1.5"):
    """Positions uniform in [-1, 1]^3; masses by ``masses``:

    * ``"uniform_0.5_1.5"``: uniform in [0.5, 1.5] / N;
    * ``"lognormal"``: lognormal(mu=0, sigma=0.5), normalised to total 1;
    * ``"equal"``: 1/N each.
    Velocities are zero.
    """
    g = rng(seed)
    pos = g.uniform(-1.0, 1.0, (n, 3))
    if masses == "uniform_0.5_1.5":
        mass = g.uniform(0.5, 1.5, n) / n
    elif masses == "lognormal":
        mass = lognormal_masses(g, n)
    elif masses == "equal":
        mass = np.full(n, 1.0 / max(n, 1))
    else:
        raise ValueError(f"unknown mass model {masses!r}")
    return _to_f32(pos, mass, None)


def lognormal_masses(g: np.random.Generator, n: int, mu: float = 0.0, sigma: float = 0.5):
    m = g.lognormal(mu, sigma, n)
    return m / m.sum()


def _plummer_f64(g: np.random.Generator, n: int, a: float, mtot: float, G: float):
    """Plummer sphere in float64: (pos[n,3], vel[n,3]) before COM removal.

    Radius: the cumulative mass M(<r)/M = r^3/(r^2+a^2)^{3/2} inverted at a
    uniform deviate X gives r = a / sqrt(X^{-2/3} - 1) (untruncated).
    Speed: v = q * v_esc(r), v_esc = sqrt(2 G M) (r^2 + a^2)^{-1/4}, with q
    drawn by rejection from g(q) ~ q^2 (1 - q^2)^{7/2} on [0, 1]; the maximum
    of that density is (2/9)(7/9)^{7/2} ~ 0.0922 < 0.1, the rejection ceiling.
    """
    x = g.uniform(0.0, 1.0, n)
    # X = 0 has probability ~2^-53 per draw; keep it finite.
    x = np.maximum(x, 1e-300)
    r = a / np.sqrt(x ** (-2.0 / 3.0) - 1.0)
    pos = r[:, None] * _isotropic(g, n)

    q = np.empty(n)
    todo = np.arange(n)
    while todo.size:
        qq = g.uniform(0.0, 1.0, todo.size)
        yy = g.uniform(0.0, 0.1, todo.size)
        ok = yy < qq * qq * (1.0 - qq * qq) ** 3.5
        q[todo[ok]] = qq[ok]
        todo = todo[~ok]
    vesc = math.sqrt(2.0 * G * mtot) * (r * r + a * a) ** -0.25
    vel = (q * vesc)[:, None] * _isotropic(g, n)
    return pos, vel


def plummer(n: int, seed: int = 0, a: float = 1.0, mtot: float = 1.0, G: float = 1.0):
    """Equal-mass Plummer sphere, centre of mass and mean velocity removed."""
    g = rng(seed)
    pos, vel = _plummer_f64(g, n, a, mtot, G)
    pos -= pos.mean(axis=0)
    vel -= vel.mean(axis=0)
    mass = np.full(n, mtot / n)
    return _to_f32(pos, mass, vel)


def two_plummer(n_a: int, n_b: int, seed: int = 0, offset: float = 4.0,
                v_bulk: float = 0.3, a: float = 1.0, G: float = 1.0):
    """Two equal-mass-per-body Plummer spheres on a head-on course along x.

    Every body has mass 1/(n_a+n_b).  Sphere A (first n_a bodies) sits at
    x = +offset moving with vx = -v_bulk; sphere B at x = -offset with
    vx = +v_bulk.  Each sphere's internal velocities come from the
    distribution function of its own mass, and each is centred (position
    and velocity) before the offset is applied.
    """
    g = rng(seed)
    n = n_a + n_b
    out_pos, out_vel = [], []
    for cnt, sign in ((n_a, +1.0), (n_b, -1.0)):
        m_sph = cnt / n
        p, v = _plummer_f64(g, cnt, a, m_sph, G)
        p -= p.mean(axis=0)
        v -= v.mean(axis=0)
        p[:, 0] += sign * offset
        v[:, 0] += -sign * v_bulk
        out_pos.append(p)
        out_vel.append(v)
    pos = np.concatenate(out_pos)
    vel = np.concatenate(out_vel)
    mass = np.full(n, 1.0 / n)
    return _to_f32(pos, mass, vel)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    eps2: float
    G: float
    dt: float
    steps: int
    seed: int
    description: str

    def generate(self):
        return make(self.name)


WORKLOADS = {
    "uniform1k": Workload(
        "uniform1k", 1024, 1e-4, 1.0, 0.0, 0, 0,
        "N=1024, uniform [-1,1]^3, masses uniform [0.5,1.5]/N, one force pass"),
    "plummer16k": Workload(
        "plummer16k", 16384, 1e-4, 1.0, 1e-3, 10, 0,
        "N=16384 Plummer (a=1, M=1), equal masses, 10 KDK steps dt=1e-3"),
    "lognormal128k": Workload(
        "lognormal128k", 131072, 1e-6, 1.0, 0.0, 0, 0,
        "N=131072 uniform [-1,1]^3, lognormal(0,0.5) masses normalised to 1, one force pass"),
    "plummer1m": Workload(
        "plummer1m", 1048576, 1e-4, 1.0, 1e-4, 1, 0,
        "N=1048576 Plummer (a=1, M=1), equal masses, one force pass + one KDK step dt=1e-4"),
    "collision1m": Workload(
        "collision1m", 1000003, 1e-4, 1.0, 1e-3, 20, 0,
        "N=1000003 two Plummer spheres (500001 + 500002) at x=+/-4, vx=-/+0.3, 20 KDK steps dt=1e-3"),
}


def make(name: str):
    """(posmass, vel) float32 [N, 4] arrays of a named workload."""
    w = WORKLOADS[name]
    if name == "uniform1k":
        return uniform_cube(w.n, w.seed, "uniform_0.5_1.5")
    if name == "lognormal128k":
        return uniform_cube(w.n, w.seed, "lognormal")
    if name in ("plummer16k", "plummer1m"):
        return plummer(w.n, w.seed)
    if name == "collision1m":
        return two_plummer(500001, 500002, w.seed)
    raise KeyError(name)
