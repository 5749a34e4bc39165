"""Double-precision CPU oracle for direct all-pairs softened gravity.

TEST INFRASTRUCTURE ONLY: the test suite, the package's smoke check and the
bench's CPU-baseline leg are the only callers.  Nothing here is used by, or
uses, the HIP library; the two share no code.  The numeric work is the C file
``nbody_oracle.c`` (gcc, -O2, OpenMP over bodies, no fast-math); this module
only builds it, marshals numpy arrays and converts the float32 body records
of the GPU path to float64 exactly.

Definitions followed (restated, cited by page title and section):

* acceleration a_i = G sum_{j!=i} m_j (x_j - x_i) / (|x_j - x_i|^2 + eps^2)^{3/2}
  -- "CUDA N-Body Simulation" README, sections 1.1-1.2;
* leapfrog kick/drift -- same README, section 1.3, closed by a second
  half-kick (kick-drift-kick);
* energy W = -G sum_{i<j} m_i m_j / sqrt(r_ij^2 + eps^2), K = sum m v^2 / 2 --
  the potential whose negative gradient is the acceleration above (not printed
  on the pages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nbody_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point this at a deliberately broken build of the same C file to
# show that the pins fail on it (see tests/test_oracle_mutants.py).
_OVERRIDE = os.environ.get("NBODY_ORACLE_LIB")

_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, OpenMP, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _OVERRIDE:
        lib = ctypes.CDLL(_OVERRIDE)
    else:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
    I64, F64 = ctypes.c_int64, ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_accel.restype = None
    lib.oracle_accel.argtypes = [_f64p, _f64p, I64, F64, F64, _f64p]
    lib.oracle_accel_rows.restype = None
    lib.oracle_accel_rows.argtypes = [_f64p, _f64p, I64, F64, F64, _i64p, I64, _f64p]
    lib.oracle_potential_rows.restype = None
    lib.oracle_potential_rows.argtypes = [_f64p, _f64p, I64, F64, F64, _i64p, I64, _f64p]
    lib.oracle_energy.restype = None
    lib.oracle_energy.argtypes = [_f64p, _f64p, _f64p, I64, F64, F64, _f64p]
    lib.oracle_kick.restype = None
    lib.oracle_kick.argtypes = [_f64p, _f64p, I64, F64]
    lib.oracle_drift.restype = None
    lib.oracle_drift.argtypes = [_f64p, _f64p, I64, F64]
    lib.oracle_kdk.restype = None
    lib.oracle_kdk.argtypes = [_f64p, _f64p, _f64p, I64, F64, F64, F64, I64, _f64p]
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _vec3(a) -> np.ndarray:
    a = np.asarray(a)
    if a.ndim != 2 or a.shape[1] not in (3, 4):
        raise ValueError("expected an [N, 3] or [N, 4] array")
    return np.ascontiguousarray(a[:, :3], dtype=np.float64)


def split_posmass(posmass):
    """float32 (or any) [N, 4] (x, y, z, m) -> float64 pos [N, 3], mass [N]."""
    pm = np.asarray(posmass)
    pos = np.ascontiguousarray(pm[:, :3], dtype=np.float64)
    mass = np.ascontiguousarray(pm[:, 3], dtype=np.float64)
    return pos, mass


def accel(pos, mass, G: float, eps2: float) -> np.ndarray:
    """float64 [N, 3] accelerations of every body."""
    pos = _vec3(pos)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    n = pos.shape[0]
    out = np.zeros((n, 3), dtype=np.float64)
    if n:
        _load().oracle_accel(pos, mass, n, float(G), float(eps2), out)
    return out


def accel_rows(pos, mass, G: float, eps2: float, rows) -> np.ndarray:
    """float64 [len(rows), 3]: the full j-sum for each listed body."""
    pos = _vec3(pos)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, 3), dtype=np.float64)
    if rows.size:
        if rows.min() < 0 or rows.max() >= pos.shape[0]:
            raise IndexError("row index out of range")
        _load().oracle_accel_rows(pos, mass, pos.shape[0], float(G), float(eps2),
                                  rows, rows.size, out)
    return out


def potential_rows(pos, mass, G: float, eps2: float, rows) -> np.ndarray:
    """float64 [len(rows)]: phi_i = -G sum_{j!=i} m_j / sqrt(r^2 + eps^2)."""
    pos = _vec3(pos)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros(rows.size, dtype=np.float64)
    if rows.size:
        if rows.min() < 0 or rows.max() >= pos.shape[0]:
            raise IndexError("row index out of range")
        _load().oracle_potential_rows(pos, mass, pos.shape[0], float(G), float(eps2),
                                      rows, rows.size, out)
    return out


ENERGY_FIELDS = ("K", "W", "E", "Px", "Py", "Pz", "M")


def energy(pos, vel, mass, G: float, eps2: float) -> dict:
    """{K, W, E, Px, Py, Pz, M} in float64."""
    pos = _vec3(pos)
    vel = _vec3(vel)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    out = np.zeros(8, dtype=np.float64)
    _load().oracle_energy(pos, vel, mass, pos.shape[0], float(G), float(eps2), out)
    return dict(zip(ENERGY_FIELDS, out[:7].tolist()))


def kick(vel, acc, h: float) -> np.ndarray:
    """Returns v + h a (float64 [N, 3])."""
    v = _vec3(vel).copy()
    a = _vec3(acc)
    _load().oracle_kick(v, a, v.shape[0], float(h))
    return v


def drift(pos, vel, dt: float) -> np.ndarray:
    """Returns x + dt v (float64 [N, 3])."""
    x = _vec3(pos).copy()
    v = _vec3(vel)
    _load().oracle_drift(x, v, x.shape[0], float(dt))
    return x


def kdk(pos, vel, mass, G: float, eps2: float, dt: float, nsteps: int):
    """nsteps of kick-drift-kick leapfrog. Returns (pos, vel, acc) float64 [N, 3]."""
    x = _vec3(pos).copy()
    v = _vec3(vel).copy()
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    a = np.zeros_like(x)
    _load().oracle_kdk(x, v, mass, x.shape[0], float(G), float(eps2), float(dt),
                       int(nsteps), a)
    return x, v, a
