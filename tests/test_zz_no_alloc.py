"""The allocation-free energy entry point, nbody_energy_static: the same
kernels as nbody_energy with the library's static device scratch in place of
a caller workspace.  Its output must equal nbody_energy's bit for bit, on
consecutive calls whose sizes differ (the second call finds the scratch as
the first left it), and sizes past the scratch must be rejected before
anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = np.float32


def with_workspace(pm, vel, G, eps2):
    n = pm.shape[0]
    ws = torch.empty(max(nb.nbody_energy_workspace_bytes(n), 16), dtype=torch.uint8, device=DEV)
    stats = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
    nb.nbody_energy(pm, vel, G, eps2, ws, stats)
    torch.cuda.synchronize()
    return stats.cpu().numpy()


def static(pm, vel, G, eps2):
    stats = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
    nb.nbody_energy_static(pm, vel, G, eps2, stats)
    torch.cuda.synchronize()
    return stats.cpu().numpy()


def largest_n():
    """The largest n whose energy scratch fits the static array."""
    lo, hi = 1, nb.NBODY_MAX_N
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if nb.nbody_energy_workspace_bytes(mid) <= nb.NBODY_ENERGY_STATIC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def test_static_scratch_equals_workspace_on_consecutive_calls():
    """A 300001-body Plummer sphere, then a 4097-body one: both bitwise equal
    to nbody_energy with a fresh workspace; the small one also against the
    oracle's energy (W to 2e-6, K and M to 1e-12)."""
    for n, seed in ((300001, 3), (4097, 4)):
        pm_np, vel_np = workloads.plummer(n, seed=seed)
        pm = torch.from_numpy(pm_np).to(DEV)
        vel = torch.from_numpy(vel_np).to(DEV)
        a = static(pm, vel, 1.0, 1e-4)
        b = with_workspace(pm, vel, 1.0, 1e-4)
        print(f"n={n}: static {a[:3]}, workspace {b[:3]}", flush=True)
        assert np.array_equal(a, b), n
        assert np.all(np.isfinite(a))
    pos, mass = oracle.split_posmass(pm_np)
    r = oracle.energy(pos, vel_np, mass, 1.0, float(F32(1e-4)))
    assert abs(a[1] - r["W"]) <= 2e-6 * abs(r["W"])
    assert abs(a[0] - r["K"]) <= 1e-12 * abs(r["K"])
    assert abs(a[6] - r["M"]) <= 1e-12 * r["M"]


def test_static_scratch_size_limit():
    """n up to the documented bound runs; one body more is rejected with
    NBODY_ERR_WORKSPACE before the library touches anything."""
    nmax = largest_n()
    print(f"largest n for the static scratch: {nmax}", flush=True)
    assert 4_000_000 <= nmax < 4_100_000
    lib = nb.load_library()
    vp = ctypes.c_void_p
    stats = torch.empty(8, dtype=torch.float64, device=DEV)
    st = vp(torch.cuda.current_stream().cuda_stream)
    assert lib.nbody_energy_static(vp(0x10000000), vp(0x20000000), nmax + 1, 1.0, 1e-4,
                                   vp(stats.data_ptr()), st) == nb.NBODY_ERR_WORKSPACE
    assert lib.nbody_energy_static(vp(0x10000000), vp(0x20000000), 0, 1.0, 1e-4,
                                   vp(stats.data_ptr()), st) == nb.NBODY_OK
