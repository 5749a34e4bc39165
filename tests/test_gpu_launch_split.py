"""Split launches: a pass whose grid would pass HIP's 2^32 work-item limit
issues its blocks in several launches.  With the per-launch block count
lowered (nbody_set_launch_block_cap), small inputs take that path, and every
pass must give bitwise the result of its single launch: each block computes
the same thing whichever launch it is in (the panel pairs by their number,
the one-sided blocks by their offset)."""
import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G, EPS2 = 0.7, 1e-4
CAPS = (1, 3, 8, 29)


def run_capped(fn, caps=CAPS):
    """fn() once without a cap, then once per cap; returns the results."""
    torch.cuda.synchronize()
    out = [fn()]
    try:
        for cap in caps:
            nb.nbody_set_launch_block_cap(cap)
            out.append(fn())
    finally:
        nb.nbody_set_launch_block_cap(0)
    return out


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().copy()


def bodies(n, seed):
    pm_np, v_np = workloads.uniform_cube(n, seed=seed, masses="lognormal")
    return torch.from_numpy(pm_np).to(DEV), torch.from_numpy(v_np).to(DEV)


def assert_all_equal(results, what):
    for k, r in enumerate(results[1:]):
        assert np.array_equal(r, results[0]), f"{what}: capped run {k + 1}"


@pytest.mark.parametrize("n", [1000, 5000])
def test_one_sided_every_variant(n):
    pm, _ = bodies(n, 300 + n)
    for v in range(nb.nbody_accel_variant_count()):
        def fn():
            out = torch.full_like(pm, float("nan"))
            nb.nbody_accel_variant(pm, G, EPS2, out, v)
            return host(out)
        assert_all_equal(run_capped(fn), f"n={n} variant {v}")


def test_one_sided_default_range_potential_and_layouts():
    n = 40000       # above the small-n variant: both defaults appear below
    pm, _ = bodies(n, 310)
    i0, ni = 1234, 20000

    def default():
        out = torch.empty_like(pm)
        nb.nbody_accel(pm, G, EPS2, out)
        return host(out)

    def small_default():
        out = torch.empty((3000, 4), dtype=torch.float32, device=DEV)
        nb.nbody_accel(pm[:3000].contiguous(), G, EPS2, out)
        return host(out)

    def share():
        out = torch.empty((ni, 4), dtype=torch.float32, device=DEV)
        nb.nbody_accel_range(pm, i0, ni, G, EPS2, out, -1)
        return host(out)

    def potential():
        out = torch.empty_like(pm)
        nb.nbody_accel_potential(pm, G, EPS2, out)
        return host(out)

    def layouts():
        pos, m = pm[:, :3].contiguous(), pm[:, 3].contiguous()
        a3 = torch.empty_like(pos)
        nb.nbody_accel_f3aos(pos, m, G, EPS2, a3)
        x, y, z = (pm[:, c].contiguous() for c in range(3))
        ax, ay, az = (torch.empty_like(x) for _ in range(3))
        nb.nbody_accel_soa(x, y, z, m, G, EPS2, ax, ay, az)
        return np.concatenate([host(a3).ravel(), host(ax), host(ay), host(az)])

    for name, fn in [("nbody_accel", default), ("nbody_accel n=3000", small_default),
                     ("range", share), ("potential", potential), ("layouts", layouts)]:
        assert_all_equal(run_capped(fn, caps=(1, 7, 100)), name)


@pytest.mark.parametrize("n", [3000, 9000])
def test_pair_symmetric_every_variant_whole_chunked_and_phases(n):
    pm, _ = bodies(n, 320 + n)
    for v in range(nb.nbody_accel_symmetric_variant_count()):
        ws = torch.empty(max(nb.nbody_accel_symmetric_workspace_bytes(n, v), 16),
                         dtype=torch.uint8, device=DEV)
        cws = torch.empty(max(nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, 32), 16),
                          dtype=torch.uint8, device=DEV)

        def whole():
            out = torch.full_like(pm, float("nan"))
            nb.nbody_accel_symmetric(pm, G, EPS2, out, ws, v)
            return host(out)

        def chunked():
            out = torch.full_like(pm, float("nan"))
            nb.nbody_accel_symmetric_chunked(pm, G, EPS2, out, cws, v, 32)
            return host(out)

        def phases():
            out = torch.full_like(pm, float("nan"))
            nb.nbody_accel_symmetric_tasks(pm, EPS2, ws, v)
            nb.nbody_accel_symmetric_reduce(n, G, out, ws, v)
            return host(out)

        ref = whole()
        for name, fn in [("whole", whole), ("chunked", chunked), ("phases", phases)]:
            res = run_capped(fn)
            assert np.array_equal(res[0], ref), f"n={n} v{v} {name} uncapped"
            assert_all_equal(res, f"n={n} v{v} {name}")


def test_pair_symmetric_potential_every_variant():
    n = 5000
    pm, _ = bodies(n, 330)
    for v in range(nb.nbody_accel_symmetric_potential_variant_count()):
        ws = torch.empty(max(nb.nbody_accel_symmetric_potential_workspace_bytes(n, v), 16),
                         dtype=torch.uint8, device=DEV)

        def fn():
            out = torch.full_like(pm, float("nan"))
            nb.nbody_accel_symmetric_potential(pm, G, EPS2, out, ws, v)
            return host(out)
        assert_all_equal(run_capped(fn), f"potential v{v}")


@pytest.mark.parametrize("n", [1, 2049, 9000])
def test_energy_and_its_static_entry(n):
    pm_np, v_np = workloads.plummer(n, seed=340 + n)
    pm, vel = torch.from_numpy(pm_np).to(DEV), torch.from_numpy(v_np).to(DEV)
    ws = torch.empty(max(nb.nbody_energy_workspace_bytes(n), 16), dtype=torch.uint8, device=DEV)

    def energy():
        st = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
        nb.nbody_energy(pm, vel, G, EPS2, ws, st)
        return host(st)

    def static():
        st = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
        nb.nbody_energy_static(pm, vel, G, EPS2, st)
        return host(st)

    ref = energy()
    assert np.all(np.isfinite(ref))
    assert_all_equal(run_capped(energy), f"energy n={n}")
    res = run_capped(static)
    assert np.array_equal(res[0], ref), f"static n={n}"
    assert_all_equal(res, f"energy static n={n}")


def test_cap_is_restored():
    """A call after the cap is lifted (0) launches whole again and gives the
    capped call's result."""
    n = 5000
    pm, _ = bodies(n, 350)
    out = torch.empty_like(pm)
    nb.nbody_set_launch_block_cap(2)
    try:
        nb.nbody_accel(pm, G, EPS2, out)
        capped = host(out)
    finally:
        nb.nbody_set_launch_block_cap(0)
    nb.nbody_accel(pm, G, EPS2, out)
    assert np.array_equal(host(out), capped)


def test_energy_past_one_launch_at_full_size():
    """12.6 million bodies make 18.9 million panel pairs of 2048 bodies, more
    blocks of 256 threads than one launch can hold (2^32 - 1 work-items), so
    the energy pair pass really goes out as two launches.  Its W must agree
    with W from the one-sided pass's potentials (nbody_accel_potential, then
    nbody_energy_from_potential; fp32 sums of 12.6 million terms, so 2e-5),
    and a repeat must be bitwise: a range launched twice or not at all would
    move W by about a tenth."""
    n = 12_600_000
    pm_np, v_np = workloads.uniform_cube(n, seed=77, masses="lognormal")
    need = nb.nbody_energy_workspace_bytes(n)
    pairs = need // 8 - 8 * (-(-n // 256))          # one double per pair after the block sums
    assert pairs * 256 > 2**32 - 1, pairs
    print(f"energy at n={n}: {pairs} panel pairs", flush=True)
    msum = float(pm_np[:, 3].astype(np.float64).sum())
    pm, vel = torch.from_numpy(pm_np).to(DEV), torch.from_numpy(v_np).to(DEV)
    del pm_np, v_np
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
    nb.nbody_energy(pm, vel, G, EPS2, ws, st)
    direct = host(st)
    nb.nbody_energy(pm, vel, G, EPS2, ws, st)
    assert np.array_equal(host(st), direct)
    acc = torch.empty_like(pm)
    nb.nbody_accel_potential(pm, G, EPS2, acc)
    wsp = torch.empty(nb.nbody_energy_from_potential_workspace_bytes(n), dtype=torch.uint8,
                      device=DEV)
    stp = torch.full((8,), float("nan"), dtype=torch.float64, device=DEV)
    nb.nbody_energy_from_potential(pm, vel, acc, wsp, stp)
    via_potential = host(stp)
    e = dict(zip(nb.ENERGY_FIELDS, direct))
    p = dict(zip(nb.ENERGY_FIELDS, via_potential))
    print(f"  W {e['W']:.12e} direct, {p['W']:.12e} from potentials", flush=True)
    assert np.isfinite(e["W"]) and e["W"] < 0
    assert abs(e["W"] - p["W"]) <= 2e-5 * abs(e["W"])
    assert abs(e["M"] - msum) <= 1e-12 * msum and abs(p["M"] - msum) <= 1e-12 * msum
