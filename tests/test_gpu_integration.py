"""Integrator and energy on the GPU: the kick/drift kernels against the
oracle's kick/drift on identical inputs, the energy reduction against the
oracle's energy, and whole kick-drift-kick runs of the project's workloads
(energy drift, momentum, the trajectory against the oracle's own float64
integration, force parity on the oracle's evolved state, time
reversibility).  No oracle input is taken from a GPU result."""
import math

import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import oracle
import workloads
from parity import assert_parity, errors, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = np.float32
ULP = 2.0 ** -23


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_leapfrog_kernel_matches_oracle_kick_drift():
    g = np.random.default_rng(1)
    n = 5000
    pm = g.uniform(-2, 2, (n, 4)).astype(F32)
    pm[:, 3] = g.uniform(0.1, 1.0, n).astype(F32)
    vel = g.uniform(-1, 1, (n, 4)).astype(F32)
    vel[:, 3] = g.uniform(-9, 9, n).astype(F32)        # w must survive untouched
    acc = g.uniform(-3, 3, (n, 4)).astype(F32)
    dt = F32(1e-2)
    tp, tv, ta = to_dev(pm), to_dev(vel), to_dev(acc)
    nb.nbody_leapfrog_step(tp, tv, ta, float(dt))
    torch.cuda.synchronize()
    x_gpu, v_gpu = tp.cpu().numpy(), tv.cpu().numpy()
    v_ref = oracle.kick(vel, acc, 0.5 * float(dt))
    x_ref = oracle.drift(pm, v_ref, float(dt))
    # v: one rounding of the exact v + h a; x: one rounding plus dt times v's.
    assert np.all(np.abs(v_gpu[:, :3] - v_ref) <= ULP * np.abs(v_ref))
    bound = ULP * (np.abs(x_ref) + float(dt) * np.abs(v_ref))
    assert np.all(np.abs(x_gpu[:, :3] - x_ref) <= bound)
    assert np.array_equal(x_gpu[:, 3], pm[:, 3])
    assert np.array_equal(v_gpu[:, 3], vel[:, 3])
    assert np.array_equal(ta.cpu().numpy(), acc)


def test_kick_kernel_matches_oracle():
    g = np.random.default_rng(2)
    n = 4099
    vel = g.uniform(-1, 1, (n, 4)).astype(F32)
    acc = g.uniform(-3, 3, (n, 4)).astype(F32)
    h = F32(5e-4)
    tv, ta = to_dev(vel), to_dev(acc)
    nb.nbody_kick(tv, ta, float(h))
    torch.cuda.synchronize()
    v = tv.cpu().numpy()
    v_ref = oracle.kick(vel, acc, float(h))
    assert np.all(np.abs(v[:, :3] - v_ref) <= ULP * np.abs(v_ref))
    assert np.array_equal(v[:, 3], vel[:, 3])


def gpu_energy(pm_np, vel_np, G, eps2):
    return nb.energy(to_dev(pm_np), to_dev(vel_np), G, eps2)


def ref_energy(pm_np, vel_np, G, eps2):
    pos, mass = oracle.split_posmass(pm_np)
    return oracle.energy(pos, vel_np, mass, float(F32(G)), float(F32(eps2)))


@pytest.mark.parametrize("n", [1, 2, 3, 65, 1000, 4097, 70000])
def test_energy_matches_oracle(n):
    pm, vel = workloads.plummer(n, seed=n) if n > 1 else (
        np.array([[0.1, 0.2, 0.3, 2.0]], F32), np.array([[1, 2, 3, 0]], F32))
    log(f"energy n={n}")
    e = gpu_energy(pm, vel, 1.0, 1e-4)
    r = ref_energy(pm, vel, 1.0, 1e-4)
    assert abs(e["K"] - r["K"]) <= 1e-12 * abs(r["K"])
    assert abs(e["M"] - r["M"]) <= 1e-12 * r["M"]
    if n > 1:
        assert abs(e["W"] - r["W"]) <= 2e-6 * abs(r["W"])
    else:
        assert e["W"] == 0.0
    # summation-order rounding of P scales with sum m |v|, not with |P| ~ 0
    mv = float((pm[:, 3].astype(np.float64) *
                np.linalg.norm(vel[:, :3].astype(np.float64), axis=1)).sum())
    for k in ("Px", "Py", "Pz"):
        assert abs(e[k] - r[k]) <= 1e-13 * mv


def test_energy_two_body_closed_form():
    pm = np.array([[0, 0, 0, 1], [3, 4, 0, 1]], F32)
    vel = np.array([[1, 0, 0, 0], [0, 2, 0, 0]], F32)
    e = gpu_energy(pm, vel, 1.0, 11.0)
    assert e["K"] == 2.5
    assert abs(e["W"] + 1.0 / 6.0) <= 1e-7
    assert (e["Px"], e["Py"], e["Pz"], e["M"]) == (1.0, 2.0, 0.0, 2.0)


def test_energy_deterministic():
    pm, vel = workloads.make("plummer16k")
    a = gpu_energy(pm, vel, 1.0, 1e-4)
    b = gpu_energy(pm, vel, 1.0, 1e-4)
    assert a == b


# The two force passes a kick-drift-kick step can use: the one-sided
# nbody_accel, and the pair-symmetric nbody_accel_symmetric (the library's
# variant for n, the pass bench.py times at 2^20 bodies).
FORCE_PATHS = ("one_sided", "symmetric")


def force_pass(path, n):
    """None (nb.kdk_step's default, nbody_accel) or a SymmetricPass for n."""
    return None if path == "one_sided" else nb.SymmetricPass(n, DEV)


def accel_with(force, pm, G, eps2, acc):
    if force is None:
        nb.nbody_accel(pm, G, eps2, acc)
    else:
        force(pm, G, eps2, acc)


def run_kdk(pm_np, vel_np, G, eps2, dt, steps, check_every=None, path="one_sided"):
    pm, vel = to_dev(pm_np), to_dev(vel_np)
    acc = torch.empty_like(pm)
    force = force_pass(path, pm.shape[0])
    accel_with(force, pm, G, eps2, acc)
    energies = [nb.energy(pm, vel, G, eps2)]
    for s in range(steps):
        nb.kdk_step(pm, vel, acc, G, eps2, dt, force=force)
        if check_every and (s + 1) % check_every == 0:
            energies.append(nb.energy(pm, vel, G, eps2))
    torch.cuda.synchronize()
    return pm, vel, acc, energies


@pytest.mark.parametrize("path", FORCE_PATHS)
def test_plummer16k_ten_steps(path):
    w = workloads.WORKLOADS["plummer16k"]
    pm0, v0 = workloads.make("plummer16k")
    pm, vel, acc, es = run_kdk(pm0, v0, w.G, w.eps2, w.dt, w.steps, check_every=w.steps,
                               path=path)
    drift = abs(es[-1]["E"] - es[0]["E"]) / abs(es[0]["E"])
    log(f"plummer16k ({path}) energy drift {drift:.3e}")
    assert drift <= 1e-4
    pm_np = pm.cpu().numpy()
    assert np.array_equal(pm_np[:, 3], pm0[:, 3])
    # trajectory against the oracle's own float64 integration
    pos0, mass0 = oracle.split_posmass(pm0)
    x_ref, v_ref, a_ref = oracle.kdk(pos0, v0, mass0, w.G, float(F32(w.eps2)),
                                     float(F32(w.dt)), w.steps)
    # accelerations at step 10: the oracle's step-10 state, rounded to float32,
    # is the input of both the GPU force pass and the oracle's force (no oracle
    # input comes from the GPU run)
    pm10 = np.concatenate([x_ref.astype(F32), pm0[:, 3:4]], axis=1)
    t10 = to_dev(pm10)
    a10 = torch.empty_like(t10)
    accel_with(force_pass(path, w.n), t10, w.G, w.eps2, a10)
    torch.cuda.synchronize()
    pos10, mass10 = oracle.split_posmass(pm10)
    assert_parity(a10.cpu().numpy(), oracle.accel(pos10, mass10, w.G, float(F32(w.eps2))),
                  f"plummer16k step-10 state ({path})")
    # the GPU run's own step-10 accelerations against the oracle run's: the
    # states differ by the trajectory error checked below, so only the
    # relative L2 bar is asserted; the worst body is reported
    l2, worst = errors(acc.cpu().numpy(), a_ref)
    log(f"plummer16k step 10 ({path}): GPU run's accel vs oracle run's accel, rel L2 {l2:.2e}, "
        f"worst body {worst:.2e}")
    assert l2 <= 1e-5
    # ten fp32 drifts round x ten times (~0.5 ulp each), so the bound scales
    # with |x|: untruncated Plummer bodies reach |x| ~ 10^2 where 1 ulp ~ 1e-5
    dx = np.abs(pm_np[:, :3] - x_ref)
    dv = np.abs(vel.cpu().numpy()[:, :3] - v_ref)
    log(f"plummer16k trajectory vs oracle: max |dx| {dx.max():.2e}, "
        f"max |dx|/(|x|+1) {(dx / (np.abs(x_ref) + 1)).max():.2e}, max |dv| {dv.max():.2e}")
    assert np.all(dx <= 2e-6 * (np.abs(x_ref) + 1.0))
    assert np.all(dv <= 2e-6 * (np.abs(v_ref) + 1.0))


@pytest.mark.parametrize("path", FORCE_PATHS)
def test_time_reversibility(path):
    pm0, v0 = workloads.plummer(4096, seed=8)
    G, eps2, dt = 1.0, 1e-4, 1e-3
    pm, vel, acc, _ = run_kdk(pm0, v0, G, eps2, dt, 10, path=path)
    vel[:, :3] = -vel[:, :3]
    force = force_pass(path, pm.shape[0])
    accel_with(force, pm, G, eps2, acc)
    for _ in range(10):
        nb.kdk_step(pm, vel, acc, G, eps2, dt, force=force)
    torch.cuda.synchronize()
    x0 = pm0[:, :3].astype(np.float64)
    dx = np.abs(pm.cpu().numpy()[:, :3] - x0)
    dv = np.abs(-vel.cpu().numpy()[:, :3] - v0[:, :3])
    log(f"reversibility ({path}): max |dx|/(|x|+1) {(dx / (np.abs(x0) + 1)).max():.2e}, "
        f"max |dv| {dv.max():.2e}")
    assert np.all(dx <= 4e-6 * (np.abs(x0) + 1.0))
    assert dv.max() <= 1e-5


@pytest.mark.parametrize("path", FORCE_PATHS)
def test_collision1m_twenty_steps(path):
    """Two Plummer spheres, N = 1000003, 20 KDK steps of dt = 1e-3:
    momentum change <= 1e-6, relative energy drift <= 1e-3, and Newton's third
    law on the final accelerations (the oracle cannot integrate 10^6 bodies in
    a test's time; step-0 parity over every body is in
    test_gpu_parity_full.py)."""
    w = workloads.WORKLOADS["collision1m"]
    pm0, v0 = workloads.make("collision1m")
    log(f"collision1m ({path}): integrating")
    pm, vel, acc, es = run_kdk(pm0, v0, w.G, w.eps2, w.dt, w.steps, check_every=w.steps,
                               path=path)
    e0, e1 = es[0], es[-1]
    dp = math.sqrt(sum((e1[k] - e0[k]) ** 2 for k in ("Px", "Py", "Pz")))
    drift = abs(e1["E"] - e0["E"]) / abs(e0["E"])
    log(f"collision1m ({path}): |dP| {dp:.3e}, energy drift {drift:.3e}")
    assert dp <= 1e-6
    assert drift <= 1e-3
    pm_np = pm.cpu().numpy()
    assert np.array_equal(pm_np[:, 3], pm0[:, 3])
    a = acc.cpu().numpy()[:, :3].astype(np.float64)
    m = pm_np[:, 3:4].astype(np.float64)
    newton = np.linalg.norm((m * a).sum(axis=0)) / (m[:, 0] * np.linalg.norm(a, axis=1)).sum()
    log(f"collision1m ({path}) step 20: |sum m a| / sum m|a| = {newton:.2e}")
    assert newton <= 1e-6
    assert np.all(a[:, :3] == a[:, :3])          # no NaN


# ---------------------------------------------------------------------------
# Potential carried in accel.w, and the O(N) energy built from it
# ---------------------------------------------------------------------------

def gpu_potential(pm_np, G=1.0, eps2=1e-4):
    t = to_dev(pm_np)
    out = torch.full_like(t, float("nan"))
    nb.nbody_accel_potential(t, G, eps2, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 4097, 16384, 70000])
def test_potential_pass(n):
    """xyz bitwise equal to nbody_accel; w = Phi_i against the oracle."""
    pm, _ = workloads.plummer(n, seed=30 + n) if n > 2 else workloads.uniform_cube(n, seed=n)
    G, eps2 = 1.5, 1e-4
    a = gpu_potential(pm, G, eps2)
    t = to_dev(pm)
    plain = torch.empty_like(t)
    nb.nbody_accel(t, G, eps2, plain)
    torch.cuda.synchronize()
    assert np.array_equal(a[:, :3], plain.cpu().numpy()[:, :3])
    if n == 1:
        assert a[0, 3] == 0.0
        return
    pos, mass = oracle.split_posmass(pm)
    rows = np.arange(n) if n <= 20000 else np.unique(np.concatenate(
        [np.arange(64), np.arange(n - 64, n), np.random.default_rng(1).choice(n, 512, False)]))
    ref = oracle.potential_rows(pos, mass, float(F32(G)), float(F32(eps2)), rows)
    got = a[rows, 3].astype(np.float64)
    l2 = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    worst = np.max(np.abs(got - ref) / np.abs(ref))
    log(f"potential n={n}: rel L2 {l2:.2e}, worst {worst:.2e}")
    assert l2 <= 1e-6 and worst <= 1e-5


@pytest.mark.parametrize("name", ["uniform1k", "plummer16k"])
def test_energy_from_potential(name):
    w = workloads.WORKLOADS[name]
    pm, vel = workloads.make(name)
    a = to_dev(gpu_potential(pm, w.G, w.eps2))
    ws = torch.empty(nb.nbody_energy_from_potential_workspace_bytes(w.n), dtype=torch.uint8,
                     device=DEV)
    stats = torch.zeros(8, dtype=torch.float64, device=DEV)
    nb.nbody_energy_from_potential(to_dev(pm), to_dev(vel), a, ws, stats)
    torch.cuda.synchronize()
    e = dict(zip(nb.ENERGY_FIELDS, stats.cpu().tolist()))
    r = ref_energy(pm, vel, w.G, w.eps2)
    direct = gpu_energy(pm, vel, w.G, w.eps2)
    assert abs(e["W"] - r["W"]) <= 2e-6 * abs(r["W"])
    assert abs(e["W"] - direct["W"]) <= 2e-6 * abs(r["W"])
    # same fp64 per-body terms as nbody_energy, summed by a different tree
    mv = float((pm[:, 3].astype(np.float64) *
                np.linalg.norm(vel[:, :3].astype(np.float64), axis=1)).sum())
    assert abs(e["K"] - direct["K"]) <= 1e-13 * abs(direct["K"]) + 1e-300
    assert abs(e["M"] - direct["M"]) <= 1e-13 * direct["M"]
    for k in ("Px", "Py", "Pz"):
        assert abs(e[k] - direct[k]) <= 1e-13 * mv, k


# ---------------------------------------------------------------------------
# Pair-symmetric pass with the potential in accel.w
# ---------------------------------------------------------------------------

# the plain pair-symmetric variant with the same (K, KP, waves) panel shape,
# and the same way of carrying the j-side sums (rotated along the lanes, or
# kept in LDS), as each potential variant: their xyz arithmetic and order are
# the same
SYM_POT_TWIN = {0: 0, 1: 1, 2: 2, 3: 3}


def gpu_sym(pm_np, G, eps2, variant, pot):
    t = to_dev(pm_np)
    n = pm_np.shape[0]
    out = torch.full_like(t, float("nan"))
    if pot:
        need = nb.nbody_accel_symmetric_potential_workspace_bytes(n, variant)
    else:
        need = nb.nbody_accel_symmetric_workspace_bytes(n, variant)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    if pot:
        nb.nbody_accel_symmetric_potential(t, G, eps2, out, ws, variant)
    else:
        nb.nbody_accel_symmetric(t, G, eps2, out, ws, variant)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_potential(a, pm, G, eps2, rows, what):
    pos, mass = oracle.split_posmass(pm)
    ref = oracle.potential_rows(pos, mass, float(F32(G)), float(F32(eps2)), rows)
    got = a[rows, 3].astype(np.float64)
    l2 = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    worst = np.max(np.abs(got - ref) / np.abs(ref))
    log(f"  potential {what}: rel L2 {l2:.2e}, worst {worst:.2e}")
    assert l2 <= 1e-6 and worst <= 1e-5


@pytest.mark.parametrize("n", [1, 2, 3, 65, 1000, 2048, 2049, 5000])
def test_symmetric_potential_every_variant(n):
    """Every potential variant: xyz bitwise equal to the plain pair-symmetric
    pass of the same panel shape, xyz against the oracle's acceleration and w
    against the oracle's potential (self term excluded)."""
    pm, _ = workloads.plummer(n, seed=200 + n) if n > 3 else workloads.uniform_cube(n, seed=n)
    G, eps2 = 1.25, 1e-4
    pos, mass = oracle.split_posmass(pm)
    ref = oracle.accel(pos, mass, float(F32(G)), float(F32(eps2)))
    for v in range(nb.nbody_accel_symmetric_potential_variant_count()):
        log(f"n={n} potential variant {v}")
        assert (nb.nbody_accel_symmetric_potential_panel(v)
                == nb.nbody_accel_symmetric_panel(SYM_POT_TWIN[v]))
        a = gpu_sym(pm, G, eps2, v, True)
        plain = gpu_sym(pm, G, eps2, SYM_POT_TWIN[v], False)
        assert np.array_equal(a[:, :3], plain[:, :3]), v
        if n == 1:
            assert np.array_equal(a, np.zeros((1, 4), F32))
            continue
        assert_parity(a, ref, f"symmetric potential n={n} v={v}")
        check_potential(a, pm, G, eps2, np.arange(n), f"n={n} v={v}")


def test_symmetric_potential_energy_plummer16k():
    """The checkpoint path: pair-symmetric pass with potentials, then the O(N)
    energy from them, against the oracle's energy."""
    w = workloads.WORKLOADS["plummer16k"]
    pm, vel = workloads.make("plummer16k")
    a = to_dev(gpu_sym(pm, w.G, w.eps2, -1, True))
    ws = torch.empty(nb.nbody_energy_from_potential_workspace_bytes(w.n), dtype=torch.uint8,
                     device=DEV)
    stats = torch.zeros(8, dtype=torch.float64, device=DEV)
    nb.nbody_energy_from_potential(to_dev(pm), to_dev(vel), a, ws, stats)
    torch.cuda.synchronize()
    e = dict(zip(nb.ENERGY_FIELDS, stats.cpu().tolist()))
    r = ref_energy(pm, vel, w.G, w.eps2)
    log(f"plummer16k W: symmetric potential {e['W']:.12e}, oracle {r['W']:.12e}")
    assert abs(e["W"] - r["W"]) <= 2e-6 * abs(r["W"])
    assert abs(e["E"] - r["E"]) <= 2e-6 * abs(r["E"])


def test_symmetric_potential_plummer1m_sampled():
    """Full size, the variant the library picks for 2^20 bodies: xyz bitwise
    equal to the plain pass's default, sampled rows of xyz and of the
    potential against the oracle."""
    w = workloads.WORKLOADS["plummer1m"]
    pm, _ = workloads.make("plummer1m")
    a = gpu_sym(pm, w.G, w.eps2, -1, True)
    plain = gpu_sym(pm, w.G, w.eps2, -1, False)
    assert np.array_equal(a[:, :3], plain[:, :3])      # default variants share a panel shape
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.n - 64, w.n),
                                     np.random.default_rng(7).choice(w.n, 192, False)]))
    pos, mass = oracle.split_posmass(pm)
    ref = oracle.accel_rows(pos, mass, w.G, float(F32(w.eps2)), rows)
    assert_parity(a[rows], ref, "symmetric potential plummer1m")
    check_potential(a, pm, w.G, w.eps2, rows, "plummer1m")


@pytest.mark.parametrize("path", FORCE_PATHS)
def test_circular_binary_one_orbit(path):
    """Equal-mass circular binary (d = 1, eps^2 = 1e-4, omega^2 = G (m1 + m2) /
    (d^2 + eps^2)^{3/2}) for one period at dt = T/1000 with the GPU's KDK
    step: the separation stays within (omega dt)^2 plus float32 rounding of d,
    and the bodies come back near their start (phase error O((omega dt)^2))."""
    eps2 = 1e-4
    m = 0.5
    omega = math.sqrt(2 * m / (1.0 + eps2) ** 1.5)
    period = 2 * math.pi / omega
    steps = 1000
    dt = float(F32(period / steps))
    pm0 = np.array([[-0.5, 0, 0, m], [0.5, 0, 0, m]], F32)
    v0 = np.array([[0, -omega * 0.5, 0, 0], [0, omega * 0.5, 0, 0]], F32)
    pm, vel = to_dev(pm0), to_dev(v0)
    acc = torch.empty_like(pm)
    force = force_pass(path, 2)
    accel_with(force, pm, 1.0, eps2, acc)
    worst = 0.0
    for k in range(steps):
        nb.kdk_step(pm, vel, acc, 1.0, eps2, dt, force=force)
        if (k + 1) % 50 == 0:
            x = pm.cpu().numpy()[:, :3].astype(np.float64)
            worst = max(worst, abs(np.linalg.norm(x[1] - x[0]) - 1.0))
    torch.cuda.synchronize()
    x = pm.cpu().numpy()[:, :3].astype(np.float64)
    log(f"circular binary ({path}): max |d - 1| {worst:.2e} (bound {(omega * dt) ** 2:.2e}), "
        f"return error {np.abs(x - pm0[:, :3]).max():.2e}")
    assert worst <= (omega * dt) ** 2 + 1e-5
    assert np.abs(x - pm0[:, :3]).max() <= 2e-3


# ---------------------------------------------------------------------------
# Streams
# ---------------------------------------------------------------------------

def test_calls_on_side_streams_run_concurrently_and_match():
    """Every entry point takes the stream it is queued on: the pair-symmetric
    pass (one call and its two phases), the one-sided pass and the energy,
    queued on two side streams with their own outputs and workspaces, match
    the same calls made one after the other on the current stream bitwise."""
    n = 20000
    pm_np, vel_np = workloads.plummer(n, seed=77)
    pm, vel = to_dev(pm_np), to_dev(vel_np)
    ws_a = torch.empty(nb.nbody_accel_symmetric_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty_like(ws_a)
    ews = torch.empty(nb.nbody_energy_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    ref_sym, ref_one = torch.empty_like(pm), torch.empty_like(pm)
    ref_stats = torch.zeros(8, dtype=torch.float64, device=DEV)
    nb.nbody_accel_symmetric(pm, 1.0, 1e-4, ref_sym, ws_a)
    nb.nbody_accel(pm, 1.0, 1e-4, ref_one)
    nb.nbody_energy(pm, vel, 1.0, 1e-4, ews, ref_stats)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    out_sym, out_two, out_one = (torch.full_like(pm, float("nan")) for _ in range(3))
    stats = torch.zeros(8, dtype=torch.float64, device=DEV)
    ews2 = torch.empty_like(ews)
    torch.cuda.synchronize()
    nb.nbody_accel_symmetric(pm, 1.0, 1e-4, out_sym, ws_a, stream=s1)
    nb.nbody_accel_symmetric_tasks(pm, 1e-4, ws_b, stream=s2)
    nb.nbody_accel(pm, 1.0, 1e-4, out_one, stream=s1)
    nb.nbody_accel_symmetric_reduce(n, 1.0, out_two, ws_b, stream=s2)
    nb.nbody_energy(pm, vel, 1.0, 1e-4, ews2, stats, stream=s2)
    s1.synchronize()
    s2.synchronize()
    assert torch.equal(out_sym, ref_sym)
    assert torch.equal(out_two, ref_sym)
    assert torch.equal(out_one, ref_one)
    assert torch.equal(stats, ref_stats)
