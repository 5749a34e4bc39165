"""nbody_kdk_run: kick-drift-kick steps run by the library (README section
1.3 read as standard kick-drift-kick, with the closing half kick) must leave
bitwise the state that nbody_leapfrog_step, the force pass and nbody_kick
leave when called one by one, for every force pass it can run, also when
the caller captures the call into a HIP graph and replays it."""
import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G, EPS2, DT = 1.0, 1e-4, 1e-3
KINDS = [nb.NBODY_PASS_ONE_SIDED, nb.NBODY_PASS_SYMMETRIC, nb.NBODY_PASS_SYMMETRIC_POTENTIAL,
         nb.NBODY_PASS_SYMMETRIC_CHUNKED]


def workspace(kind, n):
    if kind == nb.NBODY_PASS_ONE_SIDED:
        return None
    if kind == nb.NBODY_PASS_SYMMETRIC:
        need = nb.nbody_accel_symmetric_workspace_bytes(n)
    elif kind == nb.NBODY_PASS_SYMMETRIC_CHUNKED:
        need = nb.nbody_accel_symmetric_chunked_workspace_bytes(n, -1, 0)
    else:
        need = nb.nbody_accel_symmetric_potential_workspace_bytes(n)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)


def force(kind, pm, acc, ws, stream=None):
    if kind == nb.NBODY_PASS_ONE_SIDED:
        nb.nbody_accel(pm, G, EPS2, acc, stream)
    elif kind == nb.NBODY_PASS_SYMMETRIC:
        nb.nbody_accel_symmetric(pm, G, EPS2, acc, ws, stream=stream)
    elif kind == nb.NBODY_PASS_SYMMETRIC_CHUNKED:
        nb.nbody_accel_symmetric_chunked(pm, G, EPS2, acc, ws, stream=stream)
    else:
        nb.nbody_accel_symmetric_potential(pm, G, EPS2, acc, ws, stream=stream)


def start(kind, n, seed, arrays=None):
    pm_np, v_np = arrays if arrays is not None else workloads.plummer(n, seed=seed)
    pm = torch.from_numpy(pm_np).to(DEV)
    vel = torch.from_numpy(v_np).to(DEV)
    acc = torch.empty_like(pm)
    ws = workspace(kind, n)
    force(kind, pm, acc, ws)
    torch.cuda.synchronize()
    return pm, vel, acc, ws


def one_by_one(kind, pm, vel, acc, ws, steps):
    for _ in range(steps):
        nb.nbody_leapfrog_step(pm, vel, acc, DT)
        force(kind, pm, acc, ws)
        nb.nbody_kick(vel, acc, 0.5 * DT)
    torch.cuda.synchronize()


def state(*ts):
    return [t.cpu().numpy().copy() for t in ts]


@pytest.mark.parametrize("steps", [1, 2, 7])
@pytest.mark.parametrize("kind", KINDS)
def test_kdk_run_equals_the_calls_one_by_one(kind, steps):
    n = 5000
    pm, vel, acc, ws = start(kind, n, seed=40 + kind)
    ref = [t.clone() for t in (pm, vel, acc)]
    one_by_one(kind, *ref, ws, steps)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    nb.nbody_kdk_run(pm, vel, acc, G, EPS2, DT, steps, kind, workspace=ws, stream=s)
    s.synchronize()
    for w, g_, name in zip(state(*ref), state(pm, vel, acc), ("posmass", "vel", "accel")):
        assert np.array_equal(w, g_), f"kind {kind} steps {steps}: {name}"


def test_kdk_run_chunked_equals_whole_pass():
    """The step loop through the pass in column chunks (bounded workspace)
    leaves bitwise the state of the loop through the whole pass: 40000
    bodies (157 panels of 256), 3 steps of 5 column chunks each."""
    assert nb.nbody_accel_symmetric_panel(nb.nbody_accel_symmetric_variant_for_n(40000)) == 256
    n = 40000
    pm, vel, acc, ws = start(nb.NBODY_PASS_SYMMETRIC, n, seed=61)
    work = [t.clone() for t in (pm, vel, acc)]
    wsc = workspace(nb.NBODY_PASS_SYMMETRIC_CHUNKED, n)
    assert wsc.numel() < ws.numel()
    torch.cuda.synchronize()
    nb.nbody_kdk_run(pm, vel, acc, G, EPS2, DT, 3, nb.NBODY_PASS_SYMMETRIC, workspace=ws)
    nb.nbody_kdk_run(*work, G, EPS2, DT, 3, nb.NBODY_PASS_SYMMETRIC_CHUNKED, workspace=wsc)
    torch.cuda.synchronize()
    for w, g_, name in zip(state(pm, vel, acc), state(*work), ("posmass", "vel", "accel")):
        assert np.array_equal(w, g_), name


def test_kdk_run_captured_by_the_caller_and_replayed():
    """The caller captures 3 steps of nbody_kdk_run into a HIP graph (torch's
    graph capture on its own stream) and replays the graph 4 times, with its
    own eager work and a synchronisation between replays: after every replay
    the state equals, bit for bit, that of the calls made one by one for the
    same number of steps (the library records no memset into the graph)."""
    kind = nb.NBODY_PASS_SYMMETRIC
    n = 16384
    pm, vel, acc, ws = start(kind, n, seed=77)
    ref = [t.clone() for t in (pm, vel, acc)]
    work = [t.clone() for t in (pm, vel, acc)]
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        nb.nbody_kdk_run(*work, G, EPS2, DT, 3, kind, workspace=ws)
    # capturing ran nothing: the state is still the initial one
    for w, g_ in zip(state(pm, vel, acc), state(*work)):
        assert np.array_equal(w, g_)
    for r in range(4):
        g.replay()
        scratch = torch.full((1 << 20,), float(r + 1), device=DEV)   # unrelated eager work
        torch.cuda.synchronize()
        assert scratch.sum().item() == float(r + 1) * (1 << 20)
        one_by_one(kind, *ref, ws, 3)
        for w, g_, name in zip(state(*ref), state(*work), ("posmass", "vel", "accel")):
            assert np.array_equal(w, g_), f"replay {r}: {name}"


def test_kdk_run_plummer16k_ten_steps_conserves_energy():
    """The 10-step plummer16k run of the integration tests, through the
    library's step loop with its pair-symmetric pass: energy drift within
    1e-4."""
    w = workloads.WORKLOADS["plummer16k"]
    kind = nb.NBODY_PASS_SYMMETRIC
    pm, vel, acc, ws = start(kind, w.n, 0, arrays=workloads.make("plummer16k"))
    e0 = nb.energy(pm, vel, w.G, w.eps2)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    nb.nbody_kdk_run(pm, vel, acc, w.G, w.eps2, w.dt, w.steps, kind, workspace=ws, stream=s)
    s.synchronize()
    e1 = nb.energy(pm, vel, w.G, w.eps2)
    drift = abs(e1["E"] - e0["E"]) / abs(e0["E"])
    print(f"plummer16k kdk_run: energy drift {drift:.3e}", flush=True)
    assert drift <= 1e-4
