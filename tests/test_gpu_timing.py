"""The timing exports on the GPU: nbody_time_accel runs the same force pass
as the plain entry point (bitwise the same accelerations) and reports
positive times whose parts fit inside the whole; the nbody_timer events
bracket work on the stream they are recorded on.  The timing calls are the
event-timing pattern of the atomics tutorial ("CUDA programming (9)", its
timing() helper), repeated over several runs."""
import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N = 5000
G, EPS2 = 1.0, 1e-4


def plain_pass(kind, pm, ws):
    out = torch.full_like(pm, float("nan"))
    if kind == nb.NBODY_PASS_ONE_SIDED:
        nb.nbody_accel(pm, G, EPS2, out)
    elif kind == nb.NBODY_PASS_SYMMETRIC:
        nb.nbody_accel_symmetric(pm, G, EPS2, out, ws)
    elif kind == nb.NBODY_PASS_SYMMETRIC_CHUNKED:
        nb.nbody_accel_symmetric_chunked(pm, G, EPS2, out, ws)
    else:
        nb.nbody_accel_symmetric_potential(pm, G, EPS2, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def workspace(kind):
    if kind == nb.NBODY_PASS_ONE_SIDED:
        return None
    if kind == nb.NBODY_PASS_SYMMETRIC:
        need = nb.nbody_accel_symmetric_workspace_bytes(N)
    elif kind == nb.NBODY_PASS_SYMMETRIC_CHUNKED:
        need = nb.nbody_accel_symmetric_chunked_workspace_bytes(N, -1, 0)
    else:
        need = nb.nbody_accel_symmetric_potential_workspace_bytes(N)
    return torch.empty(need, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("kind", [nb.NBODY_PASS_ONE_SIDED, nb.NBODY_PASS_SYMMETRIC,
                                  nb.NBODY_PASS_SYMMETRIC_POTENTIAL,
                                  nb.NBODY_PASS_SYMMETRIC_CHUNKED])
def test_time_accel_runs_the_pass(kind):
    pm_np, _ = workloads.uniform_cube(N, seed=910 + kind, masses="lognormal")
    pm = torch.from_numpy(pm_np).to(DEV)
    ws = workspace(kind)
    ref = plain_pass(kind, pm, ws)
    out = torch.full_like(pm, float("nan"))
    reps = 4
    pass_ms, kernel_ms = nb.nbody_time_accel(pm, G, EPS2, out, kind, reps, workspace=ws)
    assert np.array_equal(out.cpu().numpy(), ref)
    assert len(pass_ms) == reps and len(kernel_ms) == reps
    for p, k in zip(pass_ms, kernel_ms):
        assert np.isfinite(p) and np.isfinite(k) and p > 0 and k > 0
        # the kernel is part of the pass (the one-sided pass is one kernel)
        assert k <= p * (1 + 1e-3) + 1e-3, (p, k)


def test_time_accel_on_a_side_stream():
    """Timed on another stream, the result is there once that stream is done."""
    pm_np, _ = workloads.plummer(N, seed=920)
    pm = torch.from_numpy(pm_np).to(DEV)
    ws = workspace(nb.NBODY_PASS_SYMMETRIC)
    ref = plain_pass(nb.NBODY_PASS_SYMMETRIC, pm, ws)
    s = torch.cuda.Stream()
    out = torch.full_like(pm, float("nan"))
    torch.cuda.synchronize()
    pass_ms, _ = nb.nbody_time_accel(pm, G, EPS2, out, nb.NBODY_PASS_SYMMETRIC, 2,
                                     workspace=ws, stream=s)
    s.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    assert all(p > 0 for p in pass_ms)


def test_timer_brackets_work_on_its_stream():
    pm_np, _ = workloads.plummer(N, seed=930)
    pm = torch.from_numpy(pm_np).to(DEV)
    out = torch.empty_like(pm)
    s = torch.cuda.Stream()
    t = nb.Timer(4)
    try:
        with torch.cuda.stream(s):
            t.mark(0, s)
            nb.nbody_accel(pm, G, EPS2, out, stream=s)
            t.mark(1, s)
            nb.nbody_accel(pm, G, EPS2, out, stream=s)
            nb.nbody_accel(pm, G, EPS2, out, stream=s)
            t.mark(2, s)
        one = t.elapsed_ms(0, 1)
        two = t.elapsed_ms(1, 2)
        assert one > 0 and two > 0
        assert abs(t.elapsed_ms(0, 2) - (one + two)) <= 1e-2 * (one + two) + 1e-3
        assert t.elapsed_ms(1, 1) == 0.0
        # a mark that was never recorded cannot be read; the failure is
        # reported once, by the status, and not left behind for the caller's
        # next HIP call
        with pytest.raises(nb.NBodyError):
            t.elapsed_ms(0, 3)
        after = torch.full((4,), 2.0, device=DEV)
        torch.cuda.synchronize()
        assert after.sum().item() == 8.0
    finally:
        t.close()


def test_binding_rejects_wrong_dtype_layout_and_rows():
    """Device tensors of the wrong dtype, a non-contiguous view, a wrong row
    width or row count are refused by the binding with a clear error, and
    the output is left untouched."""
    pm = torch.zeros((64, 4), dtype=torch.float32, device=DEV)
    out = torch.full((64, 4), 5.0, dtype=torch.float32, device=DEV)
    with pytest.raises(TypeError, match="float32"):
        nb.nbody_accel(pm.double(), G, EPS2, out)
    with pytest.raises(ValueError, match="contiguous"):
        nb.nbody_accel(torch.zeros((64, 8), device=DEV)[:, ::2], G, EPS2, out)
    with pytest.raises(ValueError, match="shape"):
        nb.nbody_accel(torch.zeros((64, 3), device=DEV), G, EPS2, out)
    with pytest.raises(ValueError, match="rows"):
        nb.nbody_accel(pm, G, EPS2, out[:32])
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)
