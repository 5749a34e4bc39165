"""Parity over every body at the three large workloads: the lognormal-mass
cube of 131072 bodies, the 2^20-body Plummer sphere and the 1,000,003-body
collision of two Plummer spheres.

Each force pass the library offers at these sizes runs once on the GPU
(through the C ABI, in the variant the library picks for n and in the launch
configuration bench.py times), and every row is compared with the
double-precision oracle on the same float32 inputs: relative L2 over all 3N
components <= 1e-5 and, for every body, |a_gpu - a_ref| / |a_ref| <= 1e-3,
with no floor ("CUDA N-Body Simulation" README, section 5.2, compares every
body of the device run with its host reference the same way).

The oracle's full pass costs N^2 double-precision interactions (about 170 s
at 2^20 on 16 host threads), so at the two 10^6-body workloads it is taken in
row chunks of 65536 bodies, one test per chunk; the last test of each
workload adds the chunks' squared sums into the all-bodies L2, reports the
oracle's full-pass time and rate, and logs the ten worst bodies of each pass
with their radius and |a_ref| (the Plummer centre, where |a_ref| is smallest,
is where a relative error would show first).
"""
import time

import numpy as np
import pytest
import torch

import direct_all_pairs_softened_amd as nb
import oracle
import workloads
from parity import BODY_TOL, L2_TOL, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = np.float32
CHUNK = 65536
WORST_KEPT = 10


class FullParity:
    """GPU results of every pass on one workload, and the running error sums
    of each pass against the oracle rows checked so far."""

    def __init__(self, name, passes):
        self.name = name
        self.w = workloads.WORKLOADS[name]
        self.pm, _ = workloads.make(name)
        self.pos, self.mass = oracle.split_posmass(self.pm)
        self.G = float(F32(self.w.G))
        self.eps2 = float(F32(self.w.eps2))
        self.gpu = passes
        self.num = {k: 0.0 for k in passes}      # sum |a_gpu - a_ref|^2
        self.den = 0.0                           # sum |a_ref|^2
        self.worst = {k: [] for k in passes}     # (rel err, row), best kept
        self.done = set()
        self.oracle_s = 0.0

    def rows(self, k):
        return np.arange(k * CHUNK, min(self.w.n, (k + 1) * CHUNK), dtype=np.int64)

    def check_chunk(self, k):
        if k in self.done:
            return
        rows = self.rows(k)
        t0 = time.perf_counter()
        ref = oracle.accel_rows(self.pos, self.mass, self.G, self.eps2, rows)
        self.oracle_s += time.perf_counter() - t0
        rn = np.linalg.norm(ref, axis=1)
        self.den += float((ref * ref).sum())
        for key, a in self.gpu.items():
            got = a[rows, :3].astype(np.float64)
            d = np.linalg.norm(got - ref, axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                rel = np.where(rn > 0, d / rn, np.where(d == 0, 0.0, np.inf))
            self.num[key] += float((d * d).sum())
            top = np.argsort(rel)[-WORST_KEPT:]
            self.worst[key] = sorted(self.worst[key] + [(float(rel[t]), int(rows[t]))
                                                        for t in top])[-WORST_KEPT:]
            chunk_l2 = float(np.sqrt((d * d).sum() / (ref * ref).sum()))
            log(f"  {self.name} rows {rows[0]}..{rows[-1]} {key}: rel L2 {chunk_l2:.2e}, "
                f"worst body {rel.max():.2e}")
            assert rel.max() <= BODY_TOL, (
                f"{self.name} {key}: body {int(rows[np.argmax(rel)])} relative error "
                f"{rel.max():.3e} > {BODY_TOL}")
        self.done.add(k)

    def finish(self):
        chunks = -(-self.w.n // CHUNK)
        for k in range(chunks):
            self.check_chunk(k)
        inter = float(self.w.n) * float(self.w.n)
        log(f"{self.name}: oracle full pass {self.oracle_s:.1f} s in {chunks} row chunks, "
            f"{inter / self.oracle_s / 1e9:.2f} x 10^9 interactions/s on "
            f"{oracle.num_threads()} threads")
        r = np.linalg.norm(self.pos, axis=1)
        for key in self.gpu:
            l2 = float(np.sqrt(self.num[key] / self.den))
            log(f"{self.name} {key}: all {self.w.n} bodies, rel L2 {l2:.3e}; worst bodies:")
            for rel, i in reversed(self.worst[key]):
                ai = self.gpu[key][i, :3].astype(np.float64)
                ref = oracle.accel_rows(self.pos, self.mass, self.G, self.eps2,
                                        np.array([i], np.int64))[0]
                log(f"    body {i:8d}  r {r[i]:10.4g}  |a_ref| {np.linalg.norm(ref):10.4g}  "
                    f"rel err {rel:.3e}  (|a_gpu| {np.linalg.norm(ai):.6g})")
            assert l2 <= L2_TOL, f"{self.name} {key}: relative L2 {l2:.3e} > {L2_TOL}"


def run(fn, n):
    out = torch.full((n, 4), float("nan"), device=DEV)
    fn(out)
    torch.cuda.synchronize()
    a = out.cpu().numpy()
    assert np.all(a[:, 3] == 0.0)
    return a


def one_sided(pm, w):
    return lambda out: nb.nbody_accel(pm, w.G, w.eps2, out)


def symmetric(pm, w):
    ws = torch.empty(nb.nbody_accel_symmetric_workspace_bytes(w.n), dtype=torch.uint8,
                     device=DEV)
    return lambda out: nb.nbody_accel_symmetric(pm, w.G, w.eps2, out, ws)


def symmetric_two_phases(pm, w):
    """The pass as bench.py launches it: the panel-pair kernel, then the reduce."""
    ws = torch.empty(nb.nbody_accel_symmetric_workspace_bytes(w.n), dtype=torch.uint8,
                     device=DEV)

    def fn(out):
        nb.nbody_accel_symmetric_tasks(pm, w.eps2, ws)
        nb.nbody_accel_symmetric_reduce(w.n, w.G, out, ws)
    return fn


def gpu_passes(name):
    w = workloads.WORKLOADS[name]
    pm_np, _ = workloads.make(name)
    pm = torch.from_numpy(pm_np).to(DEV)
    log(f"{name}: GPU passes (one-sided variant {nb.nbody_accel_variant_for_n(w.n)}, "
        f"pair-symmetric variant {nb.nbody_accel_symmetric_variant_for_n(w.n)})")
    out = {"one_sided": run(one_sided(pm, w), w.n),
           "symmetric": run(symmetric(pm, w), w.n)}
    two = run(symmetric_two_phases(pm, w), w.n)
    assert np.array_equal(two, out["symmetric"])
    return w, pm, out


# ---------------------------------------------------------------------------
# 131072 bodies, lognormal masses: the 1D pass against the 2D decompositions
# ---------------------------------------------------------------------------

def test_lognormal128k_every_body_every_decomposition():
    """Every row of every pass of the 1D-versus-2D comparison at 131072
    bodies: the one-sided and pair-symmetric passes, the split-j two-pass
    decomposition at four chunk widths, and the README's 32-wide tree first
    pass as a plain tree, FADL and fadl4, against one full oracle pass."""
    w, pm, out = gpu_passes("lognormal128k")
    for j_chunk in (32, 256, 1024, 4096):
        ws = torch.empty(nb.nbody_accel_splitj_workspace_bytes(w.n, j_chunk),
                         dtype=torch.uint8, device=DEV)
        out[f"splitj_J{j_chunk}"] = run(
            lambda o: nb.nbody_accel_splitj(pm, w.G, w.eps2, o, j_chunk, ws), w.n)
        del ws
    ws = torch.empty(nb.nbody_accel_splitj_tree_workspace_bytes(w.n, 32, 1), dtype=torch.uint8,
                     device=DEV)
    for terms in (1, 2, 4):
        out[f"splitj_tree_J32_F{terms}"] = run(
            lambda o: nb.nbody_accel_splitj_tree(pm, w.G, w.eps2, o, 32, terms, ws), w.n)
    del ws
    fp = FullParity("lognormal128k", out)
    fp.finish()


# ---------------------------------------------------------------------------
# 2^20 bodies (the headline) and 1,000,003 bodies (ragged), in row chunks
# ---------------------------------------------------------------------------

_STATE = {}


def state(name):
    if name not in _STATE:
        w, pm, out = gpu_passes(name)
        if name == "plummer1m":
            # the checkpoint pass: its xyz are the plain pass's, bit for bit
            pv = nb.nbody_accel_symmetric_potential_variant_for_n(w.n)
            ws = torch.empty(nb.nbody_accel_symmetric_potential_workspace_bytes(w.n, pv),
                             dtype=torch.uint8, device=DEV)
            pot = torch.empty_like(pm)
            nb.nbody_accel_symmetric_potential(pm, w.G, w.eps2, pot, ws, pv)
            torch.cuda.synchronize()
            assert np.array_equal(pot.cpu().numpy()[:, :3], out["symmetric"][:, :3])
            del ws, pot
            # one GPU's eighth of the i side: rows equal to a full pass of the
            # same variant, and checked against the oracle below as part of it
            ni = w.n // 8
            share = torch.empty((ni, 4), device=DEV)
            v = nb.nbody_accel_variant_for_n(ni)
            nb.nbody_accel_range(pm, 5 * ni, ni, w.G, w.eps2, share, v)
            full = torch.empty_like(pm)
            nb.nbody_accel_variant(pm, w.G, w.eps2, full, v)
            torch.cuda.synchronize()
            assert np.array_equal(share.cpu().numpy(), full.cpu().numpy()[5 * ni:6 * ni])
            out[f"one_sided_v{v}"] = full.cpu().numpy()
            del share, full
        del pm
        torch.cuda.empty_cache()
        _STATE[name] = FullParity(name, out)
    return _STATE[name]


CHUNKS_1M = range(-(-workloads.WORKLOADS["plummer1m"].n // CHUNK))
CHUNKS_COLL = range(-(-workloads.WORKLOADS["collision1m"].n // CHUNK))


@pytest.mark.parametrize("k", CHUNKS_1M)
def test_plummer1m_every_body_chunk(k):
    state("plummer1m").check_chunk(k)


def test_plummer1m_every_body_l2_and_worst_bodies():
    state("plummer1m").finish()


@pytest.mark.parametrize("k", CHUNKS_COLL)
def test_collision1m_every_body_chunk(k):
    state("collision1m").check_chunk(k)


def test_collision1m_every_body_l2_and_worst_bodies():
    state("collision1m").finish()
