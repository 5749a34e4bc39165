"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, compare against the oracle, report the error metrics.

Tolerances (fp32 accelerations against the float64 oracle on identical
float32 inputs): relative L2 over all 3N components <= 1e-5, and for every
body |a_gpu - a_ref| / |a_ref| <= 1e-3.
"""
import sys

import numpy as np

L2_TOL = 1e-5
BODY_TOL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(a_gpu, a_ref):
    """(relative L2 over all components, max per-body relative error)."""
    g = np.asarray(a_gpu, dtype=np.float64)[:, :3]
    r = np.asarray(a_ref, dtype=np.float64)[:, :3]
    diff = np.linalg.norm(g - r, axis=1)
    ref = np.linalg.norm(r, axis=1)
    denom = np.linalg.norm(r)
    l2 = float(np.linalg.norm(g - r) / denom) if denom > 0 else float(np.linalg.norm(g - r))
    with np.errstate(divide="ignore", invalid="ignore"):
        per = np.where(ref > 0, diff / ref, np.where(diff == 0, 0.0, np.inf))
    return l2, float(per.max()) if per.size else 0.0


def assert_parity(a_gpu, a_ref, what=""):
    l2, worst = errors(a_gpu, a_ref)
    log(f"  parity {what}: rel L2 {l2:.3e}, worst body {worst:.3e}")
    assert l2 <= L2_TOL, f"{what}: relative L2 {l2:.3e} > {L2_TOL}"
    assert worst <= BODY_TOL, f"{what}: per-body relative error {worst:.3e} > {BODY_TOL}"
    return l2, worst


def sample_rows(n, count, seed=0):
    """Sorted distinct rows: the first and last 64 bodies (ragged tail,
    tile edges) plus a seeded uniform sample."""
    g = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(min(64, n)), np.arange(max(0, n - 64), n)])
    rest = g.choice(n, size=min(n, count), replace=False)
    return np.unique(np.concatenate([edge, rest])).astype(np.int64)
