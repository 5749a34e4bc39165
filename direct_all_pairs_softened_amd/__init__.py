"""Direct all-pairs softened gravity on AMD MI355X (gfx950).

A thin ctypes binding over ``libnbody.so`` (C ABI in ``include/nbody.h``).
Each function here has the name and arguments of its C entry point and only
marshals arguments: it checks that tensors are CUDA (HIP) float32/float64
tensors of the right shape and contiguity, passes ``data_ptr()`` and the
current stream, and raises ``NBodyError`` on a non-zero status.  Every step of
the computation runs in the library's HIP kernels; there is no CPU fallback.
If the library is missing, ``load_library`` raises -- build it with
``python -m direct_all_pairs_softened_amd.build`` (or ``__graft_entry__.build()``).

Calls are asynchronous on the stream, like the C functions: read results
after ``torch.cuda.synchronize()`` or through stream-ordered torch ops.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnbody.so")

NBODY_OK = 0
NBODY_ERR_INVALID_ARG = -1
NBODY_ERR_ALIGNMENT = -2
NBODY_ERR_ALIAS = -3
NBODY_ERR_WORKSPACE = -4
NBODY_ERR_HIP = -5
NBODY_MAX_N = 1 << 30
NBODY_ENERGY_STATIC_SCRATCH_BYTES = 16 << 20

# Every symbol include/nbody.h declares.
EXPORTS = (
    "nbody_status_string", "nbody_abi_version",
    "nbody_accel", "nbody_accel_variant", "nbody_accel_variant_count",
    "nbody_accel_variant_info", "nbody_accel_variant_for_n",
    "nbody_accel_range", "nbody_accel_potential",
    "nbody_energy_from_potential", "nbody_energy_from_potential_workspace_bytes",
    "nbody_accel_splitj", "nbody_accel_splitj_workspace_bytes",
    "nbody_accel_splitj_tree", "nbody_accel_splitj_tree_workspace_bytes",
    "nbody_accel_symmetric", "nbody_accel_symmetric_workspace_bytes",
    "nbody_accel_symmetric_variant_count", "nbody_accel_symmetric_panel",
    "nbody_accel_symmetric_variant_for_n",
    "nbody_accel_symmetric_tasks", "nbody_accel_symmetric_reduce",
    "nbody_accel_symmetric_chunked", "nbody_accel_symmetric_chunked_workspace_bytes",
    "nbody_accel_symmetric_potential", "nbody_accel_symmetric_potential_workspace_bytes",
    "nbody_accel_symmetric_potential_variant_count", "nbody_accel_symmetric_potential_panel",
    "nbody_accel_symmetric_potential_variant_for_n",
    "nbody_accel_f3aos", "nbody_accel_soa",
    "nbody_leapfrog_step", "nbody_kick", "nbody_kdk_run",
    "nbody_energy", "nbody_energy_workspace_bytes", "nbody_energy_static",
    "nbody_timer_create", "nbody_timer_mark", "nbody_timer_elapsed_ms", "nbody_timer_destroy",
    "nbody_time_accel", "nbody_set_launch_block_cap",
)

# Force passes of nbody_time_accel.
NBODY_PASS_ONE_SIDED = 0
NBODY_PASS_SYMMETRIC = 1
NBODY_PASS_SYMMETRIC_POTENTIAL = 2
NBODY_PASS_SYMMETRIC_CHUNKED = 3

ENERGY_FIELDS = ("K", "W", "E", "Px", "Py", "Pz", "M")


class NBodyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load_library(path: str | None = None):
    """Loads libnbody.so (once) and declares every entry point's signature."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is not built; run __graft_entry__.build() or "
            "python -m direct_all_pairs_softened_amd.build")
    lib = ctypes.CDLL(p)
    c_int, c_i64, c_f, c_sz, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_size_t, ctypes.c_void_p)
    pint = ctypes.POINTER(ctypes.c_int)
    sig = {
        "nbody_status_string": (ctypes.c_char_p, [c_int]),
        "nbody_abi_version": (c_int, []),
        "nbody_accel": (c_int, [vp, c_i64, c_f, c_f, vp, vp]),
        "nbody_accel_variant": (c_int, [vp, c_i64, c_f, c_f, vp, c_int, vp]),
        "nbody_accel_variant_count": (c_int, []),
        "nbody_accel_variant_info": (c_int, [c_int, pint, pint, pint, pint, pint, pint, pint]),
        "nbody_accel_variant_for_n": (c_int, [c_i64]),
        "nbody_accel_potential": (c_int, [vp, c_i64, c_f, c_f, vp, vp]),
        "nbody_energy_from_potential": (c_int, [vp, vp, vp, c_i64, vp, c_sz, vp, vp]),
        "nbody_energy_from_potential_workspace_bytes": (c_sz, [c_i64]),
        "nbody_accel_range": (c_int, [vp, c_i64, c_i64, c_i64, c_f, c_f, vp, c_int, vp]),
        "nbody_accel_splitj": (c_int, [vp, c_i64, c_f, c_f, vp, c_i64, vp, c_sz, vp]),
        "nbody_accel_splitj_workspace_bytes": (c_sz, [c_i64, c_i64]),
        "nbody_accel_splitj_tree": (c_int, [vp, c_i64, c_f, c_f, vp, c_i64, c_int, vp, c_sz,
                                            vp]),
        "nbody_accel_splitj_tree_workspace_bytes": (c_sz, [c_i64, c_i64, c_int]),
        "nbody_accel_symmetric": (c_int, [vp, c_i64, c_f, c_f, vp, c_int, vp, c_sz, vp]),
        "nbody_accel_symmetric_workspace_bytes": (c_sz, [c_i64, c_int]),
        "nbody_accel_symmetric_variant_count": (c_int, []),
        "nbody_accel_symmetric_panel": (c_int, [c_int]),
        "nbody_accel_symmetric_variant_for_n": (c_int, [c_i64]),
        "nbody_accel_symmetric_tasks": (c_int, [vp, c_i64, c_f, c_int, vp, c_sz, vp]),
        "nbody_accel_symmetric_chunked": (c_int, [vp, c_i64, c_f, c_f, vp, c_int, c_int, vp,
                                                  c_sz, vp]),
        "nbody_accel_symmetric_chunked_workspace_bytes": (c_sz, [c_i64, c_int, c_int]),
        "nbody_accel_symmetric_reduce": (c_int, [c_i64, c_f, vp, c_int, vp, c_sz, vp]),
        "nbody_accel_symmetric_potential": (c_int, [vp, c_i64, c_f, c_f, vp, c_int, vp, c_sz,
                                                    vp]),
        "nbody_accel_symmetric_potential_workspace_bytes": (c_sz, [c_i64, c_int]),
        "nbody_accel_symmetric_potential_variant_count": (c_int, []),
        "nbody_accel_symmetric_potential_panel": (c_int, [c_int]),
        "nbody_accel_symmetric_potential_variant_for_n": (c_int, [c_i64]),
        "nbody_accel_f3aos": (c_int, [vp, vp, c_i64, c_f, c_f, vp, vp]),
        "nbody_accel_soa": (c_int, [vp, vp, vp, vp, c_i64, c_f, c_f, vp, vp, vp, vp]),
        "nbody_leapfrog_step": (c_int, [vp, vp, vp, c_f, c_i64, vp]),
        "nbody_kick": (c_int, [vp, vp, c_f, c_i64, vp]),
        "nbody_kdk_run": (c_int, [vp, vp, vp, c_i64, c_f, c_f, c_f, c_int, c_int, c_int, vp,
                                  c_sz, vp]),
        "nbody_energy": (c_int, [vp, vp, c_i64, c_f, c_f, vp, c_sz, vp, vp]),
        "nbody_energy_workspace_bytes": (c_sz, [c_i64]),
        "nbody_energy_static": (c_int, [vp, vp, c_i64, c_f, c_f, vp, vp]),
        "nbody_timer_create": (c_int, [c_int, ctypes.POINTER(vp)]),
        "nbody_timer_mark": (c_int, [vp, c_int, vp]),
        "nbody_timer_elapsed_ms": (c_int, [vp, c_int, c_int, ctypes.POINTER(c_f)]),
        "nbody_timer_destroy": (c_int, [vp]),
        "nbody_time_accel": (c_int, [vp, c_i64, c_f, c_f, vp, c_int, c_int, vp, c_sz, c_int,
                                     ctypes.POINTER(c_f), ctypes.POINTER(c_f), vp]),
        "nbody_set_launch_block_cap": (c_int, [c_i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nbody_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != NBODY_OK:
        raise NBodyError(status, where)


# ---------------------------------------------------------------------------
# argument marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, shape_tail=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape_tail is not None and tuple(t.shape[1:]) != tuple(shape_tail):
        raise ValueError(f"{name} must have shape [N, {', '.join(map(str, shape_tail))}]")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t, name, tail):
    return _dev(t, name, tail, _torch().float32)


def _n_of(t) -> int:
    return int(t.shape[0])


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def nbody_accel(posmass, G: float, eps2: float, accel_out, stream=None):
    """accel_out[i] = (a_i, 0) for float32 [N, 4] posmass."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    _check(load_library().nbody_accel(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                      _f32(accel_out, "accel_out", (4,)), _stream(stream)),
           "nbody_accel")


def nbody_accel_variant(posmass, G: float, eps2: float, accel_out, variant: int, stream=None):
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    _check(load_library().nbody_accel_variant(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                              _f32(accel_out, "accel_out", (4,)), int(variant),
                                              _stream(stream)),
           "nbody_accel_variant")


def nbody_accel_variant_count() -> int:
    return int(load_library().nbody_accel_variant_count())


def nbody_accel_variant_info(v: int) -> dict:
    vals = [ctypes.c_int() for _ in range(7)]
    _check(load_library().nbody_accel_variant_info(int(v), *[ctypes.byref(x) for x in vals]),
           "nbody_accel_variant_info")
    keys = ("bodies_per_lane", "tile", "waves_per_block", "split", "staging", "unroll",
            "lane_groups")
    return {k: x.value for k, x in zip(keys, vals)}


def nbody_accel_variant_for_n(n: int) -> int:
    return int(load_library().nbody_accel_variant_for_n(int(n)))


def nbody_accel_potential(posmass, G: float, eps2: float, accel_out, stream=None):
    """accel_out[i] = (a_i, Phi_i) with Phi_i the softened potential at body i."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    _check(load_library().nbody_accel_potential(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                                _f32(accel_out, "accel_out", (4,)),
                                                _stream(stream)),
           "nbody_accel_potential")


def nbody_energy_from_potential_workspace_bytes(n: int) -> int:
    return int(load_library().nbody_energy_from_potential_workspace_bytes(int(n)))


def nbody_energy_from_potential(posmass, vel, accel_pot, workspace, stats_out, stream=None):
    torch = _torch()
    n = _n_of(posmass)
    if _n_of(vel) != n or _n_of(accel_pot) != n:
        raise ValueError("posmass, vel and accel_pot must have N rows")
    if stats_out.numel() < 8:
        raise ValueError("stats_out needs 8 doubles")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_energy_from_potential(
        _f32(posmass, "posmass", (4,)), _f32(vel, "vel", (4,)), _f32(accel_pot, "accel_pot", (4,)),
        n, ws, nbytes, _dev(stats_out, "stats_out", None, torch.float64), _stream(stream)),
        "nbody_energy_from_potential")


def nbody_accel_range(posmass, i0: int, ni: int, G: float, eps2: float, accel_out,
                      variant: int = -1, stream=None):
    """accel_out[r] = (a_{i0+r}, 0) for r < ni, summed over all N bodies."""
    n = _n_of(posmass)
    if _n_of(accel_out) != ni:
        raise ValueError("accel_out must have ni rows")
    _check(load_library().nbody_accel_range(_f32(posmass, "posmass", (4,)), n, int(i0), int(ni),
                                            G, eps2, _f32(accel_out, "accel_out", (4,)),
                                            int(variant), _stream(stream)),
           "nbody_accel_range")


def nbody_accel_splitj_workspace_bytes(n: int, j_chunk: int) -> int:
    return int(load_library().nbody_accel_splitj_workspace_bytes(int(n), int(j_chunk)))


def nbody_accel_splitj(posmass, G: float, eps2: float, accel_out, j_chunk: int, workspace,
                       stream=None):
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_splitj(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                             _f32(accel_out, "accel_out", (4,)), int(j_chunk),
                                             ws, nbytes, _stream(stream)),
           "nbody_accel_splitj")


def nbody_accel_splitj_tree_workspace_bytes(n: int, j_chunk: int, terms: int) -> int:
    return int(load_library().nbody_accel_splitj_tree_workspace_bytes(int(n), int(j_chunk),
                                                                      int(terms)))


def nbody_accel_splitj_tree(posmass, G: float, eps2: float, accel_out, j_chunk: int, terms: int,
                            workspace, stream=None):
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_splitj_tree(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                                  _f32(accel_out, "accel_out", (4,)),
                                                  int(j_chunk), int(terms), ws, nbytes,
                                                  _stream(stream)),
           "nbody_accel_splitj_tree")


def nbody_accel_symmetric_workspace_bytes(n: int, variant: int = -1) -> int:
    return int(load_library().nbody_accel_symmetric_workspace_bytes(int(n), int(variant)))


def nbody_accel_symmetric_variant_count() -> int:
    return int(load_library().nbody_accel_symmetric_variant_count())


def nbody_accel_symmetric_panel(variant: int) -> int:
    return int(load_library().nbody_accel_symmetric_panel(int(variant)))


def nbody_accel_symmetric_variant_for_n(n: int) -> int:
    return int(load_library().nbody_accel_symmetric_variant_for_n(int(n)))


def nbody_accel_symmetric(posmass, G: float, eps2: float, accel_out, workspace,
                          variant: int = -1, stream=None):
    """Pair-symmetric force pass; workspace: a GPU tensor of at least
    nbody_accel_symmetric_workspace_bytes(N, variant) bytes."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_symmetric(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                                _f32(accel_out, "accel_out", (4,)),
                                                int(variant), ws, nbytes, _stream(stream)),
           "nbody_accel_symmetric")


def nbody_accel_symmetric_chunked_workspace_bytes(n: int, variant: int = -1,
                                                  chunk_panels: int = 0) -> int:
    return int(load_library().nbody_accel_symmetric_chunked_workspace_bytes(
        int(n), int(variant), int(chunk_panels)))


def nbody_accel_symmetric_chunked(posmass, G: float, eps2: float, accel_out, workspace,
                                  variant: int = -1, chunk_panels: int = 0, stream=None):
    """Pair-symmetric force pass in column chunks (bitwise equal to
    nbody_accel_symmetric); workspace: a GPU tensor of at least
    nbody_accel_symmetric_chunked_workspace_bytes(N, variant, chunk_panels) bytes."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_symmetric_chunked(
        _f32(posmass, "posmass", (4,)), n, G, eps2, _f32(accel_out, "accel_out", (4,)),
        int(variant), int(chunk_panels), ws, nbytes, _stream(stream)),
        "nbody_accel_symmetric_chunked")


def nbody_accel_symmetric_tasks(posmass, eps2: float, workspace, variant: int = -1, stream=None):
    """First phase of nbody_accel_symmetric: the panel-pair kernel (posmass ->
    the panel sums in workspace)."""
    n = _n_of(posmass)
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_symmetric_tasks(_f32(posmass, "posmass", (4,)), n, eps2,
                                                      int(variant), ws, nbytes, _stream(stream)),
           "nbody_accel_symmetric_tasks")


def nbody_accel_symmetric_reduce(n: int, G: float, accel_out, workspace, variant: int = -1,
                                 stream=None):
    """Second phase of nbody_accel_symmetric: the panel sums in workspace ->
    accel_out (the same n, variant and workspace as the tasks call)."""
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have n rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_symmetric_reduce(int(n), G,
                                                       _f32(accel_out, "accel_out", (4,)),
                                                       int(variant), ws, nbytes, _stream(stream)),
           "nbody_accel_symmetric_reduce")


def nbody_accel_symmetric_potential_workspace_bytes(n: int, variant: int = -1) -> int:
    return int(load_library().nbody_accel_symmetric_potential_workspace_bytes(int(n),
                                                                              int(variant)))


def nbody_accel_symmetric_potential_variant_count() -> int:
    return int(load_library().nbody_accel_symmetric_potential_variant_count())


def nbody_accel_symmetric_potential_panel(variant: int) -> int:
    return int(load_library().nbody_accel_symmetric_potential_panel(int(variant)))


def nbody_accel_symmetric_potential_variant_for_n(n: int) -> int:
    return int(load_library().nbody_accel_symmetric_potential_variant_for_n(int(n)))


def nbody_accel_symmetric_potential(posmass, G: float, eps2: float, accel_out, workspace,
                                    variant: int = -1, stream=None):
    """Pair-symmetric force pass with Phi_i in accel_out[:, 3]; workspace: a GPU
    tensor of at least nbody_accel_symmetric_potential_workspace_bytes(N, variant)
    bytes."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_accel_symmetric_potential(
        _f32(posmass, "posmass", (4,)), n, G, eps2, _f32(accel_out, "accel_out", (4,)),
        int(variant), ws, nbytes, _stream(stream)), "nbody_accel_symmetric_potential")


def nbody_accel_f3aos(pos, mass, G: float, eps2: float, accel_out, stream=None):
    """pos float32 [N, 3], mass float32 [N], accel_out float32 [N, 3]."""
    n = _n_of(pos)
    if _n_of(mass) != n or _n_of(accel_out) != n or mass.dim() != 1:
        raise ValueError("pos, mass, accel_out must have N rows; mass must be 1-D")
    _check(load_library().nbody_accel_f3aos(_f32(pos, "pos", (3,)), _f32(mass, "mass", ()),
                                            n, G, eps2, _f32(accel_out, "accel_out", (3,)),
                                            _stream(stream)),
           "nbody_accel_f3aos")


def nbody_accel_soa(x, y, z, m, G: float, eps2: float, ax, ay, az, stream=None):
    """Every array float32 [N]."""
    arrs = dict(x=x, y=y, z=z, m=m, ax=ax, ay=ay, az=az)
    n = _n_of(x)
    for k, t in arrs.items():
        if t.dim() != 1 or _n_of(t) != n:
            raise ValueError(f"{k} must be a 1-D array of N floats")
    p = {k: _f32(t, k, ()) for k, t in arrs.items()}
    _check(load_library().nbody_accel_soa(p["x"], p["y"], p["z"], p["m"], n, G, eps2,
                                          p["ax"], p["ay"], p["az"], _stream(stream)),
           "nbody_accel_soa")


def nbody_leapfrog_step(posmass, vel, accel, dt: float, stream=None):
    """In place: v += dt/2 a; x += dt v (float32 [N, 4] each)."""
    n = _n_of(posmass)
    if _n_of(vel) != n or _n_of(accel) != n:
        raise ValueError("posmass, vel, accel must have N rows")
    _check(load_library().nbody_leapfrog_step(_f32(posmass, "posmass", (4,)),
                                              _f32(vel, "vel", (4,)), _f32(accel, "accel", (4,)),
                                              dt, n, _stream(stream)),
           "nbody_leapfrog_step")


def nbody_kick(vel, accel, h: float, stream=None):
    """In place: v += h a (float32 [N, 4] each)."""
    n = _n_of(vel)
    if _n_of(accel) != n:
        raise ValueError("vel and accel must have N rows")
    _check(load_library().nbody_kick(_f32(vel, "vel", (4,)), _f32(accel, "accel", (4,)), h, n,
                                      _stream(stream)),
           "nbody_kick")


def nbody_kdk_run(posmass, vel, accel, G: float, eps2: float, dt: float, steps: int,
                  pass_kind: int = 0, variant: int = -1, workspace=None, stream=None):
    """``steps`` kick-drift-kick steps run by the library (bitwise the same as
    nbody_leapfrog_step, the force pass and nbody_kick called step by step).
    accel holds a(x) on entry and a(x_final) on return; pass_kind is one of
    NBODY_PASS_*."""
    n = _n_of(posmass)
    if _n_of(vel) != n or _n_of(accel) != n:
        raise ValueError("posmass, vel and accel must have N rows")
    if workspace is None:
        ws, nbytes = ctypes.c_void_p(), 0
    else:
        ws = _dev(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_kdk_run(_f32(posmass, "posmass", (4,)), _f32(vel, "vel", (4,)),
                                        _f32(accel, "accel", (4,)), n, G, eps2, dt, int(steps),
                                        int(pass_kind), int(variant), ws, nbytes,
                                        _stream(stream)),
           "nbody_kdk_run")


def nbody_energy_workspace_bytes(n: int) -> int:
    return int(load_library().nbody_energy_workspace_bytes(int(n)))


def nbody_energy(posmass, vel, G: float, eps2: float, workspace, stats_out, stream=None):
    """stats_out: float64 [8] GPU tensor <- {K, W, E, Px, Py, Pz, M, 0}."""
    torch = _torch()
    n = _n_of(posmass)
    if _n_of(vel) != n:
        raise ValueError("posmass and vel must have N rows")
    if stats_out.numel() < 8:
        raise ValueError("stats_out needs 8 doubles")
    ws = _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().nbody_energy(_f32(posmass, "posmass", (4,)), _f32(vel, "vel", (4,)),
                                       n, G, eps2, ws, nbytes,
                                       _dev(stats_out, "stats_out", None, torch.float64),
                                       _stream(stream)),
           "nbody_energy")


class Timer:
    """nbody_timer: ``marks`` HIP events owned by the library, recorded on the
    stream the timed work runs on (``mark``), read back with ``elapsed_ms``
    (which waits for the later event)."""

    def __init__(self, marks: int):
        self._t = ctypes.c_void_p()
        _check(load_library().nbody_timer_create(int(marks), ctypes.byref(self._t)),
               "nbody_timer_create")
        self.marks = int(marks)

    def mark(self, i: int, stream=None):
        _check(load_library().nbody_timer_mark(self._t, int(i), _stream(stream)),
               "nbody_timer_mark")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        _check(load_library().nbody_timer_elapsed_ms(self._t, int(a), int(b), ctypes.byref(ms)),
               "nbody_timer_elapsed_ms")
        return float(ms.value)

    def close(self):
        if self._t:
            load_library().nbody_timer_destroy(self._t)
            self._t = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def nbody_time_accel(posmass, G: float, eps2: float, accel_out, pass_kind: int, reps: int,
                     variant: int = -1, workspace=None, stream=None):
    """Runs ``reps`` force passes timed with the library's HIP events (waits
    for them).  Returns (pass_ms, kernel_ms), two lists of ``reps`` floats."""
    n = _n_of(posmass)
    if _n_of(accel_out) != n:
        raise ValueError("accel_out must have N rows")
    if workspace is None:
        ws, nbytes = ctypes.c_void_p(), 0
    else:
        ws = _dev(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    pass_ms = (ctypes.c_float * max(int(reps), 1))()
    kernel_ms = (ctypes.c_float * max(int(reps), 1))()
    _check(load_library().nbody_time_accel(_f32(posmass, "posmass", (4,)), n, G, eps2,
                                           _f32(accel_out, "accel_out", (4,)), int(pass_kind),
                                           int(variant), ws, nbytes, int(reps), pass_ms,
                                           kernel_ms, _stream(stream)),
           "nbody_time_accel")
    return list(pass_ms)[:reps], list(kernel_ms)[:reps]


def nbody_set_launch_block_cap(max_blocks: int) -> None:
    """Caps the blocks per kernel launch for every later call in the process
    (0 restores HIP's limit), so that small inputs take the split-launch path:
    a testing aid."""
    _check(load_library().nbody_set_launch_block_cap(int(max_blocks)),
           "nbody_set_launch_block_cap")


def nbody_energy_static(posmass, vel, G: float, eps2: float, stats_out, stream=None):
    """nbody_energy with the library's static device scratch (no workspace):
    stats_out float64 [8] GPU tensor <- {K, W, E, Px, Py, Pz, M, 0}."""
    torch = _torch()
    n = _n_of(posmass)
    if _n_of(vel) != n:
        raise ValueError("posmass and vel must have N rows")
    if stats_out.numel() < 8:
        raise ValueError("stats_out needs 8 doubles")
    _check(load_library().nbody_energy_static(_f32(posmass, "posmass", (4,)),
                                              _f32(vel, "vel", (4,)), n, G, eps2,
                                              _dev(stats_out, "stats_out", None, torch.float64),
                                              _stream(stream)),
           "nbody_energy_static")


# ---------------------------------------------------------------------------
# conveniences built only from the entry points above
# ---------------------------------------------------------------------------

def accel(posmass, G: float = 1.0, eps2: float = 1e-4, variant: int | None = None):
    """Allocates and returns float32 [N, 4] accelerations."""
    out = _torch().empty_like(posmass)
    if variant is None:
        nbody_accel(posmass, G, eps2, out)
    else:
        nbody_accel_variant(posmass, G, eps2, out, variant)
    return out


def energy(posmass, vel, G: float = 1.0, eps2: float = 1e-4) -> dict:
    """{K, W, E, Px, Py, Pz, M}; synchronises the current stream to read them."""
    torch = _torch()
    n = _n_of(posmass)
    ws = torch.empty(max(nbody_energy_workspace_bytes(n), 16), dtype=torch.uint8,
                     device=posmass.device)
    stats = torch.zeros(8, dtype=torch.float64, device=posmass.device)
    nbody_energy(posmass, vel, G, eps2, ws, stats)
    vals = stats.cpu().tolist()
    return dict(zip(ENERGY_FIELDS, vals[:7]))


class SymmetricPass:
    """nbody_accel_symmetric with its workspace allocated once, for n bodies:
    ``SymmetricPass(n, device)(posmass, G, eps2, accel_out)``."""

    def __init__(self, n: int, device, variant: int = -1):
        self.n = int(n)
        self.variant = int(variant)
        self.workspace = _torch().empty(
            max(nbody_accel_symmetric_workspace_bytes(self.n, self.variant), 16),
            dtype=_torch().uint8, device=device)

    def __call__(self, posmass, G: float, eps2: float, accel_out, stream=None):
        nbody_accel_symmetric(posmass, G, eps2, accel_out, self.workspace, self.variant, stream)


def kdk_step(posmass, vel, accel_buf, G: float, eps2: float, dt: float, stream=None,
             force=None):
    """One kick-drift-kick step: nbody_leapfrog_step, the force pass at the new
    positions, nbody_kick with dt/2.  accel_buf must hold a(x) on entry and
    holds a(x_new) on return.  force: None for nbody_accel, or a callable
    force(posmass, G, eps2, accel_out, stream) such as a SymmetricPass."""
    nbody_leapfrog_step(posmass, vel, accel_buf, dt, stream)
    if force is None:
        nbody_accel(posmass, G, eps2, accel_buf, stream)
    else:
        force(posmass, G, eps2, accel_buf, stream)
    nbody_kick(vel, accel_buf, 0.5 * dt, stream)
