"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and its pure host logic (status strings, variant table,
workspace sizes, argument validation) behaves as documented.  Nothing here
launches a kernel: every call below is rejected by validation, or is n == 0,
before the library would touch the HIP runtime."""
import ctypes
import os
import re

import pytest

import direct_all_pairs_softened_amd as nb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nbody.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nbody_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return nb.load_library()


def test_header_and_binding_agree():
    assert sorted(nb.EXPORTS) == _declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.nbody_abi_version() == 3
    for code in (0, -1, -2, -3, -4, -5):
        s = nb.status_string(code)
        assert s and s != "unknown status"
    assert nb.status_string(42) == "unknown status"


def test_variant_table(lib):
    count = nb.nbody_accel_variant_count()
    assert count >= 8
    for v in range(count):
        info = nb.nbody_accel_variant_info(v)
        assert info["bodies_per_lane"] in (1, 2, 4, 8)
        assert info["unroll"] in (1, 2, 4, 8)
        assert info["waves_per_block"] % info["split"] == 0
        assert (info["split"] * info["tile"]) % (64 * info["waves_per_block"]) == 0
        assert info["lane_groups"] in (1, 2, 4)
        assert info["tile"] % info["lane_groups"] == 0
        assert info["staging"] == 0 or info["lane_groups"] == 1
    with pytest.raises(nb.NBodyError):
        nb.nbody_accel_variant_info(count)
    for n in (1, 1000, 1024, 16384, 131072, 1 << 20, 1000003, nb.NBODY_MAX_N):
        assert 0 <= nb.nbody_accel_variant_for_n(n) < count


def test_workspace_sizes(lib):
    assert nb.nbody_accel_splitj_workspace_bytes(0, 32) == 0
    assert nb.nbody_accel_splitj_workspace_bytes(100, 31) == 0      # not a multiple of 32
    assert nb.nbody_accel_splitj_workspace_bytes(100, 16) == 0      # below 32
    assert nb.nbody_accel_splitj_workspace_bytes(131072, 32) == 4096 * 131072 * 16
    assert nb.nbody_accel_splitj_workspace_bytes(1000, 256) == 4 * 1000 * 16
    assert nb.nbody_energy_workspace_bytes(0) == 0
    assert nb.nbody_energy_workspace_bytes(-1) == 0
    assert nb.nbody_energy_workspace_bytes(1) >= 64
    assert nb.nbody_energy_workspace_bytes(1 << 20) >= 64 * ((1 << 20) // 256)


# Fake device addresses: validation rejects these calls before anything is
# enqueued or dereferenced.
A = 0x10000000
B = 0x20000000
C = 0x30000000
D = 0x40000000
vp = ctypes.c_void_p


def test_accel_validation(lib):
    f = lib.nbody_accel
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), None) == nb.NBODY_OK              # n == 0: no-op
    assert f(None, 0, 1.0, 1e-4, None, None) == nb.NBODY_OK
    assert f(None, 10, 1.0, 1e-4, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 10, 1.0, 1e-4, None, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), -1, 1.0, 1e-4, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), nb.NBODY_MAX_N + 1, 1.0, 1e-4, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 10, 1.0, 0.0, vp(B), None) == nb.NBODY_ERR_INVALID_ARG   # eps2 == 0
    assert f(vp(A), 10, 1.0, -1e-4, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 10, 1.0, float("nan"), vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 10, float("inf"), 1e-4, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A + 4), 10, 1.0, 1e-4, vp(B), None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), 10, 1.0, 1e-4, vp(B + 8), None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), 10, 1.0, 1e-4, vp(A), None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), 10, 1.0, 1e-4, vp(A + 16 * 9), None) == nb.NBODY_ERR_ALIAS
    g = lib.nbody_accel_variant
    assert g(vp(A), 10, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert g(vp(A), 10, 1.0, 1e-4, vp(B), 10 ** 6, None) == nb.NBODY_ERR_INVALID_ARG


def test_layout_variants_validation(lib):
    f3 = lib.nbody_accel_f3aos
    assert f3(vp(A), vp(B), 0, 1.0, 1e-4, vp(C), None) == nb.NBODY_OK
    assert f3(vp(A), None, 10, 1.0, 1e-4, vp(C), None) == nb.NBODY_ERR_INVALID_ARG
    assert f3(vp(A + 2), vp(B), 10, 1.0, 1e-4, vp(C), None) == nb.NBODY_ERR_ALIGNMENT
    assert f3(vp(A), vp(B), 10, 1.0, 1e-4, vp(A + 12), None) == nb.NBODY_ERR_ALIAS
    assert f3(vp(A), vp(B), 10, 1.0, 1e-4, vp(B - 8), None) == nb.NBODY_ERR_ALIAS
    soa = lib.nbody_accel_soa
    ptrs = [vp(A + k * 0x1000) for k in range(7)]
    assert soa(*ptrs[:4], 0, 1.0, 1e-4, *ptrs[4:], None) == nb.NBODY_OK
    bad = list(ptrs)
    bad[5] = None
    assert soa(*bad[:4], 10, 1.0, 1e-4, *bad[4:], None) == nb.NBODY_ERR_INVALID_ARG
    bad = list(ptrs)
    bad[6] = ptrs[0]
    assert soa(*bad[:4], 10, 1.0, 1e-4, *bad[4:], None) == nb.NBODY_ERR_ALIAS
    bad = list(ptrs)
    bad[5] = ptrs[4]
    assert soa(*bad[:4], 10, 1.0, 1e-4, *bad[4:], None) == nb.NBODY_ERR_ALIAS
    bad = list(ptrs)
    bad[2] = vp(A + 0x2001)
    assert soa(*bad[:4], 10, 1.0, 1e-4, *bad[4:], None) == nb.NBODY_ERR_ALIGNMENT


def test_splitj_validation(lib):
    f = lib.nbody_accel_splitj
    need = nb.nbody_accel_splitj_workspace_bytes(1000, 256)
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 48, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 16, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 256, None, need, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 256, vp(C), need - 1, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 256, vp(C + 8), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 256, vp(A), need, None) == nb.NBODY_ERR_ALIAS
    # more than 65535 chunks
    assert f(vp(A), 32 * 70000, 1.0, 1e-4, vp(B), 32, vp(C), 1 << 62, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), 32, None, 0, None) == nb.NBODY_OK


def test_splitj_tree_shapes_and_validation(lib):
    ws = nb.nbody_accel_splitj_tree_workspace_bytes
    # the README's 32-wide block: plain tree, FADL and fadl4
    for terms in (1, 2, 4):
        assert ws(131072, 32, terms) == 4096 * 131072 * 16
    assert ws(1000, 256, 4) == 4 * 1000 * 16          # X = 64
    assert ws(1000, 8, 1) == 125 * 1000 * 16          # X = 8
    assert ws(1000, 4, 1) == 0                        # X = 4 below the smallest tree
    assert ws(1000, 128, 1) == 0                      # X = 128 wider than a wavefront
    assert ws(1000, 48, 2) == 0                       # X = 24 not a power of two
    assert ws(1000, 32, 3) == 0                       # terms not 1, 2 or 4
    assert ws(0, 32, 1) == 0
    f = lib.nbody_accel_splitj_tree
    need = ws(1000, 32, 2)
    ok = (vp(A), 1000, 1.0, 1e-4, vp(B), 32, 2, vp(C), need, None)

    def call(**kw):
        names = ("pm", "n", "G", "eps2", "out", "chunk", "terms", "ws", "bytes", "stream")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[k] for k in names])

    assert call(terms=3) == nb.NBODY_ERR_INVALID_ARG
    assert call(chunk=48) == nb.NBODY_ERR_INVALID_ARG
    assert call(chunk=256, terms=1) == nb.NBODY_ERR_INVALID_ARG
    assert call(eps2=0.0) == nb.NBODY_ERR_INVALID_ARG
    assert call(pm=None) == nb.NBODY_ERR_INVALID_ARG
    assert call(ws=None) == nb.NBODY_ERR_WORKSPACE
    assert call(bytes=need - 1) == nb.NBODY_ERR_WORKSPACE
    assert call(ws=vp(C + 8)) == nb.NBODY_ERR_ALIGNMENT
    assert call(out=vp(B + 4)) == nb.NBODY_ERR_ALIGNMENT
    assert call(ws=vp(A)) == nb.NBODY_ERR_ALIAS
    assert call(out=vp(A + 16)) == nb.NBODY_ERR_ALIAS
    # more than 65535 chunks
    assert call(n=32 * 70000, bytes=1 << 62) == nb.NBODY_ERR_INVALID_ARG
    assert call(n=0, pm=None, out=None, ws=None, bytes=0) == nb.NBODY_OK


def test_integrator_validation(lib):
    lf = lib.nbody_leapfrog_step
    assert lf(vp(A), vp(B), vp(C), 1e-3, 0, None) == nb.NBODY_OK
    assert lf(vp(A), vp(B), vp(C), float("nan"), 10, None) == nb.NBODY_ERR_INVALID_ARG
    assert lf(vp(A), None, vp(C), 1e-3, 10, None) == nb.NBODY_ERR_INVALID_ARG
    assert lf(vp(A), vp(B + 4), vp(C), 1e-3, 10, None) == nb.NBODY_ERR_ALIGNMENT
    assert lf(vp(A), vp(A + 16), vp(C), 1e-3, 10, None) == nb.NBODY_ERR_ALIAS
    assert lf(vp(A), vp(B), vp(B), 1e-3, 10, None) == nb.NBODY_ERR_ALIAS
    k = lib.nbody_kick
    assert k(vp(A), vp(B), 5e-4, 0, None) == nb.NBODY_OK
    assert k(vp(A), vp(A), 5e-4, 10, None) == nb.NBODY_ERR_ALIAS
    assert k(vp(A), vp(B), float("inf"), 10, None) == nb.NBODY_ERR_INVALID_ARG


def test_energy_validation(lib):
    e = lib.nbody_energy
    need = nb.nbody_energy_workspace_bytes(1000)
    assert e(vp(A), vp(B), 0, 1.0, 1e-4, None, 0, None, None) == nb.NBODY_OK
    assert e(vp(A), vp(B), 1000, 1.0, 1e-4, vp(C), need, None, None) == nb.NBODY_ERR_INVALID_ARG
    assert e(vp(A), vp(B), 1000, 1.0, 1e-4, vp(C), need - 8, vp(D), None) == nb.NBODY_ERR_WORKSPACE
    assert e(vp(A), vp(B), 1000, 1.0, 1e-4, vp(C), need, vp(D + 4), None) == nb.NBODY_ERR_ALIGNMENT
    assert e(vp(A), vp(B), 1000, 1.0, 0.0, vp(C), need, vp(D), None) == nb.NBODY_ERR_INVALID_ARG
    assert e(vp(A), vp(B), 1000, 1.0, 1e-4, vp(A), need, vp(D), None) == nb.NBODY_ERR_ALIAS
    assert e(vp(A), vp(B), 1000, 1.0, 1e-4, vp(C), need, vp(B + 64), None) == nb.NBODY_ERR_ALIAS


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    pm = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        nb.nbody_accel(pm, 1.0, 1e-4, torch.zeros(4, 4))


def test_symmetric_host_side(lib):
    count = nb.nbody_accel_symmetric_variant_count()
    assert count >= 1
    for v in range(count):
        panel = nb.nbody_accel_symmetric_panel(v)
        assert panel > 0 and panel % 64 == 0
        P = -(-1000 // panel)
        assert nb.nbody_accel_symmetric_workspace_bytes(1000, v) == P * P * 3 * panel * 4
    assert nb.nbody_accel_symmetric_panel(count) == nb.NBODY_ERR_INVALID_ARG
    assert nb.nbody_accel_symmetric_workspace_bytes(0, 0) == 0
    assert nb.nbody_accel_symmetric_workspace_bytes(1000, count) == 0
    f = lib.nbody_accel_symmetric
    need = nb.nbody_accel_symmetric_workspace_bytes(1000, 0)
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), 0, None, 0, None) == nb.NBODY_OK
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), count, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 0.0, vp(B), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, vp(C), need - 4, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, None, need, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, vp(C + 4), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), 1000, 1.0, 1e-4, vp(A), 0, vp(C), need, None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, vp(B - 64), need, None) == nb.NBODY_ERR_ALIAS
    # more panel pairs than a grid holds
    assert f(vp(A), nb.NBODY_MAX_N, 1.0, 1e-4, vp(B), 0, vp(C), 1 << 62, None) == nb.NBODY_ERR_INVALID_ARG


def test_symmetric_two_phase_host_side(lib):
    """The two phases of the pair-symmetric pass check what each touches:
    the tasks phase posmass, eps2 and the workspace, the reduce G, accel_out
    and the workspace."""
    count = nb.nbody_accel_symmetric_variant_count()
    need = nb.nbody_accel_symmetric_workspace_bytes(1000, 0)
    t = lib.nbody_accel_symmetric_tasks
    assert t(vp(A), 0, 1e-4, 0, None, 0, None) == nb.NBODY_OK
    assert t(vp(A), -1, 1e-4, 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert t(vp(A), 1000, 1e-4, count, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert t(vp(A), 1000, 0.0, 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert t(vp(A), 1000, float("nan"), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert t(None, 1000, 1e-4, 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert t(vp(A + 4), 1000, 1e-4, 0, vp(C), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert t(vp(A), 1000, 1e-4, 0, vp(C), need - 4, None) == nb.NBODY_ERR_WORKSPACE
    assert t(vp(A), 1000, 1e-4, 0, vp(C + 4), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert t(vp(A), 1000, 1e-4, 0, vp(A - 64), need, None) == nb.NBODY_ERR_ALIAS
    r = lib.nbody_accel_symmetric_reduce
    assert r(0, 1.0, vp(B), 0, None, 0, None) == nb.NBODY_OK
    assert r(1000, float("inf"), vp(B), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert r(1000, 1.0, vp(B), count, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert r(1000, 1.0, None, 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert r(1000, 1.0, vp(B + 8), 0, vp(C), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert r(1000, 1.0, vp(B), 0, None, need, None) == nb.NBODY_ERR_WORKSPACE
    assert r(1000, 1.0, vp(B), 0, vp(C), need - 4, None) == nb.NBODY_ERR_WORKSPACE
    assert r(1000, 1.0, vp(B), 0, vp(B - 64), need, None) == nb.NBODY_ERR_ALIAS
    # the library's choice of variant for n when passed -1
    assert t(vp(A), 1000, 0.0, -1, vp(C), 1 << 40, None) == nb.NBODY_ERR_INVALID_ARG


def test_symmetric_potential_host_side(lib):
    count = nb.nbody_accel_symmetric_potential_variant_count()
    assert count >= 1
    for v in range(count):
        panel = nb.nbody_accel_symmetric_potential_panel(v)
        assert panel > 0 and panel % 64 == 0
        P = -(-1000 // panel)
        assert nb.nbody_accel_symmetric_potential_workspace_bytes(1000, v) == P * P * 4 * panel * 4
    for n in (1, 1000, 1 << 20):
        assert 0 <= nb.nbody_accel_symmetric_potential_variant_for_n(n) < count
    assert nb.nbody_accel_symmetric_potential_panel(count) == nb.NBODY_ERR_INVALID_ARG
    assert nb.nbody_accel_symmetric_potential_panel(-1) == nb.NBODY_ERR_INVALID_ARG
    assert nb.nbody_accel_symmetric_potential_workspace_bytes(0, 0) == 0
    assert nb.nbody_accel_symmetric_potential_workspace_bytes(1000, count) == 0
    assert (nb.nbody_accel_symmetric_potential_workspace_bytes(1000, -1)
            == nb.nbody_accel_symmetric_potential_workspace_bytes(
                1000, nb.nbody_accel_symmetric_potential_variant_for_n(1000)))
    f = lib.nbody_accel_symmetric_potential
    need = nb.nbody_accel_symmetric_potential_workspace_bytes(1000, 0)
    # the plain pass's workspace is too small for the potential pass
    assert nb.nbody_accel_symmetric_workspace_bytes(1000, 8) < need
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), 0, None, 0, None) == nb.NBODY_OK
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), count, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, float("nan"), 1e-4, vp(B), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, -1e-4, vp(B), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(None, 1000, 1.0, 1e-4, vp(B), 0, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, vp(C), need - 4, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, None, need, None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B + 8), 0, vp(C), need, None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), 1000, 1.0, 1e-4, vp(A + 16), 0, vp(C), need, None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), 0, vp(A + 64), need, None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), nb.NBODY_MAX_N, 1.0, 1e-4, vp(B), 0, vp(C), 1 << 62, None) == nb.NBODY_ERR_INVALID_ARG


def test_range_validation(lib):
    f = lib.nbody_accel_range
    assert f(vp(A), 100, 0, 0, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_OK          # empty share
    assert f(vp(A), 100, 100, 0, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_OK
    assert f(vp(A), 100, -1, 10, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 0, -1, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 95, 6, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 101, 0, 1.0, 1e-4, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 0, 10, 1.0, 1e-4, vp(B), 10 ** 6, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 0, 10, 1.0, 0.0, vp(B), -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 0, 10, 1.0, 1e-4, None, -1, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 100, 0, 10, 1.0, 1e-4, vp(B + 4), -1, None) == nb.NBODY_ERR_ALIGNMENT
    # the output may not overlap any of the n input rows, even outside the share
    assert f(vp(A), 100, 0, 10, 1.0, 1e-4, vp(A + 16 * 50), -1, None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), 100, 0, 10, 1.0, 1e-4, vp(A - 16 * 5), -1, None) == nb.NBODY_ERR_ALIAS


def test_potential_and_energy_from_potential_validation(lib):
    f = lib.nbody_accel_potential
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), None) == nb.NBODY_OK
    assert f(vp(A), 10, 1.0, 0.0, vp(B), None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 10, 1.0, 1e-4, vp(A), None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A + 8), 10, 1.0, 1e-4, vp(B), None) == nb.NBODY_ERR_ALIGNMENT
    e = lib.nbody_energy_from_potential
    need = nb.nbody_energy_from_potential_workspace_bytes(1000)
    assert need == 4 * 8 * 8
    assert e(vp(A), vp(B), vp(C), 0, None, 0, None, None) == nb.NBODY_OK
    assert e(vp(A), vp(B), None, 1000, vp(D), need, vp(D + need), None) == nb.NBODY_ERR_INVALID_ARG
    assert e(vp(A), vp(B), vp(C), 1000, vp(D), need - 1, vp(D + need), None) == nb.NBODY_ERR_WORKSPACE
    assert e(vp(A), vp(B), vp(C), 1000, vp(D), need, vp(D + need + 4), None) == nb.NBODY_ERR_ALIGNMENT
    assert e(vp(A), vp(B), vp(C), 1000, vp(C + 16), need, vp(D), None) == nb.NBODY_ERR_ALIAS
    assert e(vp(A), vp(B), vp(C), 1000, vp(D), need, vp(D + 8), None) == nb.NBODY_ERR_ALIAS


def test_timing_validation(lib):
    """nbody_time_accel and the timer calls reject bad arguments before they
    create an event or touch the stream."""
    f = lib.nbody_time_accel
    ms = (ctypes.c_float * 4)()
    INV = nb.NBODY_ERR_INVALID_ARG
    one, sym = nb.NBODY_PASS_ONE_SIDED, nb.NBODY_PASS_SYMMETRIC

    def call(n=10, G=1.0, eps2=1e-4, out=B, kind=one, v=-1, ws=None, wsb=0, reps=4, pms=ms):
        return f(vp(A), n, G, eps2, vp(out), kind, v, ws, wsb, reps, pms, None, None)

    assert call(n=0) == INV                       # nothing to time
    assert call(reps=0) == INV
    assert call(reps=(1 << 16) + 1) == INV
    assert call(kind=4) == INV
    assert call(kind=-1) == INV
    assert call(pms=None) == INV
    assert call(eps2=0.0) == INV                  # the pass's own checks
    assert call(v=10 ** 6) == INV
    assert call(out=A) == nb.NBODY_ERR_ALIAS
    assert call(out=B + 8) == nb.NBODY_ERR_ALIGNMENT
    assert call(kind=sym) == nb.NBODY_ERR_WORKSPACE
    need = nb.nbody_accel_symmetric_workspace_bytes(10)
    assert call(kind=sym, ws=vp(C), wsb=need - 1) == nb.NBODY_ERR_WORKSPACE
    assert call(kind=sym, ws=vp(A), wsb=need) == nb.NBODY_ERR_ALIAS
    chk = nb.NBODY_PASS_SYMMETRIC_CHUNKED
    need_c = nb.nbody_accel_symmetric_chunked_workspace_bytes(10, -1, 0)
    assert call(kind=chk) == nb.NBODY_ERR_WORKSPACE
    assert call(kind=chk, ws=vp(C), wsb=need_c - 1) == nb.NBODY_ERR_WORKSPACE
    assert call(kind=chk, ws=vp(B), wsb=need_c) == nb.NBODY_ERR_ALIAS
    t = vp()
    assert lib.nbody_timer_create(0, ctypes.byref(t)) == INV
    assert lib.nbody_timer_create((1 << 20) + 1, ctypes.byref(t)) == INV
    assert lib.nbody_timer_create(4, None) == INV
    assert lib.nbody_timer_mark(None, 0, None) == INV
    out = ctypes.c_float()
    assert lib.nbody_timer_elapsed_ms(None, 0, 1, ctypes.byref(out)) == INV
    assert lib.nbody_timer_destroy(None) == nb.NBODY_OK


def test_energy_static_validation(lib):
    """The allocation-free energy entry point checks its arguments, and that
    n fits its static scratch, before it looks up the scratch's address."""
    f = lib.nbody_energy_static
    INV = nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), vp(B), 0, 1.0, 1e-4, vp(C), None) == nb.NBODY_OK        # n == 0: no-op
    assert f(None, vp(B), 10, 1.0, 1e-4, vp(C), None) == INV
    assert f(vp(A), vp(B), 10, 1.0, 1e-4, None, None) == INV
    assert f(vp(A), vp(B), 10, 1.0, 0.0, vp(C), None) == INV
    assert f(vp(A), vp(B), -1, 1.0, 1e-4, vp(C), None) == INV
    assert f(vp(A + 4), vp(B), 10, 1.0, 1e-4, vp(C), None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), vp(B), 10, 1.0, 1e-4, vp(C + 4), None) == nb.NBODY_ERR_ALIGNMENT
    assert f(vp(A), vp(B), 10, 1.0, 1e-4, vp(A + 32), None) == nb.NBODY_ERR_ALIAS
    nmax = 4_063_232
    assert nb.nbody_energy_workspace_bytes(nmax) <= nb.NBODY_ENERGY_STATIC_SCRATCH_BYTES
    assert nb.nbody_energy_workspace_bytes(nmax + 1) > nb.NBODY_ENERGY_STATIC_SCRATCH_BYTES
    assert f(vp(A), vp(B), nmax + 1, 1.0, 1e-4, vp(C), None) == nb.NBODY_ERR_WORKSPACE
    assert f(vp(A), vp(B), 10 ** 7, 1.0, 1e-4, vp(C), None) == nb.NBODY_ERR_WORKSPACE


def test_symmetric_chunked_sizes_and_validation(lib):
    """Chunked workspace: one chunk's slots (the largest chunk is the last
    full one), far below the whole pass's at 10^6 bodies; bad chunk widths and
    short workspaces are rejected before anything is enqueued."""
    n = 1 << 20
    panel, P = 2048, 512
    v = nb.nbody_accel_symmetric_variant_for_n(n)
    assert nb.nbody_accel_symmetric_panel(v) == panel
    # two buffers of the largest chunk: the last one, where panels 480..511
    # take all J < 512 and panels 0..479 take 32 each
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, 32) == (
        2 * (480 * 32 + 32 * 512) * 3 * panel * 4)
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, 0) == (
        nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, 32))
    # one chunk covering every panel: one buffer, the whole pass's slots
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, P) == (
        nb.nbody_accel_symmetric_workspace_bytes(n, v))
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, 31) == 0
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(n, v, -32) == 0
    assert nb.nbody_accel_symmetric_chunked_workspace_bytes(0, v, 32) == 0
    f = lib.nbody_accel_symmetric_chunked
    need = nb.nbody_accel_symmetric_chunked_workspace_bytes(1000, -1, 32)
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), -1, 48, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(B), -1, 32, vp(C), need - 1, None) == (
        nb.NBODY_ERR_WORKSPACE)
    assert f(vp(A), 1000, 1.0, 0.0, vp(B), -1, 32, vp(C), need, None) == nb.NBODY_ERR_INVALID_ARG
    assert f(vp(A), 1000, 1.0, 1e-4, vp(A), -1, 32, vp(C), need, None) == nb.NBODY_ERR_ALIAS
    assert f(vp(A), 0, 1.0, 1e-4, vp(B), -1, 32, None, 0, None) == nb.NBODY_OK


def test_kdk_run_validation(lib):
    """nbody_kdk_run checks its steps, dt and pass, the force pass's own
    arguments and vel before it launches anything; steps == 0 and n == 0 are
    no-ops."""
    f = lib.nbody_kdk_run
    INV = nb.NBODY_ERR_INVALID_ARG
    one, sym = nb.NBODY_PASS_ONE_SIDED, nb.NBODY_PASS_SYMMETRIC
    V = A + (1 << 20)

    def call(n=10, vel=V, dt=1e-3, steps=3, kind=one, ws=None, wsb=0, pm=A, acc=B):
        return f(vp(pm), vp(vel), vp(acc), n, 1.0, 1e-4, dt, steps, kind, -1, ws, wsb, None)

    assert call(steps=-1) == INV
    assert call(dt=float("nan")) == INV
    assert call(dt=float("inf")) == INV
    assert call(kind=4) == INV
    assert call(n=0) == nb.NBODY_OK
    assert call(steps=0) == nb.NBODY_OK
    assert call(vel=0) == INV
    assert call(vel=V + 4) == nb.NBODY_ERR_ALIGNMENT
    assert call(vel=A) == nb.NBODY_ERR_ALIAS
    assert call(vel=B + 32) == nb.NBODY_ERR_ALIAS
    assert call(acc=A) == nb.NBODY_ERR_ALIAS               # the force pass's own checks
    assert call(kind=sym) == nb.NBODY_ERR_WORKSPACE
    need = nb.nbody_accel_symmetric_workspace_bytes(10)
    assert call(kind=sym, ws=vp(C), wsb=need, vel=C + 16) == nb.NBODY_ERR_ALIAS
    chk = nb.NBODY_PASS_SYMMETRIC_CHUNKED
    need_c = nb.nbody_accel_symmetric_chunked_workspace_bytes(10, -1, 0)
    assert call(kind=chk) == nb.NBODY_ERR_WORKSPACE
    assert call(kind=chk, ws=vp(C), wsb=need_c - 1) == nb.NBODY_ERR_WORKSPACE
    assert call(kind=chk, ws=vp(C), wsb=need_c, vel=C + 16) == nb.NBODY_ERR_ALIAS


def test_launch_block_cap_validation(lib):
    """nbody_set_launch_block_cap takes a non-negative block count (0 restores
    the hardware limit) and touches no GPU state."""
    assert lib.nbody_set_launch_block_cap(-1) == nb.NBODY_ERR_INVALID_ARG
    assert lib.nbody_set_launch_block_cap(5) == nb.NBODY_OK
    assert lib.nbody_set_launch_block_cap(0) == nb.NBODY_OK
    with pytest.raises(nb.NBodyError):
        nb.nbody_set_launch_block_cap(-7)


@pytest.mark.skipif(__import__("shutil").which("gcc") is None, reason="needs gcc")
def test_plain_c_client(lib, tmp_path):
    """include/nbody.h compiles as strict C99 (gcc -pedantic -Werror), and a
    C program linked against libnbody.so gets the documented answers from
    the calls that need no GPU (tests/abi_c_client.c)."""
    import subprocess
    pkg = os.path.dirname(os.path.abspath(nb.__file__))
    exe = str(tmp_path / "abi_c_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_c_client.c"),
           "-L", pkg, "-lnbody", f"-Wl,-rpath,{pkg}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_binding_rejects_host_tensors_and_non_tensors():
    """The binding only marshals device tensors: a host tensor or a numpy
    array is refused before anything reaches the library (there is no CPU
    path to fall back on)."""
    import numpy as np
    import torch
    pm = torch.zeros((8, 4), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        nb.nbody_accel(pm, 1.0, 1e-4, torch.zeros_like(pm))
    with pytest.raises(TypeError, match="torch tensor"):
        nb.nbody_accel(np.zeros((8, 4), np.float32), 1.0, 1e-4, np.zeros((8, 4), np.float32))
