"""Plant one mistake at a time in a copy of the oracle's C source, build it,
and check that the pin suite rejects it.  Runs on the CPU only; the real
oracle is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "nbody_oracle.c")

# (name, original text, mutated text): each original must occur in the source.
MUTANTS = [
    ("r_ij_sign", "const double rx = pos[3 * j + 0] - xi;", "const double rx = xi - pos[3 * j + 0];"),
    ("drop_eps2", "rz * rz + eps2;\n        const double w", "rz * rz;\n        const double w"),
    ("eps_not_squared", "rz * rz + eps2;\n        const double w", "rz * rz + sqrt(eps2);\n        const double w"),
    ("inverse_cube_to_square", "mass[j] / (d2 * sqrt(d2));", "mass[j] / d2;"),
    ("m_i_for_m_j", "mass[j] / (d2 * sqrt(d2));", "mass[i] / (d2 * sqrt(d2));"),
    ("missing_G", "out[0] = G * ax;", "out[0] = ax;"),
    ("component_swap", "ay += w * ry;", "ay += w * rz;"),
    ("pairs_counted_twice", "for (int64_t j = i + 1; j < n; ++j) {", "for (int64_t j = 0; j < n; ++j) { if (j == i) continue;"),
    ("kinetic_without_half", "K += 0.5 * mass[i]", "K += mass[i]"),
    ("potential_sign", "W *= -G;", "W *= G;"),
    ("single_half_kick", "        oracle_kick(vel, acc, n, 0.5 * dt);\n    }", "    }"),
    ("full_first_kick", "        oracle_kick(vel, acc, n, 0.5 * dt);\n        oracle_drift", "        oracle_kick(vel, acc, n, dt);\n        oracle_drift"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, orig, mut):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for {name} not found"
    bad = tmp_path / "mutant.c"
    bad.write_text(src.replace(orig, mut))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(lib), str(bad), "-lm"], check=True)
    env = dict(os.environ, NBODY_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"
