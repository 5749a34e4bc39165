/*
 * Double-precision CPU oracle for direct all-pairs softened gravity.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
 * the bench's CPU-baseline leg may load this library.  It shares no code,
 * header, constant or helper with the HIP library; it is plain C99 built by
 * gcc without -ffast-math, and every quantity is a double.  The float32
 * inputs of the GPU path are promoted exactly to double before they get here.
 *
 * Layout: pos and vel are double[n][3] (x, y, z), mass is double[n].
 *
 * What it computes (the pages' definitions, written out):
 *
 *  - acceleration: "CUDA N-Body Simulation" (LienoPC/N-BodySimulation README),
 *    sections 1.1 and 1.2: a_i = G * sum_{j != i} m_j r_ij / (|r_ij|^2 + eps^2)^{3/2}
 *    with r_ij = x_j - x_i.  The j = i term is skipped, as the README's OpenMP
 *    reference (section 5.1, CPU_compute) skips it; for eps^2 > 0 it is zero
 *    anyway (section 1.2, last paragraph).  "eps2" below is eps^2, the
 *    squared softening length (EPS2 in the README's constants table, 6.1).
 *    G is applied once per body after the j-sum (identical in exact
 *    arithmetic to applying it per pair).
 *  - kick / drift: section 1.3 of the same README: v += (dt/2) a, then
 *    x += dt v.  The closing half-kick with the new acceleration, which turns
 *    the printed scheme into kick-drift-kick leapfrog, is this project's
 *    reading (the README states only the first two updates).
 *  - energy: not printed on any page; the softened pair potential whose
 *    negative gradient is the acceleration above, pairs counted once:
 *    W = -G sum_{i<j} m_i m_j / sqrt(|x_i - x_j|^2 + eps^2), K = sum m |v|^2 / 2.
 *
 * Every loop runs j in ascending order; OpenMP only splits the outer i loop,
 * and every reduction over i is serial in ascending i afterwards, so results
 * do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One body's acceleration: the j-sum of README section 1.2 for body i,
 * excluding j == i, times G. */
static void accel_one(const double *pos, const double *mass, int64_t n,
                      double G, double eps2, int64_t i, double out[3])
{
    const double xi = pos[3 * i + 0];
    const double yi = pos[3 * i + 1];
    const double zi = pos[3 * i + 2];
    double ax = 0.0, ay = 0.0, az = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (j == i)
            continue;
        const double rx = pos[3 * j + 0] - xi;   /* r_ij = x_j - x_i */
        const double ry = pos[3 * j + 1] - yi;
        const double rz = pos[3 * j + 2] - zi;
        const double d2 = rx * rx + ry * ry + rz * rz + eps2;
        const double w = mass[j] / (d2 * sqrt(d2)); /* m_j / (r^2+eps^2)^{3/2} */
        ax += w * rx;
        ay += w * ry;
        az += w * rz;
    }
    out[0] = G * ax;
    out[1] = G * ay;
    out[2] = G * az;
}

/* All n accelerations, acc = double[n][3]. */
void oracle_accel(const double *pos, const double *mass, int64_t n,
                  double G, double eps2, double *acc)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        accel_one(pos, mass, n, G, eps2, i, acc + 3 * i);
}

/* Accelerations of the listed bodies only, acc = double[nrows][3]; each row is
 * the full j-sum over all n bodies.  Used to check samples of very large
 * inputs one body at a time. */
void oracle_accel_rows(const double *pos, const double *mass, int64_t n,
                       double G, double eps2, const int64_t *rows,
                       int64_t nrows, double *acc)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r)
        accel_one(pos, mass, n, G, eps2, rows[r], acc + 3 * r);
}

/* Potential of the listed bodies: phi_i = -G sum_{j != i} m_j / sqrt(r^2+eps^2). */
void oracle_potential_rows(const double *pos, const double *mass, int64_t n,
                           double G, double eps2, const int64_t *rows,
                           int64_t nrows, double *phi)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        double s = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (j == i)
                continue;
            const double rx = pos[3 * j + 0] - pos[3 * i + 0];
            const double ry = pos[3 * j + 1] - pos[3 * i + 1];
            const double rz = pos[3 * j + 2] - pos[3 * i + 2];
            s += mass[j] / sqrt(rx * rx + ry * ry + rz * rz + eps2);
        }
        phi[r] = -G * s;
    }
}

/* Energy and momentum: out = {K, W, K + W, Px, Py, Pz, M, 0}.
 * W sums each unordered pair once: row i holds sum_{j > i}. */
void oracle_energy(const double *pos, const double *vel, const double *mass,
                   int64_t n, double G, double eps2, double *out)
{
    double *row = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = i + 1; j < n; ++j) {
            const double rx = pos[3 * j + 0] - pos[3 * i + 0];
            const double ry = pos[3 * j + 1] - pos[3 * i + 1];
            const double rz = pos[3 * j + 2] - pos[3 * i + 2];
            s += mass[j] / sqrt(rx * rx + ry * ry + rz * rz + eps2);
        }
        row[i] = mass[i] * s;
    }
    double K = 0.0, W = 0.0, px = 0.0, py = 0.0, pz = 0.0, M = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double vx = vel[3 * i + 0], vy = vel[3 * i + 1], vz = vel[3 * i + 2];
        K += 0.5 * mass[i] * (vx * vx + vy * vy + vz * vz);
        W += row[i];
        px += mass[i] * vx;
        py += mass[i] * vy;
        pz += mass[i] * vz;
        M += mass[i];
    }
    free(row);
    W *= -G;
    out[0] = K;
    out[1] = W;
    out[2] = K + W;
    out[3] = px;
    out[4] = py;
    out[5] = pz;
    out[6] = M;
    out[7] = 0.0;
}

/* Velocity kick v += h * a (README section 1.3 with h = dt/2). */
void oracle_kick(double *vel, const double *acc, int64_t n, double h)
{
    for (int64_t k = 0; k < 3 * n; ++k)
        vel[k] += h * acc[k];
}

/* Position drift x += dt * v (README section 1.3, position full step). */
void oracle_drift(double *pos, const double *vel, int64_t n, double dt)
{
    for (int64_t k = 0; k < 3 * n; ++k)
        pos[k] += dt * vel[k];
}

/* nsteps of kick-drift-kick leapfrog, in place.  acc is double[n][3] scratch
 * owned by the caller; on return it holds a(x) at the final positions.
 * Per step: v += dt/2 a(x); x += dt v; a = a(x); v += dt/2 a. */
void oracle_kdk(double *pos, double *vel, const double *mass, int64_t n,
                double G, double eps2, double dt, int64_t nsteps, double *acc)
{
    oracle_accel(pos, mass, n, G, eps2, acc);
    for (int64_t s = 0; s < nsteps; ++s) {
        oracle_kick(vel, acc, n, 0.5 * dt);
        oracle_drift(pos, vel, n, dt);
        oracle_accel(pos, mass, n, G, eps2, acc);
        oracle_kick(vel, acc, n, 0.5 * dt);
    }
}
