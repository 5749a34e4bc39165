/*
 * Drives every entry point of the double-precision oracle once, so that the
 * oracle can be built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host (test_oracle_sanitized.py).
 *
 * Bodies come from a fixed integer hash (no part of the method's arithmetic).
 * The checks are light: every output finite, rows equal to the full pass,
 * the N = 2 softened closed form, and Newton's third law.  A non-zero exit
 * code, or a sanitizer report, fails the test.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_num_threads(void);
void oracle_accel(const double *pos, const double *mass, int64_t n, double G, double eps2,
                  double *acc);
void oracle_accel_rows(const double *pos, const double *mass, int64_t n, double G, double eps2,
                       const int64_t *rows, int64_t nrows, double *acc);
void oracle_potential_rows(const double *pos, const double *mass, int64_t n, double G,
                           double eps2, const int64_t *rows, int64_t nrows, double *phi);
void oracle_energy(const double *pos, const double *vel, const double *mass, int64_t n,
                   double G, double eps2, double *out);
void oracle_kick(double *vel, const double *acc, int64_t n, double h);
void oracle_drift(double *pos, const double *vel, int64_t n, double dt);
void oracle_kdk(double *pos, double *vel, const double *mass, int64_t n, double G, double eps2,
                double dt, int64_t nsteps, double *acc);

static double unit(uint32_t k)
{
    /* integer hash to [-1, 1) */
    k ^= k >> 16;
    k *= 0x7feb352dU;
    k ^= k >> 15;
    k *= 0x846ca68bU;
    k ^= k >> 16;
    return (double)(k >> 8) / (double)(1u << 23) - 1.0;
}

static int fail(const char *what, int64_t n)
{
    fprintf(stderr, "FAIL %s (n = %lld)\n", what, (long long)n);
    return 1;
}

static int run(int64_t n)
{
    const size_t m3 = (size_t)(n > 0 ? n : 1) * 3;
    double *pos = malloc(m3 * sizeof(double)), *vel = malloc(m3 * sizeof(double));
    double *acc = malloc(m3 * sizeof(double)), *acc2 = malloc(m3 * sizeof(double));
    double *mass = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *phi = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    int64_t *rows = malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    double e[8];
    int bad = 0;
    if (!pos || !vel || !acc || !acc2 || !mass || !phi || !rows)
        return fail("allocation", n);
    for (int64_t i = 0; i < n; ++i) {
        for (int c = 0; c < 3; ++c) {
            pos[3 * i + c] = unit((uint32_t)(6 * i + c));
            vel[3 * i + c] = 0.1 * unit((uint32_t)(6 * i + 3 + c));
        }
        mass[i] = (1.5 + unit((uint32_t)(7919 * i + 13))) / (double)n;
        rows[i] = n - 1 - i;
    }
    oracle_accel(pos, mass, n, 1.0, 1e-4, acc);
    oracle_accel_rows(pos, mass, n, 1.0, 1e-4, rows, n, acc2);
    oracle_potential_rows(pos, mass, n, 1.0, 1e-4, rows, n, phi);
    oracle_energy(pos, vel, mass, n, 1.0, 1e-4, e);
    double px = 0.0, py = 0.0, pz = 0.0, scale = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t r = rows[i];
        for (int c = 0; c < 3; ++c) {
            if (!isfinite(acc[3 * i + c]))
                bad |= fail("accel finite", n);
            if (acc2[3 * i + c] != acc[3 * r + c])
                bad |= fail("rows equal full pass", n);
        }
        if (!isfinite(phi[i]) || (n > 1 && !(phi[i] < 0.0)))
            bad |= fail("potential finite and negative", n);
        px += mass[i] * acc[3 * i];
        py += mass[i] * acc[3 * i + 1];
        pz += mass[i] * acc[3 * i + 2];
        scale += mass[i] * sqrt(acc[3 * i] * acc[3 * i] + acc[3 * i + 1] * acc[3 * i + 1] +
                                acc[3 * i + 2] * acc[3 * i + 2]);
    }
    if (n > 1 && sqrt(px * px + py * py + pz * pz) > 1e-12 * scale)
        bad |= fail("Newton's third law", n);
    for (int k = 0; k < 8; ++k)
        if (!isfinite(e[k]))
            bad |= fail("energy finite", n);
    oracle_kick(vel, acc, n, 0.5e-3);
    oracle_drift(pos, vel, n, 1e-3);
    oracle_kdk(pos, vel, mass, n, 1.0, 1e-4, 1e-3, 3, acc);
    for (int64_t k = 0; k < 3 * n; ++k)
        if (!isfinite(pos[k]) || !isfinite(vel[k]) || !isfinite(acc[k]))
            bad |= fail("kdk finite", n);
    free(pos);
    free(vel);
    free(acc);
    free(acc2);
    free(mass);
    free(phi);
    free(rows);
    return bad;
}

int main(void)
{
    int bad = 0;
    /* N = 2 at unit distance, eps^2 = 1e-4: a_1 = (1.0001^{-3/2}, 0, 0) */
    double p2[6] = {0, 0, 0, 1, 0, 0}, m2[2] = {1, 1}, a2[6];
    oracle_accel(p2, m2, 2, 1.0, 1e-4, a2);
    if (fabs(a2[0] - 1.0 / pow(1.0001, 1.5)) > 1e-15 || a2[3] != -a2[0] || a2[1] != 0.0)
        bad |= fail("two-body closed form", 2);
    const int64_t sizes[] = {0, 1, 2, 3, 97, 256};
    for (size_t s = 0; s < sizeof(sizes) / sizeof(sizes[0]); ++s)
        bad |= run(sizes[s]);
    printf("oracle driver: %d thread(s), %s\n", oracle_num_threads(), bad ? "FAILED" : "ok");
    return bad;
}
